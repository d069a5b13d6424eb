"""MXFP4 activations (fp4_quant_rows) and the MXFP4 x MXFP4 GEMM
(gemm_mxfp4_w4a4) on the GPU against the oracle: quantizer codes and scales
bit-exact; GEMM outputs within |y - ref| <= 2^-8 |ref| + 1e-4 sum|a w|
through the split-K decode path (every M <= 64) and the prefill kernel's
three tile shapes, each epilogue, padded strides, and the gate_up workload
at full size."""
import numpy as np
import pytest
import torch

import mxfp4_gemm_transformer_amd as bs
import oracle
import synth
from gpu_util import DEV, assert_within, bf16_dev, u8_dev, y_host

pytestmark = pytest.mark.gpu


def _quant_check(x_bits, pad=0):
    M, K = x_bits.shape
    if pad:
        full = np.zeros((M, K + pad), np.uint16)
        full[:, :K] = x_bits
        x = bf16_dev(full)[:, :K]
        qf = torch.full((M, K // 2 + pad), 0xAA, dtype=torch.uint8, device=DEV)
        q, s = bs.fp4_quant_rows(x, q=qf[:, :K // 2])
    else:
        q, s = bs.fp4_quant_rows(bf16_dev(x_bits))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_mxfp4_rows(x_bits)
    assert np.array_equal(s.cpu().numpy(), s_ref), "scales"
    qh = q.cpu().numpy()
    if not np.array_equal(qh, q_ref):
        bad = np.argwhere(qh != q_ref)
        m, k = bad[0]
        raise AssertionError("%d bytes differ; first (%d, %d): got %#x want %#x"
                             % (len(bad), m, k, qh[m, k], q_ref[m, k]))
    if pad:
        assert torch.all(qf[:, K // 2:] == 0xAA)


@pytest.mark.parametrize("M,K", [(1, 32), (7, 96), (64, 5120), (513, 2080), (4096, 5120)])
def test_fp4_quant_shapes(M, K):
    rng = np.random.default_rng(M + K)
    _quant_check(synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)))


def test_fp4_quant_ties_special_blocks_and_padding():
    K = 256
    grid = np.array([0, .25, .5, .75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 7], np.float32)
    rows = []
    for X in (-3, 0, 5):                             # every threshold, scaled by 2^X
        r = np.tile(np.concatenate([grid, -grid]), K // 32) * np.float32(2.0 ** X)
        r[::32] = 6.0 * 2.0 ** X                     # amax 6 * 2^X: block exponent X
        rows.append(r)
    rows.append(np.zeros(K, np.float32))             # zero blocks
    rows.append(np.full(K, -0.0, np.float32))
    rows.append(np.full(K, 1e-40, np.float32))       # subnormal amax
    rows.append(np.full(K, 3e38, np.float32))        # top of the range
    x = synth.to_bf16_bits(np.stack(rows))
    _quant_check(x)
    _quant_check(x, pad=48)


def _problem(M, N, K, seed):
    rng = np.random.default_rng(seed)
    a, sa = oracle.quant_mxfp4_rows(synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)))
    w, sw = oracle.quant_mxfp4_weights((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    b = synth.to_bf16_bits((rng.standard_normal(N) * 0.1).astype(np.float32))
    return a, sa, w, sw, b


def _run(a, sa, w, sw, b, epi, pad=0):
    M, K2 = a.shape
    N = w.shape[0]
    if pad:
        af = np.zeros((M, K2 + pad), np.uint8); af[:, :K2] = a
        wf = np.zeros((N, K2 + pad), np.uint8); wf[:, :K2] = w
        a_t, w_t = u8_dev(af)[:, :K2], u8_dev(wf)[:, :K2]
        y = torch.full((M, N + pad), float("nan"), dtype=torch.bfloat16, device=DEV)[:, :N]
    else:
        a_t, w_t, y = u8_dev(a), u8_dev(w), None
    out = bs.gemm_mxfp4_w4a4(a_t, u8_dev(sa), w_t, u8_dev(sw), bf16_dev(b) if epi else None, epi, y=y)
    return y_host(out)


@pytest.mark.parametrize("M,N,K", [
    (1, 96, 1056), (5, 2048, 512), (16, 32768 + 32, 640), (40, 2080, 1184), (64, 512, 4096),
    (65, 256, 128), (200, 320, 512), (300, 4192, 256), (513, 1024, 2048), (260, 35 * 256, 1024),
    (130, 96, 5120), (70, 160, 5248), (97, 160, 1088)])   # E8M0 rows in LDS up to K = 5120
@pytest.mark.parametrize("epi", [synth.EPI_NONE, synth.EPI_BIAS_GELU_TANH])
def test_w4a4_shapes(M, N, K, epi):
    a, sa, w, sw, b = _problem(M, N, K, seed=M + N + K + epi)
    got = _run(a, sa, w, sw, b, epi)
    ref, absum = oracle.gemm_mxfp4_w4a4(a, sa, w, sw, b if epi else None, epi)
    assert_within(got, ref, absum, "w4a4 M=%d N=%d K=%d epi=%d" % (M, N, K, epi))


# wide layers with M <= 16 (at least two 8-row groups per CU): the balanced
# decode kernel with fp4 activations and their scale rows staged in LDS;
# ragged M, one to 32 K steps, the epilogues
@pytest.mark.parametrize("M,N,K,epi", [
    (1, 4096, 1024, synth.EPI_NONE), (5, 4160, 5120, synth.EPI_BIAS_GELU_TANH),
    (9, 8192, 8192, synth.EPI_NONE), (13, 4096, 2048, synth.EPI_BIAS),
    (16, 6144, 5120, synth.EPI_BIAS_GELU_TANH), (16, 4096, 128, synth.EPI_NONE)])
def test_w4a4_wide_decode(M, N, K, epi):
    a, sa, w, sw, b = _problem(M, N, K, seed=7 * M + N + K + epi)
    got = _run(a, sa, w, sw, b, epi)
    ref, absum = oracle.gemm_mxfp4_w4a4(a, sa, w, sw, b if epi else None, epi)
    assert_within(got, ref, absum, "w4a4 wide decode M=%d N=%d K=%d epi=%d" % (M, N, K, epi))


@pytest.mark.parametrize("M", [8, 100])
def test_w4a4_padded_bias(M):
    a, sa, w, sw, b = _problem(M, 256, 512, seed=90 + M)
    got = _run(a, sa, w, sw, b, synth.EPI_BIAS, pad=32)
    ref, absum = oracle.gemm_mxfp4_w4a4(a, sa, w, sw, b, synth.EPI_BIAS)
    assert_within(got, ref, absum, "w4a4 padded M=%d" % M)


def test_w4a4_equals_w4a8_on_values_both_formats_hold():
    """Activations that are e2m1 values with unit block scales: W4A4 and
    W4A8 multiply the same numbers; both GEMMs are checked on them."""
    rng = np.random.default_rng(91)
    for M in (8, 300):
        N, K = 512, 1024
        codes = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
        a4 = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
        sa = np.full((M, K // 32), 127, np.uint8)
        e2m1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6], np.float32)
        a8 = oracle.encode_e4m3(e2m1[codes])
        w, sw = oracle.quant_mxfp4_weights((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
        y4 = bs.gemm_mxfp4_w4a4(u8_dev(a4), u8_dev(sa), u8_dev(w), u8_dev(sw))
        ref, absum = oracle.gemm_mxfp4_w4a8(a8, np.ones(M, np.float32), w, sw)
        assert_within(y_host(y4), ref, absum, "w4a4 vs w4a8 values M=%d" % M)


@pytest.mark.parametrize("M", [16, 512, 4096])
def test_gate_up_w4a4_full_size(M):
    d = synth.make("gate_up", M)
    wl = d["wl"]
    q, s = bs.fp4_quant_rows(bf16_dev(d["a_bf16"]))
    q_ref, s_ref = oracle.quant_mxfp4_rows(d["a_bf16"])
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref) and np.array_equal(s.cpu().numpy(), s_ref)
    y = bs.gemm_mxfp4_w4a4(q, s, u8_dev(d["w"]), u8_dev(d["w_scale"]))
    got = y_host(y)
    rng = np.random.default_rng(92)
    ms = np.concatenate([rng.integers(0, M, 5000), [0, M - 1]])
    ns = np.concatenate([rng.integers(0, wl.N, 5000), [wl.N - 1, 0]])
    ref, absum = oracle.gemm_mxfp4_w4a4_sampled(q_ref, s_ref, d["w"], d["w_scale"], None, 0, ms, ns)
    assert_within(got[ms, ns], ref, absum, "gate_up w4a4 M=%d" % M)
    assert np.isfinite(got).all()


def test_w4a4_rejects_k_mod_64_for_prefill():
    a = torch.zeros((100, 48), dtype=torch.uint8, device=DEV)
    sa = torch.zeros((100, 3), dtype=torch.uint8, device=DEV)
    w = torch.zeros((64, 48), dtype=torch.uint8, device=DEV)
    sw = torch.zeros((64, 3), dtype=torch.uint8, device=DEV)
    with pytest.raises(bs.BsError) as e:
        bs.gemm_mxfp4_w4a4(a, sa, w, sw)
    assert e.value.status == bs.BS_EINVAL
