"""gemm_bs_fp8 / gemm_mxfp4_w4a8 on the GPU against the oracle.

The oracle's quantized codes and scales feed both sides, so quantizer and
GEMM faults stay apart. Outputs must satisfy
|y - ref| <= 2^-8 |ref| + 1e-4 sum_k |a_k w_k| element-wise; the structured
cases (permutation, one-hot, nibble order) must be exact."""
import numpy as np
import pytest
import torch

import mxfp4_gemm_transformer_amd as bs
import oracle
import synth
from gpu_util import DEV, assert_within, bf16_dev, f32_dev, run_gemm, u8_dev, y_host

pytestmark = pytest.mark.gpu

EPIS = [synth.EPI_NONE, synth.EPI_BIAS, synth.EPI_BIAS_GELU_TANH]


def _random_problem(fmt, M, N, K, seed, wstd=0.05):
    rng = np.random.default_rng(seed)
    x = synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    a, s = oracle.quant_rows(x)
    if fmt == "fp8":
        w = oracle.encode_e4m3((rng.standard_normal((N, K)) * wstd).astype(np.float32))
        ws = rng.integers(120, 131, size=(N // 32, K // 32), dtype=np.uint8)
    else:
        w, ws = oracle.quant_mxfp4_weights((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    b = synth.to_bf16_bits((rng.standard_normal(N) * 0.1).astype(np.float32))
    return a, s, w, ws, b


def _full_check(fmt, M, N, K, epi, seed=0, ld_pad=0):
    a, s, w, ws, b = _random_problem(fmt, M, N, K, seed)
    got = run_gemm(fmt, a, s, w, ws, b if epi else None, epi, ld_pad=ld_pad)
    fn = oracle.gemm_bs_fp8 if fmt == "fp8" else oracle.gemm_mxfp4_w4a8
    ref, absum = fn(a, s, w, ws, b if epi else None, epi)
    assert_within(got, ref, absum, "%s M=%d N=%d K=%d epi=%d" % (fmt, M, N, K, epi))


# ---- decode path (M <= 64): folded (one group to M = 8, two to M = 16) and split-K, K tails
@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("M", [1, 2, 5, 8, 9, 12, 14, 15, 16, 17, 33, 64])
def test_decode_shapes(fmt, M):
    _full_check(fmt, M, 96, 1056, synth.EPI_BIAS_GELU_TANH, seed=M)


# wide layers (N >= 32768): one 8-row group per wave, activations and
# scales staged in LDS; N % 64 == 32 leaves the last workgroup half full
@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("M,K", [(1, 5120), (5, 640), (8, 128), (9, 640), (16, 1024)])
def test_decode_wide_rows(fmt, M, K):
    N = 32768 + 32
    epi = synth.EPI_BIAS_GELU_TANH if M in (5, 9) else synth.EPI_NONE
    _full_check(fmt, M, N, K, epi, seed=M + K)


# e4m3 layers of at least 2^27 weights with 2 <= M <= 16 (split-K over many
# column blocks); (32832, 4352) has a half K step at each row's end and a
# half-full last column block
@pytest.mark.parametrize("M,N,K,epi", [(3, 65536, 2304, synth.EPI_NONE),
                                       (12, 32768 + 64, 4352, synth.EPI_BIAS_GELU_TANH)])
def test_decode_wide_rows_windowed(M, N, K, epi):
    _full_check("fp8", M, N, K, epi, seed=M + K)


# more than two 8-row groups per CU on a layer the wide-layer kernel leaves
# (K % 128 = 32): the folded kernel keeps 8 waves a workgroup, one token
# group (M = 5) or two (M = 12, 16); narrower layers take 16 waves
@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("M", [5, 12, 16])
def test_decode_folded_many_groups(fmt, M):
    _full_check(fmt, M, 8192, 1056, synth.EPI_BIAS, seed=M + 1056)


# split-K (16 < M <= 64, narrow layers): K cut into S slices of whole 128-k
# steps; (2048, 1152) leaves the last three slices empty, (2080, 1184) adds
# a half-full last column block and a 32-wide K tail
@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
# (3 and 8 x 8192 x 8224: small M on a layer of >= 2^26 weights that the
# wide-layer kernel does not take, K > 8192)
@pytest.mark.parametrize("M,N,K", [(40, 2048, 1152), (17, 2080, 1184), (64, 512, 4096),
                                   (3, 8192, 8224), (8, 8192, 8224)])
def test_decode_split_k(fmt, M, N, K):
    _full_check(fmt, M, N, K, synth.EPI_BIAS_GELU_TANH if M == 17 else synth.EPI_BIAS, seed=M + K)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("K", [32, 96, 128, 160, 256, 288, 2080])
def test_decode_k_tails(fmt, K):
    _full_check(fmt, 8, 64, K, synth.EPI_BIAS, seed=K)
    _full_check(fmt, 24, 64, K, synth.EPI_NONE, seed=K + 1)


# ---- prefill path (M > 64): ragged M / N / K against the 128x128 tile
@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("M,N,K", [(65, 32, 32), (128, 128, 128), (200, 320, 544),
                                   (257, 160, 1056), (130, 416, 96)])
def test_prefill_shapes(fmt, M, N, K):
    for epi in EPIS:
        _full_check(fmt, M, N, K, epi, seed=M + N + K + epi)


# ---- prefill with K a multiple of 64 (tiles staged by LDS-mode loads):
# ragged M and N on each tile size, outputs past M / N untouched; MXFP4
# weights with their E8M0 rows in LDS (K % 128 == 0, K <= 7168, up to the
# limit) and without (K % 128 == 64, or K past the limit)
@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("M,N,K", [(65, 96, 64), (200, 320, 640), (129, 416, 128),
                                   (300, 288, 1024), (130, 96, 7168), (70, 160, 7296)])
def test_prefill_dma_shapes(fmt, M, N, K):
    for epi in EPIS:
        _full_check(fmt, M, N, K, epi, seed=M + N + K + epi)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("M,N,K", [(4000, 2016, 2048), (3900, 4064, 1024), (3900, 4064, 1088),
                                   (4000, 4192, 1024), (2000, 4000, 1088)])
def test_prefill_dma_large_tiles(fmt, M, N, K):
    # the launch plans past one round of small tiles, ragged in M and N: one
    # launch of 256x128 tiles, one of 256x256 (K % 128 == 0 and == 64), two
    # launches over column ranges (256x256 tiles in one whole round, then
    # 64x64 tiles over the 96-column rest), and 128x128 tiles two to a CU
    # (e4m3: two-step stages, here with a last half stage); y is a view into
    # a larger NaN-filled buffer
    for epi in (synth.EPI_NONE, synth.EPI_BIAS_GELU_TANH):
        a, s, w, ws, b = _random_problem(fmt, M, N, K, seed=M + N + epi)
        y_full = torch.full((M + 3, N + 64), float("nan"), dtype=torch.bfloat16, device=DEV)
        fn = bs.gemm_bs_fp8 if fmt == "fp8" else bs.gemm_mxfp4_w4a8
        fn(u8_dev(a), f32_dev(s), u8_dev(w), u8_dev(ws), bf16_dev(b) if epi else None, epi,
           y=y_full[:M, :N])
        full = y_host(y_full)
        assert np.isnan(full[M:, :]).all() and np.isnan(full[:, N:]).all()
        ms, ns = _sample_positions(M, N, 5000, epi)
        edge_m = np.concatenate([np.full(N, M - 1), np.arange(M)])
        edge_n = np.concatenate([np.arange(N), np.full(M, N - 1)])
        ms, ns = np.concatenate([ms, edge_m]), np.concatenate([ns, edge_n])
        ref, absum = oracle.gemm_sampled(fmt, a, s, w, ws, b if epi else None, epi, ms, ns)
        assert_within(full[ms, ns], ref, absum, "%s M=%d N=%d K=%d epi=%d" % (fmt, M, N, K, epi))


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("M", [8, 40, 300])
def test_padded_leading_dims(fmt, M):
    _full_check(fmt, M, 96, 256, synth.EPI_BIAS, seed=7, ld_pad=32)


# ---- exact structured pins
@pytest.mark.parametrize("M", [4, 16, 100])
def test_permutation_is_exact(M):
    # A rows of e4m3 values with a 448 in each (scale 1), W a permutation of
    # 1.0 codes: with unit block scales Y = A[:, perm]; with block scales,
    # Y = A[:, perm] * 2^(S-127). Every value is bf16-exact.
    rng = np.random.default_rng(M)
    N, K = 96, 160
    x = np.zeros((M, K), dtype=np.float32)
    codes = rng.integers(0, 0x7E, size=(M, K), dtype=np.uint8) | (rng.integers(0, 2, (M, K), dtype=np.uint8) << 7)
    vals = oracle.e4m3_table()[codes]
    vals[:, 0] = 448.0
    x_bits = synth.to_bf16_bits(vals.astype(np.float32))
    a, s = oracle.quant_rows(x_bits)
    assert np.all(s == 1.0)
    perm = rng.permutation(K)[:N]
    w = np.zeros((N, K), dtype=np.uint8)
    w[np.arange(N), perm] = 0x38
    for ws in (np.full((N // 32, K // 32), 127, np.uint8),
               rng.integers(122, 133, size=(N // 32, K // 32), dtype=np.uint8)):
        got = run_gemm("fp8", a, s, w, ws, None, synth.EPI_NONE)
        A = oracle.e4m3_table()[a]
        want = A[:, perm] * np.exp2(ws[np.arange(N) // 32, perm // 32].astype(np.float64) - 127)
        assert np.array_equal(got, want)


@pytest.mark.parametrize("M", [3, 12, 80])
def test_one_hot_isolates_block_scales(M):
    rng = np.random.default_rng(M + 1)
    N, K = 64, 512
    kstar = rng.integers(0, K, size=M)
    a = np.zeros((M, K), dtype=np.uint8)
    a[np.arange(M), kstar] = 0x38
    s = np.ones(M, dtype=np.float32)
    w = np.full((N, K), 0x38, dtype=np.uint8)
    ws = rng.integers(110, 145, size=(N // 32, K // 32), dtype=np.uint8)
    got = run_gemm("fp8", a, s, w, ws, None, synth.EPI_NONE)
    want = np.exp2(ws[np.arange(N)[None, :] // 32, kstar[:, None] // 32].astype(np.float64) - 127)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("M", [5, 16, 96])
def test_mxfp4_nibble_order_and_row_scales(M):
    rng = np.random.default_rng(M + 2)
    N, K = 64, 256
    kstar = rng.integers(0, K, size=M)
    a = np.zeros((M, K), dtype=np.uint8)
    a[np.arange(M), kstar] = 0x38
    s = np.ones(M, dtype=np.float32)
    wp = np.full((N, K // 2), 0x62, dtype=np.uint8)      # 1.0 at even k, 4.0 at odd k
    ws = rng.integers(110, 140, size=(N, K // 32), dtype=np.uint8)
    got = run_gemm("mxfp4", a, s, wp, ws, None, synth.EPI_NONE)
    base = np.where(kstar % 2 == 1, 4.0, 1.0)[:, None]
    want = base * np.exp2(ws[np.arange(N)[None, :], kstar[:, None] // 32].astype(np.float64) - 127)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("M", [8, 16, 200])
def test_cross_format_agreement(M):
    # MXFP4 with scales constant over 32-row groups equals an e4m3 32x32 problem
    rng = np.random.default_rng(M + 3)
    N, K = 128, 384
    x = synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    a, s = oracle.quant_rows(x)
    nib = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    wp = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    grid = rng.integers(118, 134, size=(N // 32, K // 32), dtype=np.uint8)
    to_e4m3 = np.array([0x00, 0x30, 0x38, 0x3C, 0x40, 0x44, 0x48, 0x4C], dtype=np.uint8)
    w8 = (to_e4m3[nib & 7] | ((nib >> 3) << 7)).astype(np.uint8)
    y4 = run_gemm("mxfp4", a, s, wp, np.repeat(grid, 32, axis=0), None, synth.EPI_NONE)
    y8 = run_gemm("fp8", a, s, w8, grid, None, synth.EPI_NONE)
    ref, absum = oracle.gemm_bs_fp8(a, s, w8, grid)
    assert_within(y4, ref, absum, "mxfp4")
    assert_within(y8, ref, absum, "fp8")


def test_zero_rows_give_bias():
    M, N, K = 9, 64, 128
    a = np.zeros((M, K), dtype=np.uint8)
    s = np.zeros(M, dtype=np.float32)
    rng = np.random.default_rng(4)
    w = oracle.encode_e4m3((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
    ws = rng.integers(120, 131, size=(N // 32, K // 32), dtype=np.uint8)
    b = synth.to_bf16_bits((rng.standard_normal(N) * 0.1).astype(np.float32))
    got = run_gemm("fp8", a, s, w, ws, b, synth.EPI_BIAS)
    want = np.array([oracle.bf16_value(v) for v in b])
    assert np.array_equal(got, np.broadcast_to(want, (M, N)))


def test_gemm_rejects_bad_arguments():
    a = torch.zeros((8, 64), dtype=torch.uint8, device=DEV)
    s = torch.ones(8, dtype=torch.float32, device=DEV)
    w = torch.zeros((64, 64), dtype=torch.uint8, device=DEV)
    ws = torch.full((2, 2), 127, dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        bs.gemm_bs_fp8(a, s, w, ws, None, bs.EPI_BIAS)            # bias missing
    lib = bs.load_library()
    import ctypes
    y = torch.empty((8, 64), dtype=torch.bfloat16, device=DEV)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib.gemm_bs_fp8(p(a), 64, p(s), p(w), 64, p(ws), None, 1, p(y), 64, 8, 64, 64, None, 0, None)
    assert st == bs.BS_EINVAL
    st = lib.gemm_bs_fp8(p(a), 64, p(s), p(w), 64, p(ws), None, 0, p(y), 64, 8, 48, 64, None, 0, None)
    assert st == bs.BS_EINVAL
    st = lib.gemm_bs_fp8(ctypes.c_void_p(a.data_ptr() + 8), 64, p(s), p(w), 64, p(ws), None, 0, p(y),
                         64, 8, 64, 64, None, 0, None)
    assert st == bs.BS_EALIGN


# ---- the workloads at full size, on sampled outputs
def _sample_positions(M, N, count, seed):
    rng = np.random.default_rng(seed)
    ms = np.concatenate([rng.integers(0, M, count), [0, M - 1, 0, M - 1]])
    ns = np.concatenate([rng.integers(0, N, count), [0, N - 1, N - 1, 0]])
    return ms, ns


@pytest.mark.parametrize("name,M", [("tiny", None), ("decode", 1), ("decode", 4), ("decode", 8),
                                    ("decode", 16), ("decode", 64), ("ffn_up", None),
                                    ("ffn_up_bias", None), ("prefill", None),
                                    ("prefill_shard", None), ("gate_up", 1),
                                    ("gate_up", 16), ("gate_up", 512), ("gate_up", 4096)])
def test_workload_full_size_sampled(name, M, seed=0):
    d = synth.make(name, M, seed=seed)
    wl = d["wl"]
    M = d["M"]
    x = bf16_dev(d["a_bf16"])
    q, s = bs.fp8_quant_rows(x)              # end to end: the GPU's own quantization
    q_ref, s_ref = oracle.quant_rows(d["a_bf16"])
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    w_t, ws_t = u8_dev(d["w"]), u8_dev(d["w_scale"])
    b_t = bf16_dev(d["bias"]) if d["bias"] is not None else None
    fn = bs.gemm_bs_fp8 if wl.fmt == "fp8" else bs.gemm_mxfp4_w4a8
    y = fn(q, s, w_t, ws_t, b_t, d["epilogue"])
    got = y_host(y)
    if M * wl.N * wl.K <= 2 ** 31:
        ofn = oracle.gemm_bs_fp8 if wl.fmt == "fp8" else oracle.gemm_mxfp4_w4a8
        ref, absum = ofn(q_ref, s_ref, d["w"], d["w_scale"], d["bias"], d["epilogue"])
        assert_within(got, ref, absum, name)
    else:
        ms, ns = _sample_positions(M, wl.N, 6000, 1)
        ref, absum = oracle.gemm_sampled(wl.fmt, q_ref, s_ref, d["w"], d["w_scale"], d["bias"],
                                         d["epilogue"], ms, ns)
        assert_within(got[ms, ns], ref, absum, name)
    assert np.isfinite(got).all()


# the same checks on a second draw of every tensor (seed 1)
@pytest.mark.parametrize("name,M", [("decode", 8), ("prefill", None), ("gate_up", 16),
                                    ("gate_up", 512)])
def test_workload_full_size_sampled_seed1(name, M):
    test_workload_full_size_sampled(name, M, seed=1)
