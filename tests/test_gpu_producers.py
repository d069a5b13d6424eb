"""Fused producers on the GPU against the oracle: add_rms_norm_quant_fp8
(RMSNorm with or without the residual add) and silu_mul_quant_fp8. Codes,
scales and the updated residual must match bit for bit.

Covers the workload shapes at full size (hidden 5120, intermediate 17408,
M in 1..4096), every thread-per-row configuration the dispatcher picks
(short rows, decode rows, long rows), ragged shapes, padded leading
dimensions, eps values, zero rows, and gates far enough out that SiLU takes
its fp64 path."""
import numpy as np
import pytest
import torch

import mxfp4_gemm_transformer_amd as bs
import oracle
import synth
from gpu_util import DEV, bf16_dev

pytestmark = pytest.mark.gpu


def _bits(t):
    torch.cuda.synchronize()
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _assert_codes(qh, q_ref, what, src=None):
    if not np.array_equal(qh, q_ref):
        bad = np.argwhere(qh != q_ref)
        m, k = bad[0]
        raise AssertionError("%s: %d codes differ; first at (%d, %d): got %#x want %#x"
                             % (what, len(bad), m, k, qh[m, k], q_ref[m, k]))


def _padded(bits, pad):
    M, K = bits.shape
    full = np.zeros((M, K + pad), dtype=np.uint16)
    full[:, :K] = bits
    return bf16_dev(full)[:, :K]


def _check_rms(x, res, w, eps, pad=0, what=""):
    M, K = x.shape
    xt = _padded(x, pad) if pad else bf16_dev(x)
    rt = None
    if res is not None:
        rt = _padded(res, pad) if pad else bf16_dev(res)
    q_out = None
    if pad:
        q_full = torch.full((M, K + pad), 0xAA, dtype=torch.uint8, device=DEV)
        q_out = q_full[:, :K]
    q, s = bs.add_rms_norm_quant_fp8(xt, rt, bf16_dev(w), eps, q=q_out)
    torch.cuda.synchronize()
    q_ref, s_ref, r_ref, h_ref = oracle.add_rms_norm_quant(x, res, w, eps)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32)), what + " scales"
    _assert_codes(q.cpu().numpy(), q_ref, what)
    if res is not None:
        got_r = _bits(rt)
        assert np.array_equal(got_r, r_ref), what + " residual"
    if pad:
        assert torch.all(q_full[:, K:] == 0xAA), "wrote past the row"


def _check_silu(gu, pad=0, what=""):
    M, I2 = gu.shape
    I = I2 // 2
    gt = _padded(gu, pad) if pad else bf16_dev(gu)
    q, s = bs.silu_mul_quant_fp8(gt)
    torch.cuda.synchronize()
    q_ref, s_ref, a_ref = oracle.silu_mul_quant(gu)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32)), what + " scales"
    _assert_codes(q.cpu().numpy(), q_ref, what)


# ------------------------------------------------------------------ RMSNorm
@pytest.mark.parametrize("M", [1, 16, 512, 4096])
def test_add_rms_workload_full_size(M):
    d = synth.producer_inputs("add_rms", M)
    _check_rms(d["x"], d["residual"], d["weight"], d["eps"], what="add_rms M=%d" % M)


@pytest.mark.parametrize("M,K", [(1, 32), (3, 96), (7, 256), (64, 1056), (65, 2080), (100, 5120),
                                 (513, 512), (600, 8192), (20, 17408), (300, 17408),
                                 (2, 32768), (530, 32768), (520, 12288), (512, 5120)])
@pytest.mark.parametrize("with_res", [True, False])
def test_rms_shapes(M, K, with_res):
    d = synth.producer_inputs("add_rms", M, K, seed=M + K)
    _check_rms(d["x"], d["residual"] if with_res else None, d["weight"], d["eps"],
               what="rms M=%d K=%d res=%d" % (M, K, with_res))


@pytest.mark.parametrize("eps", [0.0, 1e-5, 0.25])
def test_rms_eps_and_padding(eps):
    d = synth.producer_inputs("add_rms", 33, 1024, seed=5)
    _check_rms(d["x"], d["residual"], d["weight"], eps, pad=32, what="rms pad eps=%g" % eps)


def test_rms_special_rows():
    K = 512
    d = synth.producer_inputs("add_rms", 6, K, seed=9)
    x, res = d["x"].copy(), d["residual"].copy()
    x[0] = 0; res[0] = 0                                  # zero row -> scale 0
    x[1] = 0x3F80; res[1] = 0                             # constant row
    x[2] = synth.to_bf16_bits(np.full(K, 1e-30, np.float32)); res[2] = 0   # tiny row, eps dominates
    res[3] = (x[3] ^ 0x8000)                              # x + res = 0 exactly
    x[4] = synth.to_bf16_bits(np.full(K, 3e4, np.float32))  # large values
    _check_rms(x, res, d["weight"], 1e-6, what="rms special rows")


# ----------------------------------------------------------------- SiLU*up
@pytest.mark.parametrize("M", [1, 16, 512, 4096])
def test_silu_mul_workload_full_size(M):
    d = synth.producer_inputs("silu_mul", M)
    _check_silu(d["gate_up"], what="silu_mul M=%d" % M)


@pytest.mark.parametrize("M,I", [(1, 32), (5, 96), (9, 256), (64, 2048), (65, 1056), (513, 512),
                                 (33, 17408), (530, 32768), (520, 16384), (512, 17408)])
def test_silu_mul_shapes(M, I):
    d = synth.producer_inputs("silu_mul", M, I, seed=M + I)
    _check_silu(d["gate_up"], what="silu M=%d I=%d" % (M, I))


def test_silu_mul_padding_and_extreme_gates():
    rng = np.random.default_rng(41)
    M, I = 12, 1024
    g = rng.standard_normal((M, I)).astype(np.float32) * 4
    g[0] = np.linspace(-120, 120, I)            # exp(-g) overflows fp32 at the left end
    g[1] = -90.0
    g[2] = 0.0
    g[3] = np.linspace(-1e-3, 1e-3, I)
    u = rng.standard_normal((M, I)).astype(np.float32)
    u[4] = 0.0
    u[5] = 1e20
    gu = np.concatenate([synth.to_bf16_bits(g), synth.to_bf16_bits(u)], axis=1)
    _check_silu(gu, pad=40, what="silu extremes")
    _check_silu(gu, what="silu extremes")


def test_add_rms_then_gemm_end_to_end():
    """add_rms_norm_quant_fp8's (q, scale) fed straight into the MXFP4 GEMM
    at M=16: codes bit-exact, GEMM output within the acceptance bound."""
    M, K, N = 16, 512, 512
    d = synth.producer_inputs("add_rms", M, K, seed=2)
    x, res = bf16_dev(d["x"]), bf16_dev(d["residual"])
    q, s = bs.add_rms_norm_quant_fp8(x, res, bf16_dev(d["weight"]), d["eps"])
    q_ref, s_ref, _, _ = oracle.add_rms_norm_quant(d["x"], d["residual"], d["weight"], d["eps"])
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    rng = np.random.default_rng(3)
    w, ws = oracle.quant_mxfp4_weights((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
    y = bs.gemm_mxfp4_w4a8(q, s, torch.from_numpy(w).to(DEV), torch.from_numpy(ws).to(DEV))
    ref, absum = oracle.gemm_mxfp4_w4a8(q_ref, s_ref, w, ws)
    got = y.float().cpu().numpy().astype(np.float64)
    assert oracle.within_tolerance(got, ref, absum).all()
