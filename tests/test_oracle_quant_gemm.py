"""Pins of the oracle's quantizer, GEMMs and MXFP4 weight conversion.

Each check reaches the oracle's result by another route: numpy/torch float32
arithmetic and torch's float8 cast for the quantizer, dequantize-then-matmul
and exact rational brute force for the GEMMs, structured matrices whose
product is known in closed form, and the equality of the two weight formats
where their values coincide.
"""
import fractions
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _torch_e4m3(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _bf16_to_f32(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16) \
        .to(torch.float32).numpy()


_E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])


def _unpack_fp4(packed):
    lo = packed & 0xF
    hi = packed >> 4
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def _dequant_matmul_fp8(a, s, w, ws, bias, epi):
    A = _torch_e4m3(a)
    W = _torch_e4m3(w) * np.kron(np.exp2(ws.astype(np.float64) - 127), np.ones((32, 32)))
    pre = s.astype(np.float64)[:, None] * (A @ W.T)
    if epi:
        pre = pre + _bf16_to_f32(bias).astype(np.float64)[None, :]
    if epi == synth.EPI_BIAS_GELU_TANH:
        pre = torch.nn.functional.gelu(torch.from_numpy(pre), approximate="tanh").numpy()
    return pre


def _dequant_matmul_mxfp4(a, s, wp, ws, bias, epi):
    A = _torch_e4m3(a)
    W = _E2M1[_unpack_fp4(wp)] * np.repeat(np.exp2(ws.astype(np.float64) - 127), 32, axis=1)
    pre = s.astype(np.float64)[:, None] * (A @ W.T)
    if epi:
        pre = pre + _bf16_to_f32(bias).astype(np.float64)[None, :]
    if epi == synth.EPI_BIAS_GELU_TANH:
        pre = torch.nn.functional.gelu(torch.from_numpy(pre), approximate="tanh").numpy()
    return pre


# ----------------------------------------------------------------- quantizer
def _quant_reference_via_torch(x_bits):
    # s = fl32(amax / 448) and v = fl32(x / s) in numpy float32 (IEEE
    # division), then torch's nearest-even float8 cast.
    x = _bf16_to_f32(x_bits)
    amax = np.abs(x).max(axis=1)
    s = (amax / np.float32(448.0)).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        v = (x / s[:, None]).astype(np.float32)
    q = torch.from_numpy(np.ascontiguousarray(v)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return q, s, v


def test_quant_rows_matches_float32_route_on_workloads(oracle_mod):
    for name, M in (("tiny", None), ("decode", 16), ("ffn_up", 64), ("prefill", 8), ("gate_up", 4)):
        wl = synth.WORKLOADS[name]
        x = synth.activations(wl, M)
        q, s = oracle_mod.quant_rows(x)
        q_ref, s_ref, v = _quant_reference_via_torch(x)
        assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32)), name
        assert np.all(np.abs(v) <= 448.0 * (1 + 2.0 ** -23))
        # torch's cast is NaN for (464, 480); the quantizer never gets there,
        # and 448 < |v| <= 464 rounds to 448 in both.
        assert np.array_equal(q, q_ref), name


def test_quant_rows_invariants(oracle_mod):
    wl = synth.WORKLOADS["prefill"]
    x = synth.activations(wl, 32)
    q, s = oracle_mod.quant_rows(x)
    xf = _bf16_to_f32(x).astype(np.float64)
    for m in range(q.shape[0]):
        # every row holds a code of magnitude 448
        assert np.any((q[m] & 0x7F) == 0x7E)
        # dequantized error is at most half an e4m3 step of v (2^-4 relative
        # for normals) plus the subnormal half-step 2^-10, times s
        err = np.abs(_torch_e4m3(q[m]) * s[m] - xf[m])
        assert np.all(err <= s[m] * (np.abs(xf[m]) / s[m] * 2.0 ** -4 + 2.0 ** -10) * (1 + 1e-6))


def test_quant_rows_special_rows(oracle_mod):
    K = 64
    rows = np.zeros((5, K), dtype=np.float32)
    rows[1, :] = -0.0
    rows[2, 7] = -3.0                      # one nonzero: it becomes -448, the rest +0
    rows[3, :] = 1.0                       # constant row: all 448
    rows[4, :] = np.float32(1e-39)         # subnormal bf16 magnitudes
    rows[4, 5] = np.float32(-2e-39)
    x = synth.to_bf16_bits(rows)
    x[1, :] = 0x8000                       # -0.0 in every position
    q, s = oracle_mod.quant_rows(x)
    assert s[0] == 0 and np.all(q[0] == 0x00)
    assert s[1] == 0 and np.all(q[1] == 0x80)
    assert q[2, 7] == 0xFE and np.all(np.delete(q[2], 7) == 0x00)
    assert np.all(q[3] == 0x7E) and s[3] == np.float32(1.0) / np.float32(448.0)
    q_ref, s_ref, _ = _quant_reference_via_torch(x[4:5])
    assert s[4] == s_ref[0] and s[4] > 0
    assert np.array_equal(q[4], q_ref[0])


def test_quant_rows_hits_every_tie(oracle_mod):
    # A row holding 448 (so s = 1 exactly) and every midpoint between
    # adjacent e4m3 values that bf16 can hold, plus their bf16 neighbours:
    # ties must go to the even code.
    t = oracle_mod.e4m3_table()
    mids = [0.5 * (t[c] + t[c + 1]) for c in range(0x7E)]
    vals = [448.0] + mids + [-m for m in mids]
    x = synth.to_bf16_bits(np.array(vals, dtype=np.float32))
    back = _bf16_to_f32(x).astype(np.float64)
    assert np.array_equal(back, np.array(vals))     # all exactly representable
    pad = (-len(vals)) % 32
    x = np.concatenate([x, np.zeros(pad, dtype=np.uint16)])[None, :]
    q, s = oracle_mod.quant_rows(x)
    assert s[0] == np.float32(1.0)
    for i, c in enumerate(range(0x7E)):
        even = c if c % 2 == 0 else c + 1
        assert q[0, 1 + i] == even
        assert q[0, 1 + 0x7E + i] == even | 0x80


# ---------------------------------------------------------------------- GEMM
@pytest.mark.parametrize("epi", [synth.EPI_NONE, synth.EPI_BIAS, synth.EPI_BIAS_GELU_TANH])
def test_gemm_fp8_equals_dequant_matmul(oracle_mod, epi):
    rng = np.random.default_rng(3 + epi)
    M, N, K = 7, 96, 160
    x = synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    a, s = oracle_mod.quant_rows(x)
    w = oracle_mod.encode_e4m3((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
    ws = rng.integers(120, 131, size=(N // 32, K // 32), dtype=np.uint8)
    b = synth.to_bf16_bits((rng.standard_normal(N) * 0.1).astype(np.float32))
    out, absum = oracle_mod.gemm_bs_fp8(a, s, w, ws, b if epi else None, epi)
    ref = _dequant_matmul_fp8(a, s, w, ws, b, epi)
    assert np.all(np.abs(out - ref) <= 1e-12 * (absum + np.abs(ref)) + 1e-14)
    # absum bounds |pre - bias| and is itself a dequantized |A| |W|^T
    A = np.abs(_torch_e4m3(a))
    W = np.abs(_torch_e4m3(w)) * np.kron(np.exp2(ws.astype(np.float64) - 127), np.ones((32, 32)))
    assert np.allclose(absum, s[:, None] * (A @ W.T), rtol=1e-12, atol=0)


@pytest.mark.parametrize("epi", [synth.EPI_NONE, synth.EPI_BIAS, synth.EPI_BIAS_GELU_TANH])
def test_gemm_mxfp4_equals_dequant_matmul(oracle_mod, epi):
    rng = np.random.default_rng(11 + epi)
    M, N, K = 5, 64, 192
    x = synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    a, s = oracle_mod.quant_rows(x)
    wp, ws = oracle_mod.quant_mxfp4_weights((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    b = synth.to_bf16_bits((rng.standard_normal(N) * 0.1).astype(np.float32))
    out, absum = oracle_mod.gemm_mxfp4_w4a8(a, s, wp, ws, b if epi else None, epi)
    ref = _dequant_matmul_mxfp4(a, s, wp, ws, b, epi)
    assert np.all(np.abs(out - ref) <= 1e-12 * (absum + np.abs(ref)) + 1e-14)


def _frac_e4m3(c):
    return fractions.Fraction(float(_torch_e4m3(np.array([c]))[0]))


@pytest.mark.parametrize("K", [32, 64, 96, 128])
def test_gemm_fp8_exact_on_tiny_shapes(oracle_mod, K):
    # K <= 128: every term is an integer multiple of 2^-25 below 2^21, so the
    # fp64 accumulation is exact and must equal exact rational arithmetic.
    rng = np.random.default_rng(K)
    M, N = 3, 64
    a = rng.integers(0, 256, size=(M, K), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x38
    w = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    w[(w & 0x7F) == 0x7F] = 0x40
    ws = rng.integers(120, 131, size=(N // 32, K // 32), dtype=np.uint8)
    s = np.ones(M, dtype=np.float32)
    out, _ = oracle_mod.gemm_bs_fp8(a, s, w, ws)
    av = [[_frac_e4m3(c) for c in row] for row in a]
    wv = [[_frac_e4m3(c) for c in row] for row in w]
    for m in range(M):
        for n in range(N):
            acc = sum(fractions.Fraction(2) ** (int(ws[n // 32, k // 32]) - 127) * av[m][k] * wv[n][k]
                      for k in range(K))
            assert out[m, n] == float(acc)


@pytest.mark.parametrize("K", [32, 64, 128])
def test_gemm_mxfp4_exact_on_tiny_shapes(oracle_mod, K):
    rng = np.random.default_rng(100 + K)
    M, N = 3, 32
    a = rng.integers(0, 256, size=(M, K), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x38
    wp = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    ws = rng.integers(120, 131, size=(N, K // 32), dtype=np.uint8)
    s = np.ones(M, dtype=np.float32)
    out, _ = oracle_mod.gemm_mxfp4_w4a8(a, s, wp, ws)
    nib = _unpack_fp4(wp)
    for m in range(M):
        for n in range(N):
            acc = sum(fractions.Fraction(2) ** (int(ws[n, k // 32]) - 127) * _frac_e4m3(a[m, k])
                      * fractions.Fraction(float(_E2M1[nib[n, k]])) for k in range(K))
            assert out[m, n] == float(acc)


def test_gemm_fp8_permutation_identity_and_scale_shift(oracle_mod):
    # A rows hold 448 (s = 1) and e4m3 values; W is a permutation matrix of
    # 1.0 codes; with unit scales Y = A[:, perm] exactly, and with block
    # scales Y[m, n] = A[m, perm[n]] * 2^(S[n/32, perm[n]/32] - 127).
    rng = np.random.default_rng(5)
    M, N, K = 4, 96, 96
    a = rng.integers(0, 0x7E, size=(M, K), dtype=np.uint8) | (rng.integers(0, 2, size=(M, K), dtype=np.uint8) << 7)
    a[:, 0] = 0x7E
    s = np.ones(M, dtype=np.float32)
    perm = rng.permutation(K)[:N]
    w = np.zeros((N, K), dtype=np.uint8)
    w[np.arange(N), perm] = 0x38
    A = _torch_e4m3(a)
    ones = np.full((N // 32, K // 32), 127, dtype=np.uint8)
    out, _ = oracle_mod.gemm_bs_fp8(a, s, w, ones)
    assert np.array_equal(out, A[:, perm])
    ws = rng.integers(120, 131, size=(N // 32, K // 32), dtype=np.uint8)
    out, _ = oracle_mod.gemm_bs_fp8(a, s, w, ws)
    expect = A[:, perm] * np.exp2(ws[np.arange(N) // 32, perm // 32].astype(np.float64) - 127)
    assert np.array_equal(out, expect)


def test_gemm_fp8_one_hot_isolates_each_block_scale(oracle_mod):
    rng = np.random.default_rng(9)
    M, N, K = 8, 64, 256
    kstar = rng.integers(0, K, size=M)
    a = np.zeros((M, K), dtype=np.uint8)
    a[np.arange(M), kstar] = 0x38
    w = np.full((N, K), 0x38, dtype=np.uint8)
    ws = rng.integers(100, 150, size=(N // 32, K // 32), dtype=np.uint8)
    s = np.ones(M, dtype=np.float32)
    out, _ = oracle_mod.gemm_bs_fp8(a, s, w, ws)
    for m in range(M):
        for n in range(N):
            assert out[m, n] == 2.0 ** (int(ws[n // 32, kstar[m] // 32]) - 127)


def test_gemm_mxfp4_nibble_order_and_row_scales(oracle_mod):
    # one-hot A at k*; W holds 1.0 (nibble 0x2) at even k and 4.0 (0x6) at
    # odd k, so Y tells which nibble of byte k*/2 was read, and scales per
    # row per 32 k show up individually.
    rng = np.random.default_rng(13)
    M, N, K = 16, 32, 128
    kstar = rng.permutation(K)[:M]
    a = np.zeros((M, K), dtype=np.uint8)
    a[np.arange(M), kstar] = 0x38
    wp = np.full((N, K // 2), 0x62, dtype=np.uint8)
    ws = rng.integers(110, 140, size=(N, K // 32), dtype=np.uint8)
    s = np.ones(M, dtype=np.float32)
    out, _ = oracle_mod.gemm_mxfp4_w4a8(a, s, wp, ws)
    for m in range(M):
        for n in range(N):
            base = 4.0 if kstar[m] % 2 else 1.0
            assert out[m, n] == base * 2.0 ** (int(ws[n, kstar[m] // 32]) - 127)


def test_gemm_cross_format_equality(oracle_mod):
    # Every e2m1 value is an e4m3 value; with MXFP4 scales constant over each
    # 32-row group, the MXFP4 problem is an e4m3 32x32-block problem.
    rng = np.random.default_rng(21)
    M, N, K = 6, 64, 128
    x = synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    a, s = oracle_mod.quant_rows(x)
    nib = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    wp = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    grid = rng.integers(118, 136, size=(N // 32, K // 32), dtype=np.uint8)
    ws4 = np.repeat(grid, 32, axis=0)
    to_e4m3 = np.array([0x00, 0x30, 0x38, 0x3C, 0x40, 0x44, 0x48, 0x4C], dtype=np.uint8)
    w8 = to_e4m3[nib & 7] | ((nib >> 3) << 7).astype(np.uint8)
    b = synth.to_bf16_bits((rng.standard_normal(N) * 0.1).astype(np.float32))
    for epi in (synth.EPI_NONE, synth.EPI_BIAS, synth.EPI_BIAS_GELU_TANH):
        o4, ab4 = oracle_mod.gemm_mxfp4_w4a8(a, s, wp, ws4, b, epi)
        o8, ab8 = oracle_mod.gemm_bs_fp8(a, s, w8, grid, b, epi)
        assert np.array_equal(o4, o8) and np.array_equal(ab4, ab8)


def test_gemm_sampled_equals_whole(oracle_mod):
    rng = np.random.default_rng(2)
    d = synth.make("tiny")
    a, s = oracle_mod.quant_rows(d["a_bf16"])
    out, absum = oracle_mod.gemm_bs_fp8(a, s, d["w"], d["w_scale"], d["bias"], d["epilogue"])
    ms = rng.integers(0, 16, 300)
    ns = rng.integers(0, 256, 300)
    o2, ab2 = oracle_mod.gemm_sampled("fp8", a, s, d["w"], d["w_scale"], d["bias"], d["epilogue"], ms, ns)
    assert np.array_equal(o2, out[ms, ns]) and np.array_equal(ab2, absum[ms, ns])
    wp, ws = oracle_mod.quant_mxfp4_weights((rng.standard_normal((64, 256)) * 0.02).astype(np.float32))
    o4, ab4 = oracle_mod.gemm_mxfp4_w4a8(a, s, wp, ws)
    ns4 = rng.integers(0, 64, 300)
    o5, ab5 = oracle_mod.gemm_sampled("mxfp4", a, s, wp, ws, None, 0, ms, ns4)
    assert np.array_equal(o5, o4[ms, ns4]) and np.array_equal(ab5, ab4[ms, ns4])


def test_oracle_is_thread_count_invariant(oracle_mod, tmp_path):
    code = r"""
import sys, numpy as np
sys.path.insert(0, %r)
import oracle, synth
d = synth.make("tiny")
a, s = oracle.quant_rows(d["a_bf16"])
o, ab = oracle.gemm_bs_fp8(a, s, d["w"], d["w_scale"], d["bias"], 2)
np.save(sys.argv[1], np.concatenate([o.ravel(), ab.ravel(), s.astype(np.float64)]))
print(oracle.num_threads())
""" % ROOT
    res = {}
    for t in ("1", "7"):
        env = dict(os.environ, OMP_NUM_THREADS=t)
        f = str(tmp_path / ("o%s.npy" % t))
        outp = subprocess.check_output([sys.executable, "-c", code, f], env=env, text=True)
        assert outp.strip() == t
        res[t] = np.load(f)
    assert np.array_equal(res["1"], res["7"])


# ------------------------------------------------------- MXFP4 conversion
def test_mxfp4_weight_conversion_rule(oracle_mod):
    rng = np.random.default_rng(4)
    v = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    v[3, 32:64] = 0.0                                  # an all-zero group
    wp, ws = oracle_mod.quant_mxfp4_weights(v)
    nib = _unpack_fp4(wp)
    deq = _E2M1[nib] * np.repeat(np.exp2(ws.astype(np.float64) - 127), 32, axis=1)
    g = np.abs(v.astype(np.float64)).reshape(64, 8, 32)
    amax = g.max(axis=2)
    nz = amax > 0
    # the shared exponent puts each group's largest magnitude in [4, 8)
    ratio = amax[nz] / np.exp2(ws[nz].astype(np.float64) - 127)
    assert np.all((ratio >= 4) & (ratio < 8))
    assert ws[3, 1] == 0 and np.all(nib[3, 32:64] == 0)
    # every element is within half a step of e2m1 at its scale, or saturated
    unit = np.repeat(np.exp2(ws.astype(np.float64) - 127), 32, axis=1)
    x = np.abs(v) / unit
    err = np.abs(deq - v) / unit
    step = np.where(x < 2, 0.5, np.where(x < 4, 1.0, 2.0))
    assert np.all((err <= step / 2 + 1e-12) | (x > 6))
    # the sign is kept
    assert np.all((nib >= 8) == (v < 0))


def test_mxfp4_conversion_round_trips_representable_groups(oracle_mod):
    rng = np.random.default_rng(6)
    N, K = 32, 128
    X = rng.integers(-20, 5, size=(N, K // 32))
    nib = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    nib[:, ::32] = 0x7                                 # each group's max is 6 * 2^X
    v = _E2M1[nib] * np.repeat(np.exp2(X.astype(np.float64)), 32, axis=1)
    wp, ws = oracle_mod.quant_mxfp4_weights(v.astype(np.float32))
    assert np.array_equal(ws.astype(np.int64), X + 127)
    got = _unpack_fp4(wp)
    # zeros may come back with either sign only where the input was -0
    assert np.array_equal(_E2M1[got], _E2M1[nib])
