"""Pins of the oracle's static-scale quantizer and its row-wise scaled e4m3
GEMM (per-token activation scale x per-output-channel weight scale).

Routes: the dynamic quantizer (a static scale equal to the row's own scale
must give the same codes), torch's float8 cast, dequantize-then-matmul in
numpy, exact rational brute force, the block-scaled GEMM with uniform
power-of-two scales, and the sampled evaluation against the whole one."""
import fractions

import numpy as np
import pytest
import torch

import synth

F = fractions.Fraction


def _bf16(x):
    return synth.to_bf16_bits(np.asarray(x, dtype=np.float32))


def _bf16_f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16) \
        .to(torch.float64).numpy()


def _e4m3_f64(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()


# ------------------------------------------------------------ static quant
def test_static_quant_with_the_rows_own_scale_is_the_dynamic_quant(oracle_mod):
    rng = np.random.default_rng(51)
    x = _bf16(rng.standard_normal((12, 640)) * np.exp2(rng.integers(-8, 8, (12, 1))))
    q, s = oracle_mod.quant_rows(x)
    for m in range(12):
        assert np.array_equal(oracle_mod.quant_rows_static(x[m:m + 1], s[m])[0], q[m])


def test_static_quant_matches_torch_cast_and_saturates(oracle_mod):
    rng = np.random.default_rng(52)
    x = _bf16(rng.standard_normal((8, 256)) * 4)
    sc = np.float32(0.0078125)                  # |x / s| reaches ~2000: saturation
    q = oracle_mod.quant_rows_static(x, sc)
    ratio = (_bf16_f64(x) / np.float64(sc)).astype(np.float32)
    inside = np.abs(ratio) < 448
    want = torch.from_numpy(ratio).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q[inside], want[inside])
    assert np.all((q[~inside] & 0x7F) == 0x7E)
    assert np.all((q[~inside] >> 7) == (ratio[~inside] < 0))
    assert (~inside).sum() > 100


# ------------------------------------------------------------ row-wise GEMM
def _rowwise_problem(M, N, K, seed):
    rng = np.random.default_rng(seed)
    a, s = None, None
    x = _bf16(rng.standard_normal((M, K)))
    import oracle
    a, s = oracle.quant_rows(x)
    wv = _bf16(rng.standard_normal((N, K)) * 0.02)
    w, ws = oracle.quant_rows(wv)               # per-channel scales: the per-token rule on W rows
    b = _bf16(rng.standard_normal(N) * 0.1)
    return a, s, w, ws, b


@pytest.mark.parametrize("epi", [0, 1, 2])
def test_rowwise_equals_dequantized_matmul(oracle_mod, epi):
    a, s, w, ws, b = _rowwise_problem(6, 64, 256, 53)
    out, absum = oracle_mod.gemm_fp8_rowwise(a, s, w, ws, b if epi else None, epi)
    ad = _e4m3_f64(a) * s[:, None].astype(np.float64)
    wd = _e4m3_f64(w) * ws[:, None].astype(np.float64)
    pre = ad @ wd.T + (_bf16_f64(b)[None, :] if epi else 0)
    if epi == 2:
        pre = torch.nn.functional.gelu(torch.from_numpy(pre), approximate="tanh").numpy()
    assert np.allclose(out, pre, rtol=1e-12, atol=1e-12)
    assert np.allclose(absum, np.abs(ad) @ np.abs(wd).T, rtol=1e-12)


def test_rowwise_exact_against_rational_brute_force(oracle_mod):
    a, s, w, ws, b = _rowwise_problem(2, 3, 32, 54)
    out, _ = oracle_mod.gemm_fp8_rowwise(a, s, w, ws, b, 1)
    av, wv = _e4m3_f64(a), _e4m3_f64(w)
    for m in range(2):
        for n in range(3):
            acc = sum(F(float(av[m, k])) * F(float(wv[n, k])) for k in range(32))
            pre = F(float(s[m])) * F(float(ws[n])) * acc + F(float(_bf16_f64(b)[n]))
            assert abs(F(float(out[m, n])) - pre) <= abs(pre) * F(1, 2 ** 50)


def test_rowwise_equals_block_scaled_with_uniform_power_of_two_scales(oracle_mod):
    rng = np.random.default_rng(55)
    M, N, K = 4, 64, 256
    a, s = oracle_mod.quant_rows(_bf16(rng.standard_normal((M, K))))
    w = oracle_mod.encode_e4m3((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
    byte = rng.integers(118, 134, size=N // 32).astype(np.uint8)
    grid = np.repeat(byte[:, None], K // 32, axis=1)
    chan = np.repeat(np.exp2(byte.astype(np.float64) - 127), 32).astype(np.float32)
    r_out, r_abs = oracle_mod.gemm_fp8_rowwise(a, s, w, chan)
    b_out, b_abs = oracle_mod.gemm_bs_fp8(a, s, w, grid)
    assert np.allclose(r_out, b_out, rtol=1e-13, atol=0)
    assert np.allclose(r_abs, b_abs, rtol=1e-13, atol=0)


def test_rowwise_sampled_equals_whole(oracle_mod):
    a, s, w, ws, b = _rowwise_problem(5, 96, 160, 56)
    out, absum = oracle_mod.gemm_fp8_rowwise(a, s, w, ws, b, 2)
    ms = np.array([0, 4, 2, 3, 1])
    ns = np.array([0, 95, 17, 64, 33])
    o2, a2 = oracle_mod.gemm_fp8_rowwise_sampled(a, s, w, ws, b, 2, ms, ns)
    assert np.array_equal(o2, out[ms, ns]) and np.array_equal(a2, absum[ms, ns])


def test_per_channel_weight_generator_matches_the_oracle_quantizer(oracle_mod):
    wl = synth.Workload("lm_head_small", 4, 96, 512, "fp8_rowwise", synth.EPI_NONE)
    codes, scales = synth.weights(wl)
    rows = synth.weight_bf16_rows(wl, 0, wl.N)
    q, s = oracle_mod.quant_rows(rows)
    assert np.array_equal(codes, q)
    assert np.array_equal(scales.view(np.uint32), s.view(np.uint32))
    assert np.array_equal(synth.weight_bf16_rows(wl, 40, 60), rows[40:60])
