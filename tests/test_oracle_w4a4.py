"""Pins of the oracle's MXFP4 activation quantizer and its MXFP4 x MXFP4
(W4A4) GEMM.

Routes: the input generator's independent numpy OCP MX conversion, a
dequantize-then-matmul in numpy, exact rational brute force, the W4A8 GEMM
on activations representable in both formats (unit block scales), and the
sampled evaluation against the whole one."""
import fractions

import numpy as np
import pytest
import torch

import synth

F = fractions.Fraction
E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])


def _bf16(x):
    return synth.to_bf16_bits(np.asarray(x, dtype=np.float32))


def _bf16_f32(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16) \
        .to(torch.float32).numpy()


def _dequant(packed, scales):
    codes = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    codes[:, 0::2] = packed & 15
    codes[:, 1::2] = packed >> 4
    vals = E2M1[codes]
    return vals * np.repeat(np.exp2(scales.astype(np.float64) - 127), 32, axis=1)


def test_activation_quantizer_matches_the_generators_conversion(oracle_mod):
    rng = np.random.default_rng(71)
    x = rng.standard_normal((9, 640)).astype(np.float32)
    x[0, :32] = 0                                   # a zero block
    x[1, 64:96] *= 1e-30                            # tiny block
    x[2, 100] = 3e4                                 # an outlier in its block
    x[3] = np.linspace(-6, 6, 640)
    bits = _bf16(x)
    packed, scales = oracle_mod.quant_mxfp4_rows(bits)
    p2, s2 = synth._mx_quantize_rows(_bf16_f32(bits))
    assert np.array_equal(packed, p2) and np.array_equal(scales, s2)
    assert scales[0, 0] == 0 and np.all(packed[0, :16] == 0)


@pytest.mark.parametrize("epi", [0, 1, 2])
def test_w4a4_equals_dequantized_matmul(oracle_mod, epi):
    rng = np.random.default_rng(72)
    M, N, K = 5, 64, 512
    a, sa = oracle_mod.quant_mxfp4_rows(_bf16(rng.standard_normal((M, K))))
    w, sw = oracle_mod.quant_mxfp4_weights((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    b = _bf16(rng.standard_normal(N) * 0.1)
    out, absum = oracle_mod.gemm_mxfp4_w4a4(a, sa, w, sw, b if epi else None, epi)
    ad, wd = _dequant(a, sa), _dequant(w, sw)
    pre = ad @ wd.T + (_bf16_f32(b).astype(np.float64)[None, :] if epi else 0)
    if epi == 2:
        pre = torch.nn.functional.gelu(torch.from_numpy(pre), approximate="tanh").numpy()
    assert np.allclose(out, pre, rtol=1e-12, atol=1e-12)
    assert np.allclose(absum, np.abs(ad) @ np.abs(wd).T, rtol=1e-12)


def test_w4a4_exact_against_rational_brute_force(oracle_mod):
    rng = np.random.default_rng(73)
    M, N, K = 2, 3, 64
    a, sa = oracle_mod.quant_mxfp4_rows(_bf16(rng.standard_normal((M, K)) * 3))
    w, sw = oracle_mod.quant_mxfp4_weights((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
    out, _ = oracle_mod.gemm_mxfp4_w4a4(a, sa, w, sw)
    ad, wd = _dequant(a, sa), _dequant(w, sw)
    for m in range(M):
        for n in range(N):
            exact = sum(F(float(ad[m, k])) * F(float(wd[n, k])) for k in range(K))
            assert abs(F(float(out[m, n])) - exact) <= abs(exact) * F(1, 2 ** 50)


def test_w4a4_equals_w4a8_on_values_both_formats_hold(oracle_mod):
    rng = np.random.default_rng(74)
    M, N, K = 4, 96, 256
    codes = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    a_packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    a_scales = np.full((M, K // 32), 127, np.uint8)                      # unit block scales
    a_e4m3 = oracle_mod.encode_e4m3(E2M1[codes].astype(np.float32))     # the same values
    w, sw = oracle_mod.quant_mxfp4_weights((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
    o44, a44 = oracle_mod.gemm_mxfp4_w4a4(a_packed, a_scales, w, sw)
    o48, a48 = oracle_mod.gemm_mxfp4_w4a8(a_e4m3, np.ones(M, np.float32), w, sw)
    assert np.array_equal(o44, o48) and np.array_equal(a44, a48)


def test_w4a4_sampled_equals_whole(oracle_mod):
    rng = np.random.default_rng(75)
    M, N, K = 6, 128, 320
    a, sa = oracle_mod.quant_mxfp4_rows(_bf16(rng.standard_normal((M, K))))
    w, sw = oracle_mod.quant_mxfp4_weights((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    b = _bf16(rng.standard_normal(N) * 0.1)
    out, absum = oracle_mod.gemm_mxfp4_w4a4(a, sa, w, sw, b, 2)
    ms, ns = np.array([0, 5, 3, 2]), np.array([127, 0, 64, 9])
    o2, a2 = oracle_mod.gemm_mxfp4_w4a4_sampled(a, sa, w, sw, b, 2, ms, ns)
    assert np.array_equal(o2, out[ms, ns]) and np.array_equal(a2, absum[ms, ns])
