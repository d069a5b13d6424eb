"""Pins of the oracle's fused producers (RMSNorm with a residual add, and
SiLU(gate) * up, each followed by the per-token quantizer) and of its bf16
rounding of fp64 values.

Each check reaches the result by another route: torch's fp32 -> bf16 cast,
an exact rational nearest-neighbour search over all bf16 values, closed
forms on constant rows, power-of-two scaling invariance, torch's float64
rms_norm / silu (equal after bf16 rounding except next to a rounding
boundary, and never more than one bf16 step apart), torch's bf16 add.
"""
import bisect
import fractions

import numpy as np
import pytest
import torch

import synth

F = fractions.Fraction


def _bf16_bits(values_f32):
    t = torch.from_numpy(np.ascontiguousarray(values_f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _bf16_f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16) \
        .to(torch.float64).numpy()


def _steps_apart(a_bits, b_bits):
    """Distance in bf16 steps between same-sign finite bf16 values (as
    ordered integers of their magnitude bits with the sign applied)."""
    def key(b):
        b = b.astype(np.int64)
        mag = b & 0x7FFF
        return np.where(b & 0x8000, -mag, mag)
    return np.abs(key(a_bits) - key(b_bits))


# ------------------------------------------------------------ bf16 rounding
def test_bf16_round_matches_torch_on_values_exact_in_fp32(oracle_mod):
    rng = np.random.default_rng(11)
    mags = np.exp2(rng.uniform(-140, 127.9, 4000)).astype(np.float32)
    vals = np.concatenate([mags * rng.choice([-1, 1], mags.size),
                           np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, -3.0e38,
                                     3.3895e38, 1e-40, -1e-44], np.float32)]).astype(np.float32)
    want = _bf16_bits(vals)
    got = np.array([oracle_mod.bf16_round(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, want)


def _all_bf16_finite():
    bits = np.arange(0x7F80, dtype=np.uint16)           # +0 .. largest finite
    vals = _bf16_f64(bits)
    return [F(float(v)) for v in vals], bits


def test_bf16_round_is_the_nearest_even_neighbour_in_exact_arithmetic(oracle_mod):
    fr, bits = _all_bf16_finite()
    top = fr[-1]
    overflow_mid = (top + F(2) ** 128) / 2
    rng = np.random.default_rng(12)
    cases = []
    # ties and near-ties a binary32 intermediate would have blurred
    for base in [1.0, 1.5, 3.140625, 2.0 ** -126, 2.0 ** -130, 1e20, 2.0 ** 127]:
        lo = F(base)
        i = bisect.bisect_left(fr, lo)
        mid = (fr[i] + fr[i + 1]) / 2
        for d in [F(0), F(1, 2 ** 45) * fr[i], -F(1, 2 ** 45) * fr[i]]:
            cases.append(mid + d)
    cases += [F(float(v)) for v in np.exp2(rng.uniform(-135, 127.99, 2000)) * (1 + 2.0 ** -30)]
    cases += [overflow_mid, overflow_mid - F(1, 2 ** 100) * top]
    for c in cases:
        v = float(c)
        if F(v) != c:        # keep only values a double holds exactly
            continue
        got = oracle_mod.bf16_round(v)
        if c >= overflow_mid:
            assert got == 0x7F80
            continue
        j = bisect.bisect_right(fr, c) - 1
        lo, hi = fr[j], fr[j + 1]
        if c - lo < hi - c or (c - lo == hi - c and bits[j] % 2 == 0):
            want = int(bits[j])
        else:
            want = int(bits[j + 1])
        assert got == want, (v, hex(got), hex(want))
        assert oracle_mod.bf16_round(-v) == want | 0x8000


# ------------------------------------------------------------------ RMSNorm
def _row(v_bits, K):
    return np.full((1, K), v_bits, dtype=np.uint16)


@pytest.mark.parametrize("K", [32, 256, 7168])
def test_rms_constant_rows_closed_forms(oracle_mod, K):
    one = np.full(K, 0x3F80, dtype=np.uint16)                 # w = 1
    # eps = 0: a constant row normalizes to +-1
    for vb, hb in [(0x3F00, 0x3F80), (0xC140, 0xBF80), (0x0001, 0x3F80)]:
        q, s, r, h = oracle_mod.add_rms_norm_quant(_row(vb, K), None, one, 0.0)
        assert r is None and np.all(h == hb)
    # v = 0.5, eps = 0.75: mean of squares 0.25, 1/sqrt(1) -> h = 0.5
    q, s, r, h = oracle_mod.add_rms_norm_quant(_row(0x3F00, K), None, one, 0.75)
    assert np.all(h == 0x3F00)
    # w = 2 doubles it; w = -0.25 scales it exactly
    q, s, r, h = oracle_mod.add_rms_norm_quant(_row(0x3F00, K), None,
                                               np.full(K, 0x4000, np.uint16), 0.75)
    assert np.all(h == 0x3F80)
    q, s, r, h = oracle_mod.add_rms_norm_quant(_row(0x3F00, K), None,
                                               np.full(K, 0xBE80, np.uint16), 0.75)
    assert np.all(h == 0xBE00)
    # a zero row stays zero (eps > 0) and quantizes to scale 0
    q, s, r, h = oracle_mod.add_rms_norm_quant(_row(0x0000, K), None, one, 1e-6)
    assert np.all(h == 0) and s[0] == 0 and np.all(q == 0)


def test_rms_power_of_two_scaling_invariance(oracle_mod):
    rng = np.random.default_rng(21)
    x = rng.standard_normal((4, 512)).astype(np.float32)
    w = _bf16_bits(rng.uniform(0.5, 1.5, 512).astype(np.float32))
    base = oracle_mod.add_rms_norm_quant(_bf16_bits(x), None, w, 0.0)
    for j in (-20, -3, 5, 30):
        out = oracle_mod.add_rms_norm_quant(_bf16_bits(x * np.float32(2.0 ** j)), None, w, 0.0)
        for a, b in zip(base, out):
            if a is not None:
                assert np.array_equal(a, b)


@pytest.mark.parametrize("eps", [1e-6, 1e-5, 0.5])
def test_rms_against_torch_float64(oracle_mod, eps):
    rng = np.random.default_rng(22)
    M, K = 16, 2048
    x = _bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = _bf16_bits(rng.uniform(-2, 2, K).astype(np.float32))
    q, s, r, h = oracle_mod.add_rms_norm_quant(x, None, w, eps)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(_bf16_f64(x)), (K,),
                                       torch.from_numpy(_bf16_f64(w)), eps)
    ref_bits = _bf16_bits(ref.numpy().astype(np.float32))
    apart = _steps_apart(h, ref_bits)
    assert apart.max() <= 1
    assert (apart == 0).mean() > 0.995
    # unit weight, eps = 0: mean of h^2 is 1 to bf16 precision
    q, s, r, h = oracle_mod.add_rms_norm_quant(x, None, np.full(K, 0x3F80, np.uint16), 0.0)
    ms = (_bf16_f64(h) ** 2).mean(axis=1)
    assert np.all(np.abs(ms - 1.0) < 2.0 ** -7)


def test_rms_residual_add(oracle_mod):
    rng = np.random.default_rng(23)
    M, K = 8, 1024
    # magnitudes in [1/64, 4]: every bf16 sum is exact in fp32, so torch's
    # bf16 add (fp32 add, one rounding) is the correctly rounded sum
    mag = lambda: np.exp2(rng.uniform(-6, 2, (M, K))) * rng.choice([-1, 1], (M, K))
    x = _bf16_bits(mag().astype(np.float32))
    res = _bf16_bits(mag().astype(np.float32))
    w = _bf16_bits(rng.uniform(0.5, 1.5, K).astype(np.float32))
    q, s, r, h = oracle_mod.add_rms_norm_quant(x, res, w, 1e-6)
    tx = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    tr = torch.from_numpy(res.view(np.int16)).view(torch.bfloat16)
    want_r = (tx + tr).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(r, want_r)
    # the norm then runs on the new residual exactly as without a residual
    q2, s2, r2, h2 = oracle_mod.add_rms_norm_quant(r, None, w, 1e-6)
    assert np.array_equal(h, h2) and np.array_equal(q, q2) and np.array_equal(s, s2)


def test_rms_quantizer_is_applied_to_the_normalized_row(oracle_mod):
    rng = np.random.default_rng(24)
    x = _bf16_bits(rng.standard_normal((6, 768)).astype(np.float32))
    w = _bf16_bits(rng.uniform(-1, 1, 768).astype(np.float32))
    q, s, r, h = oracle_mod.add_rms_norm_quant(x, None, w, 1e-5)
    q2, s2 = oracle_mod.quant_rows(h)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    # the row's largest |h| sits at +-448 after scaling
    assert np.all(np.max(q & 0x7F, axis=1) == 0x7E)


# ----------------------------------------------------------------- SiLU*up
def test_silu_mul_against_torch_float64(oracle_mod):
    rng = np.random.default_rng(31)
    M, I = 8, 4096
    gu = _bf16_bits((rng.standard_normal((M, 2 * I)) * 3).astype(np.float32))
    q, s, a = oracle_mod.silu_mul_quant(gu)
    g = torch.from_numpy(_bf16_f64(gu[:, :I]))
    u = torch.from_numpy(_bf16_f64(gu[:, I:]))
    ref_bits = _bf16_bits((torch.nn.functional.silu(g) * u).numpy().astype(np.float32))
    apart = _steps_apart(a, ref_bits)
    assert apart.max() <= 1
    assert (apart == 0).mean() > 0.995
    q2, s2 = oracle_mod.quant_rows(a)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_silu_mul_half_order_and_limits(oracle_mod):
    I = 64
    g = np.linspace(-6, 6, I).astype(np.float32)
    gb = _bf16_bits(g)
    ones = np.full(I, 0x3F80, np.uint16)
    # up = 1: a is silu(gate) alone; swapping the halves gives silu(1) everywhere
    q, s, a = oracle_mod.silu_mul_quant(np.concatenate([gb, ones])[None])
    ref = _bf16_bits(torch.nn.functional.silu(torch.from_numpy(_bf16_f64(gb))).numpy()
                     .astype(np.float32))
    assert _steps_apart(a[0], ref).max() <= 1
    q, s, a_sw = oracle_mod.silu_mul_quant(np.concatenate([ones, gb])[None])
    assert not np.array_equal(a_sw[0], a[0])
    # gate = 0 gives zero whatever up is
    q, s, a0 = oracle_mod.silu_mul_quant(np.concatenate([np.zeros(I, np.uint16), gb])[None])
    assert np.all((a0 & 0x7FFF) == 0) and s[0] == 0
    # large gates: silu(g) = g to binary32, so a = bf16(g * up) (exact in fp32)
    big = _bf16_bits(np.full(I, 96.0, np.float32))
    q, s, a = oracle_mod.silu_mul_quant(np.concatenate([big, gb])[None])
    assert np.array_equal(a[0], _bf16_bits(96.0 * _bf16_f64(gb).astype(np.float32)))
    # very negative gates: silu(g) underflows toward -0
    neg = _bf16_bits(np.full(I, -120.0, np.float32))
    q, s, a = oracle_mod.silu_mul_quant(np.concatenate([neg, ones])[None])
    assert np.all(np.abs(_bf16_f64(a[0])) < 1e-38)


def test_producer_workload_generators_are_seeded():
    a = synth.producer_inputs("add_rms", 4, 256, seed=3)
    b = synth.producer_inputs("add_rms", 4, 256, seed=3)
    for k in a:
        if isinstance(a[k], np.ndarray):
            assert np.array_equal(a[k], b[k])
    c = synth.producer_inputs("silu_mul", 4, 256, seed=3)
    assert c["gate_up"].shape == (4, 512)
