"""Pins of the oracle's number formats against sources other than itself.

The pages name the formats only by dtype (torch.float8_e4m3fn,
torch.float4_e2m1fn_x2, "uint8 E8M0" on the vLLM DeepSeek-V4 AMD mono runner
page, AttnWeights and MonoLayerWeights); the checks below use torch's own
float8 / bfloat16 conversions (an independent implementation), the OCP
format tables and the E8M0 closed form 2^(s-127).
"""
import math

import numpy as np
import pytest
import torch


def _torch_e4m3(codes):
    t = torch.tensor(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def test_e4m3_table_equals_torch_decoder(oracle_mod):
    ours = oracle_mod.e4m3_table()
    ref = _torch_e4m3(np.arange(256))
    nan_ours = np.isnan(ours)
    assert np.array_equal(nan_ours, np.isnan(ref))
    assert np.array_equal(ours[~nan_ours], ref[~nan_ours])
    # signed zeros survive too
    assert np.array_equal(np.signbit(ours[~nan_ours]), np.signbit(ref[~nan_ours]))


def test_e4m3_spot_values_and_nan_codes(oracle_mod):
    v = oracle_mod.e4m3_value
    assert v(0x00) == 0.0 and not math.copysign(1, v(0x00)) < 0
    assert v(0x80) == 0.0 and math.copysign(1, v(0x80)) < 0
    assert v(0x01) == 2.0 ** -9          # smallest subnormal
    assert v(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert v(0x08) == 2.0 ** -6          # smallest normal
    assert v(0x38) == 1.0
    assert v(0x7E) == 448.0              # largest finite
    assert v(0xFE) == -448.0
    nan_codes = [c for c in range(256) if math.isnan(v(c))]
    assert nan_codes == [0x7F, 0xFF]


def test_e4m3_monotone_and_sign_symmetric(oracle_mod):
    t = oracle_mod.e4m3_table()
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)
    for c in range(0x7F):
        assert t[c | 0x80] == -t[c]


def test_e2m1_table_is_the_ocp_table(oracle_mod):
    t = oracle_mod.e2m1_table()
    assert list(t[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(t[8:]) == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    assert math.copysign(1, t[8]) < 0


def test_e2m1_values_are_e4m3_values(oracle_mod):
    # cross-format fact used by the cross-format GEMM pin
    e4 = oracle_mod.e4m3_table()
    codes = {0.0: 0x00, 0.5: 0x30, 1.0: 0x38, 1.5: 0x3C, 2.0: 0x40, 3.0: 0x44, 4.0: 0x48, 6.0: 0x4C}
    for val, c in codes.items():
        assert e4[c] == val


def test_e8m0_closed_form(oracle_mod):
    for s in range(255):
        assert oracle_mod.e8m0_value(s) == math.ldexp(1.0, s - 127)
    assert oracle_mod.e8m0_value(127) == 1.0
    assert oracle_mod.e8m0_value(128) == 2.0
    assert math.isnan(oracle_mod.e8m0_value(255))


def test_bf16_decoder_equals_torch(oracle_mod):
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, size=4000, dtype=np.uint32).astype(np.uint16)
    bits = np.concatenate([bits, np.array([0x0000, 0x8000, 0x0001, 0x3F80, 0x7F7F, 0xFF7F],
                                          dtype=np.uint16)])
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    for b, r in zip(bits, ref):
        o = oracle_mod.bf16_value(int(b))
        if math.isnan(r):
            assert math.isnan(o)
        else:
            assert o == r


def test_e4m3_encode_round_trips_every_finite_code(oracle_mod):
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle_mod.e4m3_encode(oracle_mod.e4m3_value(c)) == c


def test_e4m3_encode_ties_go_to_even_mantissa(oracle_mod):
    t = oracle_mod.e4m3_table()
    for c in range(0x7E):
        lo, hi = t[c], t[c + 1]
        mid = 0.5 * (lo + hi)
        even = c if c % 2 == 0 else c + 1
        assert oracle_mod.e4m3_encode(mid) == even, hex(c)
        assert oracle_mod.e4m3_encode(-mid) == even | 0x80
        below = np.nextafter(np.float32(mid), np.float32(-1))
        above = np.nextafter(np.float32(mid), np.float32(1000))
        assert oracle_mod.e4m3_encode(float(below)) == c
        assert oracle_mod.e4m3_encode(float(above)) == c + 1


def test_e4m3_encode_saturates_and_keeps_sign(oracle_mod):
    enc = oracle_mod.e4m3_encode
    for v in (448.0, 448.5, 464.0, 470.0, 480.0, 1e6, 3.4e38):
        assert enc(v) == 0x7E
        assert enc(-v) == 0xFE
    assert enc(0.0) == 0x00
    assert enc(-0.0) == 0x80
    assert enc(-1e-30) == 0x80
    assert enc(2.0 ** -10) == 0x00          # tie between 0 and 2^-9 -> even (0)
    assert enc(-2.0 ** -10) == 0x80
    assert enc(1.5 * 2.0 ** -9) == 0x02     # tie between codes 1 and 2 -> 2


def test_e4m3_encode_equals_torch_cast_below_saturation(oracle_mod):
    # torch's float8_e4m3fn cast rounds to nearest-even; within the finite
    # range it must agree with the oracle's encoder on every value.
    rng = np.random.default_rng(7)
    mag = np.exp2(rng.uniform(-14, np.log2(448.0), size=200000)).astype(np.float32)
    v = (mag * rng.choice([-1, 1], size=mag.size)).astype(np.float32)
    v = v[np.abs(v) <= 448.0]
    ours = oracle_mod.encode_e4m3(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e2m1_encode_rules(oracle_mod):
    enc = oracle_mod.e2m1_encode
    table = oracle_mod.e2m1_table()
    for c in range(16):
        assert enc(table[c]) == c
    # midpoint ties resolve to the even code
    assert enc(0.25) == 0x0
    assert enc(0.75) == 0x2
    assert enc(1.25) == 0x2
    assert enc(1.75) == 0x4
    assert enc(2.5) == 0x4
    assert enc(3.5) == 0x6
    assert enc(5.0) == 0x6
    assert enc(-5.0) == 0xE
    # just off the ties
    assert enc(np.nextafter(5.0, 10.0)) == 0x7
    assert enc(np.nextafter(0.25, 1.0)) == 0x1
    # saturation
    assert enc(7.0) == 0x7 and enc(100.0) == 0x7 and enc(-100.0) == 0xF


def test_gelu_tanh_equals_torch_and_identities(oracle_mod):
    xs = np.concatenate([np.linspace(-12, 12, 2001), [0.0, 1e-8, -1e-8, 30.0, -30.0]])
    ref = torch.nn.functional.gelu(torch.from_numpy(xs), approximate="tanh").numpy()
    ours = np.array([oracle_mod.gelu_tanh(x) for x in xs])
    # 1 + tanh(u) cancels for large negative u in both, so the bound is absolute there
    assert np.allclose(ours, ref, rtol=1e-13, atol=1e-14)
    assert oracle_mod.gelu_tanh(0.0) == 0.0
    for x in (0.1, 0.7, 1.3, 3.0, 8.0):
        assert abs(oracle_mod.gelu_tanh(x) - oracle_mod.gelu_tanh(-x) - x) < 1e-15 * (1 + x)
    assert abs(oracle_mod.gelu_tanh(20.0) / 20.0 - 1.0) < 1e-15
    # the constants of the cortiq vit.rs shader: sqrt(2/pi) ~ 0.7978845608, 0.044715
    x = 0.9
    c = 0.7978845608
    shader = 0.5 * x * (1 + math.tanh(c * (x + 0.044715 * x ** 3)))
    assert abs(oracle_mod.gelu_tanh(x) - shader) < 1e-10
