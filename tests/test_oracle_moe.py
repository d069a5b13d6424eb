"""Pins of the oracle's grouped (MoE) W4A8 GEMM: each expert's rows against
a dequantize-then-matmul of that expert alone in numpy and against the
dense W4A8 GEMM on the expert's slice, with empty experts, one expert
holding every row, and the row order the routing generator produces."""
import numpy as np
import pytest
import torch

import synth

E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])


def _dequant_w(packed, scales):
    codes = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    codes[:, 0::2] = packed & 15
    codes[:, 1::2] = packed >> 4
    return E2M1[codes] * np.repeat(np.exp2(scales.astype(np.float64) - 127), 32, axis=1)


def _e4m3(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()


def _case(oracle_mod, T0, E, topk, N, K, seed):
    rng = np.random.default_rng(seed)
    x = synth.to_bf16_bits(rng.standard_normal((T0, K)).astype(np.float32))
    row_token, off = synth.moe_routing(T0, E, topk, seed=seed)
    a, s = oracle_mod.quant_rows(x[row_token])
    w, ws = synth.moe_weights(E, N, K, seed=seed)
    b = synth.to_bf16_bits((rng.standard_normal((E, N)) * 0.1).astype(np.float32))
    return a, s, off, w, ws, b


@pytest.mark.parametrize("epi", [0, 1])
def test_grouped_equals_dequantized_matmul_per_expert(oracle_mod, epi):
    a, s, off, w, ws, b = _case(oracle_mod, 6, 8, 3, 64, 256, 81)
    out, absum = oracle_mod.gemm_mxfp4_w4a8_grouped(a, s, off, w, ws, b if epi else None, epi)
    for e in range(8):
        r0, r1 = off[e], off[e + 1]
        if r0 == r1:
            continue
        ad = _e4m3(a[r0:r1]) * s[r0:r1, None].astype(np.float64)
        ref = ad @ _dequant_w(w[e], ws[e]).T
        if epi:
            ref = ref + torch.from_numpy(b[e].view(np.int16)).view(torch.bfloat16).double().numpy()
        assert np.allclose(out[r0:r1], ref, rtol=1e-12, atol=1e-12)


def test_grouped_equals_dense_per_expert_slice(oracle_mod):
    a, s, off, w, ws, b = _case(oracle_mod, 8, 16, 4, 96, 320, 82)
    out, absum = oracle_mod.gemm_mxfp4_w4a8_grouped(a, s, off, w, ws, b, 2)
    assert np.any(np.diff(off) == 0), "the case should hold an empty expert"
    for e in range(16):
        r0, r1 = off[e], off[e + 1]
        if r0 == r1:
            continue
        o2, a2 = oracle_mod.gemm_mxfp4_w4a8(a[r0:r1], s[r0:r1], w[e], ws[e], b[e], 2)
        assert np.array_equal(out[r0:r1], o2) and np.array_equal(absum[r0:r1], a2)


def test_one_expert_holding_every_row(oracle_mod):
    rng = np.random.default_rng(83)
    a, s = oracle_mod.quant_rows(synth.to_bf16_bits(rng.standard_normal((10, 128)).astype(np.float32)))
    w, ws = synth.moe_weights(4, 64, 128, seed=83)
    off = np.array([0, 0, 10, 10, 10], np.int32)
    out, _ = oracle_mod.gemm_mxfp4_w4a8_grouped(a, s, off, w, ws)
    o2, _ = oracle_mod.gemm_mxfp4_w4a8(a, s, w[1], ws[1])
    assert np.array_equal(out, o2)


def test_routing_generator_groups_rows_by_expert():
    row_token, off = synth.moe_routing(8, 32, 8, seed=0)
    assert off[0] == 0 and off[-1] == 64 and np.all(np.diff(off) >= 0)
    for e in range(32):                        # each expert's tokens are distinct and sorted
        toks = row_token[off[e]:off[e + 1]]
        assert np.all(np.diff(toks) > 0)
    assert np.array_equal(np.bincount(row_token, minlength=8), np.full(8, 8))
