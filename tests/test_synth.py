"""The seeded workloads: determinism, value laws, and the weight preparation
checked bit for bit against the oracle's own encoders."""
import numpy as np
import pytest

import synth


def test_deterministic_and_prefix_stable():
    wl = synth.WORKLOADS["decode"]
    a64 = synth.activations(wl, 64)
    assert np.array_equal(a64, synth.activations(wl, 64))
    for M in wl.m_sweep:
        assert np.array_equal(synth.activations(wl, M), a64[:M])
    assert not np.array_equal(synth.activations(wl, 8, seed=1), a64[:8])


def test_tiny_workload_laws(oracle_mod):
    d = synth.make("tiny")
    wl = d["wl"]
    assert d["a_bf16"].shape == (16, 256) and d["w"].shape == (256, 256)
    assert d["w_scale"].shape == (8, 8) and d["bias"].shape == (256,)
    assert d["w_scale"].min() >= 120 and d["w_scale"].max() <= 130
    vals = synth.weight_values(wl)
    # every stored weight code is the oracle's encoding of its sample
    assert np.array_equal(d["w"], oracle_mod.encode_e4m3(vals))


@pytest.mark.parametrize("name", ["decode", "ffn_up", "prefill"])
def test_e4m3_weight_codes_equal_oracle_encoding(oracle_mod, name):
    wl = synth.WORKLOADS[name]
    w, ws = synth.weights(wl)
    assert w.shape == (wl.N, wl.K) and ws.shape == (wl.N // 32, wl.K // 32)
    assert ws.min() == 120 and ws.max() == 130
    rows = slice(wl.N - 64, wl.N)
    vals = synth.weight_values(wl, rows=rows)
    assert np.array_equal(w[rows], oracle_mod.encode_e4m3(vals))
    assert np.array_equal(w[:32], oracle_mod.encode_e4m3(synth.weight_values(wl, rows=slice(0, 32))))


def test_mxfp4_weights_equal_oracle_conversion(oracle_mod):
    wl = synth.WORKLOADS["gate_up"]
    rows = slice(2048 - 40, 2048 + 24)   # spans a generation chunk boundary
    vals = synth.weight_values(wl, rows=rows)
    packed, scales = synth._mx_quantize_rows(vals)
    p_ref, s_ref = oracle_mod.quant_mxfp4_weights(vals)
    assert np.array_equal(packed, p_ref) and np.array_equal(scales, s_ref)


def test_prefill_outlier_columns():
    wl = synth.WORKLOADS["prefill"]
    a = synth.activations(wl, 256)
    import torch
    x = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).float().numpy()
    col_std = x.std(axis=0)
    big = np.sum(col_std > 5)
    assert big == round(0.01 * wl.K) == 82
    assert np.all((col_std > 14) | (col_std < 1.5))


def test_bias_presence():
    assert synth.bias(synth.WORKLOADS["decode"]) is None
    assert synth.bias(synth.WORKLOADS["ffn_up"]).shape == (4096,)
    assert synth.bias(synth.WORKLOADS["ffn_up_bias"]).shape == (4096,)
