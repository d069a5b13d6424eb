"""Pins against facts the pages print, stored as small text fixtures under
tests/golden/ (each fixture names the page and section it comes from)."""
import math
import os

import numpy as np
import pytest

import mxfp4_gemm_transformer_amd as bs
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.lstrip().startswith("#")]


def _gelu_shader():
    return {k: float(v) for k, v in _lines("gelu_tanh_shader.txt")}


def test_gelu_oracle_matches_the_printed_shader_formula(oracle_mod):
    g = _gelu_shader()
    # The printed coefficient is sqrt(2/pi) to ten decimals.
    assert abs(g["c1"] - math.sqrt(2.0 / math.pi)) < 5e-11
    xs = np.concatenate([np.linspace(-8.0, 8.0, 1601), [0.0, 1e-6, -1e-6, 12.0, -12.0]])
    for x in xs:
        u = min(max(g["c1"] * (x + g["c3"] * x ** 3), g["clamp_lo"]), g["clamp_hi"])
        shader = 0.5 * x * (1.0 + math.tanh(u))
        # The oracle uses sqrt(2/pi) in full and no clamp: the printed
        # constant's last-digit rounding moves the result by < 1e-10, and the
        # clamp at |u| = 15 changes tanh by < 1e-12.
        assert abs(oracle_mod.gelu_tanh(x) - shader) <= 1e-10 * (1.0 + abs(x))


def _eval(expr, N, K):
    return {"N": N, "K": K, "N//32": N // 32, "K//32": K // 32, "K//2": K // 2}[expr]


def test_printed_scale_grid_shapes_match_the_boundary_layout():
    op = {"e4m3": 0, "fp4": 1}
    checked = 0
    for row in _lines("scale_grids.txt"):
        if row[0] == "shape":
            fmt, N, K, wr, wc, sr, sc = row[1], *map(int, row[2:])
            assert bs.weight_shape(op[fmt], N, K) == (wr, wc)
            assert bs.w_scale_shape(op[fmt], N, K) == (sr, sc)
            checked += 1
        elif row[0] == "rule":
            fmt, wr, wc, sr, sc = row[1:]
            for N, K in [(256, 256), (2048, 7168), (7168, 8192), (34816, 5120), (96, 160)]:
                assert bs.weight_shape(op[fmt], N, K) == (_eval(wr, N, K), _eval(wc, N, K))
                assert bs.w_scale_shape(op[fmt], N, K) == (_eval(sr, N, K), _eval(sc, N, K))
                checked += 1
    assert checked >= 11


@pytest.mark.parametrize("name", ["tiny", "decode", "gate_up"])
def test_generated_weights_follow_the_printed_layout(name):
    wl = synth.WORKLOADS[name]
    if wl.fmt == "mxfp4":
        wl = synth.Workload("gate_up_small", 1, 256, 512, "mxfp4", synth.EPI_NONE)
        w, ws = synth.weights(wl)
    else:
        w, ws = synth.weights(wl)
    op = 0 if wl.fmt == "fp8" else 1
    assert w.shape == bs.weight_shape(op, wl.N, wl.K)
    assert ws.shape == bs.w_scale_shape(op, wl.N, wl.K)
    if name == "decode":
        assert ws.shape == (64, 224)   # the printed wqkv_scale grid
