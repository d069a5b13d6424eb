"""bench.py's host-side pieces, on the CPU: the algorithmic bytes and FLOPs
each roofline divides by (against the per-configuration figures worked out
from the format definitions: weights, E8M0 grid, e4m3 codes and fp32 scales
of A, bf16 Y and bias), the parity sample's coverage, the CPU-baseline leg,
and the refusal of more than one GPU."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def _alg(name, M):
    return bench.algorithmic(synth.WORKLOADS[name], M)


@pytest.mark.parametrize("name,M,gemm_bytes", [
    ("tiny", 16, 78464),
    # 2048 x 7168 e4m3 + [64, 224] E8M0 + M x 7168 codes + 4M scale bytes + 2 x M x 2048 out
    ("decode", 1, 14680064 + 14336 + 7168 + 4 + 4096),
    ("decode", 8, 14784544),
    ("decode", 64, 14680064 + 14336 + 64 * 7168 + 256 + 2 * 64 * 2048),
    # 34816 x 2560 fp4 pairs + [34816, 160] E8M0 + A + out
    ("gate_up", 1, 89128960 + 5570560 + 5120 + 4 + 69632),
])
def test_algorithmic_bytes(name, M, gemm_bytes):
    assert _alg(name, M)["gemm_bytes"] == gemm_bytes


def test_algorithmic_rounded_figures():
    # the same quantities to the precision they are usually quoted at
    assert round(_alg("decode", 16)["gemm_bytes"] / 1e6, 2) == 14.87
    assert round(_alg("decode", 64)["gemm_bytes"] / 1e6, 2) == 15.42
    c3 = _alg("prefill", 4096)
    assert round(c3["gemm_bytes"] / 1e6, 1) == 151.1
    assert round(c3["gemm_flops"] / 1e9, 2) == 481.04
    c4 = _alg("ffn_up", 2048)
    assert round(c4["gemm_bytes"] / 1e6, 2) == 23.09
    assert round(c4["gemm_flops"] / 1e9, 2) == 17.18
    assert round(_alg("gate_up", 16)["gemm_bytes"] / 1e6, 2) == 95.90
    assert round(_alg("gate_up", 512)["gemm_bytes"] / 1e6, 1) == 133.0
    assert round(_alg("gate_up", 4096)["gemm_bytes"] / 1e6, 1) == 400.9
    # the quantizer moves bf16 in, codes and fp32 scales out: 3 M K + 4 M
    assert _alg("prefill", 4096)["quant_bytes"] == 3 * 4096 * 8192 + 4 * 4096


def test_sample_points_cover_every_scale_block():
    rng = np.random.default_rng(0)
    M, N = 4096, 7168
    ms, ns, how = bench._sample_points(M, N, rng)
    assert ms.min() >= 0 and ms.max() < M and ns.min() >= 0 and ns.max() < N
    # every (row block of 64, 32-column block) pair has a sampled output
    hit = np.zeros((M // 64, N // 32), dtype=bool)
    hit[ms // 64, ns // 32] = True
    assert hit.all()
    # small outputs are checked whole
    ms2, ns2, how2 = bench._sample_points(16, 256, rng)
    assert len(ms2) == 16 * 256 and "all" in how2


def test_cpu_baseline_leg_runs_the_oracle():
    wl = synth.WORKLOADS["tiny"]
    d = synth.make("tiny", 16)
    rec = bench.cpu_baseline(d, wl, 16, bench.algorithmic(wl, 16), False, 0.05)
    assert rec["kind"] == "oracle" and rec["value"] > 0 and rec["cores"] >= 1
    assert rec["gflops"] > 0 and rec["single_core"]["cores"] == 1


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
