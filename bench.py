"""Benchmark of the block-scaled linear layer on one MI355X.

A step is one pass of the whole path over one batch: per-token quantization
of bf16 activations (fp8_quant_rows) followed by the block-scaled GEMM with
its fused epilogue (gemm_bs_fp8 / gemm_mxfp4_w4a8). Inputs are resident in
HBM before timing starts. Weights rotate over >= 512 MiB of distinct copies
(twice the 256 MiB last-level cache), one copy per step, so every step reads
its weights from HBM as a real layer stack would.

Timed steps are captured once into a HIP graph and replayed, so the timing
is of GPU work, not of Python launch overhead. Output: one JSON line with
the throughput of the whole step, the roofline of the dominant kernel (its
algorithmic bytes or FLOPs per launch over its average launch time from HIP
events), and the CPU oracle's rate on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload decode --m 8]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-scaled GEMM TFLOP/s (prefill) + HBM GB/s (decode), % roofline, 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # dense fp8 MFMA
FP4_PEAK_TFLOPS = 10100.0      # dense MXFP4 MFMA
ROTATION_BYTES = 512 << 20


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None)
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--workload", default="decode",
                   choices=["tiny", "decode", "prefill", "prefill_shard", "ffn_up", "ffn_up_bias", "gate_up",
                            "gate_up_w4a4", "lm_head", "moe", "add_rms", "silu_mul"],
                   help="a GEMM workload (quantize + GEMM per step), or a fused producer "
                        "(add_rms: residual add + RMSNorm + quantize on [M, 5120]; silu_mul: "
                        "SiLU(gate) * up + quantize on [M, 2 x 17408])")
    p.add_argument("--m", type=int, default=None, help="token count (M) for sweep workloads")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="CPU oracle budget for the cpu_baseline leg (0 disables it)")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                   help="only run a plain device copy of BYTES bytes three times (the "
                        "reference for scaling FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


def kernel_source(kernel: str, M: int) -> str:
    import mxfp4_gemm_transformer_amd as bs
    csrc = os.path.join(os.path.dirname(bs.library_path()), "csrc")
    return os.path.join(csrc, "gemm_decode.hip" if M <= 64 else "gemm_prefill.hip")


def measured_traffic(kernel: str, workload: str, M: int):
    """HBM bytes per launch from the committed counter record, if it was taken
    on the kernel source as it stands (same sha256), else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get("%s %s M=%d" % (kernel, workload, M))
    except (OSError, ValueError):
        return None
    if not rec:
        return None
    with open(kernel_source(kernel, M), "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec.get("source_sha256"):
            return None
    return rec.get("traffic_bytes_per_launch")


def calibrate_copy(nbytes: int):
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": nbytes, "copies": 3}))


def algorithmic(wl, M):
    """Bytes each kernel must move and the GEMM's FLOPs, by definition."""
    N, K = wl.N, wl.K
    if wl.fmt == "mxfp4_w4a4":   # fp4 codes + one E8M0 byte per 32
        quant = 2 * M * K + M * K // 2 + M * K // 32
        a_bytes = M * K // 2 + M * K // 32
    else:
        quant = 2 * M * K + M * K + 4 * M                  # bf16 in, codes + scales out
        a_bytes = M * K + 4 * M
    w_bytes = N * K // 2 if wl.fmt in ("mxfp4", "mxfp4_w4a4") else N * K
    ws_bytes = {"fp8": (N // 32) * (K // 32), "mxfp4": N * (K // 32), "mxfp4_w4a4": N * (K // 32),
                "fp8_rowwise": 4 * N}[wl.fmt]
    gemm = w_bytes + ws_bytes + a_bytes + 2 * M * N
    if wl.epilogue:
        gemm += 2 * N
    return {"quant_bytes": quant, "gemm_bytes": gemm, "gemm_flops": 2 * M * N * K}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the layer's kernels run on one device and this "
              "build has no multi-GPU path (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    import torch
    import mxfp4_gemm_transformer_amd as bs
    import synth

    if args.workload in synth.PRODUCERS:
        bench_producer(args)
        return
    if args.workload == "moe":
        bench_moe(args)
        return

    wl = synth.WORKLOADS[args.workload]
    M = args.m if args.m is not None else wl.M
    big = 2 * M * wl.N * wl.K > 50e9
    steps = args.steps if args.steps is not None else (50 if big else 1000)
    warmup = args.warmup if args.warmup is not None else (5 if big else 50)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- inputs, resident in HBM
    d = synth.make(args.workload, M)
    x = torch.from_numpy(d["a_bf16"].view(np.int16)).view(torch.bfloat16).to(dev)
    w_host, ws_host = d["w"], d["w_scale"]
    w_bytes = w_host.nbytes + ws_host.nbytes
    copies = max(2, math.ceil(ROTATION_BYTES / w_bytes))
    w0 = torch.from_numpy(w_host).to(dev)
    ws0 = torch.from_numpy(ws_host).to(dev)
    ws_list = [w0] + [w0.clone() for _ in range(copies - 1)]
    wss_list = [ws0] + [ws0.clone() for _ in range(copies - 1)]
    bias = None
    if d["bias"] is not None:
        bias = torch.from_numpy(d["bias"].view(np.int16)).view(torch.bfloat16).to(dev)
    epi = d["epilogue"]
    w4a4 = wl.fmt == "mxfp4_w4a4"
    if w4a4:
        q = torch.empty((M, wl.K // 2), dtype=torch.uint8, device=dev)
        s = torch.empty((M, wl.K // 32), dtype=torch.uint8, device=dev)
        quant = lambda: bs.fp4_quant_rows(x, q, s)
    else:
        q = torch.empty((M, wl.K), dtype=torch.uint8, device=dev)
        s = torch.empty((M,), dtype=torch.float32, device=dev)
        quant = lambda: bs.fp8_quant_rows(x, q, s)
    y = torch.empty((M, wl.N), dtype=torch.bfloat16, device=dev)
    gemm = {"fp8": bs.gemm_bs_fp8, "mxfp4": bs.gemm_mxfp4_w4a8, "mxfp4_w4a4": bs.gemm_mxfp4_w4a4,
            "fp8_rowwise": bs.gemm_fp8_rowwise}[wl.fmt]
    work = None
    need = bs.bs_workspace_bytes({"fp8": 0, "mxfp4": 1, "fp8_rowwise": 2, "mxfp4_w4a4": 3}[wl.fmt],
                                 M, wl.N, wl.K)
    if need:
        work = torch.zeros((need,), dtype=torch.uint8, device=dev)

    def step(i):
        quant()
        gemm(q, s, ws_list[i % copies], wss_list[i % copies], bias, epi, y=y, workspace=work)

    def gemm_only(i):
        gemm(q, s, ws_list[i % copies], wss_list[i % copies], bias, epi, y=y, workspace=work)

    def quant_only(i):
        quant()

    stream = torch.cuda.Stream()

    def capture(fn, count, offset=0):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(count):
                fn(offset + i)
        return g

    # ---- warmup: eager steps, then the captured graphs' first replays
    with torch.cuda.stream(stream):
        for i in range(warmup):
            step(i)
    torch.cuda.synchronize()
    g_step = capture(step, steps)
    g_gemm = capture(gemm_only, steps)
    g_quant = capture(quant_only, steps)
    for g in (g_step, g_gemm, g_quant):
        g.replay()
    torch.cuda.synchronize()

    def timed(g):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3      # seconds

    # ---- the timed K steps (whole path), then per-kernel averages
    t0 = time.perf_counter()
    step_s = timed(g_step)
    wall_s = time.perf_counter() - t0
    gemm_s = timed(g_gemm) / steps
    quant_s = timed(g_quant) / steps

    alg = algorithmic(wl, M)
    step_bytes = alg["quant_bytes"] + alg["gemm_bytes"]
    ms_per_step = step_s / steps * 1e3
    # the binding roof: the longer of the GEMM's FLOPs at the format's MFMA
    # peak and its bytes at the HBM peak (ridge 625 flop/B for e4m3, 1262 for
    # MXFP4)
    peak = FP4_PEAK_TFLOPS if wl.fmt in ("mxfp4", "mxfp4_w4a4") else FP8_PEAK_TFLOPS
    compute_bound = alg["gemm_flops"] / (peak * 1e12) >= alg["gemm_bytes"] / (HBM_PEAK_GBS * 1e9)
    if compute_bound:
        unit = "TFLOP/s"
        value = alg["gemm_flops"] * steps / step_s / 1e12
        achieved = alg["gemm_flops"] / gemm_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
        if wl.fmt == "mxfp4":
            roof["frac_vs_fp8_rate"] = round(achieved / FP8_PEAK_TFLOPS, 4)
    else:
        unit = "GB/s"
        value = step_bytes * steps / step_s / 1e9
        achieved = alg["gemm_bytes"] / gemm_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof["kernel"] = {"fp8": "gemm_bs_fp8", "mxfp4": "gemm_mxfp4_w4a8", "mxfp4_w4a4": "gemm_mxfp4_w4a4",
                      "fp8_rowwise": "gemm_fp8_rowwise"}[wl.fmt]
    roof["traffic"] = measured_traffic(roof["kernel"], wl.name, M)
    roof["avg_launch_us"] = round(gemm_s * 1e6, 3)
    roof["algorithmic_bytes_per_launch"] = alg["gemm_bytes"]
    roof["algorithmic_flops_per_launch"] = alg["gemm_flops"]

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"mxfp4": "fp8_e4m3 x fp4_e2m1", "mxfp4_w4a4": "fp4_e2m1 x fp4_e2m1"}.get(wl.fmt, "fp8_e4m3"),
        "data": "synthetic",
        "config": {"workload": "%s M=%d N=%d K=%d (%s weights, %s scales, epilogue %s)" % (
            wl.name, M, wl.N, wl.K, "MXFP4 e2m1" if wl.fmt in ("mxfp4", "mxfp4_w4a4") else "e4m3",
            {"fp8": "32x32 E8M0", "mxfp4": "1x32 E8M0", "mxfp4_w4a4": "1x32 E8M0, MXFP4 activations",
             "fp8_rowwise": "fp32 per-channel"}[wl.fmt],
            ["none", "bias", "bias+tanh-GELU"][epi]),
            "M": M, "N": wl.N, "K": wl.K, "weight_copies_rotated": copies,
            "step": "%s + %s" % ("fp4_quant_rows" if w4a4 else "fp8_quant_rows", roof["kernel"]),
            "graph_replay": True},
        "roofline": roof,
        "kernels_us": {("fp4_quant_rows" if w4a4 else "fp8_quant_rows"): round(quant_s * 1e6, 3),
                       roof["kernel"]: round(gemm_s * 1e6, 3)},
        "step_bytes": step_bytes, "wall_s_timed_region": round(wall_s, 6),
    }
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(d, wl, M, alg, compute_bound, args.cpu_seconds)
    print(json.dumps(result))


def cpu_baseline(d, wl, M, alg, compute_bound, budget_s):
    """The CPU oracle, as it stands, on the same workload: quantization then
    the GEMM in fp64 with OpenMP over outputs. Large workloads run a bounded
    sample of output rows (all N columns of those rows)."""
    import oracle
    oracle.build()
    a_bits = d["a_bf16"]
    # rows so that one pass is about a second of work at ~1 GMAC/s/thread
    macs_per_row = wl.N * wl.K
    rows = max(1, min(M, int(2e9 / macs_per_row)))
    sample = a_bits[:rows]
    runs, t_total = 0, 0.0
    while t_total < budget_s or runs == 0:
        t0 = time.perf_counter()
        if wl.fmt == "mxfp4_w4a4":
            q, s = oracle.quant_mxfp4_rows(sample)
            oracle.gemm_mxfp4_w4a4(q, s, d["w"], d["w_scale"], d["bias"], d["epilogue"])
            t_total += time.perf_counter() - t0
            runs += 1
            if t_total > 3 * budget_s:
                break
            continue
        q, s = oracle.quant_rows(sample)
        if wl.fmt == "fp8":
            oracle.gemm_bs_fp8(q, s, d["w"], d["w_scale"], d["bias"], d["epilogue"])
        elif wl.fmt == "fp8_rowwise":
            oracle.gemm_fp8_rowwise(q, s, d["w"], d["w_scale"], d["bias"], d["epilogue"])
        else:
            oracle.gemm_mxfp4_w4a8(q, s, d["w"], d["w_scale"], d["bias"], d["epilogue"])
        t_total += time.perf_counter() - t0
        runs += 1
        if t_total > 3 * budget_s:
            break
    frac = rows / M
    if compute_bound:
        value, unit = alg["gemm_flops"] * frac * runs / t_total / 1e12, "TFLOP/s"
    else:
        step_bytes = (alg["quant_bytes"] + alg["gemm_bytes"] - d["w"].nbytes - d["w_scale"].nbytes) \
            * frac + d["w"].nbytes + d["w_scale"].nbytes
        value, unit = step_bytes * runs / t_total / 1e9, "GB/s"
    return {"value": round(value, 4), "unit": unit, "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "%d of %d token rows (all %d outputs each), %d passes of quantize + GEMM + "
                      "epilogue in %.1f s" % (rows, M, wl.N, runs, t_total),
            "cpu_model": _cpu_model()}


def bench_moe(args):
    """One step = per-token quantization of the expert-sorted rows and one
    grouped W4A8 GEMM over every expert (32 experts [4096, 7168] MXFP4, top-8
    routing of 8 decode tokens); expert-weight copies rotate over >= 512 MiB."""
    import torch
    import mxfp4_gemm_transformer_amd as bs
    import synth

    m = synth.MOE
    E, N, K, tokens, topk = m["E"], m["N"], m["K"], m["tokens"], m["topk"]
    steps = args.steps if args.steps is not None else 500
    warmup = args.warmup if args.warmup is not None else 20
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rng = np.random.default_rng(0)
    xt = synth.to_bf16_bits(rng.standard_normal((tokens, K)).astype(np.float32))
    row_token, off = synth.moe_routing(tokens, E, topk, seed=0)
    T = len(row_token)
    w_host, ws_host = synth.moe_weights(E, N, K, seed=0, distinct=4)
    copies = max(2, math.ceil(ROTATION_BYTES / (w_host.nbytes + ws_host.nbytes)))
    w0 = torch.from_numpy(w_host).to(dev)
    ws0 = torch.from_numpy(ws_host).to(dev)
    w_list = [w0] + [w0.clone() for _ in range(copies - 1)]
    ws_list = [ws0] + [ws0.clone() for _ in range(copies - 1)]
    x = torch.from_numpy(xt[row_token].view(np.int16)).view(torch.bfloat16).to(dev)
    offsets = torch.from_numpy(off).to(dev)
    q = torch.empty((T, K), dtype=torch.uint8, device=dev)
    s = torch.empty((T,), dtype=torch.float32, device=dev)
    y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)

    def gemm(i):
        bs.gemm_mxfp4_w4a8_grouped(q, s, offsets, w_list[i % copies], ws_list[i % copies], y=y,
                                   max_rows_per_expert=tokens)

    def step(i):
        bs.fp8_quant_rows(x, q, s)
        gemm(i)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(warmup):
            step(i)
    torch.cuda.synchronize()
    graphs = {}
    for name, fn in (("step", step), ("gemm", gemm)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(steps):
                fn(i)
        g.replay()
        graphs[name] = g
    torch.cuda.synchronize()

    def timed(g):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / steps

    t0 = time.perf_counter()
    step_s = timed(graphs["step"])
    wall_s = time.perf_counter() - t0
    gemm_s = timed(graphs["gemm"])
    active = int(np.count_nonzero(np.diff(off)))
    w_alg = active * (N * K // 2 + N * (K // 32))
    gemm_bytes = w_alg + T * K + 4 * T + 2 * T * N
    quant_bytes = 3 * T * K + 4 * T
    gbs = (gemm_bytes + quant_bytes) / step_s / 1e9
    achieved = gemm_bytes / gemm_s / 1e9
    result = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(step_s * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3 x fp4_e2m1", "data": "synthetic",
        "config": {"workload": "moe E=%d N=%d K=%d, %d tokens top-%d = %d rows over %d active experts "
                               "(grouped MXFP4 W4A8)" % (E, N, K, tokens, topk, T, active),
                   "E": E, "N": N, "K": K, "rows": T, "active_experts": active,
                   "weight_copies_rotated": copies, "step": "fp8_quant_rows + gemm_mxfp4_w4a8_grouped",
                   "graph_replay": True},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "gemm_mxfp4_w4a8_grouped", "avg_launch_us": round(gemm_s * 1e6, 3),
                     "algorithmic_bytes_per_launch": gemm_bytes},
        "kernels_us": {"fp8_quant_rows+gemm": round(step_s * 1e6, 3),
                       "gemm_mxfp4_w4a8_grouped": round(gemm_s * 1e6, 3)},
        "step_bytes": gemm_bytes + quant_bytes, "wall_s_timed_region": round(wall_s, 6),
    }
    if args.cpu_seconds > 0:
        import oracle
        oracle.build()
        runs, t_total = 0, 0.0
        while t_total < args.cpu_seconds or runs == 0:
            t1 = time.perf_counter()
            qh, sh = oracle.quant_rows(xt[row_token])
            oracle.gemm_mxfp4_w4a8_grouped(qh, sh, off, w_host, ws_host)
            t_total += time.perf_counter() - t1
            runs += 1
        result["cpu_baseline"] = {
            "value": round((gemm_bytes + quant_bytes) * runs / t_total / 1e9, 4), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "the whole step (%d rows), %d passes in %.1f s" % (T, runs, t_total),
            "cpu_model": _cpu_model()}
    print(json.dumps(result))


def producer_bytes(name, M, width):
    """HBM bytes a fused producer must move: bf16 inputs read, the new
    residual written (add_rms), codes and scales written."""
    if name == "add_rms":
        return 2 * M * width * 3 + 2 * width + M * width + 4 * M
    return 2 * M * 2 * width + M * width + 4 * M


def bench_producer(args):
    """One step = one fused producer call (add_rms_norm_quant_fp8 or
    silu_mul_quant_fp8) over [M, width] rows; input copies rotate over
    >= 512 MiB so each step reads its rows from HBM."""
    import torch
    import mxfp4_gemm_transformer_amd as bs
    import synth

    name = args.workload
    width, sweep = synth.PRODUCERS[name]
    M = args.m if args.m is not None else 16
    steps = args.steps if args.steps is not None else (100 if M >= 512 else 1000)
    warmup = args.warmup if args.warmup is not None else 20
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = synth.producer_inputs(name, M)
    to_dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)) \
        .view(torch.bfloat16).to(dev)
    if name == "add_rms":
        per_copy = 2 * d["x"].nbytes
        copies = max(2, math.ceil(ROTATION_BYTES / per_copy))
        xs = [to_dev(d["x"]) for _ in range(copies)]
        rs = [to_dev(d["residual"]) for _ in range(copies)]
        w = to_dev(d["weight"])
        call = lambda i: bs.add_rms_norm_quant_fp8(xs[i % copies], rs[i % copies], w, d["eps"],
                                                   q=q, scale=s)
        kernel = "add_rms_norm_quant_fp8"
    else:
        per_copy = d["gate_up"].nbytes
        copies = max(2, math.ceil(ROTATION_BYTES / per_copy))
        gus = [to_dev(d["gate_up"]) for _ in range(copies)]
        call = lambda i: bs.silu_mul_quant_fp8(gus[i % copies], q=q, scale=s)
        kernel = "silu_mul_quant_fp8"
    q = torch.empty((M, width), dtype=torch.uint8, device=dev)
    s = torch.empty((M,), dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(warmup):
            call(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(steps):
            call(i)
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        e0.record(stream)
        g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    step_s = e0.elapsed_time(e1) * 1e-3 / steps
    nbytes = producer_bytes(name, M, width)
    gbs = nbytes / step_s / 1e9
    result = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(step_s * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 -> fp8_e4m3", "data": "synthetic",
        "config": {"workload": "%s M=%d width=%d (fused %s + per-token e4m3 quantization)" % (
            name, M, width, "residual add + RMSNorm" if name == "add_rms" else "SiLU(gate) * up"),
            "M": M, "width": width, "input_copies_rotated": copies, "step": kernel,
            "graph_replay": True},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": kernel, "avg_launch_us": round(step_s * 1e6, 3),
                     "algorithmic_bytes_per_launch": nbytes},
        "kernels_us": {kernel: round(step_s * 1e6, 3)},
        "step_bytes": nbytes, "wall_s_timed_region": round(wall_s, 6),
    }
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline_producer(name, d, M, width, nbytes, args.cpu_seconds)
    print(json.dumps(result))


def cpu_baseline_producer(name, d, M, width, nbytes, budget_s):
    """The oracle's fused producer on a bounded sample of the rows."""
    import oracle
    oracle.build()
    rows = max(1, min(M, int(2e7 / width)))
    runs, t_total = 0, 0.0
    while t_total < budget_s or runs == 0:
        t0 = time.perf_counter()
        if name == "add_rms":
            oracle.add_rms_norm_quant(d["x"][:rows], d["residual"][:rows], d["weight"], d["eps"])
        else:
            oracle.silu_mul_quant(d["gate_up"][:rows])
        t_total += time.perf_counter() - t0
        runs += 1
        if t_total > 3 * budget_s:
            break
    value = nbytes * rows / M * runs / t_total / 1e9
    return {"value": round(value, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": "%d of %d rows, %d passes in %.1f s" % (rows, M, runs, t_total),
            "cpu_model": _cpu_model()}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
