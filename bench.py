"""Benchmark of the block-scaled linear layer on one MI355X.

A step is one pass of the whole path over one batch: per-token quantization
of bf16 activations (fp8_quant_rows, or fp4_quant_rows for W4A4) followed by
the block-scaled GEMM with its fused epilogue (gemm_bs_fp8 / gemm_mxfp4_w4a8
/ ...). Inputs are resident in HBM before timing starts.

The default run prints one JSON line with both halves of the metric: the
decode projection (M=8, N=2048, K=7168, HBM-bound) as the headline `value`
and `roofline`, and under "prefill" the compute-bound prefill projection
(M=4096, N=7168, K=8192) with its TFLOP/s, MFMA roofline, kernel times,
parity re-check and CPU-oracle baseline.

Timing protocol (DRAM-cold weights, the sly-radiance README's decode-cell
method): the weights exist as >= 512 MiB of identical copies (twice the
256 MiB Infinity Cache). Before every timed graph replay an untimed graph
touches every copy once in order 0, 1, ..., C-1; the timed graph then runs
its K launches on copies 0, 1, 2, ... (mod C). Every timed launch therefore
reads a copy that was last touched about 512 MiB of weight traffic earlier,
whatever K is. Timed launches are captured once into HIP graphs and timed
with HIP events on the stream they run on: the whole step, the GEMM alone
and the quantizer alone, each K launches.

Parity re-check: the output of the timed step replay (every timed launch
computes the same values: the copies are identical) is compared with the
CPU oracle: quantized codes and scales bit for bit on every row, GEMM outputs
within |y - ref| <= 2^-8 |ref| + 1e-4 sum_k |a_k w_k| on every output when
there are at most 2^21 of them, else on rows m = 0 mod 64 (one output in
every 32-column block of each) plus 4096 random outputs.

    python bench.py [--steps K] [--warmup W]            # both halves
    python bench.py --workload decode --m 64            # one workload
    python bench.py --workload ceiling                  # streaming-read / empty-launch ceilings
    python bench.py --workload mfma_rate                # scaled-MFMA rate per operand format
    python bench.py --workload fused_step --m 16        # fused RMSNorm producer + gate_up GEMM
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
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
GEMM_WORKLOADS = ["tiny", "decode", "prefill", "prefill_shard", "ffn_up", "ffn_up_bias",
                  "gate_up", "gate_up_w4a4", "lm_head"]
KERNEL_NAME = {"fp8": "gemm_bs_fp8", "mxfp4": "gemm_mxfp4_w4a8", "mxfp4_w4a4": "gemm_mxfp4_w4a4",
               "fp8_rowwise": "gemm_fp8_rowwise"}


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None)
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--workload", default="default",
                   choices=["default"] + GEMM_WORKLOADS +
                           ["moe", "moe_prefill", "add_rms", "silu_mul", "ceiling", "mfma_rate",
                            "fused_step"],
                   help="default: the decode and prefill projections in one line; a GEMM "
                        "workload (quantize + GEMM per step); moe / moe_prefill (grouped W4A8, 8 or "
                        "512 tokens routed top-8 over 32 experts); a fused "
                        "producer (add_rms: residual add + RMSNorm + quantize on [M, 5120]; "
                        "silu_mul: SiLU(gate) * up + quantize on [M, 2 x 17408]); ceiling "
                        "(streaming read of rotated buffers and an empty launch); mfma_rate "
                        "(scaled MFMAs per operand format); fused_step (add_rms producer then "
                        "the MXFP4 gate_up GEMM, against the unfused chain)")
    p.add_argument("--m", type=int, default=None, help="token count (M) for sweep workloads")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="CPU oracle budget for each cpu_baseline leg (0 disables it)")
    p.add_argument("--no-check", action="store_true",
                   help="skip the parity re-check of the timed output against the oracle")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                   help="only run a plain device copy of BYTES bytes three times (the "
                        "reference for scaling FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


# ----------------------------------------------------------------- helpers
def kernel_sources(M: int):
    """The sources a GEMM call at M rows compiles from (its counters are only
    valid for these exact files)."""
    csrc = os.path.join(ROOT, "mxfp4_gemm_transformer_amd", "csrc")
    main = "gemm_decode.hip" if M <= 64 else "gemm_prefill.hip"
    return [os.path.join(csrc, main), os.path.join(csrc, "bs_device.hpp")]


def sources_sha256(M: int) -> str:
    h = hashlib.sha256()
    for path in kernel_sources(M):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str, M: int):
    """Beyond-L2 bytes per launch from the committed counter record, if it
    was taken on the kernel sources as they stand (same sha256), else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get("%s %s M=%d" % (kernel, workload, M))
    except (OSError, ValueError):
        return None
    if not rec or rec.get("sources_sha256") != sources_sha256(M):
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
    return {"quant_bytes": quant, "gemm_bytes": gemm, "gemm_flops": 2 * M * N * K,
            "weight_bytes": w_bytes + ws_bytes}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


class Graphs:
    """HIP graphs captured on one side stream, replayed and timed with HIP
    events recorded on that same stream."""

    def __init__(self):
        import torch
        self.torch = torch
        self.stream = torch.cuda.Stream()

    def capture(self, fn, count):
        g = self.torch.cuda.CUDAGraph()
        with self.torch.cuda.graph(g, stream=self.stream):
            for i in range(count):
                fn(i)
        return g

    def eager(self, fn, count):
        with self.torch.cuda.stream(self.stream):
            for i in range(count):
                fn(i)
        self.torch.cuda.synchronize()

    def replay(self, g):
        with self.torch.cuda.stream(self.stream):
            g.replay()
        self.torch.cuda.synchronize()

    def timed(self, g, flush=None, replays=1):
        """Seconds for `replays` back-to-back replays of g; `flush` is
        replayed first, untimed."""
        torch = self.torch
        if flush is not None:
            self.replay(flush)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(self.stream):
            e0.record(self.stream)
            for _ in range(replays):
                g.replay()
            e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3


# Launches each kernel's own timing averages over (whole rotation cycles,
# replayed back to back), so that a graph's launch latency is spread over
# about this many launches whatever --steps is.
KERNEL_TIMING_LAUNCHES = 200


# --------------------------------------------------------- parity re-check
def _sample_points(M, N, rng):
    """Every output when there are at most 2^21, else rows m = 0 mod 64 with
    one output in each 32-column block (the column inside the block varies
    with the row) plus 4096 random outputs."""
    if M * N <= (1 << 21):
        mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        return mm.ravel(), nn.ravel(), "all %d outputs" % (M * N)
    rows = np.arange(0, M, 64)
    blocks = np.arange(N // 32)
    mm = np.repeat(rows, len(blocks))
    nn = (np.tile(blocks, len(rows)) * 32 + (mm // 64 + np.tile(blocks, len(rows)) * 7) % 32)
    rm = rng.integers(0, M, 4096)
    rn = rng.integers(0, N, 4096)
    return (np.concatenate([mm, rm]), np.concatenate([nn, rn]),
            "rows m = 0 mod 64 x one output per 32-column block (%d) + 4096 random" % len(mm))


def parity_check(wl, d, q_gpu, s_gpu, y_gpu):
    """The timed output against the oracle; returns a summary dict."""
    import oracle
    oracle.build()
    x = d["a_bf16"]
    M, N = x.shape[0], wl.N
    if wl.fmt == "mxfp4_w4a4":
        q_ref, s_ref = oracle.quant_mxfp4_rows(x)
        quant_ok = bool(np.array_equal(q_gpu, q_ref) and np.array_equal(s_gpu, s_ref))
    else:
        q_ref, s_ref = oracle.quant_rows(x)
        quant_ok = bool(np.array_equal(q_gpu, q_ref) and
                        np.array_equal(s_gpu.view(np.uint32), s_ref.view(np.uint32)))
    ms, ns, how = _sample_points(M, N, np.random.default_rng(1234))
    if wl.fmt == "mxfp4_w4a4":
        ref, absum = oracle.gemm_mxfp4_w4a4_sampled(q_ref, s_ref, d["w"], d["w_scale"], d["bias"],
                                                    d["epilogue"], ms, ns)
    elif wl.fmt == "fp8_rowwise":
        ref, absum = oracle.gemm_fp8_rowwise_sampled(q_ref, s_ref, d["w"], d["w_scale"], d["bias"],
                                                     d["epilogue"], ms, ns)
    else:
        ref, absum = oracle.gemm_sampled(wl.fmt, q_ref, s_ref, d["w"], d["w_scale"], d["bias"],
                                         d["epilogue"], ms, ns)
    got = y_gpu[ms, ns].astype(np.float64)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-4 * absum
    err = np.abs(got - ref)
    ok = bool(np.all(err <= bound))
    return {"quant_bit_exact": quant_ok, "gemm_within_tolerance": ok,
            "gemm_points": int(ms.size), "gemm_sample": how,
            "max_err_over_bound": round(float(np.max(err / bound)), 4), "ok": quant_ok and ok}


# ------------------------------------------------------ GEMM workload record
def gemm_record(name, M, steps, warmup, cpu_seconds, check):
    """Time one GEMM workload (quantize + GEMM per step) and return its record."""
    import torch
    import mxfp4_gemm_transformer_amd as bs
    import synth

    wl = synth.WORKLOADS[name]
    M = wl.M if M is None else M
    big = 2 * M * wl.N * wl.K > 50e9
    steps = steps if steps is not None else (50 if big else 1000)
    warmup = warmup if warmup is not None else (5 if big else 50)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    d = synth.make(name, M)
    x = torch.from_numpy(d["a_bf16"].view(np.int16)).view(torch.bfloat16).to(dev)
    w_host, ws_host = d["w"], d["w_scale"]
    copies = max(2, math.ceil(ROTATION_BYTES / (w_host.nbytes + ws_host.nbytes)))
    w0 = torch.from_numpy(w_host).to(dev)
    ws0 = torch.from_numpy(ws_host).to(dev)
    w_list = [w0] + [w0.clone() for _ in range(copies - 1)]
    wsc_list = [ws0] + [ws0.clone() for _ in range(copies - 1)]
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

    def gemm_only(i):
        gemm(q, s, w_list[i % copies], wsc_list[i % copies], bias, epi, y=y, workspace=work)

    def step(i):
        quant()
        gemm_only(i)

    def quant_only(i):
        quant()

    G = Graphs()
    G.eager(step, warmup)                      # warm-up: eager steps
    g_flush = G.capture(gemm_only, copies)     # touches every weight copy once, in order
    g_step = G.capture(step, steps)
    g_quant = G.capture(quant_only, steps)
    for g in (g_flush, g_step, g_quant):
        G.replay(g)                            # first replays, untimed

    t0 = time.perf_counter()
    step_s = G.timed(g_step, flush=g_flush)
    wall_s = time.perf_counter() - t0
    parity = None
    if check:
        parity = parity_check(wl, d, q.cpu().numpy(), s.cpu().numpy(), y.float().cpu().numpy())
    # each kernel's average launch time: the GEMM over whole rotation cycles
    # (the flush graph: one launch per weight copy, each copy last touched a
    # cycle earlier), the quantizer over its own graph, both replayed back to
    # back to about KERNEL_TIMING_LAUNCHES launches
    r_gemm = max(1, math.ceil(KERNEL_TIMING_LAUNCHES / copies))
    gemm_s = G.timed(g_flush, flush=g_flush, replays=r_gemm) / (r_gemm * copies)
    r_quant = max(1, math.ceil(KERNEL_TIMING_LAUNCHES / steps))
    quant_s = G.timed(g_quant, replays=r_quant) / (r_quant * steps)

    alg = algorithmic(wl, M)
    step_bytes = alg["quant_bytes"] + alg["gemm_bytes"]
    fp4w = wl.fmt in ("mxfp4", "mxfp4_w4a4")
    peak = FP4_PEAK_TFLOPS if fp4w else FP8_PEAK_TFLOPS
    # the binding roof: the longer of the GEMM's FLOPs at the format's MFMA
    # peak and its bytes at the HBM peak (ridge 625 flop/B e4m3, 1262 MXFP4)
    compute_bound = alg["gemm_flops"] / (peak * 1e12) >= alg["gemm_bytes"] / (HBM_PEAK_GBS * 1e9)
    kernel = KERNEL_NAME[wl.fmt]
    if compute_bound:
        unit = "TFLOP/s"
        value = alg["gemm_flops"] * steps / step_s / 1e12
        achieved = alg["gemm_flops"] / gemm_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4)}
    else:
        unit = "GB/s"
        value = step_bytes * steps / step_s / 1e9
        achieved = alg["gemm_bytes"] / gemm_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof["traffic"] = measured_traffic(kernel, wl.name, M)
    roof["traffic_kind"] = ("bytes beyond L2 per launch (FETCH_SIZE x 2 + WRITE_SIZE; reads served "
                            "by the Infinity Cache count too)")
    roof["kernel"] = kernel
    roof["avg_launch_us"] = round(gemm_s * 1e6, 3)
    roof["algorithmic_bytes_per_launch"] = alg["gemm_bytes"]
    roof["algorithmic_flops_per_launch"] = alg["gemm_flops"]
    qname = "fp4_quant_rows" if w4a4 else "fp8_quant_rows"
    rec = {
        "value": round(value, 2), "unit": unit, "steps": steps, "warmup": warmup,
        "ms_per_step": round(step_s / steps * 1e3, 5),
        "dtype": {"mxfp4": "fp8_e4m3 x fp4_e2m1", "mxfp4_w4a4": "fp4_e2m1 x fp4_e2m1"}.get(
            wl.fmt, "fp8_e4m3"),
        "config": {"workload": "%s M=%d N=%d K=%d (%s weights, %s scales, epilogue %s)" % (
            wl.name, M, wl.N, wl.K, "MXFP4 e2m1" if fp4w else "e4m3",
            {"fp8": "32x32 E8M0", "mxfp4": "1x32 E8M0", "mxfp4_w4a4": "1x32 E8M0, MXFP4 activations",
             "fp8_rowwise": "fp32 per-channel"}[wl.fmt],
            ["none", "bias", "bias+tanh-GELU"][epi]),
            "M": M, "N": wl.N, "K": wl.K, "weight_copies_rotated": copies,
            "rotation": "every copy touched in order before each timed replay",
            "step": "%s + %s" % (qname, kernel), "graph_replay": True,
            "kernel_timing": "GEMM: a graph of one launch per weight copy, replayed %d time(s) "
                             "(%d launches); quantizer: its %d-launch graph, replayed %d time(s)" % (
                                 r_gemm, r_gemm * copies, steps, r_quant)},
        "roofline": roof,
        "kernels_us": {qname: round(quant_s * 1e6, 3), kernel: round(gemm_s * 1e6, 3)},
        "step_bytes": step_bytes, "wall_s_timed_region": round(wall_s, 6),
    }
    if fp4w and compute_bound:
        roof["frac_vs_fp8_rate"] = round(achieved / FP8_PEAK_TFLOPS, 4)
    if compute_bound:
        # the scaled MFMA the kernel issues (32x32x64, weights as the A
        # operand), measured now on random operands: the rate this GEMM could
        # reach if it did nothing but MFMAs
        pair = (4 if fp4w else 0, 4 if w4a4 else 0)
        rate = measured_mfma_rate(G, pair)
        roof["measured_mfma_tflops"] = {"operands": "%s weights x %s activations, 32x32x64" % (
            "fp4" if pair[0] else "fp8", "fp4" if pair[1] else "fp8"), "value": rate}
        roof["frac_vs_measured_mfma"] = round(achieved / rate, 4)
        roof["peak_derived"] = derived_peak("fp4" if w4a4 else "fp8")
    if parity is not None:
        rec["parity"] = parity
    if cpu_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline(d, wl, M, alg, compute_bound, cpu_seconds)
    return rec


def cpu_baseline(d, wl, M, alg, compute_bound, budget_s):
    """The CPU oracle, as it stands, on the same workload: quantization then
    the GEMM in fp64 with OpenMP over outputs. Large workloads run a bounded
    sample of token rows (all N outputs of each)."""
    import oracle
    oracle.build()
    # rows so that one pass is about a second of work at ~1 GMAC/s/thread
    rows = max(1, min(M, int(2e9 / (wl.N * wl.K))))
    sample = d["a_bf16"][:rows]
    def one_pass():
        if wl.fmt == "mxfp4_w4a4":
            qa, sa = oracle.quant_mxfp4_rows(sample)
            oracle.gemm_mxfp4_w4a4(qa, sa, d["w"], d["w_scale"], d["bias"], d["epilogue"])
            return
        qa, sa = oracle.quant_rows(sample)
        fn = {"fp8": oracle.gemm_bs_fp8, "fp8_rowwise": oracle.gemm_fp8_rowwise,
              "mxfp4": oracle.gemm_mxfp4_w4a8}[wl.fmt]
        fn(qa, sa, d["w"], d["w_scale"], d["bias"], d["epilogue"])

    runs, t_total = 0, 0.0
    while t_total < budget_s or runs == 0:
        t0 = time.perf_counter()
        one_pass()
        t_total += time.perf_counter() - t0
        runs += 1
        if t_total > 3 * budget_s:
            break
    frac = rows / M

    def rate(runs_, t_):
        if compute_bound:
            return alg["gemm_flops"] * frac * runs_ / t_ / 1e12, "TFLOP/s"
        wb = alg["weight_bytes"]
        step_bytes = (alg["quant_bytes"] + alg["gemm_bytes"] - wb) * frac + wb
        return step_bytes * runs_ / t_ / 1e9, "GB/s"
    value, unit = rate(runs, t_total)
    rec = {"value": round(value, 4), "unit": unit, "cores": oracle.num_threads(), "kind": "oracle",
           "sample": "%d of %d token rows (all %d outputs each), %d passes of quantize + GEMM + "
                     "epilogue in %.1f s" % (rows, M, wl.N, runs, t_total),
           "cpu_model": _cpu_model(),
           "gflops": round(alg["gemm_flops"] * frac * runs / t_total / 1e9, 3)}
    if not compute_bound and rows * wl.N * wl.K <= (1 << 27):
        # small workloads (the tiny GEMM, the decode projection): the same
        # sample on one core too, for about a third of the budget
        cores = oracle.num_threads()
        oracle.set_num_threads(1)
        try:
            r1, t1s = 0, 0.0
            while t1s < budget_s / 3 or r1 == 0:
                t0 = time.perf_counter()
                one_pass()
                t1s += time.perf_counter() - t0
                r1 += 1
        finally:
            oracle.set_num_threads(cores)
        v1, _ = rate(r1, t1s)
        rec["single_core"] = {"value": round(v1, 4), "unit": unit, "cores": 1,
                              "gflops": round(alg["gemm_flops"] * frac * r1 / t1s / 1e9, 3),
                              "sample": "the same, %d passes in %.1f s" % (r1, t1s)}
    return rec


def line(rec, n_gpus=1):
    """The contract's JSON line from a workload record."""
    out = {"metric": METRIC, "value": rec["value"], "unit": rec["unit"], "n_gpus": n_gpus,
           "steps": rec["steps"], "warmup": rec["warmup"], "ms_per_step": rec["ms_per_step"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": rec["dtype"],
           "data": "synthetic"}
    for k, v in rec.items():
        if k not in out:
            out[k] = v
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the layer's kernels run on one device and the "
              "library has no multi-GPU path (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    import synth
    check = not args.no_check
    wl_name = args.workload
    if wl_name in synth.PRODUCERS:
        result = bench_producer(args)
    elif wl_name in ("moe", "moe_prefill"):
        result = bench_moe(args)
    elif wl_name == "ceiling":
        result = bench_ceiling(args)
    elif wl_name == "mfma_rate":
        result = bench_mfma_rate(args)
    elif wl_name == "fused_step":
        result = bench_fused_step(args)
    elif wl_name == "default":
        dec = gemm_record("decode", args.m if args.m is not None else 8, args.steps, args.warmup,
                          args.cpu_seconds, check)
        pre = gemm_record("prefill", None, args.steps, args.warmup, args.cpu_seconds, check)
        result = line(dec)
        result["prefill"] = {k: pre[k] for k in ("value", "unit", "steps", "warmup", "ms_per_step",
                                                 "dtype", "config", "roofline", "kernels_us",
                                                 "parity", "cpu_baseline") if k in pre}
    else:
        result = line(gemm_record(wl_name, args.m, args.steps, args.warmup, args.cpu_seconds,
                                  check))
    print(json.dumps(result), flush=True)
    bad = [r for r in (result.get("parity"), (result.get("prefill") or {}).get("parity"))
           if r is not None and not r["ok"]]
    if bad:
        print("parity re-check FAILED: %s" % bad, file=sys.stderr)
        sys.exit(1)


# ------------------------------------------------------------ other modes
def bench_moe(args):
    """One step = per-token quantization of the expert-sorted rows and one
    grouped W4A8 GEMM over every expert (32 experts [4096, 7168] MXFP4, top-8
    routing of 8 decode tokens, or of 512 prefill tokens for moe_prefill);
    expert-weight copies rotate as for the GEMM workloads."""
    import torch
    import mxfp4_gemm_transformer_amd as bs
    import synth

    m = synth.MOE_PREFILL if args.workload == "moe_prefill" else synth.MOE
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

    max_rows = int(np.diff(off).max())

    def gemm(i):
        bs.gemm_mxfp4_w4a8_grouped(q, s, offsets, w_list[i % copies], ws_list[i % copies], y=y,
                                   max_rows_per_expert=max_rows)

    def step(i):
        bs.fp8_quant_rows(x, q, s)
        gemm(i)

    G = Graphs()
    G.eager(step, warmup)
    g_flush = G.capture(gemm, copies)
    g_step = G.capture(step, steps)
    for g in (g_flush, g_step):
        G.replay(g)
    t0 = time.perf_counter()
    step_s = G.timed(g_step, flush=g_flush) / steps
    wall_s = time.perf_counter() - t0
    parity = None
    big = T * N * K > (1 << 33)     # the prefill routing: outputs sampled per expert
    if not args.no_check:
        import oracle
        qh, sh = oracle.quant_rows(xt[row_token])
        got = y.float().cpu().numpy().astype(np.float64)
        qok = bool(np.array_equal(q.cpu().numpy(), qh))
        if big:
            rng_c = np.random.default_rng(11)
            ok, pts = True, 0
            for e in range(E):
                r0, r1 = int(off[e]), int(off[e + 1])
                if r0 == r1:
                    continue
                ms = np.concatenate([np.arange(r1 - r0), rng_c.integers(0, r1 - r0, 64)])
                ns = np.concatenate([np.arange(r1 - r0) * 29 % N, rng_c.integers(0, N, 64)])
                ref, absum = oracle.gemm_sampled("mxfp4", qh[r0:r1], sh[r0:r1], w_host[e], ws_host[e],
                                                 None, 0, ms, ns)
                g = got[r0 + ms, ns]
                ok &= bool(np.all(np.abs(g - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-4 * absum))
                pts += ms.size
            how = "every row, one column each, plus 64 random outputs per expert"
        else:
            ref, absum = oracle.gemm_mxfp4_w4a8_grouped(qh, sh, off, w_host, ws_host)
            ok = bool(np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-4 * absum))
            pts, how = int(ref.size), "all outputs"
        parity = {"quant_bit_exact": qok, "gemm_within_tolerance": ok,
                  "gemm_points": pts, "gemm_sample": how, "ok": ok and qok}
    r_gemm = max(1, math.ceil(KERNEL_TIMING_LAUNCHES / copies))
    gemm_s = G.timed(g_flush, flush=g_flush, replays=r_gemm) / (r_gemm * copies)
    active = int(np.count_nonzero(np.diff(off)))
    w_alg = active * (N * K // 2 + N * (K // 32))
    gemm_bytes = w_alg + T * K + 4 * T + 2 * T * N
    quant_bytes = 3 * T * K + 4 * T
    achieved = gemm_bytes / gemm_s / 1e9
    rec = {
        "value": round((gemm_bytes + quant_bytes) / step_s / 1e9, 2), "unit": "GB/s",
        "steps": steps, "warmup": warmup, "ms_per_step": round(step_s * 1e3, 5),
        "dtype": "fp8_e4m3 x fp4_e2m1",
        "config": {"workload": "%s E=%d N=%d K=%d, %d tokens top-%d = %d rows over %d active "
                               "experts (grouped MXFP4 W4A8)" % (args.workload, E, N, K, tokens, topk,
                                                                  T, active),
                   "E": E, "N": N, "K": K, "rows": T, "active_experts": active,
                   "weight_copies_rotated": copies,
                   "step": "fp8_quant_rows + gemm_mxfp4_w4a8_grouped", "graph_replay": True},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "gemm_mxfp4_w4a8_grouped", "avg_launch_us": round(gemm_s * 1e6, 3),
                     "algorithmic_bytes_per_launch": gemm_bytes,
                     "algorithmic_flops_per_launch": 2 * T * N * K,
                     "tflops": round(2 * T * N * K / gemm_s / 1e12, 1),
                     "max_rows_per_expert": max_rows},
        "kernels_us": {"fp8_quant_rows+gemm": round(step_s * 1e6, 3),
                       "gemm_mxfp4_w4a8_grouped": round(gemm_s * 1e6, 3)},
        "step_bytes": gemm_bytes + quant_bytes, "wall_s_timed_region": round(wall_s, 6),
    }
    if parity is not None:
        rec["parity"] = parity
    if args.cpu_seconds > 0:
        import oracle
        oracle.build()
        # the whole step, or for the prefill routing the first two rows of
        # every expert (all N outputs each)
        keep = np.concatenate([np.arange(off[e], min(off[e] + 2, off[e + 1])) for e in range(E)]) \
            if big else np.arange(T)
        counts = np.array([min(2, off[e + 1] - off[e]) if big else off[e + 1] - off[e]
                           for e in range(E)])
        off_s = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        xs = xt[row_token][keep]
        runs, t_total = 0, 0.0
        while t_total < args.cpu_seconds or runs == 0:
            t1 = time.perf_counter()
            qh, sh = oracle.quant_rows(xs)
            oracle.gemm_mxfp4_w4a8_grouped(qh, sh, off_s, w_host, ws_host)
            t_total += time.perf_counter() - t1
            runs += 1
        frac = len(keep) / T
        step_b = (gemm_bytes + quant_bytes - w_alg) * frac + w_alg
        rec["cpu_baseline"] = {
            "value": round(step_b * runs / t_total / 1e9, 4), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "%d of %d rows (all %d outputs each), %d passes in %.1f s" % (
                len(keep), T, N, runs, t_total),
            "cpu_model": _cpu_model()}
    return line(rec)


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
    width, _ = synth.PRODUCERS[name]
    M = args.m if args.m is not None else 16
    steps = args.steps if args.steps is not None else (100 if M >= 512 else 1000)
    warmup = args.warmup if args.warmup is not None else 20
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = synth.producer_inputs(name, M)
    to_dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)) \
        .view(torch.bfloat16).to(dev)
    q = torch.empty((M, width), dtype=torch.uint8, device=dev)
    s = torch.empty((M,), dtype=torch.float32, device=dev)
    if name == "add_rms":
        copies = max(2, math.ceil(ROTATION_BYTES / (2 * d["x"].nbytes)))
        xs = [to_dev(d["x"]) for _ in range(copies)]
        rs = [to_dev(d["residual"]) for _ in range(copies)]
        w = to_dev(d["weight"])
        call = lambda i: bs.add_rms_norm_quant_fp8(xs[i % copies], rs[i % copies], w, d["eps"],
                                                   q=q, scale=s)
        kernel = "add_rms_norm_quant_fp8"
    else:
        copies = max(2, math.ceil(ROTATION_BYTES / d["gate_up"].nbytes))
        gus = [to_dev(d["gate_up"]) for _ in range(copies)]
        call = lambda i: bs.silu_mul_quant_fp8(gus[i % copies], q=q, scale=s)
        kernel = "silu_mul_quant_fp8"
    G = Graphs()
    G.eager(call, warmup)
    g_flush = G.capture(call, copies)
    g = G.capture(call, steps)
    G.replay(g_flush)
    G.replay(g)
    t0 = time.perf_counter()
    step_s = G.timed(g, flush=g_flush) / steps
    wall_s = time.perf_counter() - t0
    nbytes = producer_bytes(name, M, width)
    gbs = nbytes / step_s / 1e9
    rec = {
        "value": round(gbs, 2), "unit": "GB/s", "steps": steps, "warmup": warmup,
        "ms_per_step": round(step_s * 1e3, 5), "dtype": "bf16 -> fp8_e4m3",
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
        rec["cpu_baseline"] = cpu_baseline_producer(name, d, M, width, nbytes, args.cpu_seconds)
    return line(rec)


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


def _bench_lib():
    """libbsbench.so: the ceiling microbenchmarks (built with the layer)."""
    path = os.path.join(ROOT, "mxfp4_gemm_transformer_amd", "libbsbench.so")
    if not os.path.exists(path):
        raise RuntimeError("libbsbench.so is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.bsb_stream_read.argtypes = [vp, i64, vp, i32, i32, vp]
    lib.bsb_stream_read.restype = i32
    lib.bsb_empty.argtypes = [i32, vp]
    lib.bsb_empty.restype = i32
    lib.bsb_mfma_rate.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, vp]
    lib.bsb_stream_read_shared.argtypes = [vp, i64, vp, i64, vp, i32, i32, vp]
    lib.bsb_stream_read_shared.restype = i32
    lib.bsb_l2_read.argtypes = [vp, i32, i32, i32, i32, vp, vp]
    lib.bsb_l2_read.restype = i32
    lib.bsb_mfma_rate.restype = i32
    ip = ctypes.POINTER(ctypes.c_int)
    lib.bsb_device_info.argtypes = [ip, ip, ip, ip]
    lib.bsb_device_info.restype = i32
    return lib


# Dense MFMA work per CU per engine clock on gfx950: a 32x32x64 MFMA with
# 8-bit operands is 131072 flops in 64 cycles on each of a CU's 4 SIMDs;
# 4-bit operands on both sides double it.
MFMA_FLOP_PER_CLK_CU = {"fp8": 8192, "fp4": 16384}


def derived_peak(kind):
    """The dense MFMA peak of an operand kind from the device's own compute
    unit count and peak engine clock, beside AMD's published figure."""
    lib = _bench_lib()
    v = [ctypes.c_int(0) for _ in range(4)]
    if lib.bsb_device_info(*[ctypes.byref(x) for x in v]) != 0:
        return None
    cus, sclk_khz, mclk_khz, bus_bits = (x.value for x in v)
    tf = cus * MFMA_FLOP_PER_CLK_CU[kind] * sclk_khz * 1e3 / 1e12
    return {"value": round(tf, 1), "unit": "TFLOP/s",
            "from": "%d CUs x %d flop/clk x %.3f GHz (device-reported peak engine clock)" % (
                cus, MFMA_FLOP_PER_CLK_CU[kind], sclk_khz / 1e6),
            "memory": "%d-bit bus, %.3f GHz memory clock (device-reported)" % (bus_bits, mclk_khz / 1e6)}


def bench_ceiling(args):
    """Ceilings for the HBM-bound lines, in the same graph-replay harness:
    a plain streaming read of rotated buffers of the decode layer's size
    (14,784,544 bytes, the algorithmic bytes of the M=8 decode GEMM) and of
    the MXFP4 gate_up layer's weights (94,766,080 bytes), over a sweep of
    launch shapes (the best is reported), and an empty kernel."""
    import torch
    lib = _bench_lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    steps = args.steps if args.steps is not None else 200
    warmup = args.warmup if args.warmup is not None else 20
    num_cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    G = Graphs()
    out = {"num_cus": num_cus, "stream_read": [], "steps": steps}

    def ck(st):
        if st != 0:
            raise RuntimeError("microbenchmark launch failed (hipError %d)" % st)

    for nbytes in (14784544, 94766080):
        nb = (nbytes + 15) // 16 * 16
        copies = max(2, math.ceil(ROTATION_BYTES / nb))
        bufs = [torch.full((nb,), 0x5A, dtype=torch.uint8, device=dev) for _ in range(copies)]
        best, sweep = None, []
        for blocks_per_cu in (1, 2, 4, 8):
            for unroll in (1, 2, 4, 8, 16):
                blocks = blocks_per_cu * num_cus
                if blocks * 256 * 16 * unroll > 4 * nb:
                    continue
                fn = lambda i: ck(lib.bsb_stream_read(ctypes.c_void_p(bufs[i % copies].data_ptr()),
                                                      nb, ctypes.c_void_p(sink.data_ptr()), blocks,
                                                      unroll, ctypes.c_void_p(G.stream.cuda_stream)))
                G.eager(fn, warmup)
                g_flush = G.capture(fn, copies)
                G.replay(g_flush)
                # timed as the GEMMs are: whole rotation cycles, back to back
                r = max(1, math.ceil(KERNEL_TIMING_LAUNCHES / copies))
                us = G.timed(g_flush, flush=g_flush, replays=r) / (r * copies) * 1e6
                rec = {"bytes": nb, "blocks": blocks, "unroll": unroll, "us": round(us, 3),
                       "GBps": round(nb / us / 1e3, 1), "frac": round(nb / us / 1e3 / HBM_PEAK_GBS, 4)}
                sweep.append([blocks, unroll, round(us, 3)])
                if best is None or us < best["us"]:
                    best = rec
        best["copies_rotated"] = copies
        best["sweep_blocks_unroll_us"] = sweep
        out["stream_read"].append(best)
        del bufs
        torch.cuda.empty_cache()
    # the decode layer's weights (14,784,544 - 57,344 - 4 x 8 bytes of activations and
    # scales, rounded) with every workgroup also reading the 57,344 activation bytes
    # of 8 tokens, as the decode GEMM without a split K does
    nb = 14727168
    copies = max(2, math.ceil(ROTATION_BYTES / nb))
    bufs = [torch.full((nb,), 0x5A, dtype=torch.uint8, device=dev) for _ in range(copies)]
    act = torch.full((8 * 7168,), 0x5A, dtype=torch.uint8, device=dev)
    shared = []
    for blocks_per_cu in (1, 2, 4, 8):
        for unroll in (1, 2, 4, 8, 16):
            blocks = blocks_per_cu * num_cus
            if blocks * 256 * 16 * unroll > 4 * nb:
                continue
            fn = lambda i: ck(lib.bsb_stream_read_shared(
                ctypes.c_void_p(bufs[i % copies].data_ptr()), nb, ctypes.c_void_p(act.data_ptr()),
                act.numel(), ctypes.c_void_p(sink.data_ptr()), blocks, unroll,
                ctypes.c_void_p(G.stream.cuda_stream)))
            G.eager(fn, warmup)
            g_flush = G.capture(fn, copies)
            G.replay(g_flush)
            r = max(1, math.ceil(KERNEL_TIMING_LAUNCHES / copies))
            shared.append([blocks, unroll,
                           round(G.timed(g_flush, flush=g_flush, replays=r) / (r * copies) * 1e6, 3)])
    out["stream_read_plus_shared_57344_per_workgroup"] = {
        "bytes": nb, "best_us": min(r[2] for r in shared), "sweep_blocks_unroll_us": shared}
    del bufs
    torch.cuda.empty_cache()
    # per-CU read rate from L2, into registers and with LDS-mode loads into
    # LDS (the prefill kernels' staging), 1 or 2 workgroups of 256 per CU,
    # each re-reading its own region (2 MiB per XCD in all, L2-resident)
    l2 = {}
    buf = torch.full((num_cus * 65536,), 0x5A, dtype=torch.uint8, device=dev)
    for per_cu, chunk in ((1, 65536), (2, 32768)):
        iters = 64 * 65536 // chunk
        for dma in (0, 1):
            fn = lambda i: ck(lib.bsb_l2_read(ctypes.c_void_p(buf.data_ptr()), chunk, iters,
                                              per_cu * num_cus, dma, ctypes.c_void_p(sink.data_ptr()),
                                              ctypes.c_void_p(G.stream.cuda_stream)))
            G.eager(fn, 3)
            g = G.capture(fn, 10)
            G.replay(g)
            us = G.timed(g) / 10 * 1e6
            l2["%d workgroup(s) per CU, %s" % (per_cu, "LDS-mode loads" if dma else "registers")] = {
                "us": round(us, 2), "GBps_per_CU": round(per_cu * chunk * iters / us / 1e3, 1)}
    out["l2_read_per_cu"] = l2
    del buf
    fn = lambda i: ck(lib.bsb_empty(num_cus, ctypes.c_void_p(G.stream.cuda_stream)))
    G.eager(fn, warmup)
    g = G.capture(fn, steps)
    G.replay(g)
    out["empty_kernel_us"] = round(G.timed(g) / steps * 1e6, 3)
    dec = out["stream_read"][0]
    return {"metric": "HBM ceilings: streaming read and launch cost, 1 GPU", "value": dec["GBps"],
            "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
            "ms_per_step": round(dec["us"] * 1e-3, 6), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "u8", "data": "synthetic",
            "config": {"workload": "ceiling: streaming read of rotated buffers (best launch shape) "
                                   "and an empty kernel"},
            "ceiling": out}


def measure_mfma_rates(G, lib, dev, iters=2048, reps=5, random_bits=0):
    """Dense scaled-MFMA rate (TFLOP/s) per shape and operand-format pair:
    4 waves per workgroup, 2 workgroups per CU, register operands (a fixed
    pattern of small values, or pseudo-random bits)."""
    import torch
    num_cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.zeros(256, dtype=torch.float32, device=dev)
    blocks, waves = 2 * num_cus, 4
    res = {}
    for shape, sname in ((1, "32x32x64"), (0, "16x16x128")):
        flops = blocks * waves * 4 * iters * (2 * 32 * 32 * 64 if shape else 2 * 16 * 16 * 128)
        for fa, fb, fname in ((0, 0, "fp8 x fp8"), (4, 0, "fp4 x fp8"), (0, 4, "fp8 x fp4"),
                              (4, 4, "fp4 x fp4")):
            def fn(i):
                st = lib.bsb_mfma_rate(shape, fa, fb, iters, blocks, waves, random_bits,
                                       ctypes.c_void_p(sink.data_ptr()),
                                       ctypes.c_void_p(G.stream.cuda_stream))
                if st != 0:
                    raise RuntimeError("bsb_mfma_rate failed (hipError %d)" % st)
            G.eager(fn, 2)
            g = G.capture(fn, reps)
            G.replay(g)
            s = G.timed(g) / reps
            res["%s %s" % (sname, fname)] = round(flops / s / 1e12, 1)
    return res, {"blocks": blocks, "waves_per_block": waves, "mfma_per_wave": 4 * iters}


def measured_mfma_rate(G, pair, iters=2048, reps=3):
    """TFLOP/s of back-to-back 32x32x64 scaled MFMAs of one operand-format
    pair (weights, activations) on random operands, 2 workgroups of 4 waves
    per CU."""
    import torch
    lib = _bench_lib()
    dev = torch.device("cuda:0")
    num_cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.zeros(256, dtype=torch.float32, device=dev)
    blocks, waves = 2 * num_cus, 4

    def fn(i):
        st = lib.bsb_mfma_rate(1, pair[0], pair[1], iters, blocks, waves, 1,
                               ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(G.stream.cuda_stream))
        if st != 0:
            raise RuntimeError("bsb_mfma_rate failed (hipError %d)" % st)
    G.eager(fn, 1)
    g = G.capture(fn, reps)
    G.replay(g)
    s = G.timed(g) / reps
    return round(blocks * waves * 4 * iters * 2 * 32 * 32 * 64 / s / 1e12, 1)


def bench_mfma_rate(args):
    """The scaled MFMA's dense rate per operand format on this GPU: the
    ceiling of each GEMM variant (e4m3 x e4m3; W4A8's fp4 weights with e4m3
    activations; W4A4's fp4 x fp4)."""
    import torch
    lib = _bench_lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    G = Graphs()
    rates, shape = measure_mfma_rates(G, lib, dev)
    rates_rnd, _ = measure_mfma_rates(G, lib, dev, random_bits=1)
    best = rates["32x32x64 fp8 x fp8"]
    return {"metric": "scaled MFMA rate per operand format, 1 GPU", "value": best,
            "unit": "TFLOP/s", "n_gpus": 1, "steps": 5, "warmup": 2, "ms_per_step": None,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3",
            "data": "synthetic",
            "config": {"workload": "mfma_rate: back-to-back V_MFMA_SCALE_F32 with register operands",
                       **shape},
            "rates_tflops": rates, "rates_tflops_random_operands": rates_rnd,
            "published_peaks_tflops": {"fp8": FP8_PEAK_TFLOPS, "fp4": FP4_PEAK_TFLOPS}}


def bench_fused_step(args):
    """The decode-time value of the fused producer: a step of
    add_rms_norm_quant_fp8 (residual add + RMSNorm + e4m3 quantization in one
    kernel) then the MXFP4 gate_up GEMM (N=34816, K=5120), against the
    unfused chain (residual add, RMSNorm in torch, then fp8_quant_rows, then
    the same GEMM) and against quantize + GEMM alone (the norm assumed done
    elsewhere). Weights rotate as for the GEMM workloads."""
    import torch
    import mxfp4_gemm_transformer_amd as bs
    import synth

    M = args.m if args.m is not None else 16
    steps = args.steps if args.steps is not None else 500
    warmup = args.warmup if args.warmup is not None else 20
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.WORKLOADS["gate_up"]
    w_host, ws_host = synth.weights(wl)
    pi = synth.producer_inputs("add_rms", M, width=wl.K)
    copies = max(2, math.ceil(ROTATION_BYTES / (w_host.nbytes + ws_host.nbytes)))
    w0 = torch.from_numpy(w_host).to(dev)
    ws0 = torch.from_numpy(ws_host).to(dev)
    w_list = [w0] + [w0.clone() for _ in range(copies - 1)]
    wsc_list = [ws0] + [ws0.clone() for _ in range(copies - 1)]
    to_dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)) \
        .view(torch.bfloat16).to(dev)
    x = to_dev(pi["x"])
    res0 = to_dev(pi["residual"])
    res = res0.clone()
    gamma = to_dev(pi["weight"])
    q = torch.empty((M, wl.K), dtype=torch.uint8, device=dev)
    s = torch.empty((M,), dtype=torch.float32, device=dev)
    y = torch.empty((M, wl.N), dtype=torch.bfloat16, device=dev)
    h = torch.empty((M, wl.K), dtype=torch.bfloat16, device=dev)
    need = bs.bs_workspace_bytes(1, M, wl.N, wl.K)
    work = torch.zeros((need,), dtype=torch.uint8, device=dev) if need else None

    def gemm(i):
        bs.gemm_mxfp4_w4a8(q, s, w_list[i % copies], wsc_list[i % copies], y=y, workspace=work)

    def fused(i):
        # the residual is updated in place each step (it grows by x; the
        # normalized row does not change scale), as in a layer stack
        bs.add_rms_norm_quant_fp8(x, res, gamma, pi["eps"], q=q, scale=s)
        gemm(i)

    def unfused(i):
        r = x + res0
        hf = torch.nn.functional.rms_norm(r.float(), (wl.K,), gamma.float(), pi["eps"])
        h.copy_(hf)
        bs.fp8_quant_rows(h, q, s)
        gemm(i)

    def quant_gemm(i):
        bs.fp8_quant_rows(x, q, s)
        gemm(i)

    G = Graphs()
    g_flush = G.capture(gemm, copies)
    times = {}
    for name, fn in (("fused", fused), ("unfused", unfused), ("quant_gemm", quant_gemm),
                     ("gemm", gemm)):
        G.eager(fn, warmup)
        g = G.capture(fn, steps)
        G.replay(g_flush)
        G.replay(g)
        times[name] = G.timed(g, flush=g_flush) / steps * 1e6
    parity = None
    if not args.no_check:
        import oracle
        res.copy_(res0)
        G.eager(fused, 1)
        qf, sf, _, _ = oracle.add_rms_norm_quant(pi["x"], pi["residual"], pi["weight"], pi["eps"])
        qok = bool(np.array_equal(q.cpu().numpy(), qf) and
                   np.array_equal(s.cpu().numpy().view(np.uint32), sf.view(np.uint32)))
        ms, ns, how = _sample_points(M, wl.N, np.random.default_rng(7))
        ref, absum = oracle.gemm_sampled("mxfp4", qf, sf, w_host, ws_host, None, 0, ms, ns)
        got = y.float().cpu().numpy()[ms, ns].astype(np.float64)
        ok = bool(np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-4 * absum))
        parity = {"quant_bit_exact": qok, "gemm_within_tolerance": ok, "gemm_points": int(ms.size),
                  "gemm_sample": how, "ok": qok and ok}
    fused_us = times["fused"]
    return {"metric": "fused producer + GEMM decode step latency, 1 GPU",
            "value": round(fused_us, 3), "unit": "us/step", "n_gpus": 1, "steps": steps,
            "warmup": warmup, "ms_per_step": round(fused_us * 1e-3, 6), "higher_is_better": False,
            "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3 x fp4_e2m1",
            "data": "synthetic",
            "config": {"workload": "fused_step M=%d: add_rms_norm_quant_fp8 [M, %d] then "
                                   "gemm_mxfp4_w4a8 N=%d K=%d" % (M, wl.K, wl.N, wl.K),
                       "M": M, "weight_copies_rotated": copies, "graph_replay": True},
            "us_per_step": {"fused: add_rms_norm_quant_fp8 + gemm": round(fused_us, 3),
                            "unfused: add + rms_norm (torch) + fp8_quant_rows + gemm":
                                round(times["unfused"], 3),
                            "fp8_quant_rows + gemm (no norm)": round(times["quant_gemm"], 3),
                            "gemm alone": round(times["gemm"], 3)},
            "parity": parity}


if __name__ == "__main__":
    main()
