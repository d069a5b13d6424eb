"""Summaries of rocprofv3 CSV output for profiles/.

    python rocprof_summary.py trace DIR            # per-kernel durations from --kernel-trace
    python rocprof_summary.py pmc DIR              # per-kernel counter values from --pmc
    python rocprof_summary.py mfma DIR             # MFMA busy and clock per kernel (--pmc
                                                   # SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE ...)
    python rocprof_summary.py traffic KEY M ALG_BYTES KERNELS FETCH_DIR WRITE_DIR CAL_FETCH_DIR CAL_WRITE_DIR
        # bytes beyond L2 per call of the kernels whose names contain one of
        # the comma-separated KERNELS substrings (medians per dispatch, added
        # over the kernels of one call), FETCH_SIZE and WRITE_SIZE each scaled
        # by what the counter reads for bench.py --calibrate-copy; the record
        # goes into profiles/traffic.json under KEY ("<entry point> <workload>
        # M=<M>") with the sha256 of the kernel sources bench.py checks

DIR is the -d directory of a rocprofv3 run with --output-format csv; every
matching CSV below it is read. Output is a Markdown table on stdout. Kernel
names are shortened to their first 90 characters.

Durations: the median over dispatches (rocprofv3's own average is also shown;
it includes warm-up launches). MFMA utilisation: SQ_VALU_MFMA_BUSY_CYCLES
summed over the GPU divided by GRBM_GUI_ACTIVE x SIMDs (1024 on MI355X),
the clock as GRBM_GUI_ACTIVE over the dispatch's duration.
"""
from __future__ import annotations

import csv
import glob
import os
import statistics
import sys

SIMDS = 1024          # 256 CUs x 4 SIMDs


def _rows(directory: str, suffix: str):
    for path in sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True)):
        with open(path, newline="") as f:
            yield from csv.DictReader(f)


def _short(name: str) -> str:
    name = name.strip()
    return name if len(name) <= 90 else name[:87] + "..."


def durations(directory: str):
    """{kernel: [duration ns per dispatch]} from kernel_trace.csv."""
    out = {}
    for r in _rows(directory, "kernel_trace.csv"):
        d = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        out.setdefault(r["Kernel_Name"], []).append(d)
    return out


def trace_table(directory: str) -> str:
    stats = {r["Name"]: r for r in _rows(directory, "kernel_stats.csv")}
    durs = durations(directory)
    lines = ["| kernel | calls | median ns | average ns | min ns | max ns |",
             "|---|---:|---:|---:|---:|---:|"]
    for name, ds in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        avg = stats.get(name, {}).get("AverageNs")
        lines.append("| `%s` | %d | %.1f | %s | %d | %d |" % (
            _short(name), len(ds), statistics.median(ds),
            "%.1f" % float(avg) if avg else "%.1f" % statistics.mean(ds), min(ds), max(ds)))
    return "\n".join(lines)


def counters(directory: str):
    """{kernel: {counter: [value per dispatch]}} and {kernel: [duration ns]}
    from counter_collection.csv (values summed over a dispatch's rows)."""
    per = {}
    dur = {}
    for r in _rows(directory, "counter_collection.csv"):
        key = (r["Kernel_Name"], r.get("Dispatch_Id") or r.get("Correlation_Id"))
        name, v = r["Counter_Name"], float(r["Counter_Value"])
        cur = per.setdefault(key, {})
        # GRBM counters count GPU-wide cycles: one value per dispatch (the
        # largest instance); the others add up over their instances
        if name.startswith("GRBM_"):
            cur[name] = max(cur.get(name, 0.0), v)
        else:
            cur[name] = cur.get(name, 0.0) + v
        if r.get("Start_Timestamp") and r.get("End_Timestamp"):
            dur[key] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    out, odur = {}, {}
    for (kname, _), cs in per.items():
        for c, v in cs.items():
            out.setdefault(kname, {}).setdefault(c, []).append(v)
    for (kname, _), d in dur.items():
        odur.setdefault(kname, []).append(d)
    return out, odur


def pmc_table(directory: str) -> str:
    cs, _ = counters(directory)
    names = sorted({c for k in cs.values() for c in k})
    lines = ["| kernel | dispatches | " + " | ".join("%s (median)" % n for n in names) + " |",
             "|---|---:|" + "---:|" * len(names)]
    for kname, k in sorted(cs.items(), key=lambda kv: kv[0]):
        n = max(len(v) for v in k.values())
        lines.append("| `%s` | %d | " % (_short(kname), n) +
                     " | ".join("%.1f" % statistics.median(k[c]) if c in k else "" for c in names) + " |")
    return "\n".join(lines)


def mfma_table(directory: str) -> str:
    cs, durs = counters(directory)
    lines = ["| kernel | dispatches | MFMA busy / (GRBM_GUI_ACTIVE x 1024 SIMDs) | clock GHz | "
             "median ns |", "|---|---:|---:|---:|---:|"]
    for kname, k in sorted(cs.items(), key=lambda kv: kv[0]):
        if "SQ_VALU_MFMA_BUSY_CYCLES" not in k or "GRBM_GUI_ACTIVE" not in k:
            continue
        busy = statistics.median(k["SQ_VALU_MFMA_BUSY_CYCLES"])
        act = statistics.median(k["GRBM_GUI_ACTIVE"])
        d = statistics.median(durs[kname]) if kname in durs else None
        lines.append("| `%s` | %d | %.3f | %s | %s |" % (
            _short(kname), len(k["GRBM_GUI_ACTIVE"]), busy / (act * SIMDS) if act else 0.0,
            "%.2f" % (act / d) if d else "", "%.0f" % d if d else ""))
    return "\n".join(lines)


def _median_kb(directory, counter, substrs):
    cs, _ = counters(directory)
    total, found = 0.0, []
    for kname, k in cs.items():
        if counter in k and any(sub in kname for sub in substrs):
            total += statistics.median(k[counter])
            found.append(_short(kname))
    if not found:
        raise SystemExit("no kernel matching %s with %s in %s" % (substrs, counter, directory))
    return total, found


def traffic(key, M, alg, kernels, fdir, wdir, cfdir, cwdir):
    import hashlib
    import json
    root = os.path.dirname(os.path.abspath(__file__))
    subs = kernels.split(",")
    fetch_kb, names = _median_kb(fdir, "FETCH_SIZE", subs)
    write_kb, _ = _median_kb(wdir, "WRITE_SIZE", subs)
    copy_bytes = 268435456
    cal_f, _ = _median_kb(cfdir, "FETCH_SIZE", ["copyBuffer"])
    cal_w, _ = _median_kb(cwdir, "WRITE_SIZE", ["copyBuffer"])
    fs, wsc = copy_bytes / 1024.0 / cal_f, copy_bytes / 1024.0 / cal_w
    total = int(round(fetch_kb * 1024 * fs + write_kb * 1024 * wsc))
    csrc = os.path.join(root, "mxfp4_gemm_transformer_amd", "csrc")
    h = hashlib.sha256()
    for name in ("gemm_decode.hip" if int(M) <= 64 else "gemm_prefill.hip", "bs_device.hpp"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    path = os.path.join(root, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    rec[key] = {"kernels": names, "fetch_kb_per_call": round(fetch_kb, 2),
                "write_kb_per_call": round(write_kb, 2), "fetch_scale": round(fs, 4),
                "write_scale": round(wsc, 4), "traffic_bytes_per_launch": total,
                "algorithmic_bytes_per_launch": int(alg),
                "traffic_over_algorithmic": round(total / int(alg), 3),
                "sources_sha256": h.hexdigest()}
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({key: rec[key]}, indent=1))


def main():
    if len(sys.argv) == 10 and sys.argv[1] == "traffic":
        traffic(*sys.argv[2:])
        return
    if len(sys.argv) != 3 or sys.argv[1] not in ("trace", "pmc", "mfma"):
        print(__doc__)
        sys.exit(2)
    mode, directory = sys.argv[1], sys.argv[2]
    print({"trace": trace_table, "pmc": pmc_table, "mfma": mfma_table}[mode](directory))


if __name__ == "__main__":
    main()
