"""Build libbsgemm.so (the layer) and libbsbench.so (bench.py's ceiling
microbenchmarks) for gfx950 in-tree with hipcc (no GPU needed)."""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libbsgemm.so")
BENCH_SRC = os.path.join(PKG, "bench_kernels")
BENCH_LIB = os.path.join(PKG, "libbsbench.so")
OBJ_DIR = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # keep hipcc from forming packed fp32 arithmetic on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _link(objs, out):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libbsgemm.so and libbsbench.so;
    returns the path of libbsgemm.so."""
    os.makedirs(OBJ_DIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
        cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
        if verbose:
            print(" ".join(cmd))
        return obj

    bench_srcs = sorted(glob.glob(os.path.join(BENCH_SRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one, sources() + bench_srcs))
    _link(objs[:len(objs) - len(bench_srcs)], LIB)
    _link(objs[len(objs) - len(bench_srcs):], BENCH_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
