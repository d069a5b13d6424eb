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


def build_host_sanitized() -> str:
    """libbsgemm_hostsan.so: the C ABI's host code (argument checks, the
    architecture gate, dispatch) built with AddressSanitizer and
    UndefinedBehaviorSanitizer, linked with the kernels as built by build().
    Device code is not instrumented. Load it through BSGEMM_LIB in a process
    that preloads clang's ASan runtime (asan_runtime())."""
    if not os.path.exists(os.path.join(OBJ_DIR, "gemm_decode.hip.o")):
        build()
    api = os.path.join(CSRC, "bsgemm_api.hip")
    obj = os.path.join(OBJ_DIR, "bsgemm_api.hostsan.o")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g"]
    r = subprocess.run([HIPCC, *flags, *san, "-c", api, "-o", obj], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (api, r.stderr))
    kernels = [os.path.join(OBJ_DIR, os.path.basename(src) + ".o") for src in sources()
               if os.path.basename(src) != "bsgemm_api.hip"]
    out = os.path.join(PKG, "libbsgemm_hostsan.so")
    tmp = out + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host",
                        "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libasan",
                        obj, *kernels, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, out)
    return out


def asan_runtime() -> str:
    """clang's shared ASan runtime, which libbsgemm_hostsan.so links against."""
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("clang's libclang_rt.asan-x86_64.so was not found under /opt/rocm/llvm")
    return found[-1]


if __name__ == "__main__":
    print(build(verbose=True))
