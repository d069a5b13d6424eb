"""The CPU tests again under AddressSanitizer and UndefinedBehaviorSanitizer:
the oracle's pins against a sanitizer build of bs_oracle.c (gcc), and the C
ABI's host-side checks against a build of its host code with both
sanitizers (hipcc, host side only; the kernels are not instrumented). Each
runs in a child process that preloads the sanitizer runtime; any report
fails the child (UndefinedBehaviorSanitizer does not recover)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")


def _run(env_extra, preload, tests):
    env = dict(os.environ)
    env.update(env_extra)
    # the runtime first; anything already preloaded keeps its place after it
    env["LD_PRELOAD"] = ":".join(p for p in (preload, os.environ.get("LD_PRELOAD", "")) if p)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=23"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu and not slow",
           "-p", "no:cacheprovider", *[os.path.join(TESTS, t) for t in tests]]
    r = subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    return out


def test_oracle_under_asan_ubsan():
    import oracle
    lib = oracle.build_sanitized()
    asan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    out = _run({"BS_ORACLE_LIB": lib}, asan,
               ["test_oracle_codecs.py", "test_oracle_quant_gemm.py", "test_oracle_producers.py",
                "test_oracle_moe.py", "test_oracle_rowwise.py", "test_oracle_w4a4.py",
                "test_golden.py"])
    assert " passed" in out


def test_host_checks_under_asan_ubsan():
    from mxfp4_gemm_transformer_amd import _build
    lib = _build.build_host_sanitized()
    out = _run({"BSGEMM_LIB": lib}, _build.asan_runtime(), ["test_lib_host.py"])
    assert " passed" in out
