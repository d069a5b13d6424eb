"""Host-side checks of the C ABI, runnable without a GPU: the library loads,
exports every function include/bsgemm.h declares, and rejects bad arguments
on the host before touching a device."""
import ctypes
import os
import re

import pytest

import mxfp4_gemm_transformer_amd as bs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "bsgemm.h")

# A 16-byte-aligned fake address: only ever passed to calls that must fail
# validation, which happens before any device access.
FAKE = ctypes.c_void_p(0x10000)


def _declared():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, re.M)))


def test_header_declares_the_binding_names():
    assert _declared() == sorted(bs.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = bs.load_library()
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings_and_workspace():
    for st in (0, -1, -2, -3, -4, -5):
        assert bs.bs_status_string(st)
    assert bs.bs_status_string(7) == "unknown status"
    assert bs.bs_workspace_bytes(0, 8, 2048, 7168) == 0
    assert bs.bs_workspace_bytes(1, 4096, 34816, 5120) == 0
    # split-K decode (8 < M <= 64): S fp32 partial sums [S][M][N], S from N and K
    assert bs.bs_workspace_bytes(0, 64, 2048, 7168) == 8 * 64 * 2048 * 4
    assert bs.bs_workspace_bytes(1, 16, 2048, 7168) == 8 * 16 * 2048 * 4
    assert bs.bs_workspace_bytes(0, 9, 32, 32) == 1 * 9 * 32 * 4
    assert bs.bs_workspace_bytes(0, 65, 2048, 7168) == 0
    # 2 <= M <= 8 on layers of >= 2^26 weights: split-K too (S = 5 at K = 5120)
    assert bs.bs_workspace_bytes(2, 8, 248320, 5120) == 5 * 8 * 248320 * 4
    assert bs.bs_workspace_bytes(2, 1, 248320, 5120) == 0
    assert bs.bs_workspace_bytes(0, 8, 7168, 8192) == 0            # 2^25.8 weights


def _gemm(fn, a=FAKE, lda=64, s=FAKE, w=FAKE, ldw=64, ws=FAKE, bias=None, epi=0, y=FAKE, ldy=64,
          M=8, N=64, K=64, work=None, work_bytes=0):
    return fn(a, lda, s, w, ldw, ws, bias, epi, y, ldy, M, N, K, work, work_bytes, None)


@pytest.mark.parametrize("name", ["gemm_bs_fp8", "gemm_mxfp4_w4a8"])
def test_gemm_argument_checks(name):
    lib = bs.load_library()
    fn = getattr(lib, name)
    E = bs.BS_EINVAL
    assert _gemm(fn, a=None) == E
    assert _gemm(fn, s=None) == E
    assert _gemm(fn, w=None) == E
    assert _gemm(fn, ws=None) == E
    assert _gemm(fn, y=None) == E
    assert _gemm(fn, M=0) == E
    assert _gemm(fn, N=48) == E                    # N % 32
    assert _gemm(fn, K=80) == E                    # K % 32
    assert _gemm(fn, N=0) == E
    assert _gemm(fn, epi=3) == E
    assert _gemm(fn, epi=-1) == E
    assert _gemm(fn, epi=1) == E                   # bias required
    assert _gemm(fn, epi=2) == E
    assert _gemm(fn, lda=32) == E                  # ld_a < K
    assert _gemm(fn, ldy=32) == E                  # ld_y < N
    assert _gemm(fn, ldw=16) == E                  # ld_w < row bytes
    assert _gemm(fn, lda=(1 << 22) + 16) == E      # row strides above 4 MiB
    assert _gemm(fn, ldw=(1 << 22) + 16) == E
    A = bs.BS_EALIGN
    assert _gemm(fn, a=ctypes.c_void_p(0x10008)) == A
    assert _gemm(fn, w=ctypes.c_void_p(0x10004)) == A
    assert _gemm(fn, y=ctypes.c_void_p(0x10002)) == A
    assert _gemm(fn, lda=72) == A
    assert _gemm(fn, ldw=72) == A
    assert _gemm(fn, ldy=68) == A
    assert _gemm(fn, s=ctypes.c_void_p(0x10002)) == A
    assert _gemm(fn, bias=ctypes.c_void_p(0x10001), epi=1) == A
    # 8 < M <= 64 needs the split-K workspace: too small, missing, misaligned
    need = bs.bs_workspace_bytes(0 if name == "gemm_bs_fp8" else 1, 16, 64, 64)
    assert need > 0
    W = bs.BS_EWORKSPACE
    assert _gemm(fn, M=16) == W
    assert _gemm(fn, M=16, work=FAKE, work_bytes=need - 4) == W
    assert _gemm(fn, M=16, work=None, work_bytes=need) == W
    assert _gemm(fn, M=16, work=ctypes.c_void_p(0x10008), work_bytes=need) == A


def test_quant_argument_checks():
    lib = bs.load_library()
    q = lambda x=FAKE, ldx=64, qq=FAKE, ldq=64, s=FAKE, M=4, K=64: lib.fp8_quant_rows(x, ldx, qq, ldq, s, M, K, None)
    assert q(x=None) == bs.BS_EINVAL
    assert q(qq=None) == bs.BS_EINVAL
    assert q(s=None) == bs.BS_EINVAL
    assert q(M=0) == bs.BS_EINVAL
    assert q(K=48) == bs.BS_EINVAL
    assert q(K=0) == bs.BS_EINVAL
    assert q(ldx=32) == bs.BS_EINVAL
    assert q(ldq=32) == bs.BS_EINVAL
    assert q(x=ctypes.c_void_p(0x10008)) == bs.BS_EALIGN
    assert q(qq=ctypes.c_void_p(0x10001)) == bs.BS_EALIGN
    assert q(ldx=68) == bs.BS_EALIGN
    assert q(ldq=72) == bs.BS_EALIGN
    assert q(s=ctypes.c_void_p(0x10002)) == bs.BS_EALIGN


def test_rowwise_and_static_argument_checks():
    lib = bs.load_library()
    E, A = bs.BS_EINVAL, bs.BS_EALIGN
    fn = lib.gemm_fp8_rowwise
    assert _gemm(fn, ws=None) == E
    assert _gemm(fn, ws=ctypes.c_void_p(0x10008)) == A            # fp32 scales need 16 bytes
    assert _gemm(fn, a=None) == E
    assert _gemm(fn, N=48) == E
    assert bs.bs_workspace_bytes(2, 16, 2048, 7168) == bs.bs_workspace_bytes(0, 16, 2048, 7168)

    def st(x=FAKE, ldx=64, s=FAKE, q=FAKE, ldq=64, so=FAKE, M=4, K=64):
        return lib.fp8_quant_rows_static(x, ldx, s, q, ldq, so, M, K, None)

    assert st(x=None) == E
    assert st(s=None) == E
    assert st(q=None) == E
    assert st(M=0) == E
    assert st(K=48) == E
    assert st(ldx=32) == E
    assert st(ldq=32) == E
    assert st(x=ctypes.c_void_p(0x10008)) == A
    assert st(s=ctypes.c_void_p(0x10002)) == A
    assert st(so=ctypes.c_void_p(0x10002)) == A
    assert st(ldq=72) == A


def test_w4a4_argument_checks():
    lib = bs.load_library()
    E, A, W = bs.BS_EINVAL, bs.BS_EALIGN, bs.BS_EWORKSPACE
    fn = lib.gemm_mxfp4_w4a4
    need = bs.bs_workspace_bytes(3, 8, 64, 64)
    assert need > 0 and bs.bs_workspace_bytes(3, 65, 64, 64) == 0
    ok = dict(work=FAKE, work_bytes=need)
    assert _gemm(fn, a=None, **ok) == E
    assert _gemm(fn, s=None, **ok) == E
    assert _gemm(fn, lda=16, **ok) == E                              # < K/2
    assert _gemm(fn, M=100, K=96, lda=48, ldw=48, **ok) == E         # prefill needs K % 64 == 0
    assert _gemm(fn, lda=40, ldw=32, **ok) == A
    assert _gemm(fn, M=8, lda=32, ldw=32) == W                       # missing workspace
    q = lambda x=FAKE, ldx=64, qq=FAKE, ldq=32, s=FAKE, M=4, K=64: lib.fp4_quant_rows(x, ldx, qq, ldq, s, M, K, None)
    assert q(x=None) == E
    assert q(s=None) == E
    assert q(K=48) == E
    assert q(ldq=16) == E                                            # < K/2
    assert q(ldq=40) == A
    assert q(x=ctypes.c_void_p(0x10008)) == A


def test_grouped_argument_checks():
    lib = bs.load_library()
    E_, A = bs.BS_EINVAL, bs.BS_EALIGN

    def g(a=FAKE, lda=64, s=FAKE, off=FAKE, E=4, mr=8, w=FAKE, ldw=32, wst=32 * 64, ws=FAKE,
          b=None, epi=0, y=FAKE, ldy=64, T=8, N=64, K=64):
        return lib.gemm_mxfp4_w4a8_grouped(a, lda, s, off, E, mr, w, ldw, wst, ws, b, epi, y, ldy,
                                           T, N, K, None)

    assert g(off=None) == E_
    assert g(a=None) == E_
    assert g(E=0) == E_
    assert g(E=70000) == E_
    assert g(mr=0) == E_
    assert g(N=48) == E_
    assert g(wst=32 * 63) == E_                 # experts overlap
    assert g(ldw=16) == E_                      # < K/2
    assert g(epi=1) == E_                       # bias required
    assert g(off=ctypes.c_void_p(0x10002)) == A
    assert g(wst=32 * 64 + 8) == A
    assert g(ldw=40, wst=40 * 64) == A


def test_producer_argument_checks():
    lib = bs.load_library()
    E, A = bs.BS_EINVAL, bs.BS_EALIGN

    def rms(x=FAKE, ldx=64, r=FAKE, ldr=64, w=FAKE, eps=1e-6, q=FAKE, ldq=64, s=FAKE, M=4, K=64):
        return lib.add_rms_norm_quant_fp8(x, ldx, r, ldr, w, eps, q, ldq, s, M, K, None)

    assert rms(x=None) == E
    assert rms(w=None) == E
    assert rms(q=None) == E
    assert rms(s=None) == E
    assert rms(M=0) == E
    assert rms(K=48) == E
    assert rms(K=32768 + 32, ldx=40000, ldr=40000, ldq=40000) == E    # longer than 32768
    assert rms(ldx=32) == E
    assert rms(ldr=32) == E
    assert rms(ldq=32) == E
    assert rms(eps=-1.0) == E
    assert rms(eps=float("nan")) == E
    assert rms(x=ctypes.c_void_p(0x10008)) == A
    assert rms(r=ctypes.c_void_p(0x10008)) == A
    assert rms(w=ctypes.c_void_p(0x10002)) == A
    assert rms(q=ctypes.c_void_p(0x10001)) == A
    assert rms(ldx=68) == A
    assert rms(ldr=68) == A
    assert rms(ldq=72) == A
    assert rms(s=ctypes.c_void_p(0x10002)) == A
    assert rms(r=None, ldr=0, x=ctypes.c_void_p(0x10008)) == A     # no residual: its stride is unused

    def silu(gu=FAKE, ld=128, q=FAKE, ldq=64, s=FAKE, M=4, I=64):
        return lib.silu_mul_quant_fp8(gu, ld, q, ldq, s, M, I, None)

    assert silu(gu=None) == E
    assert silu(q=None) == E
    assert silu(s=None) == E
    assert silu(M=0) == E
    assert silu(I=48) == E
    assert silu(I=32768 + 32, ld=70000, ldq=40000) == E
    assert silu(ld=127) == E                                          # < 2I
    assert silu(ldq=32) == E
    assert silu(gu=ctypes.c_void_p(0x10008)) == A
    assert silu(ld=132) == A
    assert silu(ldq=72) == A
    assert silu(s=ctypes.c_void_p(0x10002)) == A


def test_valid_call_without_a_gpu_is_refused_by_the_arch_gate():
    import subprocess
    import sys
    # Run in a child with no visible devices so a machine with a GPU never launches on
    # the fake addresses: the gate must answer BS_EARCH before any launch.
    # E8M0 scale grids may start at any byte address: grids at odd addresses
    # pass every host check too (G1, G3), for the block-scaled, MXFP4 and
    # W4A4 GEMMs
    code = ("import ctypes,sys; sys.path.insert(0, %r); import mxfp4_gemm_transformer_amd as bs;"
            "lib=bs.load_library(); F=ctypes.c_void_p(0x10000);"
            "G1=ctypes.c_void_p(0x10001); G3=ctypes.c_void_p(0x10003);"
            "wk=bs.bs_workspace_bytes(3,8,64,64);"
            "print(lib.fp8_quant_rows(F,64,F,64,F,4,64,None),"
            " lib.gemm_bs_fp8(F,64,F,F,64,F,None,0,F,64,8,64,64,None,0,None),"
            " lib.gemm_bs_fp8(F,64,F,F,64,G1,None,0,F,64,8,64,64,None,0,None),"
            " lib.gemm_mxfp4_w4a8(F,128,F,F,64,G3,None,0,F,64,200,64,128,None,0,None),"
            " lib.gemm_mxfp4_w4a4(F,64,G1,F,64,G3,None,0,F,64,8,64,64,F,wk,None))") % ROOT
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1",
               CUDA_VISIBLE_DEVICES="-1")
    out = subprocess.check_output([sys.executable, "-c", code], env=env, text=True, timeout=120)
    assert out.split() == [str(bs.BS_EARCH)] * 5


def test_binding_refuses_tensors_off_the_device():
    # every pointer argument must be a device tensor on the operands' device:
    # a host tensor would reach a kernel as a host address
    import torch
    cpu = torch.zeros(4, dtype=torch.float32)
    with pytest.raises(ValueError, match="a_scale must be a device tensor"):
        bs._on(cpu, "a_scale", torch.device("cuda:0"))
    with pytest.raises(ValueError, match="workspace"):
        bs._workspace(torch.zeros(16, dtype=torch.uint8), 16, torch.device("cuda:0"), None)
    # no workspace needed and none given: nothing is allocated
    assert bs._workspace(None, 0, torch.device("cuda:0"), None) is None
