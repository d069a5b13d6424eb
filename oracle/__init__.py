"""CPU oracle for the block-scaled low-precision linear layer.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library never does, and
this package never imports the product library. The arithmetic lives in
``bs_oracle.c`` (plain C, fp64, OpenMP over output elements); this module
builds it with gcc and marshals numpy arrays to it with ctypes.

Parity status of each function (the pins are the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py``):

* e4m3 / e2m1 / E8M0 / bf16 decoders: pinned (exhaustive tables against
  torch's independent float8 decoder, closed-form spot values, NaN codes).
* e4m3 / e2m1 encoders: pinned (round trips, exhaustive midpoint ties,
  torch's float8 cast on random values).
* quantizer: pinned (invariants: exact scale, a +-448 code per row, error
  bound, special rows).
* GEMMs (both weight formats, all epilogues): pinned (dequantize-then-matmul
  in numpy, exact rational brute force on tiny shapes, identity /
  permutation / one-hot / scale-shift structures, cross-format equality,
  torch's tanh GELU).
* MXFP4 weight preparation: pinned (OCP rule properties, exact round trip
  of representable groups, the input generator's independent numpy path).
* bf16 rounding of fp64 values: pinned (torch's fp32 -> bf16 cast on values
  exact in fp32, exact rational nearest-neighbour search on values that are
  not, overflow and signed zeros).
* grouped (MoE) W4A8 GEMM: pinned (each expert's rows equal the dense W4A8
  GEMM on that expert alone; empty experts, one expert holding every row;
  the expert order of the rows).
* MXFP4 activation quantizer and the W4A4 GEMM: pinned (the quantizer is
  the weight conversion applied to activation rows, checked against the
  generator's independent numpy conversion; the GEMM against
  dequantize-then-matmul, exact rational brute force, and the W4A8 GEMM
  where the activations are representable in both formats).
* static-scale quantizer: pinned (equals the dynamic quantizer when given
  the row's own scale; saturation beyond 448 s; torch's float8 cast).
* row-wise scaled GEMM (per-token x per-channel fp32 scales): pinned
  (dequantize-then-matmul in numpy, exact rational brute force, equality
  with the block-scaled GEMM when the channel scales are uniform powers of
  two, sampled = whole).
* fused producers (RMSNorm with residual add, SiLU * up, each followed by
  the quantizer): pinned (closed forms on constant rows and eps, power-of-two
  scaling invariance, torch's float64 rms_norm and silu within one bf16
  step, torch's bf16 residual add, gate/up half order, the quantizer applied
  to the returned intermediate).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bs_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SAN_LIB_PATH = os.path.join(_HERE, "liboracle_san.so")
# BS_ORACLE_LIB loads another build of bs_oracle.c (the sanitizer build of
# build_sanitized(), under a process started with its runtime preloaded)
_LOAD_PATH = os.environ.get("BS_ORACLE_LIB") or None

EPI_NONE, EPI_BIAS, EPI_BIAS_GELU_TANH = 0, 1, 2

_lib = None


def build(force: bool = False) -> str:
    """Compile bs_oracle.c into liboracle.so next to it (gcc, -O2, OpenMP,
    no fast-math) and return the library path."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC",
                               "-shared", "-Wall", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_sanitized() -> str:
    """Compile bs_oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer
    (gcc, -O1, OpenMP) into liboracle_san.so; load it through BS_ORACLE_LIB in
    a process that preloads gcc's libasan."""
    tmp = _SAN_LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-fPIC", "-shared", "-Wall",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-fno-omit-frame-pointer", _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _SAN_LIB_PATH)
    return _SAN_LIB_PATH


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(_LOAD_PATH or build())
        u8, f64, i64 = ctypes.c_uint8, ctypes.c_double, ctypes.c_int64
        vp = ctypes.c_void_p
        lib.or_e4m3_value.argtypes = [u8]
        lib.or_e4m3_value.restype = f64
        lib.or_e2m1_value.argtypes = [u8]
        lib.or_e2m1_value.restype = f64
        lib.or_e8m0_value.argtypes = [u8]
        lib.or_e8m0_value.restype = f64
        lib.or_bf16_value.argtypes = [ctypes.c_uint16]
        lib.or_bf16_value.restype = f64
        lib.or_e4m3_encode.argtypes = [f64]
        lib.or_e4m3_encode.restype = u8
        lib.or_e2m1_encode.argtypes = [f64]
        lib.or_e2m1_encode.restype = u8
        lib.or_gelu_tanh.argtypes = [f64]
        lib.or_gelu_tanh.restype = f64
        lib.or_quant_rows.argtypes = [vp, i64, i64, i64, vp, i64, vp]
        lib.or_quant_rows.restype = None
        gemm = [vp, i64, vp, vp, i64, vp, vp, ctypes.c_int, i64, i64, i64, vp, vp]
        lib.or_gemm_bs_fp8.argtypes = gemm
        lib.or_gemm_bs_fp8.restype = None
        lib.or_gemm_mxfp4_w4a8.argtypes = gemm
        lib.or_gemm_mxfp4_w4a8.restype = None
        sampled = [vp, i64, vp, vp, i64, vp, vp, ctypes.c_int, i64, i64, vp, vp, vp, vp]
        lib.or_gemm_bs_fp8_sampled.argtypes = sampled
        lib.or_gemm_bs_fp8_sampled.restype = None
        lib.or_gemm_mxfp4_w4a8_sampled.argtypes = sampled
        lib.or_gemm_mxfp4_w4a8_sampled.restype = None
        lib.or_encode_e4m3.argtypes = [vp, i64, vp]
        lib.or_encode_e4m3.restype = None
        lib.or_quant_mxfp4_weights.argtypes = [vp, i64, i64, vp, vp]
        lib.or_quant_mxfp4_weights.restype = None
        lib.or_gemm_mxfp4_w4a8_grouped.argtypes = [vp, i64, vp, vp, i64, vp, i64, i64, vp, vp,
                                                   ctypes.c_int, i64, i64, i64, vp, vp]
        lib.or_gemm_mxfp4_w4a8_grouped.restype = None
        lib.or_quant_mxfp4_rows.argtypes = [vp, i64, i64, i64, vp, vp]
        lib.or_quant_mxfp4_rows.restype = None
        w4 = [vp, i64, vp, vp, i64, vp, vp, ctypes.c_int, i64, i64, i64, vp, vp]
        lib.or_gemm_mxfp4_w4a4.argtypes = w4
        lib.or_gemm_mxfp4_w4a4.restype = None
        lib.or_gemm_mxfp4_w4a4_sampled.argtypes = [vp, i64, vp, vp, i64, vp, vp, ctypes.c_int,
                                                   i64, i64, vp, vp, vp, vp]
        lib.or_gemm_mxfp4_w4a4_sampled.restype = None
        lib.or_quant_rows_static.argtypes = [vp, i64, i64, i64, ctypes.c_float, vp, i64]
        lib.or_quant_rows_static.restype = None
        rw = [vp, i64, vp, vp, i64, vp, vp, ctypes.c_int, i64, i64, i64, vp, vp]
        lib.or_gemm_fp8_rowwise.argtypes = rw
        lib.or_gemm_fp8_rowwise.restype = None
        lib.or_gemm_fp8_rowwise_sampled.argtypes = [vp, i64, vp, vp, i64, vp, vp, ctypes.c_int,
                                                    i64, i64, vp, vp, vp, vp]
        lib.or_gemm_fp8_rowwise_sampled.restype = None
        lib.or_bf16_round.argtypes = [f64]
        lib.or_bf16_round.restype = ctypes.c_uint16
        lib.or_add_rms_norm_quant.argtypes = [vp, i64, vp, i64, vp, f64, i64, i64, vp, i64, vp, i64,
                                              vp, i64, vp]
        lib.or_add_rms_norm_quant.restype = None
        lib.or_silu_mul_quant.argtypes = [vp, i64, i64, i64, vp, i64, vp, i64, vp]
        lib.or_silu_mul_quant.restype = None
        lib.or_num_threads.argtypes = []
        lib.or_num_threads.restype = ctypes.c_int
        lib.or_set_num_threads.argtypes = [ctypes.c_int]
        lib.or_set_num_threads.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a: np.ndarray, dtype) -> np.ndarray:
    assert a.dtype == dtype, (a.dtype, dtype)
    return np.ascontiguousarray(a)


# ------------------------------------------------------------------ codecs
def e4m3_value(code: int) -> float:
    return _load().or_e4m3_value(int(code))


def e2m1_value(nibble: int) -> float:
    return _load().or_e2m1_value(int(nibble))


def e8m0_value(s: int) -> float:
    return _load().or_e8m0_value(int(s))


def bf16_value(bits: int) -> float:
    return _load().or_bf16_value(int(bits))


def e4m3_encode(v: float) -> int:
    return int(_load().or_e4m3_encode(float(v)))


def e2m1_encode(v: float) -> int:
    return int(_load().or_e2m1_encode(float(v)))


def gelu_tanh(v: float) -> float:
    return _load().or_gelu_tanh(float(v))


def e4m3_table() -> np.ndarray:
    """fp64 value of each of the 256 e4m3fn codes."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e2m1_table() -> np.ndarray:
    return np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def encode_e4m3(values: np.ndarray) -> np.ndarray:
    """Element-wise e4m3fn encoding of float32 values (nearest, ties even,
    saturating)."""
    v = _c(values, np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    _load().or_encode_e4m3(_ptr(v), v.size, _ptr(out))
    return out


# --------------------------------------------------------------- quantizer
def quant_rows(x_bf16: np.ndarray):
    """Per-token e4m3 quantization of bf16 bits [M, K] (uint16).
    Returns (codes uint8 [M, K], scales float32 [M])."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M,), dtype=np.float32)
    _load().or_quant_rows(_ptr(x), K, M, K, _ptr(q), K, _ptr(s))
    return q, s


def quant_rows_static(x_bf16: np.ndarray, scale: float) -> np.ndarray:
    """e4m3 codes of bf16 bits [M, K] divided by one given fp32 scale."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.uint8)
    _load().or_quant_rows_static(_ptr(x), K, M, K, float(np.float32(scale)), _ptr(q), K)
    return q


# ---------------------------------------------------------- fused producers
def bf16_round(v: float) -> int:
    """Bits of the nearest bfloat16 to v (ties even, overflow to infinity)."""
    return int(_load().or_bf16_round(float(v)))


def add_rms_norm_quant(x_bf16, residual_bf16, weight_bf16, eps):
    """RMSNorm (with the residual added first when given) then the per-token
    quantizer. bf16 bits in (uint16 [M, K], [M, K] or None, [K]); returns
    (codes uint8 [M, K], scales float32 [M], new residual uint16 [M, K] or
    None, normalized row h uint16 [M, K])."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    w = _c(weight_bf16, np.uint16)
    assert w.shape == (K,)
    r = None if residual_bf16 is None else _c(residual_bf16, np.uint16)
    if r is not None:
        assert r.shape == (M, K)
    r_out = None if r is None else np.empty((M, K), dtype=np.uint16)
    h = np.empty((M, K), dtype=np.uint16)
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M,), dtype=np.float32)
    _load().or_add_rms_norm_quant(_ptr(x), K, _ptr(r), K, _ptr(w), float(eps), M, K,
                                  _ptr(r_out), K, _ptr(h), K, _ptr(q), K, _ptr(s))
    return q, s, r_out, h


def silu_mul_quant(gate_up_bf16):
    """SiLU(gate) * up then the per-token quantizer; gate_up bf16 bits
    [M, 2I] (gate in the first I columns). Returns (codes uint8 [M, I],
    scales float32 [M], the bf16 product row a uint16 [M, I])."""
    gu = _c(gate_up_bf16, np.uint16)
    M, I2 = gu.shape
    assert I2 % 2 == 0
    I = I2 // 2
    a = np.empty((M, I), dtype=np.uint16)
    q = np.empty((M, I), dtype=np.uint8)
    s = np.empty((M,), dtype=np.float32)
    _load().or_silu_mul_quant(_ptr(gu), I2, M, I, _ptr(a), I, _ptr(q), I, _ptr(s))
    return q, s, a


# ------------------------------------------------------------------- GEMMs
def gemm_bs_fp8(a_codes, a_scale, w_codes, w_scale, bias_bf16=None, epilogue=EPI_NONE):
    """fp64 output and absum [M, N] of the 32x32-block-scaled e4m3 GEMM."""
    a = _c(a_codes, np.uint8)
    s = _c(a_scale, np.float32)
    w = _c(w_codes, np.uint8)
    ws = _c(w_scale, np.uint8)
    M, K = a.shape
    N = w.shape[0]
    assert w.shape == (N, K) and ws.shape == (N // 32, K // 32) and s.shape == (M,)
    b = None if bias_bf16 is None else _c(bias_bf16, np.uint16)
    if epilogue != EPI_NONE:
        assert b is not None and b.shape == (N,)
    out = np.empty((M, N), dtype=np.float64)
    absum = np.empty((M, N), dtype=np.float64)
    _load().or_gemm_bs_fp8(_ptr(a), K, _ptr(s), _ptr(w), K, _ptr(ws), _ptr(b),
                           int(epilogue), M, N, K, _ptr(out), _ptr(absum))
    return out, absum


def gemm_mxfp4_w4a8(a_codes, a_scale, w_packed, w_scale, bias_bf16=None, epilogue=EPI_NONE):
    """fp64 output and absum [M, N] of the MXFP4-weight GEMM."""
    a = _c(a_codes, np.uint8)
    s = _c(a_scale, np.float32)
    w = _c(w_packed, np.uint8)
    ws = _c(w_scale, np.uint8)
    M, K = a.shape
    N = w.shape[0]
    assert w.shape == (N, K // 2) and ws.shape == (N, K // 32) and s.shape == (M,)
    b = None if bias_bf16 is None else _c(bias_bf16, np.uint16)
    if epilogue != EPI_NONE:
        assert b is not None and b.shape == (N,)
    out = np.empty((M, N), dtype=np.float64)
    absum = np.empty((M, N), dtype=np.float64)
    _load().or_gemm_mxfp4_w4a8(_ptr(a), K, _ptr(s), _ptr(w), K // 2, _ptr(ws), _ptr(b),
                               int(epilogue), M, N, K, _ptr(out), _ptr(absum))
    return out, absum


def gemm_sampled(fmt, a_codes, a_scale, w, w_scale, bias_bf16, epilogue, ms, ns):
    """fp64 output and absum at the sampled positions (ms[i], ns[i]).
    fmt is "fp8" (w e4m3 [N, K], scales [N/32, K/32]) or "mxfp4"
    (w packed [N, K/2], scales [N, K/32])."""
    a = _c(a_codes, np.uint8)
    s = _c(a_scale, np.float32)
    w = _c(w, np.uint8)
    ws = _c(w_scale, np.uint8)
    K = a.shape[1]
    b = None if bias_bf16 is None else _c(bias_bf16, np.uint16)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    out = np.empty(ms.shape, dtype=np.float64)
    absum = np.empty(ms.shape, dtype=np.float64)
    if fmt == "fp8":
        fn, ldw = _load().or_gemm_bs_fp8_sampled, K
    else:
        fn, ldw = _load().or_gemm_mxfp4_w4a8_sampled, K // 2
    fn(_ptr(a), K, _ptr(s), _ptr(w), ldw, _ptr(ws), _ptr(b), int(epilogue), K,
       ms.size, _ptr(ms), _ptr(ns), _ptr(out), _ptr(absum))
    return out, absum


def gemm_mxfp4_w4a8_grouped(a_codes, a_scale, offsets, w_packed, w_scale, bias_bf16=None,
                            epilogue=EPI_NONE):
    """Grouped (MoE) W4A8 GEMM: rows [offsets[e], offsets[e+1]) of A use
    expert e's weights w_packed[e] [N, K/2] with scales w_scale[e] [N, K/32]
    and bias_bf16[e] [N]. Returns fp64 out and absum [offsets[-1], N]."""
    a = _c(a_codes, np.uint8)
    s = _c(a_scale, np.float32)
    off = _c(offsets, np.int32)
    w = _c(w_packed, np.uint8)
    ws = _c(w_scale, np.uint8)
    E, N, K2 = w.shape
    K = 2 * K2
    T = int(off[-1])
    assert off.shape == (E + 1,) and off[0] == 0 and np.all(np.diff(off) >= 0)
    assert a.shape[0] >= T and a.shape[1] == K and ws.shape == (E, N, K // 32)
    b = None if bias_bf16 is None else _c(bias_bf16, np.uint16)
    out = np.empty((T, N), dtype=np.float64)
    absum = np.empty((T, N), dtype=np.float64)
    _load().or_gemm_mxfp4_w4a8_grouped(_ptr(a), K, _ptr(s), _ptr(off), E, _ptr(w), K2, N * K2,
                                       _ptr(ws), _ptr(b), int(epilogue), T, N, K, _ptr(out),
                                       _ptr(absum))
    return out, absum


def quant_mxfp4_rows(x_bf16: np.ndarray):
    """MXFP4 (OCP MX) quantization of bf16 activation rows [M, K]:
    (packed uint8 [M, K/2], E8M0 scales uint8 [M, K/32])."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    packed = np.empty((M, K // 2), dtype=np.uint8)
    scales = np.empty((M, K // 32), dtype=np.uint8)
    _load().or_quant_mxfp4_rows(_ptr(x), K, M, K, _ptr(packed), _ptr(scales))
    return packed, scales


def gemm_mxfp4_w4a4(a_packed, a_scales, w_packed, w_scales, bias_bf16=None, epilogue=EPI_NONE):
    """fp64 output and absum [M, N] of the MXFP4 x MXFP4 GEMM."""
    a = _c(a_packed, np.uint8)
    sa = _c(a_scales, np.uint8)
    w = _c(w_packed, np.uint8)
    sw = _c(w_scales, np.uint8)
    M, K2 = a.shape
    K = 2 * K2
    N = w.shape[0]
    assert w.shape == (N, K2) and sa.shape == (M, K // 32) and sw.shape == (N, K // 32)
    b = None if bias_bf16 is None else _c(bias_bf16, np.uint16)
    out = np.empty((M, N), dtype=np.float64)
    absum = np.empty((M, N), dtype=np.float64)
    _load().or_gemm_mxfp4_w4a4(_ptr(a), K2, _ptr(sa), _ptr(w), K2, _ptr(sw), _ptr(b),
                               int(epilogue), M, N, K, _ptr(out), _ptr(absum))
    return out, absum


def gemm_mxfp4_w4a4_sampled(a_packed, a_scales, w_packed, w_scales, bias_bf16, epilogue, ms, ns):
    a = _c(a_packed, np.uint8)
    sa = _c(a_scales, np.uint8)
    w = _c(w_packed, np.uint8)
    sw = _c(w_scales, np.uint8)
    K2 = a.shape[1]
    b = None if bias_bf16 is None else _c(bias_bf16, np.uint16)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    out = np.empty(ms.shape, dtype=np.float64)
    absum = np.empty(ms.shape, dtype=np.float64)
    _load().or_gemm_mxfp4_w4a4_sampled(_ptr(a), K2, _ptr(sa), _ptr(w), K2, _ptr(sw), _ptr(b),
                                       int(epilogue), 2 * K2, ms.size, _ptr(ms), _ptr(ns),
                                       _ptr(out), _ptr(absum))
    return out, absum


def gemm_fp8_rowwise(a_codes, a_scale, w_codes, w_scale_f32, bias_bf16=None,
                     epilogue=EPI_NONE):
    """fp64 output and absum [M, N] of the row-wise scaled e4m3 GEMM
    (per-token a_scale [M] x per-channel w_scale [N], both fp32)."""
    a = _c(a_codes, np.uint8)
    s = _c(a_scale, np.float32)
    w = _c(w_codes, np.uint8)
    ws = _c(w_scale_f32, np.float32)
    M, K = a.shape
    N = w.shape[0]
    assert w.shape == (N, K) and ws.shape == (N,) and s.shape == (M,)
    b = None if bias_bf16 is None else _c(bias_bf16, np.uint16)
    out = np.empty((M, N), dtype=np.float64)
    absum = np.empty((M, N), dtype=np.float64)
    _load().or_gemm_fp8_rowwise(_ptr(a), K, _ptr(s), _ptr(w), K, _ptr(ws), _ptr(b),
                                int(epilogue), M, N, K, _ptr(out), _ptr(absum))
    return out, absum


def gemm_fp8_rowwise_sampled(a_codes, a_scale, w_codes, w_scale_f32, bias_bf16, epilogue, ms, ns):
    a = _c(a_codes, np.uint8)
    s = _c(a_scale, np.float32)
    w = _c(w_codes, np.uint8)
    ws = _c(w_scale_f32, np.float32)
    K = a.shape[1]
    b = None if bias_bf16 is None else _c(bias_bf16, np.uint16)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    out = np.empty(ms.shape, dtype=np.float64)
    absum = np.empty(ms.shape, dtype=np.float64)
    _load().or_gemm_fp8_rowwise_sampled(_ptr(a), K, _ptr(s), _ptr(w), K, _ptr(ws), _ptr(b),
                                        int(epilogue), K, ms.size, _ptr(ms), _ptr(ns),
                                        _ptr(out), _ptr(absum))
    return out, absum


def quant_mxfp4_weights(values: np.ndarray):
    """OCP MX conversion of float32 weights [N, K] to (packed [N, K/2],
    scales [N, K/32])."""
    v = _c(values, np.float32)
    N, K = v.shape
    packed = np.empty((N, K // 2), dtype=np.uint8)
    scales = np.empty((N, K // 32), dtype=np.uint8)
    _load().or_quant_mxfp4_weights(_ptr(v), N, K, _ptr(packed), _ptr(scales))
    return packed, scales


def num_threads() -> int:
    return int(_load().or_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops from now on."""
    _load().or_set_num_threads(int(n))


def within_tolerance(y, ref, absum):
    """The acceptance bound |y - ref| <= 2^-8 |ref| + 1e-4 absum, element-wise."""
    y = np.asarray(y, dtype=np.float64)
    return np.abs(y - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-4 * absum
