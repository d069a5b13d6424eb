"""Block-scaled low-precision linear layer on AMD Instinct MI355X (gfx950).

A thin binding of the C ABI in ``include/bsgemm.h`` (``libbsgemm.so``, built
in-tree by ``__graft_entry__.build()``): the functions below check tensor
dtypes, shapes and strides, allocate outputs with torch when none are given,
and pass raw device pointers and torch's current HIP stream to the library.
Every step of the computation runs in the library's HIP kernels; there is no
fallback path. Importing works without a GPU; the first call that needs the
library raises if it was not built.

    q, s = fp8_quant_rows(x)                               # bf16 [M, K]
    y = gemm_bs_fp8(q, s, w, w_scale, bias, EPI_BIAS)      # e4m3 W, 32x32 E8M0
    y = gemm_mxfp4_w4a8(q, s, w4, w4_scale)                # fp4x2 W, 1x32 E8M0
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["fp8_quant_rows", "fp8_quant_rows_static", "add_rms_norm_quant_fp8",
           "silu_mul_quant_fp8", "gemm_bs_fp8", "gemm_bs_fp8_noalloc", "gemm_mxfp4_w4a8", "gemm_fp8_rowwise",
           "fp4_quant_rows", "gemm_mxfp4_w4a4", "gemm_mxfp4_w4a8_grouped", "bs_workspace_bytes",
           "bs_status_string", "BsError", "EPI_NONE", "EPI_BIAS", "EPI_BIAS_GELU_TANH",
           "weight_shape", "w_scale_shape", "library_path", "load_library",
           "EXPORTED_SYMBOLS"]

EPI_NONE, EPI_BIAS, EPI_BIAS_GELU_TANH = 0, 1, 2
BS_OK, BS_EINVAL, BS_EALIGN, BS_EARCH, BS_EWORKSPACE, BS_ELAUNCH = 0, -1, -2, -3, -4, -5
NOALLOC_SCRATCH_BYTES = 16 << 20      # BS_NOALLOC_SCRATCH_BYTES of include/bsgemm.h

EXPORTED_SYMBOLS = ("fp8_quant_rows", "fp8_quant_rows_static", "add_rms_norm_quant_fp8",
                    "silu_mul_quant_fp8", "gemm_bs_fp8", "gemm_bs_fp8_noalloc", "gemm_mxfp4_w4a8", "gemm_fp8_rowwise",
                    "fp4_quant_rows", "gemm_mxfp4_w4a4", "gemm_mxfp4_w4a8_grouped", "bs_workspace_bytes", "bs_status_string")

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbsgemm.so")
# BSGEMM_LIB loads another build of the same sources (the host-sanitizer
# build of _build.build_host_sanitized(), for the CPU tests)
_LOAD_PATH = os.environ.get("BSGEMM_LIB") or _LIB_PATH
_lib = None


class BsError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s failed: %s (status %d)" % (what, bs_status_string(status), status))
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libbsgemm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LOAD_PATH):
            raise RuntimeError("%s is not built; run __graft_entry__.build() "
                               "(hipcc --offload-arch=gfx950) first" % os.path.basename(_LOAD_PATH))
        lib = ctypes.CDLL(_LOAD_PATH)
        i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.fp8_quant_rows.argtypes = [vp, i64, vp, i64, vp, i64, i64, vp]
        lib.fp8_quant_rows.restype = i32
        lib.add_rms_norm_quant_fp8.argtypes = [vp, i64, vp, i64, vp, ctypes.c_double, vp, i64, vp,
                                               i64, i64, vp]
        lib.add_rms_norm_quant_fp8.restype = i32
        lib.silu_mul_quant_fp8.argtypes = [vp, i64, vp, i64, vp, i64, i64, vp]
        lib.silu_mul_quant_fp8.restype = i32
        gemm = [vp, i64, vp, vp, i64, vp, vp, i32, vp, i64, i64, i64, i64, vp, ctypes.c_size_t, vp]
        lib.gemm_bs_fp8.argtypes = gemm
        lib.gemm_bs_fp8.restype = i32
        lib.gemm_mxfp4_w4a8.argtypes = gemm
        lib.gemm_bs_fp8_noalloc.argtypes = gemm[:13] + [vp]
        lib.gemm_bs_fp8_noalloc.restype = i32
        lib.gemm_mxfp4_w4a8.restype = i32
        lib.gemm_fp8_rowwise.argtypes = gemm
        lib.gemm_fp8_rowwise.restype = i32
        lib.gemm_mxfp4_w4a4.argtypes = gemm
        lib.gemm_mxfp4_w4a4.restype = i32
        lib.gemm_mxfp4_w4a8_grouped.argtypes = [vp, i64, vp, vp, i64, i64, vp, i64, i64, vp, vp,
                                                i32, vp, i64, i64, i64, i64, vp]
        lib.gemm_mxfp4_w4a8_grouped.restype = i32
        lib.fp4_quant_rows.argtypes = [vp, i64, vp, i64, vp, i64, i64, vp]
        lib.fp4_quant_rows.restype = i32
        lib.fp8_quant_rows_static.argtypes = [vp, i64, vp, vp, i64, vp, i64, i64, vp]
        lib.fp8_quant_rows_static.restype = i32
        lib.bs_workspace_bytes.argtypes = [i32, i64, i64, i64]
        lib.bs_workspace_bytes.restype = ctypes.c_size_t
        lib.bs_status_string.argtypes = [i32]
        lib.bs_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def bs_status_string(status: int) -> str:
    return load_library().bs_status_string(int(status)).decode()


def bs_workspace_bytes(op: int, M: int, N: int, K: int) -> int:
    return int(load_library().bs_workspace_bytes(int(op), int(M), int(N), int(K)))


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _u8(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype in (torch.float8_e4m3fn, getattr(torch, "float4_e2m1fn_x2", None)):
        t = t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise TypeError("%s must be uint8 / float8_e4m3fn bytes, got %s" % (name, t.dtype))
    return t


def _matrix(t: torch.Tensor, name: str, rows: int, cols: int) -> int:
    """Check a row-major [rows, cols] view with unit column stride; return its row stride."""
    if t.dim() != 2 or tuple(t.shape) != (rows, cols) or t.stride(1) != 1:
        raise ValueError("%s must be a [%d, %d] row-major view, got shape %s strides %s"
                         % (name, rows, cols, tuple(t.shape), t.stride()))
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    return t.stride(0) if rows > 1 else max(t.stride(0), cols)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _on(t: torch.Tensor, name: str, device: torch.device) -> torch.Tensor:
    """Refuse a tensor that is not on `device` (a host pointer handed to a
    kernel would fault on the GPU instead of raising here)."""
    if not t.is_cuda or t.device != device:
        raise ValueError("%s must be a device tensor on %s, got %s" % (name, device, t.device))
    return t


def _torch_stream(stream):
    if stream is None:
        return None
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(getattr(stream, "cuda_stream", stream)))


def _alloc(shape, dtype, device, stream, zero=False):
    """A new tensor owned by the caching allocator on the stream the kernels
    run on, so that its memory is not handed to other work before they end."""
    s = _torch_stream(stream)
    if s is None:
        return torch.zeros(shape, dtype=dtype, device=device) if zero else \
            torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(s):
        return torch.zeros(shape, dtype=dtype, device=device) if zero else \
            torch.empty(shape, dtype=dtype, device=device)


def _workspace(workspace, need: int, device: torch.device, stream):
    """The split-K workspace: the caller's (a contiguous device tensor on the
    same device), or a new one of `need` bytes."""
    if workspace is None:
        return _alloc((need,), torch.uint8, device, stream) if need else None
    _on(workspace, "workspace", device)
    if not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor")
    return workspace


def fp8_quant_rows(x: torch.Tensor, q: torch.Tensor | None = None,
                   scale: torch.Tensor | None = None, stream=None):
    """Per-token e4m3 quantization of bf16 x [M, K]. Returns (q uint8 [M, K],
    scale fp32 [M])."""
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    M, K = x.shape
    ldx = _matrix(x, "x", M, K)
    q, ldq, scale = _quant_outputs(q, scale, M, K, x.device, stream)
    st = load_library().fp8_quant_rows(_ptr(x), ldx, _ptr(q), ldq, _ptr(scale), M, K,
                                       ctypes.c_void_p(_stream(stream)))
    if st != BS_OK:
        raise BsError(st, "fp8_quant_rows")
    return q, scale


def _quant_outputs(q, scale, M, K, device, stream):
    if q is None:
        q = _alloc((M, K), torch.uint8, device, stream)
    q = _on(_u8(q, "q"), "q", device)
    ldq = _matrix(q, "q", M, K)
    if scale is None:
        scale = _alloc((M,), torch.float32, device, stream)
    if scale.dtype != torch.float32 or scale.shape != (M,) or not scale.is_contiguous():
        raise ValueError("scale must be a contiguous fp32 [M] tensor")
    _on(scale, "scale", device)
    return q, ldq, scale


def add_rms_norm_quant_fp8(x: torch.Tensor, residual: torch.Tensor | None, weight: torch.Tensor,
                           eps: float, q: torch.Tensor | None = None,
                           scale: torch.Tensor | None = None, stream=None):
    """RMSNorm of x (+ residual, which is updated in place to the bf16 sum)
    with the bf16 weight [K], then per-token e4m3 quantization. Returns
    (q uint8 [M, K], scale fp32 [M])."""
    if x.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise TypeError("x and weight must be bfloat16")
    M, K = x.shape
    ldx = _matrix(x, "x", M, K)
    ldr = 0
    if residual is not None:
        if residual.dtype != torch.bfloat16:
            raise TypeError("residual must be bfloat16")
        ldr = _matrix(_on(residual, "residual", x.device), "residual", M, K)
    if weight.shape != (K,) or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous bf16 [K] tensor")
    _on(weight, "weight", x.device)
    q, ldq, scale = _quant_outputs(q, scale, M, K, x.device, stream)
    st = load_library().add_rms_norm_quant_fp8(_ptr(x), ldx, _ptr(residual), ldr, _ptr(weight),
                                               float(eps), _ptr(q), ldq, _ptr(scale), M, K,
                                               ctypes.c_void_p(_stream(stream)))
    if st != BS_OK:
        raise BsError(st, "add_rms_norm_quant_fp8")
    return q, scale


def silu_mul_quant_fp8(gate_up: torch.Tensor, q: torch.Tensor | None = None,
                       scale: torch.Tensor | None = None, stream=None):
    """SiLU(gate) * up of gate_up [M, 2I] (gate first), then per-token e4m3
    quantization. Returns (q uint8 [M, I], scale fp32 [M])."""
    if gate_up.dtype != torch.bfloat16:
        raise TypeError("gate_up must be bfloat16")
    M, I2 = gate_up.shape
    if I2 % 2:
        raise ValueError("gate_up must have an even number of columns")
    I = I2 // 2
    ldgu = _matrix(gate_up, "gate_up", M, I2)
    q, ldq, scale = _quant_outputs(q, scale, M, I, gate_up.device, stream)
    st = load_library().silu_mul_quant_fp8(_ptr(gate_up), ldgu, _ptr(q), ldq, _ptr(scale), M, I,
                                           ctypes.c_void_p(_stream(stream)))
    if st != BS_OK:
        raise BsError(st, "silu_mul_quant_fp8")
    return q, scale


def weight_shape(op: int, N: int, K: int) -> tuple:
    """Byte shape of the weight operand: e4m3 [N, K] (op 0, and op 2 with
    per-channel scales) or fp4 e2m1 packed two per byte [N, K/2] (op 1)."""
    return (N, K // 2) if op == 1 else (N, K)


def w_scale_shape(op: int, N: int, K: int) -> tuple:
    """Shape of the uint8 E8M0 scale grid, row-major: one scale per 32x32
    block [N/32, K/32] for e4m3 weights (op 0), one per row per 32 along K
    [N, K/32] for MXFP4 weights (op 1)."""
    return (N // 32, K // 32) if op == 0 else (N, K // 32)


def _gemm(fn_name, op, a, a_scale, w, w_scale, bias, epilogue, y, workspace, stream):
    a = _u8(a, "a")
    w = _u8(w, "w")
    M, K = a.shape
    N = w.shape[0]
    lda = _matrix(a, "a", M, K)
    ldw = _matrix(w, "w", N, weight_shape(op, N, K)[1])
    if a_scale.dtype != torch.float32 or a_scale.shape != (M,) or not a_scale.is_contiguous():
        raise ValueError("a_scale must be a contiguous fp32 [M] tensor")
    if op == 2:
        if w_scale.dtype != torch.float32 or tuple(w_scale.shape) != (N,) \
                or not w_scale.is_contiguous():
            raise ValueError("w_scale must be a contiguous fp32 [N] tensor")
    elif w_scale.dtype != torch.uint8 or tuple(w_scale.shape) != w_scale_shape(op, N, K) \
            or not w_scale.is_contiguous():
        raise ValueError("w_scale must be a contiguous uint8 %s tensor"
                         % (w_scale_shape(op, N, K),))
    if epilogue != EPI_NONE:
        if bias is None or bias.dtype != torch.bfloat16 or bias.shape != (N,) \
                or not bias.is_contiguous():
            raise ValueError("this epilogue needs a contiguous bf16 bias [N]")
        _on(bias, "bias", a.device)
    _on(w, "w", a.device)
    _on(a_scale, "a_scale", a.device)
    _on(w_scale, "w_scale", a.device)
    if y is None:
        y = _alloc((M, N), torch.bfloat16, a.device, stream)
    if y.dtype != torch.bfloat16:
        raise TypeError("y must be bfloat16")
    ldy = _matrix(_on(y, "y", a.device), "y", M, N)
    workspace = _workspace(workspace, bs_workspace_bytes(op, M, N, K), a.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fn = getattr(load_library(), fn_name)
    st = fn(_ptr(a), lda, _ptr(a_scale), _ptr(w), ldw, _ptr(w_scale),
            _ptr(bias if epilogue != EPI_NONE else None), int(epilogue), _ptr(y), ldy, M, N, K,
            _ptr(workspace), ws_bytes, ctypes.c_void_p(_stream(stream)))
    if st != BS_OK:
        raise BsError(st, fn_name)
    return y


def gemm_bs_fp8(a, a_scale, w, w_scale, bias=None, epilogue=EPI_NONE, y=None, workspace=None,
                stream=None):
    """y [M, N] bf16 = epilogue(a_scale[m] * sum_k a[m,k] w[n,k] 2^(S[n/32,k/32]-127) (+ bias)).
    a: e4m3 [M, K]; w: e4m3 [N, K]; w_scale: uint8 E8M0 [N/32, K/32]."""
    return _gemm("gemm_bs_fp8", 0, a, a_scale, w, w_scale, bias, epilogue, y, workspace, stream)


def gemm_bs_fp8_noalloc(a, a_scale, w, w_scale, bias=None, epilogue=EPI_NONE, y=None,
                        stream=None):
    """gemm_bs_fp8 through the entry point that allocates nothing: the split-K
    partial sums use the library's per-device scratch array
    (NOALLOC_SCRATCH_BYTES) instead of a workspace. y [M, N] bf16 must be
    given. Calls that overlap in time on one device race on that array."""
    if y is None:
        raise ValueError("gemm_bs_fp8_noalloc needs the output y: it allocates nothing")
    a = _u8(a, "a")
    w = _on(_u8(w, "w"), "w", a.device)
    M, K = a.shape
    N = w.shape[0]
    lda = _matrix(a, "a", M, K)
    ldw = _matrix(w, "w", N, K)
    if a_scale.dtype != torch.float32 or a_scale.shape != (M,) or not a_scale.is_contiguous():
        raise ValueError("a_scale must be a contiguous fp32 [M] tensor")
    if w_scale.dtype != torch.uint8 or tuple(w_scale.shape) != w_scale_shape(0, N, K) \
            or not w_scale.is_contiguous():
        raise ValueError("w_scale must be a contiguous uint8 %s tensor" % (w_scale_shape(0, N, K),))
    _on(a_scale, "a_scale", a.device)
    _on(w_scale, "w_scale", a.device)
    if epilogue != EPI_NONE:
        if bias is None or bias.dtype != torch.bfloat16 or bias.shape != (N,) \
                or not bias.is_contiguous():
            raise ValueError("this epilogue needs a contiguous bf16 bias [N]")
        _on(bias, "bias", a.device)
    if y.dtype != torch.bfloat16:
        raise TypeError("y must be bfloat16")
    ldy = _matrix(_on(y, "y", a.device), "y", M, N)
    st = load_library().gemm_bs_fp8_noalloc(
        _ptr(a), lda, _ptr(a_scale), _ptr(w), ldw, _ptr(w_scale),
        _ptr(bias if epilogue != EPI_NONE else None), int(epilogue), _ptr(y), ldy, M, N, K,
        ctypes.c_void_p(_stream(stream)))
    if st != BS_OK:
        raise BsError(st, "gemm_bs_fp8_noalloc")
    return y


def gemm_fp8_rowwise(a, a_scale, w, w_scale, bias=None, epilogue=EPI_NONE, y=None,
                     workspace=None, stream=None):
    """y [M, N] bf16 = epilogue(a_scale[m] * w_scale[n] * sum_k a[m,k] w[n,k] (+ bias)).
    a: e4m3 [M, K]; w: e4m3 [N, K]; w_scale: fp32 [N], one per output channel."""
    return _gemm("gemm_fp8_rowwise", 2, a, a_scale, w, w_scale, bias, epilogue, y, workspace,
                 stream)


def fp8_quant_rows_static(x: torch.Tensor, scale: torch.Tensor, q: torch.Tensor | None = None,
                          scale_out: torch.Tensor | None = None, stream=None):
    """e4m3 codes of bf16 x [M, K] divided by one given scale (a device fp32
    tensor of one element). Returns (q uint8 [M, K], scale_out fp32 [M] filled
    with that scale)."""
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    if scale.dtype != torch.float32 or scale.numel() != 1 or not scale.is_cuda:
        raise ValueError("scale must be a one-element fp32 device tensor")
    M, K = x.shape
    ldx = _matrix(x, "x", M, K)
    _on(scale, "scale", x.device)
    q, ldq, scale_out = _quant_outputs(q, scale_out, M, K, x.device, stream)
    st = load_library().fp8_quant_rows_static(_ptr(x), ldx, _ptr(scale), _ptr(q), ldq,
                                              _ptr(scale_out), M, K,
                                              ctypes.c_void_p(_stream(stream)))
    if st != BS_OK:
        raise BsError(st, "fp8_quant_rows_static")
    return q, scale_out


def gemm_mxfp4_w4a8_grouped(a, a_scale, expert_offsets, w, w_scale, bias=None,
                            epilogue=EPI_NONE, y=None, max_rows_per_expert=None, stream=None):
    """Grouped (MoE) W4A8 GEMM. a: e4m3 [T, K] rows sorted by expert;
    expert_offsets: int32 device [E + 1]; w: fp4x2 [E, N, K/2]; w_scale:
    uint8 [E, N, K/32]; bias: bf16 [E, N] or None. Returns y bf16 [T, N]
    (rows outside every expert's range are left as they are)."""
    a = _u8(a, "a")
    w = _u8(w, "w")
    T, K = a.shape
    E, N, K2 = w.shape
    if K2 * 2 != K:
        raise ValueError("w must be [E, N, K/2]")
    lda = _matrix(a, "a", T, K)
    if w.stride(2) != 1 or w.stride(1) < K2 or not w.is_cuda:
        raise ValueError("w must be a device [E, N, K/2] tensor with unit column stride")
    if a_scale.dtype != torch.float32 or a_scale.shape != (T,) or not a_scale.is_contiguous():
        raise ValueError("a_scale must be a contiguous fp32 [T] tensor")
    if expert_offsets.dtype != torch.int32 or expert_offsets.shape != (E + 1,) \
            or not expert_offsets.is_contiguous() or not expert_offsets.is_cuda:
        raise ValueError("expert_offsets must be a contiguous int32 device [E + 1] tensor")
    if w_scale.dtype != torch.uint8 or tuple(w_scale.shape) != (E, N, K // 32) \
            or not w_scale.is_contiguous():
        raise ValueError("w_scale must be a contiguous uint8 [E, N, K/32] tensor")
    if epilogue != EPI_NONE:
        if bias is None or bias.dtype != torch.bfloat16 or tuple(bias.shape) != (E, N) \
                or not bias.is_contiguous():
            raise ValueError("this epilogue needs a contiguous bf16 bias [E, N]")
        _on(bias, "bias", a.device)
    for t, name in ((w, "w"), (a_scale, "a_scale"), (expert_offsets, "expert_offsets"),
                    (w_scale, "w_scale")):
        _on(t, name, a.device)
    if y is None:
        y = _alloc((T, N), torch.bfloat16, a.device, stream, zero=True)
    ldy = _matrix(_on(y, "y", a.device), "y", T, N)
    mr = T if max_rows_per_expert is None else int(max_rows_per_expert)
    st = load_library().gemm_mxfp4_w4a8_grouped(
        _ptr(a), lda, _ptr(a_scale), _ptr(expert_offsets), E, mr, _ptr(w), w.stride(1),
        w.stride(0), _ptr(w_scale), _ptr(bias if epilogue != EPI_NONE else None), int(epilogue),
        _ptr(y), ldy, T, N, K, ctypes.c_void_p(_stream(stream)))
    if st != BS_OK:
        raise BsError(st, "gemm_mxfp4_w4a8_grouped")
    return y


def fp4_quant_rows(x: torch.Tensor, q: torch.Tensor | None = None,
                   scale: torch.Tensor | None = None, stream=None):
    """MXFP4 quantization of bf16 x [M, K]: (q uint8 [M, K/2] two e2m1 codes
    per byte, low nibble = even k; scale uint8 E8M0 [M, K/32])."""
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    M, K = x.shape
    ldx = _matrix(x, "x", M, K)
    if q is None:
        q = _alloc((M, K // 2), torch.uint8, x.device, stream)
    ldq = _matrix(_on(_u8(q, "q"), "q", x.device), "q", M, K // 2)
    if scale is None:
        scale = _alloc((M, K // 32), torch.uint8, x.device, stream)
    if scale.dtype != torch.uint8 or tuple(scale.shape) != (M, K // 32) or not scale.is_contiguous():
        raise ValueError("scale must be a contiguous uint8 [M, K/32] tensor")
    _on(scale, "scale", x.device)
    st = load_library().fp4_quant_rows(_ptr(x), ldx, _ptr(q), ldq, _ptr(scale), M, K,
                                       ctypes.c_void_p(_stream(stream)))
    if st != BS_OK:
        raise BsError(st, "fp4_quant_rows")
    return q, scale


def gemm_mxfp4_w4a4(a, a_scale, w, w_scale, bias=None, epilogue=EPI_NONE, y=None,
                    workspace=None, stream=None):
    """y [M, N] bf16 = epilogue(sum_kb 2^(Sa[m,kb]-127) 2^(Sw[n,kb]-127) sum a w (+ bias)).
    a: fp4x2 [M, K/2] with E8M0 a_scale [M, K/32]; w: fp4x2 [N, K/2] with
    w_scale [N, K/32]."""
    a = _u8(a, "a")
    w = _u8(w, "w")
    M, K2 = a.shape
    K = 2 * K2
    N = w.shape[0]
    lda = _matrix(a, "a", M, K2)
    ldw = _matrix(w, "w", N, K2)
    for t, name, rows in ((a_scale, "a_scale", M), (w_scale, "w_scale", N)):
        if t.dtype != torch.uint8 or tuple(t.shape) != (rows, K // 32) or not t.is_contiguous():
            raise ValueError("%s must be a contiguous uint8 [%d, %d] tensor" % (name, rows, K // 32))
        _on(t, name, a.device)
    _on(w, "w", a.device)
    if epilogue != EPI_NONE:
        if bias is None or bias.dtype != torch.bfloat16 or bias.shape != (N,) \
                or not bias.is_contiguous():
            raise ValueError("this epilogue needs a contiguous bf16 bias [N]")
        _on(bias, "bias", a.device)
    if y is None:
        y = _alloc((M, N), torch.bfloat16, a.device, stream)
    if y.dtype != torch.bfloat16:
        raise TypeError("y must be bfloat16")
    ldy = _matrix(_on(y, "y", a.device), "y", M, N)
    workspace = _workspace(workspace, bs_workspace_bytes(3, M, N, K), a.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().gemm_mxfp4_w4a4(_ptr(a), lda, _ptr(a_scale), _ptr(w), ldw, _ptr(w_scale),
                                        _ptr(bias if epilogue != EPI_NONE else None),
                                        int(epilogue), _ptr(y), ldy, M, N, K, _ptr(workspace),
                                        ws_bytes, ctypes.c_void_p(_stream(stream)))
    if st != BS_OK:
        raise BsError(st, "gemm_mxfp4_w4a4")
    return y


def gemm_mxfp4_w4a8(a, a_scale, w, w_scale, bias=None, epilogue=EPI_NONE, y=None,
                    workspace=None, stream=None):
    """As gemm_bs_fp8 with fp4 e2m1 weights packed [N, K/2] (low nibble = even
    k) and one E8M0 scale per row per 32 k, w_scale [N, K/32]."""
    return _gemm("gemm_mxfp4_w4a8", 1, a, a_scale, w, w_scale, bias, epilogue, y, workspace,
                 stream)
