"""Helpers shared by the GPU parity tests: moving seeded inputs to the device
and comparing GEMM outputs with the oracle at the acceptance bound."""
import numpy as np
import torch

import mxfp4_gemm_transformer_amd as bs
import oracle

DEV = torch.device("cuda:0")


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def u8_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def f32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def y_host(y: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def assert_within(got, ref, absum, what=""):
    ok = oracle.within_tolerance(got, ref, absum)
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError("%s: %d of %d outside |y-ref| <= 2^-8|ref| + 1e-4 absum; first at %s:"
                             " got %r ref %r absum %r" % (what, len(bad), ok.size, i, got[i],
                                                          ref[i], absum[i]))


def run_gemm(fmt, a, s, w, ws, bias, epi, ld_pad=0):
    """Run the GPU GEMM on host arrays (optionally with padded leading
    dimensions) and return y as float64 [M, N]."""
    M, K = a.shape
    N = w.shape[0]
    if ld_pad:
        a_full = np.zeros((M, K + ld_pad), dtype=np.uint8)
        a_full[:, :K] = a
        a_t = u8_dev(a_full)[:, :K]
        w_full = np.zeros((N, w.shape[1] + ld_pad), dtype=np.uint8)
        w_full[:, :w.shape[1]] = w
        w_t = u8_dev(w_full)[:, :w.shape[1]]
        y_t = torch.full((M, N + ld_pad), float("nan"), dtype=torch.bfloat16, device=DEV)[:, :N]
    else:
        a_t, w_t, y_t = u8_dev(a), u8_dev(w), None
    b_t = bf16_dev(bias) if bias is not None else None
    fn = bs.gemm_bs_fp8 if fmt == "fp8" else bs.gemm_mxfp4_w4a8
    y = fn(a_t, f32_dev(s), w_t, u8_dev(ws), b_t, epi, y=y_t)
    return y_host(y)
