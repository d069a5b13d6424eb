"""Seeded synthetic workloads for the block-scaled linear layer.

Both the CPU oracle's tests and the GPU library's tests and benchmark draw
their inputs here; this module holds random draws and the offline weight
preparation that turns drawn weight values into stored codes, nothing of the
layer's own arithmetic (activation quantization, decoding, the GEMM or its
epilogue).

Every tensor has its own PCG64 stream, keyed by (seed, tensor id), so a
tensor does not change when another one's shape does: W is the same across
an M sweep, and A for M rows is the first M rows of A for more rows.

Workloads (shapes from the vLLM DeepSeek-V4 AMD mono runner page's weight
tables, the flash-rt groot_n17 ViT fc1 site and the sly-radiance README's
fused gate_up):

  tiny     M=16,  N=256,   K=256,  e4m3 W, 32x32 E8M0, bias epilogue
  decode   M in {1,4,8,16,64}, N=2048, K=7168, e4m3 W (wqkv's [2048, 7168]
           with its [64, 224] scale grid), no bias
  prefill  M=4096, N=7168, K=8192, e4m3 W, 1% of A's columns scaled x20
  prefill_shard  the prefill layer's share on one of eight GPUs when its
           output columns are split: M=4096, N=896, K=8192 (28 scale-block
           rows), the same laws and its own draws
  ffn_up   M=2048, N=4096, K=1024, e4m3 W, bias + tanh-GELU (second variant
           bias only)
  gate_up  M in {1,16,512,4096}, N=34816, K=5120, MXFP4 W (e2m1 + 1x32 E8M0)
  gate_up_w4a4  the gate_up layer with MXFP4 activations too (W4A4: the
           activations quantized per 32 by the OCP MX rule)
  lm_head  M in {1,8,16}, N=248320, K=5120, e4m3 W with one fp32 scale per
           output channel (the sly-radiance README's fp8 lm_head: weight
           quantized per output channel, per-token fp8 activations)

Value laws: A ~ N(0,1) rounded to bf16; e4m3 W = nearest e4m3 code of an
N(0, 0.05) sample; 32x32 scale bytes uniform on [120, 130]; bias ~ N(0, 0.1)
rounded to bf16; MXFP4 W from N(0, 0.02) samples by the OCP MX conversion;
per-channel e4m3 W from N(0, 0.02) samples rounded to bf16, each row
quantized with scale amax/448 (the per-token rule applied to weight rows).

Fused-producer inputs (the sly-radiance README's add_rms_quant and
silu_mul_quant feed the 5120-wide gate_up and the 17408-wide down
projection of the same model):

  add_rms   x [M, 5120] ~ N(0,1), residual ~ N(0, 2^2), norm weight
            ~ U(0.5, 1.5), all rounded to bf16; eps = 1e-6
  silu_mul  gate_up [M, 2*17408] ~ N(0, 1.5^2) rounded to bf16 (gate in
            the first half)
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

EPI_NONE, EPI_BIAS, EPI_BIAS_GELU_TANH = 0, 1, 2

# tensor ids of the per-tensor streams
_T_A, _T_OUTLIER, _T_W, _T_WS, _T_BIAS = 0, 1, 2, 3, 4
_T_RES, _T_GAMMA, _T_GU = 5, 6, 7


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    fmt: str               # "fp8" (e4m3 W, 32x32 scales), "mxfp4", "mxfp4_w4a4" or "fp8_rowwise"
    epilogue: int
    outlier_frac: float = 0.0
    m_sweep: tuple = ()


WORKLOADS = {
    "tiny": Workload("tiny", 16, 256, 256, "fp8", EPI_BIAS),
    "decode": Workload("decode", 8, 2048, 7168, "fp8", EPI_NONE, m_sweep=(1, 4, 8, 16, 64)),
    "prefill": Workload("prefill", 4096, 7168, 8192, "fp8", EPI_NONE, outlier_frac=0.01),
    "prefill_shard": Workload("prefill_shard", 4096, 896, 8192, "fp8", EPI_NONE,
                              outlier_frac=0.01),
    "ffn_up": Workload("ffn_up", 2048, 4096, 1024, "fp8", EPI_BIAS_GELU_TANH),
    "ffn_up_bias": Workload("ffn_up_bias", 2048, 4096, 1024, "fp8", EPI_BIAS),
    "gate_up": Workload("gate_up", 16, 34816, 5120, "mxfp4", EPI_NONE, m_sweep=(1, 16, 512, 4096)),
    "gate_up_w4a4": Workload("gate_up_w4a4", 4096, 34816, 5120, "mxfp4_w4a4", EPI_NONE,
                             m_sweep=(16, 512, 4096)),
    "lm_head": Workload("lm_head", 8, 248320, 5120, "fp8_rowwise", EPI_NONE, m_sweep=(1, 8, 16)),
}


def _rng(seed: int, tensor: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tensor,))))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), torch's round-to-nearest-even cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def activations(wl: Workload, M: int | None = None, seed: int = 0) -> np.ndarray:
    """bf16 bits [M, K]: N(0,1) samples; for the prefill workload
    round(frac*K) distinct columns are multiplied by 20 before rounding."""
    M = wl.M if M is None else M
    a = _rng(seed, _T_A).standard_normal((M, wl.K), dtype=np.float32)
    if wl.outlier_frac > 0:
        cols = _rng(seed, _T_OUTLIER).choice(wl.K, size=int(round(wl.outlier_frac * wl.K)),
                                             replace=False)
        a[:, cols] *= np.float32(20.0)
    return to_bf16_bits(a)


def weight_values(wl: Workload, seed: int = 0, rows: slice | None = None) -> np.ndarray:
    """float32 weight samples [N, K] (or a slice of rows) before encoding."""
    std = 0.05 if wl.fmt == "fp8" else 0.02
    rng = _rng(seed, _T_W)
    if rows is None or rows == slice(None):
        return rng.standard_normal((wl.N, wl.K), dtype=np.float32) * np.float32(std)
    start, stop = rows.start or 0, rows.stop
    rng.standard_normal((start, wl.K), dtype=np.float32)  # advance the stream
    return rng.standard_normal((stop - start, wl.K), dtype=np.float32) * np.float32(std)


def _encode_e4m3_weights(v: np.ndarray) -> np.ndarray:
    # Offline weight preparation with torch's float8_e4m3fn cast (nearest,
    # ties to even). The samples are far below the format's range, where the
    # cast and a saturating encoder agree; a CPU test compares the result
    # with the oracle's encoder on every generated value of the tiny
    # workload and on samples of the others.
    assert np.abs(v).max() < 448.0
    return torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _mx_quantize_rows(v: np.ndarray):
    # Offline OCP MX conversion of weight rows: per 32 consecutive k, the
    # shared exponent floor(log2 amax) - 2, its E8M0 byte (clamped to
    # [0, 254]), and each element's nearest e2m1 code (ties to the even
    # code, saturating at 6) of v / 2^exponent. A CPU test checks the
    # result bit for bit against the oracle's own conversion.
    n, K = v.shape
    g = v.reshape(n, K // 32, 32).astype(np.float64)
    amax = np.abs(g).max(axis=2)
    _, ex = np.frexp(amax)
    byte = np.where(amax > 0, np.clip(ex - 1 - 2 + 127, 0, 254), 0).astype(np.int64)
    x = g / np.ldexp(1.0, byte - 127)[..., None]
    a = np.minimum(np.abs(x), 6.0)
    lo = np.searchsorted(_E2M1_GRID, a, side="right") - 1          # grid[lo] <= a
    hi = np.minimum(lo + 1, 7)
    mid = 0.5 * (_E2M1_GRID[lo] + _E2M1_GRID[hi])
    code = np.where(a < mid, lo, np.where(a > mid, hi, np.where(lo & 1, hi, lo)))
    code = np.where(a >= 6.0, 7, code)
    code = code | np.where(np.signbit(x), 8, 0)
    code = code.reshape(n, K).astype(np.uint8)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, byte.astype(np.uint8)


def _rowwise_quantize_rows(v_bf16: np.ndarray):
    # Offline per-output-channel weight quantization: per row, the scale
    # fl32(amax / 448) and each element's e4m3 code of fl32(w / scale) by
    # torch's float8_e4m3fn cast (nearest, ties even; |w / scale| <= 448 up
    # to the fp32 rounding of the division, which the cast rounds to 448).
    # A CPU test checks the result bit for bit against the oracle's
    # per-token quantizer applied to the weight rows.
    t = torch.from_numpy(np.ascontiguousarray(v_bf16).view(np.int16)).view(torch.bfloat16).float()
    amax = t.abs().amax(dim=1)
    scale = (amax.double() / 448.0).float()
    safe = torch.where(scale > 0, scale, torch.ones_like(scale))
    q = (t / safe[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return q, scale.numpy()


def weight_bf16_rows(wl: Workload, r0: int, r1: int, seed: int = 0) -> np.ndarray:
    """bf16 bits of weight rows [r0, r1) for the per-channel workloads."""
    rng = _rng(seed, _T_W)
    if r0:
        rng.standard_normal((r0, wl.K), dtype=np.float32)   # advance the stream
    return to_bf16_bits(rng.standard_normal((r1 - r0, wl.K), dtype=np.float32) * np.float32(0.02))


def weights(wl: Workload, seed: int = 0):
    """(W, W scales): e4m3 codes [N, K] with E8M0 [N/32, K/32] uniform on
    [120, 130]; MXFP4 packed [N, K/2] with E8M0 [N, K/32]; or e4m3 codes
    [N, K] with one fp32 scale per row [N] (fmt "fp8_rowwise")."""
    if wl.fmt == "fp8_rowwise":
        codes = np.empty((wl.N, wl.K), dtype=np.uint8)
        scales = np.empty((wl.N,), dtype=np.float32)
        rng = _rng(seed, _T_W)
        chunk = 8192
        for r0 in range(0, wl.N, chunk):
            r1 = min(wl.N, r0 + chunk)
            v = to_bf16_bits(rng.standard_normal((r1 - r0, wl.K), dtype=np.float32) * np.float32(0.02))
            codes[r0:r1], scales[r0:r1] = _rowwise_quantize_rows(v)
        return codes, scales
    if wl.fmt == "fp8":
        w = _encode_e4m3_weights(weight_values(wl, seed))
        ws = _rng(seed, _T_WS).integers(120, 131, size=(wl.N // 32, wl.K // 32),
                                        dtype=np.uint8)
        return w, ws
    packed = np.empty((wl.N, wl.K // 2), dtype=np.uint8)
    scales = np.empty((wl.N, wl.K // 32), dtype=np.uint8)
    rng = _rng(seed, _T_W)
    chunk = 2048
    for r0 in range(0, wl.N, chunk):
        r1 = min(wl.N, r0 + chunk)
        v = rng.standard_normal((r1 - r0, wl.K), dtype=np.float32) * np.float32(0.02)
        packed[r0:r1], scales[r0:r1] = _mx_quantize_rows(v)
    return packed, scales


def bias(wl: Workload, seed: int = 0):
    """bf16 bits [N] ~ N(0, 0.1), or None for workloads without a bias."""
    if wl.epilogue == EPI_NONE:
        return None
    b = _rng(seed, _T_BIAS).standard_normal((wl.N,), dtype=np.float32) * np.float32(0.1)
    return to_bf16_bits(b)


def make(name: str, M: int | None = None, seed: int = 0) -> dict:
    """All inputs of a workload: A bf16 bits, W, W scales, bias, epilogue."""
    wl = WORKLOADS[name]
    w, ws = weights(wl, seed)
    return {"wl": wl, "M": wl.M if M is None else M, "a_bf16": activations(wl, M, seed),
            "w": w, "w_scale": ws, "bias": bias(wl, seed), "epilogue": wl.epilogue}


# grouped MoE W4A8: the mono runner page's routed-expert layout (w13
# [experts, 2 inter, hidden / 2] fp4x2, scales [experts * 2 inter, hidden/32])
# at hidden = 7168 (its projection widths); the expert count, intermediate
# size and routing are this workload's choice: 32 local experts, 2 inter =
# 4096, top-8 routing of a decode batch of 8 tokens.
MOE = {"E": 32, "N": 4096, "K": 7168, "tokens": 8, "topk": 8}
# the same experts at prefill: 512 tokens routed top-8 (4096 rows, about 128
# per expert)
MOE_PREFILL = {"E": 32, "N": 4096, "K": 7168, "tokens": 512, "topk": 8}
_T_ROUTE = 8


def moe_routing(tokens: int, E: int, topk: int, seed: int = 0):
    """(row_token [tokens * topk], offsets [E + 1] int32): each token picks
    topk distinct experts uniformly; rows are the (token, expert) pairs
    sorted by expert (then token)."""
    rng = _rng(seed, _T_ROUTE)
    pairs = [(int(e), t) for t in range(tokens) for e in rng.choice(E, size=topk, replace=False)]
    pairs.sort()
    row_token = np.array([t for _, t in pairs], dtype=np.int64)
    counts = np.bincount([e for e, _ in pairs], minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return row_token, offsets


def moe_weights(E: int, N: int, K: int, seed: int = 0, distinct: int | None = None):
    """MXFP4 expert weights [E, N, K/2] and scales [E, N, K/32] from
    N(0, 0.02) samples by the OCP MX conversion; with `distinct`, expert e
    holds a copy of expert e % distinct (a large bench configuration drawn
    quickly)."""
    distinct = E if distinct is None else distinct
    packed = np.empty((E, N, K // 2), dtype=np.uint8)
    scales = np.empty((E, N, K // 32), dtype=np.uint8)
    rng = _rng(seed, _T_W)
    for e in range(distinct):
        for r0 in range(0, N, 2048):
            r1 = min(N, r0 + 2048)
            v = rng.standard_normal((r1 - r0, K), dtype=np.float32) * np.float32(0.02)
            packed[e, r0:r1], scales[e, r0:r1] = _mx_quantize_rows(v)
    for e in range(distinct, E):
        packed[e] = packed[e % distinct]
        scales[e] = scales[e % distinct]
    return packed, scales


# fused producers: name -> (row width at full size, M sweep)
PRODUCERS = {
    "add_rms": (5120, (1, 16, 512, 4096)),
    "silu_mul": (17408, (1, 16, 512, 4096)),
}
RMS_EPS = 1e-6


def producer_inputs(name: str, M: int, width: int | None = None, seed: int = 0) -> dict:
    """Inputs of a fused producer as bf16 bits. add_rms: x [M, width],
    residual [M, width], weight [width], eps. silu_mul: gate_up [M, 2 width]."""
    width = PRODUCERS[name][0] if width is None else width
    if name == "add_rms":
        x = _rng(seed, _T_A).standard_normal((M, width), dtype=np.float32)
        r = _rng(seed, _T_RES).standard_normal((M, width), dtype=np.float32) * np.float32(2.0)
        g = _rng(seed, _T_GAMMA).uniform(0.5, 1.5, width).astype(np.float32)
        return {"x": to_bf16_bits(x), "residual": to_bf16_bits(r), "weight": to_bf16_bits(g),
                "eps": RMS_EPS, "M": M, "K": width}
    if name == "silu_mul":
        gu = _rng(seed, _T_GU).standard_normal((M, 2 * width), dtype=np.float32) * np.float32(1.5)
        return {"gate_up": to_bf16_bits(gu), "M": M, "I": width}
    raise KeyError(name)
