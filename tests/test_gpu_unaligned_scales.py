"""E8M0 scale grids at any byte address: the GEMMs take the grid pointers
(the block-scaled weights' grid, MXFP4 activations' grid) as plain bytes, so
a grid that starts 1, 2 or 3 bytes past an aligned address (a slice of a
larger byte buffer) must give the same outputs as an aligned one, on every
kernel a shape can reach: the folded and split-K decode, the wide-layer
decode (which reads whole 4-byte scale words and so takes the folded path
for an unaligned grid), the prefill tiles with per-step scale loads and
with the tile's scale rows staged once (MXFP4, K % 128 == 0), W4A4, and the
grouped MoE GEMM."""
import numpy as np
import pytest
import torch

import mxfp4_gemm_transformer_amd as bs
import oracle
import synth
from gpu_util import DEV, assert_within, bf16_dev, f32_dev, u8_dev, y_host

pytestmark = pytest.mark.gpu


def _at(host: np.ndarray, off: int) -> torch.Tensor:
    """A contiguous device copy of `host` whose first byte is `off` bytes past
    a 256-byte aligned address (inside a larger buffer)."""
    n = host.size
    buf = torch.zeros(n + 256, dtype=torch.uint8, device=DEV)
    t = buf[off:off + n].view(host.shape)
    t.copy_(u8_dev(host))
    assert t.data_ptr() % 256 == off
    return t


def _problem(fmt, M, N, K, seed):
    rng = np.random.default_rng(seed)
    x = synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    a, s = oracle.quant_rows(x)
    if fmt == "fp8":
        w = oracle.encode_e4m3((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
        ws = rng.integers(120, 131, size=(N // 32, K // 32), dtype=np.uint8)
    else:
        w, ws = oracle.quant_mxfp4_weights((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    b = synth.to_bf16_bits((rng.standard_normal(N) * 0.1).astype(np.float32))
    return a, s, w, ws, b


# (fmt, M, N, K): folded decode (one and two token groups), split-K decode,
# the wide-layer decode shape, prefill tiles (e4m3: per-step scale loads;
# MXFP4 K % 128 == 0: staged scale rows; K % 128 == 64: per-step loads)
CASES = [("fp8", 8, 256, 1024), ("fp8", 16, 256, 1024), ("fp8", 33, 256, 1024),
         ("fp8", 200, 384, 1024), ("mxfp4", 1, 256, 1024), ("mxfp4", 33, 256, 1024),
         ("mxfp4", 1, 32768 + 32, 640), ("mxfp4", 200, 384, 1024), ("mxfp4", 200, 384, 1088)]


@pytest.mark.parametrize("fmt,M,N,K", CASES)
@pytest.mark.parametrize("off", [1, 2, 3])
def test_unaligned_weight_scale_grid(fmt, M, N, K, off):
    a, s, w, ws, b = _problem(fmt, M, N, K, seed=M + N + K + off)
    epi = synth.EPI_BIAS
    fn = bs.gemm_bs_fp8 if fmt == "fp8" else bs.gemm_mxfp4_w4a8
    y = fn(u8_dev(a), f32_dev(s), u8_dev(w), _at(ws, off), bf16_dev(b), epi)
    ref, absum = (oracle.gemm_bs_fp8 if fmt == "fp8" else oracle.gemm_mxfp4_w4a8)(a, s, w, ws, b, epi)
    assert_within(y_host(y), ref, absum, "%s M=%d N=%d K=%d grid at +%d" % (fmt, M, N, K, off))


@pytest.mark.parametrize("M,N,K", [(8, 256, 1024), (16, 32768 + 32, 640), (200, 384, 1024)])
@pytest.mark.parametrize("off", [1, 2])
def test_unaligned_w4a4_scale_grids(M, N, K, off):
    rng = np.random.default_rng(M + K + off)
    a, sa = oracle.quant_mxfp4_rows(synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)))
    w, sw = oracle.quant_mxfp4_weights((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    b = synth.to_bf16_bits((rng.standard_normal(N) * 0.1).astype(np.float32))
    y = bs.gemm_mxfp4_w4a4(u8_dev(a), _at(sa, off), u8_dev(w), _at(sw, 4 - off), bf16_dev(b),
                           synth.EPI_BIAS)
    ref, absum = oracle.gemm_mxfp4_w4a4(a, sa, w, sw, b, synth.EPI_BIAS)
    assert_within(y_host(y), ref, absum, "w4a4 M=%d N=%d K=%d grids at +%d/+%d" % (M, N, K, off, 4 - off))


# rows per expert: a few (the grouped decode kernel) and about 60 (the
# grouped prefill tiles, scale rows staged since K % 128 == 0)
@pytest.mark.parametrize("T0,topk", [(8, 4), (120, 4)])
def test_unaligned_grouped_scale_grid(T0, topk):
    E, N, K = 8, 128, 512
    rng = np.random.default_rng(T0)
    x = synth.to_bf16_bits(rng.standard_normal((T0, K)).astype(np.float32))
    row_token, off = synth.moe_routing(T0, E, topk, seed=T0)
    a, s = oracle.quant_rows(x[row_token])
    w, ws = synth.moe_weights(E, N, K, seed=T0)
    T = a.shape[0]
    y = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    bs.gemm_mxfp4_w4a8_grouped(u8_dev(a), f32_dev(s), torch.from_numpy(off).to(DEV), u8_dev(w),
                               _at(ws, 1), None, synth.EPI_NONE, y=y,
                               max_rows_per_expert=int(np.diff(off).max()))
    ref, absum = oracle.gemm_mxfp4_w4a8_grouped(a, s, off, w, ws)
    assert_within(y_host(y), ref, absum, "grouped T0=%d grid at +1" % T0)
