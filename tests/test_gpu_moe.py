"""Grouped (MoE) W4A8 GEMM on the GPU against the oracle: expert-sorted
token rows, device offsets, empty experts, experts with more rows than one
pass takes (and a too-small row bound), bias per expert, rows outside every
expert left untouched, and the 32-expert decode workload at full size."""
import numpy as np
import pytest
import torch

import mxfp4_gemm_transformer_amd as bs
import oracle
import synth
from gpu_util import DEV, assert_within, bf16_dev, f32_dev, u8_dev, y_host

pytestmark = pytest.mark.gpu


def _case(T0, E, topk, N, K, seed, distinct=None):
    rng = np.random.default_rng(seed)
    x = synth.to_bf16_bits(rng.standard_normal((T0, K)).astype(np.float32))
    row_token, off = synth.moe_routing(T0, E, topk, seed=seed)
    a, s = oracle.quant_rows(x[row_token])
    w, ws = synth.moe_weights(E, N, K, seed=seed, distinct=distinct)
    b = synth.to_bf16_bits((rng.standard_normal((E, N)) * 0.1).astype(np.float32))
    return a, s, off, w, ws, b


def _run(a, s, off, w, ws, b, epi, max_rows=None, extra_rows=0):
    T, K = a.shape
    N = w.shape[1]
    a_full = np.zeros((T + extra_rows, K), np.uint8); a_full[:T] = a
    s_full = np.ones(T + extra_rows, np.float32); s_full[:T] = s
    y = torch.full((T + extra_rows, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    bs.gemm_mxfp4_w4a8_grouped(u8_dev(a_full), f32_dev(s_full),
                               torch.from_numpy(off).to(DEV), u8_dev(w), u8_dev(ws),
                               bf16_dev(b) if epi else None, epi, y=y, max_rows_per_expert=max_rows)
    return y_host(y)


@pytest.mark.parametrize("T0,E,topk,N,K", [(6, 8, 3, 64, 256), (8, 16, 4, 128, 320),
                                           (8, 32, 8, 256, 1056)])
@pytest.mark.parametrize("epi", [synth.EPI_NONE, synth.EPI_BIAS_GELU_TANH])
def test_grouped_shapes(T0, E, topk, N, K, epi):
    a, s, off, w, ws, b = _case(T0, E, topk, N, K, seed=T0 + E + N + K)
    got = _run(a, s, off, w, ws, b, epi, max_rows=T0)
    ref, absum = oracle.gemm_mxfp4_w4a8_grouped(a, s, off, w, ws, b if epi else None, epi)
    assert_within(got, ref, absum, "moe T0=%d E=%d N=%d K=%d" % (T0, E, N, K))


@pytest.mark.parametrize("max_rows", [8, 16, 40, None])
def test_grouped_many_rows_per_expert(max_rows):
    """~27 rows per expert: several 8-token groups, several passes when the
    row bound is too small."""
    a, s, off, w, ws, b = _case(40, 3, 2, 96, 512, seed=5)
    assert np.diff(off).max() > 16
    got = _run(a, s, off, w, ws, b, synth.EPI_BIAS, max_rows=max_rows, extra_rows=5)
    ref, absum = oracle.gemm_mxfp4_w4a8_grouped(a, s, off, w, ws, b, synth.EPI_BIAS)
    T = off[-1]
    assert_within(got[:T], ref, absum, "moe many rows max_rows=%s" % max_rows)
    assert np.isnan(got[T:]).all(), "rows outside every expert were written"


def test_grouped_empty_and_single_expert():
    rng = np.random.default_rng(7)
    K, N, E = 256, 64, 5
    a, s = oracle.quant_rows(synth.to_bf16_bits(rng.standard_normal((12, K)).astype(np.float32)))
    w, ws = synth.moe_weights(E, N, K, seed=7)
    b = synth.to_bf16_bits((rng.standard_normal((E, N)) * 0.1).astype(np.float32))
    for off in (np.array([0, 0, 12, 12, 12, 12], np.int32), np.array([0, 0, 0, 0, 0, 12], np.int32),
                np.array([0, 3, 3, 7, 7, 12], np.int32)):
        got = _run(a, s, off, w, ws, b, synth.EPI_BIAS, max_rows=12)
        ref, absum = oracle.gemm_mxfp4_w4a8_grouped(a, s, off, w, ws, b, synth.EPI_BIAS)
        assert_within(got, ref, absum, "moe offsets %s" % off)


def test_moe_workload_full_size():
    m = synth.MOE
    a, s, off, w, ws, b = _case(m["tokens"], m["E"], m["topk"], m["N"], m["K"], seed=0, distinct=4)
    got = _run(a, s, off, w, ws, b, synth.EPI_NONE, max_rows=m["tokens"])
    ref, absum = oracle.gemm_mxfp4_w4a8_grouped(a, s, off, w, ws)
    assert_within(got, ref, absum, "moe workload")


# ---- prefill-sized expert batches (more than 32 rows per expert): the
# grouped form of the large-M tiles; ragged rows per expert, empty experts,
# a row bound below the largest expert (its workgroups then take further
# m-tiles), K with and without the tile's scale rows in LDS
def _explicit(rows, N, K, seed):
    rng = np.random.default_rng(seed)
    E = len(rows)
    off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    T = int(off[-1])
    a, s = oracle.quant_rows(synth.to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32)))
    w, ws = synth.moe_weights(E, N, K, seed=seed)
    b = synth.to_bf16_bits((rng.standard_normal((E, N)) * 0.1).astype(np.float32))
    return a, s, off, w, ws, b


@pytest.mark.parametrize("rows,N,K,max_rows", [
    ([0, 1, 64, 65, 130, 300, 0, 33], 288, 1024, None),     # 256x256 tiles, scale rows in LDS
    ([0, 1, 64, 65, 130, 300, 0, 33], 288, 1024, 100),      # 128x128, bound below the largest expert
    ([150, 0, 129, 33, 160], 288, 1024, None),               # 160x256 tiles
    ([300, 140, 0, 20], 288, 1024, 150),                     # 160x256, two m-tiles for one expert
    ([150, 7], 64, 256, None),                               # 160x256, fewer stages than buffers
    ([170, 5, 192, 0, 161], 544, 1024, None),                # 192x256 tiles
    ([40, 50, 0, 64], 160, 512, 64),                          # 64x64 tiles
    ([200, 0, 77, 129], 96, 1088, 200),                       # K % 128 = 64: one-step stages
])
@pytest.mark.parametrize("epi", [synth.EPI_NONE, synth.EPI_BIAS_GELU_TANH])
def test_grouped_prefill_sized_experts(rows, N, K, max_rows, epi):
    a, s, off, w, ws, b = _explicit(rows, N, K, seed=sum(rows) + N + K)
    mr = max(rows) if max_rows is None else max_rows
    assert mr > 32
    got = _run(a, s, off, w, ws, b, epi, max_rows=mr, extra_rows=3)
    ref, absum = oracle.gemm_mxfp4_w4a8_grouped(a, s, off, w, ws, b if epi else None, epi)
    T = off[-1]
    assert_within(got[:T], ref, absum, "moe prefill rows=%s N=%d K=%d bound=%s" % (rows, N, K, mr))
    assert np.isnan(got[T:]).all(), "rows outside every expert were written"


def test_grouped_prefill_workload_sampled():
    # 32 experts of [4096, 7168] MXFP4, 512 tokens routed top-8 (4096 rows,
    # about 128 per expert); outputs sampled per expert against the dense
    # oracle GEMM of that expert
    m = synth.MOE_PREFILL
    a, s, off, w, ws, b = _case(m["tokens"], m["E"], m["topk"], m["N"], m["K"], seed=0, distinct=4)
    max_rows = int(np.diff(off).max())
    assert max_rows > 32
    T, K = a.shape
    N = w.shape[1]
    y = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    bs.gemm_mxfp4_w4a8_grouped(u8_dev(a), f32_dev(s), torch.from_numpy(off).to(DEV), u8_dev(w),
                               u8_dev(ws), y=y, max_rows_per_expert=max_rows)
    got = y_host(y)
    rng = np.random.default_rng(3)
    for e in range(m["E"]):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r0 == r1:
            continue
        ms = np.concatenate([np.arange(r1 - r0), rng.integers(0, r1 - r0, 64)])
        ns = np.concatenate([rng.integers(0, N, r1 - r0), rng.integers(0, N, 64)])
        ref, absum = oracle.gemm_sampled("mxfp4", a[r0:r1], s[r0:r1], w[e], ws[e], None,
                                         synth.EPI_NONE, ms, ns)
        assert_within(got[r0 + ms, ns], ref, absum, "moe prefill workload expert %d" % e)
