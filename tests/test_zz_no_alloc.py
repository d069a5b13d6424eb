"""gemm_bs_fp8_noalloc (the entry point that allocates nothing: split-K
partial sums in the library's per-device scratch array) against gemm_bs_fp8
with a workspace, through the C ABI: identical outputs (the split-K
reduction adds the slices in a fixed order), within the oracle's tolerance,
on two calls in a row, the second with a smaller input; shapes that need
more scratch than the array holds are refused."""
import numpy as np
import pytest
import torch

import mxfp4_gemm_transformer_amd as bs
import oracle
import synth
from gpu_util import DEV, assert_within, bf16_dev, f32_dev, u8_dev, y_host

pytestmark = pytest.mark.gpu


def _problem(M, N, K, seed):
    rng = np.random.default_rng(seed)
    a, s = oracle.quant_rows(synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)))
    w = oracle.encode_e4m3((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
    ws = rng.integers(120, 131, size=(N // 32, K // 32), dtype=np.uint8)
    b = synth.to_bf16_bits((rng.standard_normal(N) * 0.1).astype(np.float32))
    return a, s, w, ws, b


@pytest.mark.parametrize("first,second", [((64, 2048, 7168, 0), (16, 1024, 2048, 2)),
                                          ((40, 2080, 1184, 1), (17, 96, 256, 0))])
def test_noalloc_matches_workspace_entry_point(first, second):
    for M, N, K, epi in (first, second):
        assert 0 < bs.bs_workspace_bytes(0, M, N, K) <= bs.NOALLOC_SCRATCH_BYTES
        a, s, w, ws, b = _problem(M, N, K, seed=M + N + K)
        A, S, W, WS = u8_dev(a), f32_dev(s), u8_dev(w), u8_dev(ws)
        B = bf16_dev(b) if epi else None
        y_ref = bs.gemm_bs_fp8(A, S, W, WS, B, epi)
        y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        bs.gemm_bs_fp8_noalloc(A, S, W, WS, B, epi, y=y)
        got, want = y_host(y), y_host(y_ref)
        assert np.array_equal(got, want), "M=%d N=%d K=%d" % (M, N, K)
        ref, absum = oracle.gemm_bs_fp8(a, s, w, ws, b if epi else None, epi)
        assert_within(got, ref, absum, "noalloc M=%d N=%d K=%d epi=%d" % (M, N, K, epi))


def test_noalloc_without_split_k_and_refusals():
    # M <= 8 on a narrow layer needs no scratch: the same kernels as gemm_bs_fp8
    a, s, w, ws, b = _problem(8, 2048, 7168, seed=3)
    A, S, W, WS = u8_dev(a), f32_dev(s), u8_dev(w), u8_dev(ws)
    y = torch.empty((8, 2048), dtype=torch.bfloat16, device=DEV)
    bs.gemm_bs_fp8_noalloc(A, S, W, WS, y=y)
    assert np.array_equal(y_host(y), y_host(bs.gemm_bs_fp8(A, S, W, WS)))
    # more scratch than the array holds: refused before any launch
    M, N, K = 64, 66560, 1024
    assert bs.bs_workspace_bytes(0, M, N, K) > bs.NOALLOC_SCRATCH_BYTES
    a2 = torch.zeros((M, K), dtype=torch.uint8, device=DEV)
    y2 = torch.zeros((M, N), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(bs.BsError) as e:
        bs.gemm_bs_fp8_noalloc(a2, torch.ones(M, dtype=torch.float32, device=DEV),
                               torch.zeros((N, K), dtype=torch.uint8, device=DEV),
                               torch.full((N // 32, K // 32), 127, dtype=torch.uint8, device=DEV),
                               y=y2)
    assert e.value.status == bs.BS_EWORKSPACE
    assert not y2.any()
