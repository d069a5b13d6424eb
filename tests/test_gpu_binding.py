"""The Python binding's device checks and stream handling, and the decode
dispatcher's limits, on the GPU.

- Every pointer argument must be a tensor on the operands' device: a host
  tensor is refused with ValueError before anything launches.
- Outputs and the split-K workspace the binding allocates belong to the
  stream the kernels run on, so a call on a side stream matches the same call
  on the current stream.
- Wide decode layers whose workgroups own more rows than their 1024 threads
  can stage epilogue operands for (8 rows per group, 128 groups a workgroup
  at N = 262144 on 256 CUs) take another kernel and stay correct with a bias.
"""
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
    x = synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    a, s = oracle.quant_rows(x)
    w = oracle.encode_e4m3((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
    ws = rng.integers(120, 131, size=(N // 32, K // 32), dtype=np.uint8)
    b = synth.to_bf16_bits((rng.standard_normal(N) * 0.1).astype(np.float32))
    return a, s, w, ws, b


def test_host_tensors_are_refused():
    a, s, w, ws, b = _problem(8, 64, 256, seed=3)
    A, S, W, WS, B = u8_dev(a), f32_dev(s), u8_dev(w), u8_dev(ws), bf16_dev(b)
    for kw in ({"a_scale": torch.from_numpy(s)}, {"w_scale": torch.from_numpy(ws)},
               {"bias": torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)}):
        args = {"a": A, "a_scale": S, "w": W, "w_scale": WS, "bias": B}
        args.update(kw)
        with pytest.raises(ValueError, match="device tensor"):
            bs.gemm_bs_fp8(args["a"], args["a_scale"], args["w"], args["w_scale"], args["bias"],
                           bs.EPI_BIAS)
    # a workspace on the host, for a split-K call (M = 16)
    a16, s16, w16, ws16, _ = _problem(16, 2048, 1024, seed=4)
    assert bs.bs_workspace_bytes(0, 16, 2048, 1024) > 0
    with pytest.raises(ValueError, match="workspace"):
        bs.gemm_bs_fp8(u8_dev(a16), f32_dev(s16), u8_dev(w16), u8_dev(ws16),
                       workspace=torch.zeros(1 << 20, dtype=torch.uint8))
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="scale"):
        bs.fp8_quant_rows(x, scale=torch.zeros(4, dtype=torch.float32))


def test_split_k_on_a_side_stream():
    # the binding allocates y and the workspace on the side stream the
    # kernels run on; other work on the current stream cannot take them
    a, s, w, ws, b = _problem(16, 2048, 7168, seed=5)
    A, S, W, WS = u8_dev(a), f32_dev(s), u8_dev(w), u8_dev(ws)
    ref_dev = y_host(bs.gemm_bs_fp8(A, S, W, WS))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(4):
        outs.append(bs.gemm_bs_fp8(A, S, W, WS, stream=side))
        junk = torch.empty(bs.bs_workspace_bytes(0, 16, 2048, 7168), dtype=torch.uint8,
                           device=DEV).fill_(0xFF)   # current-stream work meanwhile
    torch.cuda.current_stream().wait_stream(side)
    del junk
    ref, absum = oracle.gemm_bs_fp8(a, s, w, ws)
    assert_within(ref_dev, ref, absum, "current stream")
    for y in outs:
        got = y_host(y)
        assert np.array_equal(got, ref_dev)


@pytest.mark.parametrize("fmt", ["mxfp4", "fp8_rowwise"])
@pytest.mark.parametrize("M", [1, 12])
def test_wide_decode_layer_with_bias(fmt, M):
    # 262144 rows at K = 640: 128 groups of 8 rows per workgroup on 256 CUs,
    # more bias entries than threads for the units kernel
    N, K = 262144, 640
    rng = np.random.default_rng(M + 11)
    a, s = oracle.quant_rows(synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)))
    b = synth.to_bf16_bits((rng.standard_normal(N) * 0.1).astype(np.float32))
    if fmt == "mxfp4":
        w, ws = oracle.quant_mxfp4_weights((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
        y = bs.gemm_mxfp4_w4a8(u8_dev(a), f32_dev(s), u8_dev(w), u8_dev(ws), bf16_dev(b),
                               bs.EPI_BIAS)
        ref, absum = oracle.gemm_mxfp4_w4a8(a, s, w, ws, b, bs.EPI_BIAS)
    else:
        w, ws = oracle.quant_rows(synth.to_bf16_bits((rng.standard_normal((N, K)) * 0.02)
                                                     .astype(np.float32)))
        y = bs.gemm_fp8_rowwise(u8_dev(a), f32_dev(s), u8_dev(w), f32_dev(ws), bf16_dev(b),
                                bs.EPI_BIAS)
        ref, absum = oracle.gemm_fp8_rowwise(a, s, w, ws, b, bs.EPI_BIAS)
    assert_within(y_host(y), ref, absum, "%s M=%d N=%d K=%d bias" % (fmt, M, N, K))
