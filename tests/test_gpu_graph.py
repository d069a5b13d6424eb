"""The calls are capture-safe: quantize + GEMM recorded into a HIP graph and
replayed several times, with eager work and synchronisation between the
replays, give the eager result bit for bit on every replay (decode, wide
decode, split-K decode and prefill paths; each kernel is deterministic).
The split-K workspace is filled with NaN before each replay: its contents
on entry must not matter."""
import numpy as np
import pytest
import torch

import mxfp4_gemm_transformer_amd as bs
import synth
from gpu_util import DEV, bf16_dev, u8_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt,M,N,K,epi", [("fp8", 8, 2048, 1024, synth.EPI_BIAS_GELU_TANH),
                                           ("mxfp4", 4, 32768 + 32, 640, synth.EPI_NONE),
                                           ("fp8", 24, 2048, 1024, synth.EPI_BIAS),
                                           ("mxfp4", 64, 1024 + 32, 2080, synth.EPI_BIAS_GELU_TANH),
                                           ("fp8", 300, 1024, 512, synth.EPI_BIAS),
                                           ("mxfp4", 512, 4096 + 96, 256, synth.EPI_BIAS)])
def test_graph_replays_match_eager(fmt, M, N, K, epi):
    rng = np.random.default_rng(M + N)
    x = bf16_dev(synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)))
    if fmt == "fp8":
        w = u8_dev(rng.integers(0, 0x7E, size=(N, K), dtype=np.uint8) |
                   (rng.integers(0, 2, size=(N, K), dtype=np.uint8) << 7))
        ws = u8_dev(rng.integers(120, 131, size=(N // 32, K // 32), dtype=np.uint8))
        gemm = bs.gemm_bs_fp8
    else:
        w = u8_dev(rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8))
        ws = u8_dev(rng.integers(120, 131, size=(N, K // 32), dtype=np.uint8))
        gemm = bs.gemm_mxfp4_w4a8
    b = bf16_dev(synth.to_bf16_bits((rng.standard_normal(N) * 0.1).astype(np.float32)))
    bias = b if epi else None
    q = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    s = torch.empty((M,), dtype=torch.float32, device=DEV)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    need = bs.bs_workspace_bytes(0 if fmt == "fp8" else 1, M, N, K)
    work = torch.full((max(need, 4) // 4,), float("nan"), dtype=torch.float32, device=DEV)

    bs.fp8_quant_rows(x, q, s)
    gemm(q, s, w, ws, bias, epi, y=y, workspace=work)
    torch.cuda.synchronize()
    y_eager, q_eager, s_eager = y.clone(), q.clone(), s.clone()

    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        bs.fp8_quant_rows(x, q, s)
        gemm(q, s, w, ws, bias, epi, y=y, workspace=work)
    for r in range(4):
        y.fill_(float("nan"))
        work.fill_(float("nan"))
        q.zero_()
        s.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(q, q_eager), "replay %d: codes" % r
        assert torch.equal(s, s_eager), "replay %d: scales" % r
        assert torch.equal(y.view(torch.int16), y_eager.view(torch.int16)), "replay %d: y" % r
        # eager work between replays
        bs.fp8_quant_rows(x[: max(1, M // 2)])
        torch.cuda.synchronize()
