"""fp8_quant_rows on the GPU against the oracle: codes and scales bit-exact.

Covers every workload's activations at full size, the M sweeps, ragged and
padded shapes, every e4m3 rounding tie, zero / single-value / subnormal rows,
and rows long enough for the two-pass kernel."""
import numpy as np
import pytest
import torch

import mxfp4_gemm_transformer_amd as bs
import oracle
import synth
from gpu_util import DEV, bf16_dev

pytestmark = pytest.mark.gpu


def _check(x_bits, ld_pad=0):
    M, K = x_bits.shape
    if ld_pad:
        full = np.zeros((M, K + ld_pad), dtype=np.uint16)
        full[:, :K] = x_bits
        x = bf16_dev(full)[:, :K]
        q_full = torch.full((M, K + ld_pad), 0xAA, dtype=torch.uint8, device=DEV)
        q, s = bs.fp8_quant_rows(x, q=q_full[:, :K])
    else:
        q, s = bs.fp8_quant_rows(bf16_dev(x_bits))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_rows(x_bits)
    qh = q.cpu().numpy()
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    if not np.array_equal(qh, q_ref):
        bad = np.argwhere(qh != q_ref)
        m, k = bad[0]
        raise AssertionError("%d codes differ; first at (%d, %d): got %#x want %#x (x bits %#x)"
                             % (len(bad), m, k, qh[m, k], q_ref[m, k], x_bits[m, k]))
    if ld_pad:
        assert torch.all(q_full[:, K:] == 0xAA), "wrote past the row"


@pytest.mark.parametrize("name,M", [("tiny", None), ("decode", 1), ("decode", 4), ("decode", 8),
                                    ("decode", 16), ("decode", 64), ("ffn_up", None),
                                    ("gate_up", 1), ("gate_up", 16), ("gate_up", 512),
                                    ("gate_up", 4096)])
def test_quant_workloads(name, M):
    _check(synth.activations(synth.WORKLOADS[name], M))


def test_quant_prefill_full_size():
    # 4096 x 8192 with 82 outlier columns x20
    _check(synth.activations(synth.WORKLOADS["prefill"]))


@pytest.mark.parametrize("M,K", [(3, 32), (17, 96), (5, 544), (300, 4128), (33, 8192 + 32),
                                 (2, 65536 + 64), (1, 131072),
                                 # one row: 512 threads of one to four chunks, or
                                 # 256 threads past that
                                 (1, 2080), (1, 8192 + 32), (1, 16384 + 32),
                                 # many rows: 64 / 256 / 512 threads a row, 1-3 chunks a
                                 # thread, and rows too long for 512 threads
                                 (513, 96), (700, 2080), (600, 4128), (1030, 8224),
                                 (512, 16384), (520, 32768)])
def test_quant_ragged_shapes(M, K):
    rng = np.random.default_rng(M * 1000 + K)
    x = synth.to_bf16_bits((rng.standard_normal((M, K)) * rng.uniform(0.01, 50, (M, 1))).astype(np.float32))
    _check(x)


@pytest.mark.parametrize("pad", [16, 48])
def test_quant_padded_leading_dims(pad):
    rng = np.random.default_rng(pad)
    x = synth.to_bf16_bits(rng.standard_normal((37, 224)).astype(np.float32))
    _check(x, ld_pad=pad)


def test_quant_every_tie_and_its_neighbours():
    t = oracle.e4m3_table()
    mids = np.array([0.5 * (t[c] + t[c + 1]) for c in range(0x7E)], dtype=np.float32)
    bits = synth.to_bf16_bits(mids)
    # each midpoint, its bf16 neighbours below and above, and negatives
    nb = np.concatenate([bits, bits - 1, bits + 1]).astype(np.uint16)
    row = np.concatenate([synth.to_bf16_bits(np.array([448.0], dtype=np.float32)), nb, nb | 0x8000])
    row = np.concatenate([row, np.zeros((-row.size) % 32, dtype=np.uint16)])
    _check(row[None, :].repeat(3, axis=0))


def test_quant_special_rows():
    K = 256
    rows = np.zeros((6, K), dtype=np.float32)
    rows[2, 100] = -3.0
    rows[3, :] = 1.0
    rows[4, :] = np.float32(1e-39)
    rows[4, 5] = np.float32(-2.5e-39)
    rows[5, ::2] = 3.0e38
    rows[5, 1::2] = -1.0
    x = synth.to_bf16_bits(rows)
    x[1, :] = 0x8000
    _check(x)


def test_quant_random_bit_patterns():
    # every finite bf16 magnitude class, scaled rows
    rng = np.random.default_rng(5)
    x = rng.integers(0, 1 << 16, size=(64, 1024), dtype=np.uint32).astype(np.uint16)
    x[(x & 0x7F80) == 0x7F80] &= 0xBFFF      # drop Inf/NaN
    _check(x)


def test_quant_rejects_bad_arguments():
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(bs.BsError) as e:
        bs.fp8_quant_rows(x[:, :48])           # K not a multiple of 32
    assert e.value.status == bs.BS_EINVAL
    with pytest.raises(bs.BsError) as e:
        bs.fp8_quant_rows(torch.zeros((4, 68), dtype=torch.bfloat16, device=DEV)[:, 4:68])
    assert e.value.status == bs.BS_EALIGN
