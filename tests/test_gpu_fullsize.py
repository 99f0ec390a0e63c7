"""GPU parity at the full workload sizes, on sampled rows the oracle computes one by one.

The GPU computes every row of the rank's share in the same launch configuration
the benchmark times; the oracle computes a seeded sample of rows (first/last
rows, zigzag half boundaries, document starts and ends, random rows) against
the whole global sequence.
"""
import numpy as np
import pytest
import torch

import oracle
import sequence_parallelism_amd as ra
import synth
from tests.gpu_common import (TOL_LSE_BF16, TOL_O_BF16, device_bits, max_abs, oracle_inputs, rank_inputs,
                              sample_rows, to_device)

pytestmark = pytest.mark.gpu


def _check_sampled(g, w, rank, rows, gq, gk, gv, out_dtype=torch.float32):
    qr, kr, vr = rank_inputs(g, w.cp, rank, w.partition)
    out, lse = ra.ra_forward(qr, kr, vr, g.cu_seqlens, w.cp, rank, w.partition, out_dtype=out_dtype)
    torch.cuda.synchronize()
    O, L = oracle.attention_rank(gq, gk, gv, g.cu_seqlens, w.cp, rank, w.partition, rows=rows)
    o = out[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    l = lse[:, torch.from_numpy(rows).cuda()].cpu().numpy()
    eo, el = max_abs(o, O), max_abs(l, L)
    assert np.all(np.isfinite(out.float().cpu().numpy()))
    assert eo <= TOL_O_BF16 and el <= TOL_LSE_BF16, f"rank {rank}: max-abs O {eo:.3e} LSE {el:.3e}"
    return eo, el


@pytest.fixture(scope="module")
def llama7b():
    g = synth.make_global_inputs(synth.LLAMA7B_ZIGZAG, 0)
    return g, oracle_inputs(g)


@pytest.mark.parametrize("rank", [0, 3])
def test_llama7b_zigzag_sampled(llama7b, rank):
    g, (gq, gk, gv) = llama7b
    w = synth.LLAMA7B_ZIGZAG
    rows = sample_rows(w.s_total // w.cp, extra=(4095, 4096, 127, 128, 8191), seed=rank)
    _check_sampled(g, w, rank, rows, gq, gk, gv)


def test_llama7b_zigzag_bf16_output(llama7b):
    g, (gq, gk, gv) = llama7b
    w = synth.LLAMA7B_ZIGZAG
    _check_sampled(g, w, 0, sample_rows(8192, seed=5), gq, gk, gv, out_dtype=torch.bfloat16)


def test_gqa_striped_sampled():
    w = synth.GQA_STRIPED
    g = synth.make_global_inputs(w, 0)
    gq, gk, gv = oracle_inputs(g)
    for rank in (0, 7):
        _check_sampled(g, w, rank, sample_rows(w.s_total // w.cp, seed=rank), gq, gk, gv)


def test_packed_documents_all_ranks_sampled():
    w = synth.PACKED_ZIGZAG
    g = synth.make_global_inputs(w, 0)
    gq, gk, gv = oracle_inputs(g)
    cu = g.cu_seqlens
    for rank in range(w.cp):
        pos = oracle.positions(w.partition, w.s_total, w.cp, rank)
        # rows at document starts / ends that this rank holds
        idx = np.searchsorted(pos, np.concatenate([cu[1:-1] - 1, cu[1:-1]]))
        rows = sample_rows(w.s_total // w.cp, extra=idx[:12], n_random=8, seed=rank)
        _check_sampled(g, w, rank, rows, gq, gk, gv)


def test_ulysses_path_sampled():
    """[S/N=32768, H=32, d=128] x 4 simulated ranks permuted to [131072, 8, 128],
    causal attention over 131072 tokens for rank 0's 8 heads, inverse permute."""
    n, sl, H, d = 4, 32768, 32, 128
    xq = synth.make_ulysses_inputs(n, sl, H, d, seed=0, tid=synth.TID_Q)
    xk = synth.make_ulysses_inputs(n, sl, H, d, seed=0, tid=synth.TID_K)
    xv = synth.make_ulysses_inputs(n, sl, H, d, seed=0, tid=synth.TID_V)
    yq = ra.ulysses_permute(to_device(xq, "bf16"), n)
    yk = ra.ulysses_permute(to_device(xk, "bf16"), n)
    yv = ra.ulysses_permute(to_device(xv, "bf16"), n)
    S = n * sl
    out, lse = ra.ra_forward(yq[0], yk[0:1], yv[0:1], None, 1, 0, "contiguous", out_dtype=torch.float32)
    o_all = torch.zeros((n, S, H // n, d), dtype=torch.bfloat16, device="cuda")
    ra.ra_forward(yq[0], yk[0:1], yv[0:1], None, 1, 0, "contiguous", out=o_all[0])
    back = ra.ulysses_permute(o_all, n, inverse=True)
    torch.cuda.synchronize()
    # oracle: device 0 holds every token of heads 0..7
    gq = synth.bf16_bits_to_f64(oracle.ulysses_permute(xq, n)[0])
    gk = synth.bf16_bits_to_f64(oracle.ulysses_permute(xk, n)[0])
    gv = synth.bf16_bits_to_f64(oracle.ulysses_permute(xv, n)[0])
    rows = sample_rows(S, extra=(sl - 1, sl, 2 * sl, 3 * sl - 1), n_random=16)
    O, L = oracle.attention_rank(gq, gk, gv, None, 1, 0, "contiguous", rows=rows)
    ri = torch.from_numpy(rows).cuda()
    assert max_abs(out[ri].cpu().numpy(), O) <= TOL_O_BF16
    assert max_abs(lse[:, ri].cpu().numpy(), L) <= TOL_LSE_BF16
    # the inverse permute returns device 0's heads to the sequence-split layout, bit-exactly
    exp_back = oracle.ulysses_permute(device_bits(o_all), n, inverse=True)
    assert np.array_equal(device_bits(back), exp_back)
    assert np.array_equal(device_bits(back)[:, :, : H // n], device_bits(o_all[0]).reshape(n, sl, H // n, d))
