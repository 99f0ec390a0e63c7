"""GPU parity of the per-document zigzag partition (RA_PART_DOC_ZIGZAG).

The reorder (cp_reorder_docs) and the tile classification are bit-exact
against the oracle; attention and its gradients are checked at the same bars
as the other partitions (max-abs 1e-2 on O and 1e-3 on LSE for bf16 inputs,
1e-4 for fp32; the backward's derived per-element bound), including padding
slots (O = 0, LSE = -inf, zero gradients) and, at the packed-document
workload's full size, sampled rows of two ranks.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
import sequence_parallelism_amd as ra
import synth
from oracle.partition import local_length, positions
from tests.bwd_common import bwd_case, check_rank
from tests.gpu_common import (TOL_LSE_BF16, TOL_LSE_F32, TOL_O_BF16, TOL_O_F32, device_bits, max_abs, o_err,
                              oracle_inputs, rank_inputs, sample_rows, to_device)

pytestmark = pytest.mark.gpu

CUS = {
    "one": None,
    "three": np.array([0, 700, 701, 2048], dtype=np.int32),
    "many": np.concatenate([[0], np.cumsum([1, 2, 3, 64, 65, 127, 128, 129, 500, 1129])]).astype(np.int32),
}


@pytest.mark.parametrize("name,cp,h,d,elem", [("one", 4, 2, 128, 2), ("three", 8, 3, 64, 2),
                                              ("many", 2, 1, 5, 4), ("many", 3, 2, 128, 2),
                                              ("three", 4, 64, 128, 2), ("many", 3, 1, 8, 2),
                                              ("one", 2, 8, 128, 4)])
def test_reorder_docs_bit_exact(name, cp, h, d, elem):
    cu = CUS[name]
    S = 2048 if cu is None else int(cu[-1])
    rng = np.random.default_rng(cp * 7 + d)
    dt = np.uint16 if elem == 2 else np.uint32
    x = rng.integers(0, np.iinfo(dt).max, size=(S, h, d), dtype=dt)
    tdt = torch.bfloat16 if elem == 2 else torch.float32
    xd = torch.from_numpy(x.view(np.int16 if elem == 2 else np.int32)).view(tdt).cuda()
    y = ra.cp_reorder_docs(xd, cp, cu)
    assert y.shape[1] == local_length("doc_zigzag", S, cp, cu) == ra.ra_local_length(S, cp, "doc_zigzag", cu)
    ref = oracle.cp_reorder(x, cp, "doc_zigzag", cu_seqlens=cu)
    assert np.array_equal(device_bits(y).view(dt), ref)
    back = ra.cp_reorder_docs(y, cp, cu, inverse=True, s_total=S)
    assert np.array_equal(device_bits(back).view(dt), x)


@pytest.mark.parametrize("name,cp,bm,bn,causal", [("three", 4, 128, 64, True), ("many", 2, 64, 64, True),
                                                  ("many", 3, 64, 128, False), ("one", 8, 32, 32, True),
                                                  ("three", 2, 16, 128, True)])
def test_classification_bit_exact(name, cp, bm, bn, causal):
    cu = CUS[name]
    S = 2048 if cu is None else int(cu[-1])
    for rank in range(cp):
        got = ra.ra_classify(S, cp, rank, "doc_zigzag", bm, bn, cu, causal=causal).cpu().numpy()
        exp = oracle.classify_tiles(S, cp, rank, "doc_zigzag", cu, bm, bn, causal)
        assert np.array_equal(got, exp), f"rank {rank}"


def _check(g, cp, rank, causal=True, out_dtype=torch.float32):
    qr, kr, vr = rank_inputs(g, cp, rank, "doc_zigzag")
    out, lse = ra.ra_forward(qr, kr, vr, g.cu_seqlens, cp, rank, "doc_zigzag", causal=causal, out_dtype=out_dtype,
                             s_total=g.q.shape[0])
    torch.cuda.synchronize()
    gq, gk, gv = oracle_inputs(g)
    O, L = oracle.attention_rank(gq, gk, gv, g.cu_seqlens, cp, rank, "doc_zigzag", causal)
    o, l = out.float().cpu().numpy(), lse.cpu().numpy()
    tol_o, tol_l = (TOL_O_BF16, TOL_LSE_BF16) if g.dtype == "bf16" else (TOL_O_F32, TOL_LSE_F32)
    eo, el = o_err(o, O, out_dtype == torch.bfloat16), max_abs(l, L)
    assert eo <= tol_o and el <= tol_l, f"rank {rank}: max-abs O {eo:.3e} LSE {el:.3e}"
    pad = positions("doc_zigzag", g.q.shape[0], cp, rank, g.cu_seqlens) < 0
    assert np.all(o[pad] == 0) and np.all(np.isneginf(l[:, pad]))


def _case(S, hq, hkv, d, dtype, seed, docs="loguniform", doc_lo=16):
    w = synth.Workload("doczz", S, hq, hkv, d, 1, "contiguous", 0, dtype, docs=docs, doc_lo=doc_lo,
                       doc_hi=max(doc_lo + 1, S // 3))
    return synth.make_global_inputs(w, seed)


@pytest.mark.parametrize("cp,causal", list(itertools.product([1, 2, 4, 8], [True, False])))
def test_forward_bf16(cp, causal):
    g = _case(3000, 4, 2, 128, "bf16", seed=cp + 20 * causal)
    for rank in sorted({0, cp // 2, cp - 1}):
        _check(g, cp, rank, causal)


@pytest.mark.parametrize("cp,d", [(4, 128), (3, 64)])
def test_plan_then_planned_call_matches_ra_forward(cp, d):
    """ra_plan + ra_forward_planned (the per-document zigzag entry point) gives
    ra_forward's outputs bit for bit, on every rank and twice from one plan."""
    g = _case(3000, 4, 2, d, "bf16", seed=40 + cp)
    S = g.q.shape[0]
    for rank in range(cp):
        qr, kr, vr = rank_inputs(g, cp, rank, "doc_zigzag")
        out, lse = ra.ra_forward(qr, kr, vr, g.cu_seqlens, cp, rank, "doc_zigzag", s_total=S)
        plan = ra.ra_plan(S, 4, 2, d, g.cu_seqlens, cp, rank, "doc_zigzag")
        assert plan.s_local == qr.shape[0]
        for _ in range(2):
            o2, l2 = ra.ra_forward_planned(qr, kr, vr, plan)
            torch.cuda.synchronize()
            assert torch.equal(o2, out) and torch.equal(l2, lse), f"rank {rank}"


def test_forward_d64_bf16_output_and_fp32():
    g = _case(1500, 2, 2, 64, "bf16", seed=31)
    for rank in range(3):
        _check(g, 3, rank, out_dtype=torch.bfloat16)
    g = _case(700, 2, 1, 64, "f32", seed=32)
    for rank in range(2):
        _check(g, 2, rank)


@pytest.mark.parametrize("cp", [2, 4])
def test_backward(cp):
    g, gdo = bwd_case(2500, 4, 2, 128, "bf16", seed=40 + cp, docs="loguniform")
    for rank in sorted({0, cp - 1}):
        check_rank(g, gdo, cp, rank, "doc_zigzag")


def test_packed_documents_full_size_sampled():
    """131072 packed tokens, log-uniform documents in [512, 32768], CP=8, per-document
    zigzag: sampled rows of ranks 0 and 7 (document starts and ends, padding, random)."""
    w = synth.PACKED_ZIGZAG
    g = synth.make_global_inputs(w, 0)
    gq, gk, gv = oracle_inputs(g)
    S = w.s_total
    for rank in (0, 7):
        qr, kr, vr = rank_inputs(g, w.cp, rank, "doc_zigzag")
        out, lse = ra.ra_forward(qr, kr, vr, g.cu_seqlens, w.cp, rank, "doc_zigzag", out_dtype=torch.float32)
        torch.cuda.synchronize()
        pos = positions("doc_zigzag", S, w.cp, rank, g.cu_seqlens)
        edges = np.flatnonzero(np.diff((pos >= 0).astype(np.int8)) != 0)
        rows = sample_rows(len(pos), extra=np.concatenate([edges, edges + 1])[:24], n_random=12, seed=rank)
        O, L = oracle.attention_rows(gq[np.maximum(pos[rows], 0)], pos[rows], gk, gv, np.arange(S), g.cu_seqlens, S,
                                     True)
        o = out[torch.from_numpy(rows).cuda()].cpu().numpy()
        l = lse[:, torch.from_numpy(rows).cuda()].cpu().numpy()
        eo, el = max_abs(o, O), max_abs(l, L)
        assert eo <= TOL_O_BF16 and el <= TOL_LSE_BF16, f"rank {rank}: max-abs O {eo:.3e} LSE {el:.3e}"
