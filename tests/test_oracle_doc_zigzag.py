"""Pins of the per-document zigzag partition (doc_zigzag) in the oracle (CPU only).

Checked against the independent pure-Python tier (positions, attention and tile
classification), against the whole-sequence result (every rank's rows put back
by position reproduce attention of the packed sequence), and against the
properties the partition is for: every real token is held exactly once, every
rank holds the same number of tokens, and causal work is balanced across ranks
where the global zigzag of packed documents is not.
"""
import itertools

import numpy as np
import pytest

import oracle
import synth
from oracle import brute
from oracle.partition import (DOC_GRANULE, doc_zigzag_piece_bounds, doc_zigzag_rank_runs, local_length,
                              positions, visible_counts)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


CUS = [None, [0, 5, 6, 40], [0, 1, 2, 3, 100], [0, 300], [0, 600, 700], [0, 1000, 1001, 2600]]


def _total(cuv):
    return 40 if cuv is None else cuv[-1]


@pytest.mark.parametrize("cu,cp", list(itertools.product(range(len(CUS)), [1, 2, 3, 4])))
def test_positions_match_brute_force_and_cover_once(cu, cp):
    cuv = CUS[cu]
    S = _total(cuv)
    cu_np = None if cuv is None else np.array(cuv, dtype=np.int32)
    seen = []
    sl = local_length("doc_zigzag", S, cp, cu_np)
    widths = []
    for r in range(cp):
        p = positions("doc_zigzag", S, cp, r, cu_np)
        b = brute.brute_positions("doc_zigzag", S, cp, r, cuv)
        assert [int(x) if x >= 0 else None for x in p] == b
        assert len(p) == sl and sl % DOC_GRANULE == 0
        seen.extend(int(x) for x in p if x >= 0)
        # every run of consecutive positions starts on a granule boundary of the local order
        starts = [i for i in range(sl) if p[i] >= 0 and (i == 0 or p[i - 1] != p[i] - 1)]
        assert all(i % DOC_GRANULE == 0 for i in starts)
        widths.append(sum(s for _, _, s in doc_zigzag_rank_runs(cu_np, S, cp, r)))
    assert sorted(seen) == list(range(S))
    assert max(widths) == sl  # no rank's slots end in a whole granule of padding by choice


@pytest.mark.parametrize("L,cp", [(1, 1), (40, 2), (300, 4), (510, 4), (4096, 8), (5000, 3), (20149, 8), (131072, 8)])
def test_piece_bounds(L, cp):
    """Inner bounds are multiples of 256 within 128 of the zigzag cut k L / 2CP
    (so pieces differ from L / 2CP by at most 256); bounds ascend from 0 to L."""
    b = doc_zigzag_piece_bounds(L, cp)
    n = 2 * cp
    assert b[0] == 0 and b[n] == L and np.all(np.diff(b) >= 0)
    for k in range(1, n):
        assert b[k] == L or b[k] % DOC_GRANULE == 0
        assert b[k] == L or abs(2 * n * b[k] - 2 * k * L) <= n * DOC_GRANULE
    if L % (n * DOC_GRANULE) == 0:  # the plain zigzag cut
        assert np.array_equal(b, np.arange(n + 1) * (L // n))


def test_one_document_is_the_zigzag_split():
    """A single document whose zigzag pieces are whole granules is held exactly as
    the global zigzag holds the sequence."""
    S, cp = 8192, 4
    for r in range(cp):
        np.testing.assert_array_equal(positions("doc_zigzag", S, cp, r, np.array([0, S])),
                                      positions("zigzag", S, cp, r))


@pytest.mark.parametrize("cp,causal", [(1, True), (2, True), (3, False), (2, False)])
def test_attention_matches_brute_force(cp, causal):
    cu = [0, 7, 8, 30, 45]
    S, hq, hkv, d = 45, 2, 1, 3
    q, k, v = _rand((S, hq, d), 1), _rand((S, hkv, d), 2), _rand((S, hkv, d), 3)
    for r in range(cp):
        O, L = oracle.attention_rank(q, k, v, np.array(cu, dtype=np.int32), cp, r, "doc_zigzag", causal)
        Ob, Lb = brute.brute_attention_rank(q.tolist(), k.tolist(), v.tolist(), cu, cp, r, "doc_zigzag", causal)
        np.testing.assert_allclose(O, np.array(Ob), rtol=0, atol=1e-12)
        np.testing.assert_allclose(L, np.array(Lb), rtol=0, atol=1e-12)
        pos = positions("doc_zigzag", S, cp, r, np.array(cu))
        assert np.all(O[pos < 0] == 0) and np.all(np.isneginf(L[:, pos < 0]))


@pytest.mark.parametrize("cu", [[0, 100, 101, 333, 512], [0, 700, 701, 1500, 2048]])
def test_ranks_reassemble_the_whole_sequence(cu):
    cu = np.array(cu, dtype=np.int32)
    S, hq, hkv, d, cp = int(cu[-1]), 4, 2, 8, 4
    q, k, v = _rand((S, hq, d), 4), _rand((S, hkv, d), 5), _rand((S, hkv, d), 6)
    O1, L1 = oracle.attention_rank(q, k, v, cu, 1, 0, "contiguous")
    Og = np.zeros_like(O1)
    for r in range(cp):
        O, L = oracle.attention_rank(q, k, v, cu, cp, r, "doc_zigzag")
        pos = positions("doc_zigzag", S, cp, r, cu)
        Og[pos[pos >= 0]] = O[pos >= 0]
        np.testing.assert_allclose(L[:, pos >= 0], L1[:, pos[pos >= 0]], rtol=0, atol=1e-12)
        # the ring steps merge to the same rows
        Om, Lm = oracle.merge_steps(oracle.step_partials(q, k, v, cu, cp, r, "doc_zigzag"))
        np.testing.assert_allclose(Om, O, rtol=0, atol=1e-12)
    np.testing.assert_allclose(Og, O1, rtol=0, atol=1e-12)


@pytest.mark.parametrize("cu,cp,bm,bn", [([0, 30, 31, 140, 200], 2, 64, 64), ([0, 30, 31, 140, 200], 3, 128, 64),
                                         ([0, 30, 31, 140, 200], 2, 64, 32), ([0, 30, 31, 140, 200], 4, 64, 128),
                                         ([0, 600, 700], 2, 128, 64), ([0, 600, 700], 2, 256, 64)])
def test_classification_matches_brute_force(cu, cp, bm, bn):
    S = cu[-1]
    for r in range(cp):
        got = oracle.classify_tiles(S, cp, r, "doc_zigzag", np.array(cu, dtype=np.int32), bm, bn)
        exp = brute.brute_classify(S, cp, r, "doc_zigzag", cu, bm, bn)
        assert got.tolist() == exp


def test_cp_reorder_round_trip_with_padding():
    cu = np.array([0, 70, 71, 200], dtype=np.int32)
    x = _rand((200, 3, 4), 7)
    y = oracle.cp_reorder(x, 2, "doc_zigzag", cu_seqlens=cu)
    assert y.shape == (2, local_length("doc_zigzag", 200, 2, cu), 3, 4)
    for r in range(2):
        pos = positions("doc_zigzag", 200, 2, r, cu)
        assert np.all(y[r][pos < 0] == 0)
        np.testing.assert_array_equal(y[r][pos >= 0], x[pos[pos >= 0]])
    back = oracle.cp_reorder(y, 2, "doc_zigzag", inverse=True, cu_seqlens=cu, s_total=200)
    np.testing.assert_array_equal(back, x)


def test_doc_zigzag_balances_packed_documents():
    """On the packed-document workload (131072 tokens, log-uniform documents, CP=8)
    the global zigzag's per-rank causal work differs several-fold; per-document
    zigzag brings every rank within a few percent of the mean. What is left comes
    from moving the piece bounds to multiples of 256 tokens."""
    w = synth.PACKED_ZIGZAG
    cu = synth.loguniform_cu_seqlens(0, w.s_total, w.doc_lo, w.doc_hi)
    glob = [visible_counts(positions("zigzag", w.s_total, w.cp, r), cu, w.s_total, True).sum() for r in range(w.cp)]
    doc = [visible_counts(positions("doc_zigzag", w.s_total, w.cp, r, cu), cu, w.s_total, True).sum()
           for r in range(w.cp)]
    assert sum(glob) == sum(doc)  # the same pairs, differently distributed
    assert max(glob) / min(glob) > 2.0
    assert max(doc) / min(doc) < 1.08 and max(doc) / np.mean(doc) < 1.03
