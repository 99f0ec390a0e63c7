"""Pins of the oracle's attention, step partials and LSE merge (CPU only).

Each test checks the oracle against something other than itself: the
pure-Python brute force, torch's fp64 scaled_dot_product_attention, closed
forms, a hand-computed golden case, or invariants the pages fix.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from oracle.partition import positions, visible_counts

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _to_list(x):
    return x.tolist()


CASES = []
for part, cp, docs, (hq, hkv), causal in itertools.product(
        ["contiguous", "zigzag", "striped"], [1, 2, 4], [False, True], [(2, 2), (4, 2), (4, 1)], [True, False]):
    CASES.append((part, cp, docs, hq, hkv, causal))


@pytest.mark.parametrize("part,cp,docs,hq,hkv,causal", CASES)
def test_dense_matches_brute_force(part, cp, docs, hq, hkv, causal):
    S, d = 16, 4
    seed = CASES.index((part, cp, docs, hq, hkv, causal))
    q = _rand((S, hq, d), seed)
    k = _rand((S, hkv, d), seed + 1)
    v = _rand((S, hkv, d), seed + 2)
    cu = np.array([0, 5, 6, 16], dtype=np.int32) if docs else None
    for r in range(cp):
        O, L = oracle.attention_rank(q, k, v, cu, cp, r, part, causal)
        Ob, Lb = brute.brute_attention_rank(_to_list(q), _to_list(k), _to_list(v),
                                            None if cu is None else cu.tolist(), cp, r, part, causal)
        np.testing.assert_allclose(O, np.array(Ob), rtol=0, atol=1e-12)
        np.testing.assert_allclose(L, np.array(Lb), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2)])
def test_cp1_equals_torch_sdpa(causal, hq, hkv):
    """CP=1, one document: the textbook softmax(QK^T/sqrt(d) + mask) V, from
    torch's fp64 CPU scaled_dot_product_attention (GQA via enable_gqa, which
    maps query head h to KV head h // (hq/hkv))."""
    S, d = 48, 16
    q, k, v = _rand((S, hq, d), 1), _rand((S, hkv, d), 2), _rand((S, hkv, d), 3)
    O, L = oracle.attention_rank(q, k, v, None, 1, 0, "contiguous", causal)
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                           enable_gqa=(hq != hkv))
    np.testing.assert_allclose(O, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    # LSE from torch's logsumexp of the explicitly masked scores
    kk = np.repeat(k, hq // hkv, axis=1)
    s = torch.einsum("ihc,jhc->hij", torch.from_numpy(q), torch.from_numpy(kk)) / math.sqrt(d)
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(S, S, dtype=torch.bool), 1), -math.inf)
    np.testing.assert_allclose(L, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


def test_documents_equal_independent_sequences():
    """Packed documents with cu_seqlens ([XTuner-09] 9.5: no attention across
    documents) equal running causal attention on each document on its own."""
    S, hq, hkv, d = 40, 4, 2, 8
    cu = np.array([0, 7, 8, 25, 40], dtype=np.int32)
    q, k, v = _rand((S, hq, d), 4), _rand((S, hkv, d), 5), _rand((S, hkv, d), 6)
    O, L = oracle.attention_rank(q, k, v, cu, 1, 0, "contiguous", True)
    for a, b in zip(cu[:-1], cu[1:]):
        tq = torch.from_numpy(q[a:b]).permute(1, 0, 2)[None]
        tk = torch.from_numpy(k[a:b]).permute(1, 0, 2)[None]
        tv = torch.from_numpy(v[a:b]).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, enable_gqa=True)
        np.testing.assert_allclose(O[a:b], ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_one_token_per_rank_golden():
    """S = CP = 4, one token per rank, hand-computed values (tests/golden)."""
    rows = []
    with open(os.path.join(GOLDEN, "one_token_per_rank.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append(line.split())
    S = 4
    q = np.full((S, 1, 1), math.log(2.0))
    k = np.arange(S, dtype=np.float64).reshape(S, 1, 1)
    v = k.copy()
    for case, cu in (("causal", None), ("docs_0_2_4", np.array([0, 2, 4], dtype=np.int32))):
        for r in range(4):
            for part in ("contiguous", "striped"):
                O, L = oracle.attention_rank(q, k, v, cu, 4, r, part, True)
                (exp_row,) = [x for x in rows if x[0] == case and int(x[1]) == r]
                num, den, arg = map(float, exp_row[2:])
                assert abs(O[0, 0, 0] - num / den) < 1e-14
                assert abs(L[0, 0] - math.log(arg)) < 1e-14
                # the ring steps and their merge give the same value
                Om, Lm = oracle.merge_steps(oracle.step_partials(q, k, v, cu, 4, r, part, True))
                assert abs(Om[0, 0, 0] - num / den) < 1e-14
                assert abs(Lm[0, 0] - math.log(arg)) < 1e-14


def test_closed_forms():
    S, hq, hkv, d, cp = 32, 2, 1, 8, 2
    cu = np.array([0, 3, 20, 32], dtype=np.int32)
    k, v = _rand((S, hkv, d), 7), _rand((S, hkv, d), 8)
    for part in ("contiguous", "zigzag", "striped"):
        for r in range(cp):
            pos = positions(part, S, cp, r)
            # Q = 0: uniform weights over the visible keys; LSE = ln(n_vis)
            O, L = oracle.attention_rank(np.zeros((S, hq, d)), k, v, cu, cp, r, part, True)
            starts = np.array([cu[np.searchsorted(cu, p, side="right") - 1] for p in pos])
            for i, p in enumerate(pos):
                mean = v[starts[i]:p + 1, 0, :].mean(axis=0)
                np.testing.assert_allclose(O[i, 0], mean, atol=1e-13)
                assert abs(L[0, i] - math.log(p - starts[i] + 1)) < 1e-13
            # V constant: O == constant
            q = _rand((S, hq, d), 9)
            O, _ = oracle.attention_rank(q, k, np.full((S, hkv, d), 2.5), cu, cp, r, part, True)
            np.testing.assert_allclose(O, 2.5, atol=1e-13)
            # a row whose only visible key is itself: O = v_p, LSE = s_pp
            O, L = oracle.attention_rank(q, k, v, cu, cp, r, part, True)
            for i, p in enumerate(pos):
                if p in (0, 3, 20):
                    np.testing.assert_allclose(O[i, 1], v[p, 0], atol=1e-14)
                    assert abs(L[1, i] - q[p, 1] @ k[p, 0] / math.sqrt(d)) < 1e-13


@pytest.mark.parametrize("part", ["contiguous", "zigzag", "striped"])
@pytest.mark.parametrize("docs", [False, True])
def test_I1_chunk_and_merge_equals_unchunked(part, docs):
    S, hq, hkv, d, cp = 64, 4, 2, 8, 4
    cu = np.array([0, 10, 11, 40, 64], dtype=np.int32) if docs else None
    q, k, v = _rand((S, hq, d), 10), _rand((S, hkv, d), 11), _rand((S, hkv, d), 12)
    for r in range(cp):
        O, L = oracle.attention_rank(q, k, v, cu, cp, r, part, True)
        Om, Lm = oracle.merge_steps(oracle.step_partials(q, k, v, cu, cp, r, part, True))
        np.testing.assert_allclose(Om, O, atol=1e-12)
        np.testing.assert_allclose(Lm, L, atol=1e-12)


def test_I2_merge_order_does_not_matter():
    S, hq, hkv, d, cp = 64, 2, 2, 8, 4
    q, k, v = _rand((S, hq, d), 13), _rand((S, hkv, d), 14), _rand((S, hkv, d), 15)
    parts = oracle.step_partials(q, k, v, None, cp, 3, "zigzag", True)
    ref_o, ref_l = oracle.merge_steps(parts)
    for perm in itertools.permutations(range(cp)):
        o, l = oracle.merge_steps([parts[i] for i in perm])
        np.testing.assert_allclose(o, ref_o, atol=1e-13)
        np.testing.assert_allclose(l, ref_l, atol=1e-13)
    # pairwise tree
    a = oracle.lse_merge(*parts[0][1:], *parts[1][1:])
    b = oracle.lse_merge(*parts[2][1:], *parts[3][1:])
    o, l = oracle.lse_merge(*a, *b)
    np.testing.assert_allclose(o, ref_o, atol=1e-13)
    np.testing.assert_allclose(l, ref_l, atol=1e-13)


def test_I3_invisible_keys_do_not_matter():
    """Perturbing K/V at positions no row of the rank can see (future tokens,
    other documents) leaves O and LSE bit-identical."""
    S, hq, hkv, d, cp = 64, 2, 1, 8, 4
    cu = np.array([0, 30, 64], dtype=np.int32)
    q, k, v = _rand((S, hq, d), 16), _rand((S, hkv, d), 17), _rand((S, hkv, d), 18)
    for part in ("contiguous", "zigzag", "striped"):
        for r in range(cp):
            pos = positions(part, S, cp, r)
            O, L = oracle.attention_rank(q, k, v, cu, cp, r, part, True)
            # keys visible to at least one row of this rank
            vis = oracle.visible_matrix(pos, np.arange(S), cu, S, True).any(axis=0)
            k2, v2 = k.copy(), v.copy()
            k2[~vis] = 1e3 * _rand(k2[~vis].shape, 19)
            v2[~vis] = 1e3 * _rand(v2[~vis].shape, 20)
            O2, L2 = oracle.attention_rank(q, k2, v2, cu, cp, r, part, True)
            assert np.array_equal(O, O2) and np.array_equal(L, L2)


def test_I4_partition_invariance():
    S, hq, hkv, d = 64, 2, 2, 8
    cu = np.array([0, 17, 64], dtype=np.int32)
    q, k, v = _rand((S, hq, d), 21), _rand((S, hkv, d), 22), _rand((S, hkv, d), 23)
    ref_o, ref_l = oracle.attention_rank(q, k, v, cu, 1, 0, "contiguous", True)
    for part in ("contiguous", "zigzag", "striped"):
        for cp in (2, 4, 8):
            go = np.zeros_like(ref_o)
            gl = np.zeros_like(ref_l)
            for r in range(cp):
                pos = positions(part, S, cp, r)
                O, L = oracle.attention_rank(q, k, v, cu, cp, r, part, True)
                go[pos] = O
                gl[:, pos] = L
            np.testing.assert_allclose(go, ref_o, atol=1e-12)
            np.testing.assert_allclose(gl, ref_l, atol=1e-12)


def test_I5_merge_with_empty_partial_is_identity():
    o = _rand((5, 3, 4), 24)
    lse = _rand((3, 5), 25)
    zero = np.zeros_like(o)
    ninf = np.full_like(lse, -np.inf)
    for args in ((o, lse, zero, ninf), (zero, ninf, o, lse)):
        mo, ml = oracle.lse_merge(*args)
        np.testing.assert_array_equal(mo, o)
        np.testing.assert_allclose(ml, lse, atol=0, rtol=0)
    mo, ml = oracle.lse_merge(zero, ninf, zero, ninf)
    assert np.all(mo == 0) and np.all(np.isneginf(ml))


def test_merge_hand_example():
    # partial a: LSE ln 1, O 1 ; partial b: LSE ln 3, O 0 -> LSE ln 4, O 1/4
    o, l = oracle.lse_merge(np.ones((1, 1, 1)), np.zeros((1, 1)), np.zeros((1, 1, 1)),
                            np.full((1, 1), math.log(3.0)))
    assert abs(o[0, 0, 0] - 0.25) < 1e-15 and abs(l[0, 0] - math.log(4.0)) < 1e-15


def test_I6_visible_pair_totals():
    """Closed forms for the number of visible (q, k) pairs per rank (one head)."""
    for S, cp in ((32768, 4), (65536, 8), (4096, 2)):
        sl = S // cp
        for r in range(cp):
            n = int(visible_counts(positions("zigzag", S, cp, r), None, S, True).sum())
            assert n == S * S // (2 * cp) + S // (2 * cp)
            n = int(visible_counts(positions("contiguous", S, cp, r), None, S, True).sum())
            assert n == sl * (r * sl) + sl * (sl + 1) // 2
            n = int(visible_counts(positions("striped", S, cp, r), None, S, True).sum())
            assert n == sl * (r + 1) + cp * sl * (sl - 1) // 2
    # the counts quoted for the Llama-2-7B-shaped and GQA workloads
    assert int(visible_counts(positions("zigzag", 32768, 4, 0), None, 32768, True).sum()) == 134221824
    assert int(visible_counts(positions("striped", 65536, 8, 0), None, 65536, True).sum()) == 268410880
    assert int(visible_counts(positions("striped", 65536, 8, 7), None, 65536, True).sum()) == 268468224
    # counts agree with the dense visibility matrix on a small case with documents
    cu = np.array([0, 9, 30, 64], dtype=np.int32)
    for part in ("contiguous", "zigzag", "striped"):
        pos = positions(part, 64, 4, 1)
        dense = oracle.visible_matrix(pos, np.arange(64), cu, 64, True).sum(axis=1)
        np.testing.assert_array_equal(dense, visible_counts(pos, cu, 64, True))
        dense = oracle.visible_matrix(pos, np.arange(64), cu, 64, False).sum(axis=1)
        np.testing.assert_array_equal(dense, visible_counts(pos, cu, 64, False))


def test_online_softmax_reading():
    """The online-softmax update of [SP-concept] section 二 reproduces dense
    attention with the factor exp(m_old - m_new) on O; the printed inverse does not."""
    S, hq, hkv, d = 64, 2, 1, 8
    cu = np.array([0, 20, 64], dtype=np.int32)
    q, k, v = _rand((S, hq, d), 26), _rand((S, hkv, d), 27), _rand((S, hkv, d), 28)
    pos = np.arange(S)
    O, L = oracle.attention_rows(q, pos, k, v, pos, cu, S, True)
    Ob, Lb = oracle.online_softmax_blocks(q, pos, k, v, pos, cu, S, True, block=8)
    np.testing.assert_allclose(Ob, O, atol=1e-12)
    np.testing.assert_allclose(Lb, L, atol=1e-12)
    Oi, _ = oracle.online_softmax_blocks(q, pos, k, v, pos, cu, S, True, block=8, rescale_reading="inverse")
    assert np.max(np.abs(Oi - O)) > 1e-3


def test_step_partial_empty_rows():
    """A step whose chunk holds no visible key for a row yields (O=0, LSE=-inf)."""
    S, cp = 16, 4
    q, k, v = _rand((S, 1, 4), 29), _rand((S, 1, 4), 30), _rand((S, 1, 4), 31)
    parts = oracle.step_partials(q, k, v, None, cp, 0, "contiguous", True)
    # rank 0, contiguous: steps t>0 visit chunks 3,2,1 -- all in the future
    for s, O_t, L_t in parts[1:]:
        assert np.all(O_t == 0) and np.all(np.isneginf(L_t))
    assert [p[0] for p in parts] == [0, 3, 2, 1]


def test_ring_chunk_order_follows_the_send_to_next_ring():
    """[CP-TE] 2.2 and [SP-concept] (Ring Attention): at every step each rank sends
    the KV chunk it holds to the next rank and receives the previous rank's. The
    hand-simulated passing gives the chunk each rank holds at each step; the tiny
    ring simulation's rank 2 of 4 visits chunks 2, 1, 0, 3."""
    for cp in (1, 2, 3, 4, 8):
        held = list(range(cp))
        seen = [[] for _ in range(cp)]
        for _ in range(cp):
            for r in range(cp):
                seen[r].append(held[r])
            held = [held[(r - 1) % cp] for r in range(cp)]  # receive from the previous rank
        for r in range(cp):
            assert oracle.ring_chunk_order(cp, r) == seen[r]
    assert oracle.ring_chunk_order(4, 2) == [2, 1, 0, 3]
