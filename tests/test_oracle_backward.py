"""Pins of the oracle's attention gradients (CPU only).

The gradients are derived by the chain rule (the pages print none), so each
test checks them against something that does not share that derivation:
torch's autograd through an explicitly masked fp64 softmax, central finite
differences of the pure-Python brute-force forward, a hand-worked golden case,
closed forms, and exact identities of softmax attention.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as bwd
from oracle import brute
from oracle.partition import positions

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _autograd(gq, gk, gv, dout, cu, cp, rank, part, causal, scale=None):
    """Gradients of <dout, O> by torch autograd, the mask built from the
    brute-force position map and document lookup."""
    S, hq, d = gq.shape
    hkv = gk.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    pos = brute.brute_positions(part, S, cp, rank)
    mask = torch.zeros(len(pos), S, dtype=torch.bool)
    for i, pq in enumerate(pos):
        for pk in range(S):
            ok = (not causal or pk <= pq) and brute.brute_doc_of(pk, cu) == brute.brute_doc_of(pq, cu)
            mask[i, pk] = ok
    tq = torch.tensor(gq, requires_grad=True)
    tk = torch.tensor(gk, requires_grad=True)
    tv = torch.tensor(gv, requires_grad=True)
    rows = tq[torch.tensor(pos)]                                   # [R, hq, d]
    kk = tk.repeat_interleave(hq // hkv, dim=1)                    # [S, hq, d]
    vv = tv.repeat_interleave(hq // hkv, dim=1)
    s = torch.matmul(rows.permute(1, 0, 2), kk.permute(1, 2, 0)) * scale   # [hq, R, S]
    s = s.masked_fill(~mask[None], -math.inf)
    o = torch.matmul(torch.softmax(s, dim=-1), vv.permute(1, 0, 2))        # [hq, R, d]
    loss = (o.permute(1, 0, 2) * torch.tensor(dout)).sum()
    loss.backward()
    return tq.grad.numpy()[pos], tk.grad.numpy(), tv.grad.numpy()


CASES = list(itertools.product(["contiguous", "zigzag", "striped"], [1, 2, 4], [False, True],
                               [(2, 2), (4, 1)], [True, False]))


@pytest.mark.parametrize("part,cp,docs,heads,causal", CASES)
def test_backward_matches_torch_autograd(part, cp, docs, heads, causal):
    hq, hkv = heads
    S, d = 24, 5
    seed = CASES.index((part, cp, docs, heads, causal))
    gq, gk, gv = _rand((S, hq, d), seed), _rand((S, hkv, d), seed + 100), _rand((S, hkv, d), seed + 200)
    cu = np.array([0, 7, 8, 24], dtype=np.int32) if docs else None
    for r in range(cp):
        dout = _rand((S // cp, hq, d), seed + 300 + r)
        dq, dk, dv = oracle.attention_rank_backward(gq, gk, gv, dout, cu, cp, r, part, causal)
        tq, tk, tv = _autograd(gq, gk, gv, dout, None if cu is None else cu.tolist(), cp, r, part, causal)
        np.testing.assert_allclose(dq, tq, rtol=0, atol=1e-12)
        np.testing.assert_allclose(dk, tk, rtol=0, atol=1e-12)
        np.testing.assert_allclose(dv, tv, rtol=0, atol=1e-12)


def test_backward_matches_finite_differences_of_brute_force():
    """Central differences of <dO, O> with the pure-Python forward, every input entry."""
    S, hq, hkv, d, cp, part = 8, 2, 1, 3, 2, "zigzag"
    cu = [0, 3, 8]
    gq, gk, gv = _rand((S, hq, d), 1), _rand((S, hkv, d), 2), _rand((S, hkv, d), 3)
    for r in range(cp):
        dout = _rand((S // cp, hq, d), 4 + r)

        def loss(q, k, v):
            O, _ = brute.brute_attention_rank(q.tolist(), k.tolist(), v.tolist(), cu, cp, r, part, True)
            return float((np.array(O) * dout).sum())

        dq, dk, dv = oracle.attention_rank_backward(gq, gk, gv, dout, np.array(cu, dtype=np.int32), cp, r, part)
        pos = positions(part, S, cp, r)
        eps = 1e-5
        for name, x, grad in (("q", gq, None), ("k", gk, dk), ("v", gv, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args_p = {"q": gq, "k": gk, "v": gv}
                args_m = dict(args_p)
                args_p[name], args_m[name] = xp, xm
                num[idx] = (loss(args_p["q"], args_p["k"], args_p["v"]) -
                            loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * eps)
            if name == "q":
                np.testing.assert_allclose(dq, num[pos], rtol=0, atol=1e-8)
                other = np.setdiff1d(np.arange(S), pos)
                assert np.abs(num[other]).max() < 1e-8  # other ranks' rows do not enter this loss
            else:
                np.testing.assert_allclose(grad, num, rtol=0, atol=1e-8)


def test_backward_golden_one_token_per_rank():
    rows = []
    with open(os.path.join(GOLDEN, "backward_one_token_per_rank.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append(line.split())
    S = 4
    q = np.full((S, 1, 1), math.log(2.0))
    k = np.arange(S, dtype=np.float64).reshape(S, 1, 1)
    v = k.copy()
    dout = np.ones((1, 1, 1))
    for case, cu in (("causal", None), ("docs_0_2_4", np.array([0, 2, 4], dtype=np.int32))):
        exp = {int(x[1]): list(map(float, x[2:])) for x in rows if x[0] == case}
        for part in ("contiguous", "striped", "zigzag"):
            cp = 4 if part != "zigzag" else 2  # zigzag with S = 4 holds two tokens per rank
            dk_sum, dv_sum = np.zeros((S, 1, 1)), np.zeros((S, 1, 1))
            for r in range(cp):
                pos = positions(part, S, cp, r)
                dq, dk, dv = oracle.attention_rank_backward(q, k, v, np.ones((len(pos), 1, 1)), cu, cp, r, part)
                for i, p in enumerate(pos):
                    assert abs(dq[i, 0, 0] - exp[p][0] / exp[p][1]) < 1e-14
                dk_sum += dk
                dv_sum += dv
            for p in range(S):
                assert abs(dv_sum[p, 0, 0] - exp[p][2] / exp[p][3]) < 1e-14
                assert abs(dk_sum[p, 0, 0] - math.log(2.0) * exp[p][4] / exp[p][5]) < 1e-14
        # the ring steps of each rank give the same sums
        for r in range(4):
            steps = oracle.ring_step_gradients(q, k, v, dout, cu, 4, r, "contiguous")
            assert abs(sum(st[1][0, 0, 0] for st in steps) - exp[r][0] / exp[r][1]) < 1e-14


def test_backward_closed_forms():
    S, hq, hkv, d, cp = 32, 4, 2, 6, 2
    cu = np.array([0, 3, 20, 32], dtype=np.int32)
    gq, gk, gv = _rand((S, hq, d), 11), _rand((S, hkv, d), 12), _rand((S, hkv, d), 13)
    for part in ("contiguous", "zigzag", "striped"):
        for r in range(cp):
            pos = positions(part, S, cp, r)
            dout = _rand((len(pos), hq, d), 14 + r)
            # V rows all equal: O does not depend on the scores, so dQ = dK = 0
            vc = np.broadcast_to(_rand((1, hkv, d), 15), (S, hkv, d)).copy()
            dq, dk, dv = oracle.attention_rank_backward(gq, gk, vc, dout, cu, cp, r, part)
            assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13
            # one document per token: each row sees only itself -> dQ = dK = 0, dV = own dO (group sum)
            cu1 = np.arange(S + 1, dtype=np.int32)
            dq, dk, dv = oracle.attention_rank_backward(gq, gk, gv, dout, cu1, cp, r, part)
            assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13
            exp_dv = np.zeros((S, hkv, d))
            exp_dv[pos] = dout.reshape(len(pos), hkv, hq // hkv, d).sum(axis=2)
            np.testing.assert_allclose(dv, exp_dv, rtol=0, atol=1e-13)
            # Q = 0: uniform weights over the visible keys, so dK = 0 and
            # dV_k = sum over the rows i that see k of dO_i / n_vis(i)
            dq, dk, dv = oracle.attention_rank_backward(np.zeros_like(gq), gk, gv, dout, cu, cp, r, part)
            assert np.abs(dk).max() < 1e-13
            exp_dv = np.zeros((S, hkv, d))
            for i, p in enumerate(pos):
                start = cu[np.searchsorted(cu, p, side="right") - 1]
                grp = dout[i].reshape(hkv, hq // hkv, d).sum(axis=1)
                exp_dv[start:p + 1] += grp / (p - start + 1)
            np.testing.assert_allclose(dv, exp_dv, rtol=0, atol=1e-13)


@pytest.mark.parametrize("part", ["contiguous", "zigzag", "striped"])
def test_backward_identities(part):
    """Exact identities of softmax attention, per KV-head group:
       sum_k dK_k = 0               (each row of dS sums to zero)
       <Q, dQ> = <K, dK>            (scores are unchanged by Q -> aQ, K -> K/a)
       sum_k dV_k = sum_i dO_i      (each row of P sums to one)
       <V, dV> = sum_i <dO_i, O_i>"""
    S, hq, hkv, d, cp = 48, 4, 2, 8, 4
    cu = np.array([0, 9, 30, 48], dtype=np.int32)
    gq, gk, gv = _rand((S, hq, d), 21), _rand((S, hkv, d), 22), _rand((S, hkv, d), 23)
    grp = hq // hkv
    for r in range(cp):
        pos = positions(part, S, cp, r)
        dout = _rand((len(pos), hq, d), 24 + r)
        dq, dk, dv = oracle.attention_rank_backward(gq, gk, gv, dout, cu, cp, r, part)
        O, _ = oracle.attention_rank(gq, gk, gv, cu, cp, r, part)
        for g in range(hkv):
            hs = slice(g * grp, (g + 1) * grp)
            assert np.abs(dk[:, g].sum(axis=0)).max() < 1e-12
            assert abs((gq[pos][:, hs] * dq[:, hs]).sum() - (gk[:, g] * dk[:, g]).sum()) < 1e-12
            np.testing.assert_allclose(dv[:, g].sum(axis=0), dout[:, hs].sum(axis=(0, 1)), rtol=0, atol=1e-12)
            assert abs((gv[:, g] * dv[:, g]).sum() - (dout[:, hs] * O[:, hs]).sum()) < 1e-12


@pytest.mark.parametrize("part", ["contiguous", "zigzag", "striped"])
def test_ring_steps_partition_the_sums(part):
    """Per-step gradients: dq sums over the steps to the unchunked dq, each
    chunk's dk / dv are the unchunked ones at that chunk's positions, and the
    ranks' contributions add up to the gradient of the whole sequence (CP = 1)."""
    S, hq, hkv, d, cp = 32, 2, 1, 4, 4
    cu = np.array([0, 11, 32], dtype=np.int32)
    gq, gk, gv = _rand((S, hq, d), 31), _rand((S, hkv, d), 32), _rand((S, hkv, d), 33)
    gdout = _rand((S, hq, d), 34)
    dk_tot, dv_tot = np.zeros((S, hkv, d)), np.zeros((S, hkv, d))
    dq_glob = np.zeros((S, hq, d))
    for r in range(cp):
        pos = positions(part, S, cp, r)
        dout = gdout[pos]
        dq, dk, dv = oracle.attention_rank_backward(gq, gk, gv, dout, cu, cp, r, part)
        steps = oracle.ring_step_gradients(gq, gk, gv, dout, cu, cp, r, part)
        assert [s[0] for s in steps] == oracle.ring_chunk_order(cp, r)
        np.testing.assert_allclose(sum(s[1] for s in steps), dq, rtol=0, atol=1e-13)
        for owner, _, dk_t, dv_t in steps:
            p = positions(part, S, cp, owner)
            np.testing.assert_allclose(dk_t, dk[p], rtol=0, atol=1e-13)
            np.testing.assert_allclose(dv_t, dv[p], rtol=0, atol=1e-13)
        dk_tot += dk
        dv_tot += dv
        dq_glob[pos] = dq
    dq1, dk1, dv1 = oracle.attention_rank_backward(gq, gk, gv, gdout, cu, 1, 0, "contiguous")
    np.testing.assert_allclose(dq_glob, dq1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk_tot, dk1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv_tot, dv1, rtol=0, atol=1e-12)


def test_softmax_grad_terms():
    """P reproduces the forward O; rows of dS sum to zero; scale * dS K is dq."""
    S, hq, hkv, d = 20, 2, 1, 4
    cu = np.array([0, 6, 20], dtype=np.int32)
    gq, gk, gv = _rand((S, hq, d), 41), _rand((S, hkv, d), 42), _rand((S, hkv, d), 43)
    pos = positions("zigzag", S, 2, 1)
    dout = _rand((len(pos), hq, d), 44)
    O, _ = oracle.attention_rank(gq, gk, gv, cu, 2, 1, "zigzag")
    dq, _, _ = oracle.attention_rank_backward(gq, gk, gv, dout, cu, 2, 1, "zigzag")
    for h in range(hq):
        P, dP, dS = bwd.softmax_grad_terms(gq[pos], pos, gk, gv, np.arange(S), dout, cu, S, h)
        np.testing.assert_allclose(P @ gv[:, 0], O[:, h], rtol=0, atol=1e-13)
        assert np.abs(dS.sum(axis=1)).max() < 1e-13
        np.testing.assert_allclose(dS @ gk[:, 0] / math.sqrt(d), dq[:, h], rtol=0, atol=1e-13)
