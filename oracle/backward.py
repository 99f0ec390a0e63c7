"""Gradients of one CP rank's ring attention (oracle; test infrastructure only).

The pages train with these layers (the DeepSpeed-Ulysses vs Ring-Attention
how-to page, section 4, measures memory after the forward and after the
backward of every step; the Context Parallelism page, section 4, reports
training throughput), and the Sequence Parallelism concept page (section
"為什麼需要序列並行？") notes that activations are either kept for the backward
or recomputed. They print no backward equations, so the gradients here are the
chain rule applied to the forward's definition (oracle/attention.py):

    s_ik = scale * q_i . k_k,   P_ik = exp(s_ik - LSE_i) on visible pairs, else 0
    O_i  = sum_k P_ik v_k

For an upstream gradient dO of the rank's output rows (the loss is any function
of O; its gradient enters only through dO):

    dV_k  = sum_i P_ik dO_i
    dP_ik = dO_i . v_k
    dS_ik = P_ik * (dP_ik - sum_k' P_ik' dP_ik')       (softmax Jacobian)
    dQ_i  = scale * sum_k dS_ik k_k
    dK_k  = scale * sum_i dS_ik q_i

Under GQA the KV head g(h) = h // (hq/hkv) is shared, so dK / dV of a KV head
sum over the query heads of its group. P is the softmax over ALL keys the row
sees (the LSE of the whole ring), so one ring step's contribution is the same
sums restricted to that step's keys: dQ sums over steps, and the dK / dV of a
chunk come only from the step that visits it (reading: the pages do not
describe the ring backward; this is the plainest decomposition of the sums).

Dense fp64 numpy; the score, probability and gradient matrices are
materialised per head in row blocks. Everything is computed from q, k, v and
dO; nothing is taken from a forward result.
"""
from __future__ import annotations

import math

import numpy as np

from .partition import positions, visible_matrix
from .attention import ring_chunk_order, _row_blocks


def attention_rows_backward(q_rows, pos_q, k_rows, v_rows, pos_k, dout, cu_seqlens, s_total, causal=True,
                            scale=None):
    """Gradients of masked softmax attention of query rows against key rows.

    q_rows, dout [R, hq, d]; k_rows, v_rows [K, hkv, d]; pos_q [R], pos_k [K]
    global positions. Returns dq [R, hq, d], dk [K, hkv, d], dv [K, hkv, d]
    (fp64): the gradient of <dout, O> with O the attention of the given rows.
    Rows with no visible key contribute nothing."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k_rows = np.asarray(k_rows, dtype=np.float64)
    v_rows = np.asarray(v_rows, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    R, hq, d = q_rows.shape
    K, hkv, _ = k_rows.shape
    if hq % hkv:
        raise ValueError("hq must be a multiple of hkv")
    group = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = np.zeros((R, hq, d))
    dk = np.zeros((K, hkv, d))
    dv = np.zeros((K, hkv, d))
    if R == 0 or K == 0:
        return dq, dk, dv
    pos_q = np.asarray(pos_q, dtype=np.int64)
    pos_k = np.asarray(pos_k, dtype=np.int64)
    for r0, r1 in _row_blocks(R, K, budget=1 << 24):
        vis = visible_matrix(pos_q[r0:r1], pos_k, cu_seqlens, s_total, causal)
        any_vis = vis.any(axis=1)
        for h in range(hq):
            g = h // group
            s = np.where(vis, (q_rows[r0:r1, h, :] @ k_rows[:, g, :].T) * scale, -np.inf)
            m = np.where(any_vis, s.max(axis=1), 0.0)
            e = np.exp(s - m[:, None])
            tot = e.sum(axis=1)
            P = np.where(any_vis[:, None], e / np.where(any_vis, tot, 1.0)[:, None], 0.0)
            dO = dout[r0:r1, h, :]
            dP = dO @ v_rows[:, g, :].T
            dS = P * (dP - (P * dP).sum(axis=1)[:, None])
            dq[r0:r1, h, :] = scale * (dS @ k_rows[:, g, :])
            dk[:, g, :] += scale * (dS.T @ q_rows[r0:r1, h, :])
            dv[:, g, :] += P.T @ dO
    return dq, dk, dv


def attention_rank_backward(gq, gk, gv, dout, cu_seqlens, cp, rank, partition, causal=True, scale=None):
    """Gradients for rank `rank`'s query rows against the whole global sequence.

    gq [S, hq, d], gk / gv [S, hkv, d] in global order; dout [S_l, hq, d] in the
    rank's local row order. Returns dq [S_l, hq, d] (local order) and this
    rank's contributions dk, dv [S, hkv, d] in GLOBAL order."""
    S = gq.shape[0]
    pos_q = positions(partition, S, cp, rank, cu_seqlens)
    pos_k = np.arange(S, dtype=np.int64)
    return attention_rows_backward(gq[np.maximum(pos_q, 0)], pos_q, gk, gv, pos_k, dout, cu_seqlens, S, causal,
                                   scale)


def ring_step_gradients(gq, gk, gv, dout, cu_seqlens, cp, rank, partition, causal=True, scale=None):
    """The backward ring of one rank, step by step: a list over t = 0..CP-1 of
    (owner, dq_t [S_l,hq,d], dk_t [S_l,hkv,d], dv_t [S_l,hkv,d]), where owner =
    (rank - t) mod CP is the chunk visited at step t and dk_t / dv_t are in that
    chunk's local order. Probabilities use the row's softmax over all steps."""
    S = gq.shape[0]
    pos_q = positions(partition, S, cp, rank, cu_seqlens)
    pos_k = np.arange(S, dtype=np.int64)
    q_rows = np.asarray(gq[np.maximum(pos_q, 0)], dtype=np.float64)
    k_all = np.asarray(gk, dtype=np.float64)
    v_all = np.asarray(gv, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    R, hq, d = q_rows.shape
    hkv = k_all.shape[1]
    group = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    order = ring_chunk_order(cp, rank)
    chunk_pos = [positions(partition, S, cp, s, cu_seqlens) for s in order]
    out = [(s, np.zeros((R, hq, d)), np.zeros((len(p), hkv, d)), np.zeros((len(p), hkv, d)))
           for s, p in zip(order, chunk_pos)]
    for r0, r1 in _row_blocks(R, S, budget=1 << 24):
        vis = visible_matrix(pos_q[r0:r1], pos_k, cu_seqlens, S, causal)
        any_vis = vis.any(axis=1)
        for h in range(hq):
            g = h // group
            s = np.where(vis, (q_rows[r0:r1, h, :] @ k_all[:, g, :].T) * scale, -np.inf)
            m = np.where(any_vis, s.max(axis=1), 0.0)
            e = np.exp(s - m[:, None])
            tot = e.sum(axis=1)
            P = np.where(any_vis[:, None], e / np.where(any_vis, tot, 1.0)[:, None], 0.0)
            dO = dout[r0:r1, h, :]
            dP = dO @ v_all[:, g, :].T
            D = (P * dP).sum(axis=1)
            for (owner, dq_t, dk_t, dv_t), p in zip(out, chunk_pos):
                P_t, dS_t = P[:, p], P[:, p] * (dP[:, p] - D[:, None])
                dq_t[r0:r1, h, :] += scale * (dS_t @ k_all[p, g, :])
                dk_t[:, g, :] += scale * (dS_t.T @ q_rows[r0:r1, h, :])
                dv_t[:, g, :] += P_t.T @ dO
    return out


def softmax_grad_terms(q_rows, pos_q, k_rows, v_rows, pos_k, dout, cu_seqlens, s_total, h, causal=True, scale=None):
    """P, dP and dS of one query head h as dense [R, K] fp64 matrices (small
    inputs only), for tests that bound rounding by sums of absolute terms."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k_rows = np.asarray(k_rows, dtype=np.float64)
    v_rows = np.asarray(v_rows, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    hq, d = q_rows.shape[1], q_rows.shape[2]
    g = h // (hq // k_rows.shape[1])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    vis = visible_matrix(np.asarray(pos_q), np.asarray(pos_k), cu_seqlens, s_total, causal)
    any_vis = vis.any(axis=1)
    s = np.where(vis, (q_rows[:, h, :] @ k_rows[:, g, :].T) * scale, -np.inf)
    m = np.where(any_vis, s.max(axis=1), 0.0)
    e = np.exp(s - m[:, None])
    tot = e.sum(axis=1)
    P = np.where(any_vis[:, None], e / np.where(any_vis, tot, 1.0)[:, None], 0.0)
    dP = dout[:, h, :] @ v_rows[:, g, :].T
    dS = P * (dP - (P * dP).sum(axis=1)[:, None])
    return P, dP, dS
