"""Dense fp64 attention for one CP rank, its per-step partials and the LSE merge
(oracle; test infrastructure only).

Definition ([SP-concept] section "二、Ring Attention 的塊級線上 Softmax":
S = Q K^T / sqrt(d_k), softmax over keys, times V; the block-wise result is
mathematically equal to full attention):

    s_ik  = scale * sum_c q[i,h,c] * k[k,g(h),c]          scale = 1/sqrt(d) by default
    LSE_i = ln sum_{k visible} exp(s_ik)                   natural log of the scaled scores
    O_i   = sum_{k visible} exp(s_ik - LSE_i) * v[k,g(h)]

g(h) = h // (hq/hkv): consecutive query heads share one KV head (GQA reading,
[How-to] section 2 only says GQA has fewer KV heads). A row with no visible key
has O = 0 and LSE = -inf (reading: the pages are silent on empty rows).

The dense tier materialises the masked score matrix [rows x keys] per head
(masked entries = -inf), in row blocks to bound memory.

Ring steps ([CP-TE] section 2.2, [SP-concept] "Ring Attention 的不同思路": each
device sends its KV block to the next device and receives the previous one's):
at step t rank r holds the KV chunk of rank (r - t) mod CP.

LSE merge (follows from the online-softmax update of [SP-concept] section 二,
applied at chunk granularity; [LongCtx] "线索三": attention aggregates exactly
across blocks):
    LSE = ln(e^{LSE_a} + e^{LSE_b})
    O   = e^{LSE_a - LSE} O_a + e^{LSE_b - LSE} O_b
with -inf meaning an empty partial (weight 0).
"""
from __future__ import annotations

import math

import numpy as np

from .partition import positions, visible_matrix

NEG_INF = -np.inf


def ring_chunk_order(cp: int, rank: int) -> list:
    """KV chunk (owner rank) visited by `rank` at steps t = 0..CP-1."""
    return [(rank - t) % cp for t in range(cp)]


def _row_blocks(n_rows: int, n_keys: int, budget: int = 1 << 25):
    step = max(1, min(n_rows, budget // max(1, n_keys)))
    for r0 in range(0, n_rows, step):
        yield r0, min(n_rows, r0 + step)


def attention_rows(q_rows, pos_q, k_rows, v_rows, pos_k, cu_seqlens, s_total, causal=True, scale=None):
    """Masked softmax attention of query rows against key rows (fp64).

    q_rows [R, hq, d]; k_rows, v_rows [K, hkv, d]; pos_q [R], pos_k [K] are global
    positions. Returns O [R, hq, d] and LSE [hq, R] (natural log)."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k_rows = np.asarray(k_rows, dtype=np.float64)
    v_rows = np.asarray(v_rows, dtype=np.float64)
    R, hq, d = q_rows.shape
    K, hkv, _ = k_rows.shape
    if hq % hkv:
        raise ValueError("hq must be a multiple of hkv")
    group = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    O = np.zeros((R, hq, d), dtype=np.float64)
    LSE = np.full((hq, R), NEG_INF, dtype=np.float64)
    if R == 0 or K == 0:
        return O, LSE
    pos_q = np.asarray(pos_q, dtype=np.int64)
    pos_k = np.asarray(pos_k, dtype=np.int64)
    for r0, r1 in _row_blocks(R, K):
        vis = visible_matrix(pos_q[r0:r1], pos_k, cu_seqlens, s_total, causal)
        any_vis = vis.any(axis=1)
        for h in range(hq):
            g = h // group
            s = (q_rows[r0:r1, h, :] @ k_rows[:, g, :].T) * scale
            s = np.where(vis, s, NEG_INF)
            m = np.where(any_vis, s.max(axis=1), 0.0)
            e = np.exp(s - m[:, None])  # exp(-inf) = 0 for masked entries
            tot = e.sum(axis=1)
            with np.errstate(divide="ignore"):
                lse = np.where(any_vis, m + np.log(tot), NEG_INF)
            w = np.where(any_vis[:, None], e / np.where(any_vis, tot, 1.0)[:, None], 0.0)
            O[r0:r1, h, :] = w @ v_rows[:, g, :]
            LSE[h, r0:r1] = lse
    return O, LSE


def _rank_rows(s_total, cp, rank, partition, rows, cu_seqlens=None):
    pos_q = positions(partition, s_total, cp, rank, cu_seqlens)
    if rows is not None:
        pos_q = pos_q[np.asarray(rows, dtype=np.int64)]
    return pos_q


def attention_rank(gq, gk, gv, cu_seqlens, cp, rank, partition, causal=True, scale=None, rows=None):
    """Unchunked attention for rank `rank`'s query rows against the whole global
    sequence. gq [S, hq, d], gk/gv [S, hkv, d] in global order (fp64).
    `rows` optionally selects local row indices. Returns (O [R,hq,d], LSE [hq,R])."""
    S = gq.shape[0]
    pos_q = _rank_rows(S, cp, rank, partition, rows, cu_seqlens)
    pos_k = np.arange(S, dtype=np.int64)
    return attention_rows(gq[np.maximum(pos_q, 0)], pos_q, gk, gv, pos_k, cu_seqlens, S, causal, scale)


def step_partials(gq, gk, gv, cu_seqlens, cp, rank, partition, causal=True, scale=None, rows=None):
    """Per-step partial results of the ring: a list over t = 0..CP-1 of
    (chunk_owner, O_t [R,hq,d], LSE_t [hq,R]), attention restricted to the keys of
    the chunk visited at step t."""
    S = gq.shape[0]
    pos_q = _rank_rows(S, cp, rank, partition, rows, cu_seqlens)
    q_rows = gq[np.maximum(pos_q, 0)]
    out = []
    for s in ring_chunk_order(cp, rank):
        pos_k = positions(partition, S, cp, s, cu_seqlens)
        kk = np.maximum(pos_k, 0)
        O_t, L_t = attention_rows(q_rows, pos_q, gk[kk], gv[kk], pos_k, cu_seqlens, S, causal, scale)
        out.append((s, O_t, L_t))
    return out


def lse_merge(o_a, lse_a, o_b, lse_b):
    """Merge two normalised partials through their LSE. o [R,h,d], lse [h,R]."""
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    mx = np.maximum(lse_a, lse_b)
    empty = np.isneginf(mx)
    mx_safe = np.where(empty, 0.0, mx)
    tot = np.exp(lse_a - mx_safe) + np.exp(lse_b - mx_safe)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, NEG_INF, mx_safe + np.log(np.where(empty, 1.0, tot)))
    lse_safe = np.where(empty, 0.0, lse)
    wa = np.where(empty, 0.0, np.exp(lse_a - lse_safe))  # [h, R]
    wb = np.where(empty, 0.0, np.exp(lse_b - lse_safe))
    o = wa.T[:, :, None] * np.asarray(o_a, dtype=np.float64) + wb.T[:, :, None] * np.asarray(o_b, dtype=np.float64)
    return o, lse


def merge_steps(partials):
    """Left fold of lse_merge over [(owner, O_t, LSE_t), ...] or [(O_t, LSE_t), ...]."""
    it = [p[-2:] for p in partials]
    o, lse = it[0]
    for o_b, lse_b in it[1:]:
        o, lse = lse_merge(o, lse, o_b, lse_b)
    return o, lse


def online_softmax_blocks(q_rows, pos_q, k_rows, v_rows, pos_k, cu_seqlens, s_total, causal=True,
                          scale=None, block=16, rescale_reading="factor"):
    """Block-wise online softmax over key blocks, in the order and notation of
    [SP-concept] section 二:
        m^(i) = max(m^(i-1), rowmax(S_i));  P_i = exp(S_i - m^(i))
        l^(i) = exp(m^(i-1) - m^(i)) l^(i-1) + rowsum(P_i)
        O^(i) = F * O^(i-1) + P_i V_i;  finally O / l.
    The page prints F as diag(exp(m^(i-1) - m^(i)))^(-1). Reading taken: F is
    exp(m^(i-1) - m^(i)), the same factor as in the l update (rescale_reading=
    "factor"); "inverse" applies the printed inverse, kept only so that a test
    can show it does not reproduce attention. Returns (O, LSE)."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    R, hq, d = q_rows.shape
    K, hkv, _ = k_rows.shape
    group = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    vis_all = visible_matrix(pos_q, pos_k, cu_seqlens, s_total, causal)
    O = np.zeros((R, hq, d))
    LSE = np.full((hq, R), NEG_INF)
    for h in range(hq):
        g = h // group
        m = np.full(R, NEG_INF)
        l = np.zeros(R)
        acc = np.zeros((R, d))
        for b0 in range(0, K, block):
            b1 = min(K, b0 + block)
            S_i = (q_rows[:, h, :] @ np.asarray(k_rows[b0:b1, g, :], dtype=np.float64).T) * scale
            S_i = np.where(vis_all[:, b0:b1], S_i, NEG_INF)
            m_new = np.maximum(m, S_i.max(axis=1))
            m_safe = np.where(np.isneginf(m_new), 0.0, m_new)
            P = np.exp(S_i - m_safe[:, None])
            alpha = np.exp(m - m_safe)  # exp(-inf) = 0 when nothing was seen yet
            l = alpha * l + P.sum(axis=1)
            if rescale_reading == "factor":
                F = alpha
            elif rescale_reading == "inverse":
                with np.errstate(divide="ignore", over="ignore"):
                    F = np.where(alpha > 0, 1.0 / np.where(alpha > 0, alpha, 1.0), 0.0)
            else:
                raise ValueError(rescale_reading)
            acc = F[:, None] * acc + P @ np.asarray(v_rows[b0:b1, g, :], dtype=np.float64)
            m = m_new
        seen = l > 0
        O[:, h, :] = np.where(seen[:, None], acc / np.where(seen, l, 1.0)[:, None], 0.0)
        with np.errstate(divide="ignore"):
            LSE[h] = np.where(seen, m + np.log(np.where(seen, l, 1.0)), NEG_INF)
    return O, LSE
