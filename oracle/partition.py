"""Partition maps, document maps and the visibility rule (oracle; test infrastructure only).

positions(): which global token positions a CP rank holds, in its local order.
  contiguous -- rank r holds [r*S/CP, (r+1)*S/CP): the plain sequence split of
                [How-to] section 1/3 (seq_len_local = full_seq_len / sp_size)
                and of [SP-concept] "Ring Attention 的不同思路" (device i holds
                Q_i K_i V_i).
  zigzag     -- named, not defined, on [LongCtx] (timeline "zigzag/stripe 重排")
                and [How-to] section 5 (load balancing for the causal mask).
                Reading: split S into 2*CP equal chunks; rank r holds chunk r
                followed by chunk 2*CP-1-r. Needs S % (2*CP) == 0.
  striped    -- [LongCtx] timeline (Striped Attention: striped reorder fixes
                the causal imbalance of Ring). Reading: rank r holds positions
                r, r+CP, r+2CP, ... in increasing order. Needs S % CP == 0.

Documents: cu_seqlens [n_docs+1] are packed-document offsets ([XTuner-09]
section 9.5): tokens of different documents must not attend to each other.

Visibility of key position pk from query position pq ([CP-TE] sections 3.3
and 5.2: the causal mask uses global positions, following the CP split):
    vis(pq, pk) = (not causal or pk <= pq) and doc(pq) == doc(pk)
"""
from __future__ import annotations

import numpy as np


def positions(partition: str, s_total: int, cp: int, rank: int) -> np.ndarray:
    """Global positions held by `rank`, in its local order (int64 [S/CP])."""
    if partition == "contiguous":
        if s_total % cp:
            raise ValueError("S must be divisible by CP")
        sl = s_total // cp
        return np.arange(rank * sl, (rank + 1) * sl, dtype=np.int64)
    if partition == "zigzag":
        if s_total % (2 * cp):
            raise ValueError("S must be divisible by 2*CP for zigzag")
        half = s_total // (2 * cp)
        first = np.arange(rank * half, (rank + 1) * half, dtype=np.int64)
        mirror = 2 * cp - 1 - rank
        second = np.arange(mirror * half, (mirror + 1) * half, dtype=np.int64)
        return np.concatenate([first, second])
    if partition == "striped":
        if s_total % cp:
            raise ValueError("S must be divisible by CP")
        return np.arange(rank, s_total, cp, dtype=np.int64)
    raise ValueError(f"unknown partition {partition!r}")


def doc_bounds(cu_seqlens, s_total: int):
    """Per position p: (start, end) of the document holding p (end exclusive).

    With no cu_seqlens the whole sequence is one document."""
    if cu_seqlens is None:
        start = np.zeros(s_total, dtype=np.int64)
        end = np.full(s_total, s_total, dtype=np.int64)
        return start, end
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    p = np.arange(s_total, dtype=np.int64)
    j = np.searchsorted(cu, p, side="right") - 1  # cu[j] <= p < cu[j+1]
    return cu[j], cu[j + 1]


def visible_matrix(pos_q: np.ndarray, pos_k: np.ndarray, cu_seqlens, s_total: int, causal: bool) -> np.ndarray:
    """Boolean [len(pos_q), len(pos_k)]: vis(pq, pk) as defined above."""
    start, _ = doc_bounds(cu_seqlens, s_total)
    pq = np.asarray(pos_q, dtype=np.int64)[:, None]
    pk = np.asarray(pos_k, dtype=np.int64)[None, :]
    same_doc = start[pq] == start[pk]
    if causal:
        return same_doc & (pk <= pq)
    return same_doc


def visible_counts(pos_q: np.ndarray, cu_seqlens, s_total: int, causal: bool) -> np.ndarray:
    """Number of visible keys (over the whole sequence) for each query position."""
    start, end = doc_bounds(cu_seqlens, s_total)
    pq = np.asarray(pos_q, dtype=np.int64)
    if causal:
        return pq - start[pq] + 1
    return end[pq] - start[pq]
