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
  doc_zigzag -- per-document zigzag for packed documents. [How-to] section 2
                notes that variable lengths magnify Ring's load imbalance (and
                that ring-flash-attention adds balancing and variable-length
                handling), and [LongCtx]'s timeline names dynamic CP for it,
                without a layout. Reading: every document j (length L_j, from
                cu_seqlens) is cut into 2*CP contiguous pieces at the bounds
                b_k = min(L_j, G * round(k * L_j / (2*CP*G))), k = 0..2*CP
                (halves rounded up, b_{2CP} = L_j), G = 256 tokens: the zigzag
                cut of the document with every inner bound moved to the
                nearest multiple of G. Piece pair p of document j is piece p
                and piece 2*CP-1-p; rank r holds pair p = (r + j) mod CP,
                document after document, piece p first, each non-empty piece
                padded at its end to a multiple of G slots (only a document's
                last non-empty piece is ever short of one). Every rank's slots
                are then padded at the end to S_l, the largest rank's count.
                Padding slots have position -1: they see nothing and nothing
                sees them. Pairs are the zigzag's balanced halves; rotating
                them by document spreads the rounding and the padded last
                pieces over the ranks, and bounds on multiples of G keep
                whole query tiles of G rows inside one document.

Documents: cu_seqlens [n_docs+1] are packed-document offsets ([XTuner-09]
section 9.5): tokens of different documents must not attend to each other.

Visibility of key position pk from query position pq ([CP-TE] sections 3.3
and 5.2: the causal mask uses global positions, following the CP split):
    vis(pq, pk) = (not causal or pk <= pq) and doc(pq) == doc(pk)
"""
from __future__ import annotations

import numpy as np


DOC_GRANULE = 256  # doc_zigzag piece bounds fall on multiples of this many tokens


def doc_zigzag_piece_bounds(L: int, cp: int, g: int = DOC_GRANULE) -> np.ndarray:
    """Document-relative bounds b_0..b_{2CP} of the 2*CP pieces of a document of
    length L: k*L/(2CP) rounded to the nearest multiple of g (halves up), capped
    at L, and b_{2CP} = L."""
    n = 2 * cp
    k = np.arange(n + 1, dtype=np.int64)
    b = g * ((2 * k * L + n * g) // (2 * n * g))  # g * floor(k L / (n g) + 1/2)
    b = np.minimum(b, L)
    b[n] = L
    return b


def doc_zigzag_rank_runs(cu_seqlens, s_total: int, cp: int, rank: int, g: int = DOC_GRANULE):
    """Runs (first position, tokens, slots) of `rank` in local order, before the
    end padding: for every document, piece p = (rank + j) mod CP and then piece
    2*CP-1-p, empty pieces left out, each padded to a multiple of g slots."""
    cu = np.asarray([0, s_total] if cu_seqlens is None else cu_seqlens, dtype=np.int64)
    runs = []
    for j in range(len(cu) - 1):
        b = doc_zigzag_piece_bounds(int(cu[j + 1] - cu[j]), cp, g)
        p = (rank + j) % cp
        for piece in (p, 2 * cp - 1 - p):
            n_tok = int(b[piece + 1] - b[piece])
            if n_tok > 0:
                runs.append((int(cu[j] + b[piece]), n_tok, g * -(-n_tok // g)))
    return runs


def local_length(partition: str, s_total: int, cp: int, cu_seqlens=None) -> int:
    """Tokens each rank holds (padding included for doc_zigzag: the largest
    rank's slot count)."""
    if partition == "doc_zigzag":
        return max(sum(s for _, _, s in doc_zigzag_rank_runs(cu_seqlens, s_total, cp, r)) for r in range(cp))
    return s_total // cp


def positions(partition: str, s_total: int, cp: int, rank: int, cu_seqlens=None) -> np.ndarray:
    """Global positions held by `rank`, in its local order (int64 [S_l]; -1 marks
    doc_zigzag padding)."""
    if partition == "doc_zigzag":
        out = np.full(local_length("doc_zigzag", s_total, cp, cu_seqlens), -1, dtype=np.int64)
        at = 0
        for first, n_tok, slots in doc_zigzag_rank_runs(cu_seqlens, s_total, cp, rank):
            out[at:at + n_tok] = np.arange(first, first + n_tok)
            at += slots
        return out
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
    """Boolean [len(pos_q), len(pos_k)]: vis(pq, pk) as defined above (a padding
    position -1 on either side is never visible)."""
    start, _ = doc_bounds(cu_seqlens, s_total)
    pq = np.asarray(pos_q, dtype=np.int64)[:, None]
    pk = np.asarray(pos_k, dtype=np.int64)[None, :]
    valid = (pq >= 0) & (pk >= 0)
    same_doc = valid & (start[np.maximum(pq, 0)] == start[np.maximum(pk, 0)])
    if causal:
        return same_doc & (pk <= pq)
    return same_doc


def visible_counts(pos_q: np.ndarray, cu_seqlens, s_total: int, causal: bool) -> np.ndarray:
    """Number of visible keys (over the whole sequence) for each query position
    (0 for padding)."""
    start, end = doc_bounds(cu_seqlens, s_total)
    pq = np.asarray(pos_q, dtype=np.int64)
    p = np.maximum(pq, 0)
    n = (p - start[p] + 1) if causal else (end[p] - start[p])
    return np.where(pq >= 0, n, 0)
