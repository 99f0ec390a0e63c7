"""Per-tile mask classification by brute force (oracle; test infrastructure only).

For rank r, ring step t (KV chunk s = (r - t) mod CP, [CP-TE] section 2.2) and
a tile I x J of the local query / key index grid (bm x bn; edge tiles hold only
the in-range indices), count visible (q, k) pairs with the visibility rule of
oracle.partition ([CP-TE] sections 3.3 and 5.2, [XTuner-09] section 9.5):
    SKIP    (0) no visible pair in the tile
    PARTIAL (1) some but not all pairs visible
    FULL    (2) every in-range pair visible
"""
from __future__ import annotations

import numpy as np

from .attention import ring_chunk_order
from .partition import local_length, positions, visible_matrix

SKIP, PARTIAL, FULL = 0, 1, 2


def classify_tiles(s_total, cp, rank, partition, cu_seqlens, bm, bn, causal=True, return_counts=False):
    """int8 [CP, ceil(S_l/bm), ceil(S_l/bn)] tile classes (and, optionally, the
    int64 visible-pair counts per tile)."""
    sl = local_length(partition, s_total, cp, cu_seqlens)
    nqt = -(-sl // bm)
    nkt = -(-sl // bn)
    pos_q = positions(partition, s_total, cp, rank, cu_seqlens)
    cls = np.zeros((cp, nqt, nkt), dtype=np.int8)
    counts = np.zeros((cp, nqt, nkt), dtype=np.int64)
    kt_starts = np.arange(0, sl, bn)
    for t, s in enumerate(ring_chunk_order(cp, rank)):
        pos_k = positions(partition, s_total, cp, s, cu_seqlens)
        for I in range(nqt):
            r0, r1 = I * bm, min(sl, (I + 1) * bm)
            vis = visible_matrix(pos_q[r0:r1], pos_k, cu_seqlens, s_total, causal)
            per_tile = np.add.reduceat(vis.sum(axis=0, dtype=np.int64), kt_starts)
            sizes = (r1 - r0) * (np.minimum(kt_starts + bn, sl) - kt_starts)
            counts[t, I] = per_tile
            cls[t, I] = np.where(per_tile == 0, SKIP, np.where(per_tile == sizes, FULL, PARTIAL))
    if return_counts:
        return cls, counts
    return cls
