"""Pure-Python brute-force tier for tiny inputs (oracle; test infrastructure only).

Written independently of the numpy tier: explicit loops, math.exp, and the
definitions restated directly (no shared helpers beyond the input lists).
Used only to pin the numpy tier on tiny shapes (S <= 64, d <= 16).

  position maps: [How-to] section 3 (contiguous split), [LongCtx] timeline
  (zigzag / striped, readings as in oracle.partition);
  visibility: [CP-TE] sections 3.3 / 5.2 and [XTuner-09] section 9.5;
  scores and softmax: [SP-concept] section 二 (S = Q K^T / sqrt(d_k)).
"""
from __future__ import annotations

import math


def brute_piece_bound(L, n, k, g):
    """The multiple of g nearest to k*L/n (the larger one on a tie), at most L:
    candidates compared in integers, |m*g*n - k*L|."""
    if k == n:
        return L
    best = None
    for m in range(L // g + 2):
        dist = abs(m * g * n - k * L)
        if best is None or dist <= best[0]:
            best = (dist, m)
    return min(L, best[1] * g)


def brute_positions(partition, S, cp, r, cu=None, g=256):
    """Positions of rank r in local order; None marks doc_zigzag padding."""
    out = []
    sl = S // cp
    if partition == "doc_zigzag":
        bounds = cu if cu is not None else [0, S]
        n = 2 * cp
        ranks = []
        for rr in range(cp):
            mine = []
            for j in range(len(bounds) - 1):
                L = bounds[j + 1] - bounds[j]
                pair = (rr + j) % cp
                for k in (pair, n - 1 - pair):
                    lo, hi = brute_piece_bound(L, n, k, g), brute_piece_bound(L, n, k + 1, g)
                    piece = [bounds[j] + t for t in range(lo, hi)]
                    while len(piece) % g:
                        piece.append(None)
                    mine.extend(piece)
            ranks.append(mine)
        width = max(len(x) for x in ranks)
        return ranks[r] + [None] * (width - len(ranks[r]))
    if partition == "contiguous":
        for i in range(sl):
            out.append(r * sl + i)
    elif partition == "zigzag":
        half = S // (2 * cp)
        for i in range(half):
            out.append(r * half + i)
        for i in range(half):
            out.append((2 * cp - 1 - r) * half + i)
    elif partition == "striped":
        for i in range(sl):
            out.append(r + i * cp)
    else:
        raise ValueError(partition)
    return out


def brute_doc_of(p, cu):
    if cu is None:
        return 0
    for j in range(len(cu) - 1):
        if cu[j] <= p < cu[j + 1]:
            return j
    raise ValueError("position outside cu_seqlens")


def brute_attention_rank(q, k, v, cu, cp, r, partition, causal=True, scale=None):
    """q: nested lists [S][hq][d]; k, v: [S][hkv][d]. Returns (O [R][hq][d], LSE [hq][R])."""
    S = len(q)
    hq = len(q[0])
    hkv = len(k[0])
    d = len(q[0][0])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    pos = brute_positions(partition, S, cp, r, cu)
    O = [[[0.0] * d for _ in range(hq)] for _ in pos]
    LSE = [[-math.inf] * len(pos) for _ in range(hq)]
    for i, pq in enumerate(pos):
        if pq is None:
            continue
        for h in range(hq):
            g = (h * hkv) // hq
            keys = []
            for pk in range(S):
                if causal and pk > pq:
                    continue
                if brute_doc_of(pk, cu) != brute_doc_of(pq, cu):
                    continue
                sc = 0.0
                for c in range(d):
                    sc += q[pq][h][c] * k[pk][g][c]
                keys.append((pk, sc * scale))
            if not keys:
                continue
            mx = max(sc for _, sc in keys)
            tot = 0.0
            for _, sc in keys:
                tot += math.exp(sc - mx)
            lse = mx + math.log(tot)
            LSE[h][i] = lse
            for pk, sc in keys:
                w = math.exp(sc - lse)
                for c in range(d):
                    O[i][h][c] += w * v[pk][g][c]
    return O, LSE


def brute_classify(S, cp, r, partition, cu, bm, bn, causal=True):
    """Nested list [CP][nqt][nkt] of 0/1/2 (skip/partial/full), by counting pairs."""
    pos_q = brute_positions(partition, S, cp, r, cu)
    sl = len(pos_q)
    nqt = (sl + bm - 1) // bm
    nkt = (sl + bn - 1) // bn
    out = []
    for t in range(cp):
        s = (r - t) % cp
        pos_k = brute_positions(partition, S, cp, s, cu)
        grid = []
        for I in range(nqt):
            row = []
            for J in range(nkt):
                n_vis = 0
                n_all = 0
                for i in range(I * bm, min(sl, (I + 1) * bm)):
                    for j in range(J * bn, min(sl, (J + 1) * bn)):
                        n_all += 1
                        pq, pk = pos_q[i], pos_k[j]
                        ok = (pq is not None and pk is not None and (not causal or pk <= pq)
                              and brute_doc_of(pq, cu) == brute_doc_of(pk, cu))
                        n_vis += 1 if ok else 0
                row.append(0 if n_vis == 0 else (2 if n_vis == n_all else 1))
            grid.append(row)
        out.append(grid)
    return out
