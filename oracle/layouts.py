"""Local permutation kernels' definitions (oracle; test infrastructure only).

cp_reorder: global sequence [S, ...] <-> rank-major partitioned [CP, S/CP, ...]
  out[r, i] = in[pos_r[i]]  with pos_r from oracle.partition.positions
  (contiguous / zigzag / striped; see that module for the readings).

ulysses_permute: the Ulysses all-to-all layout change done locally for N
simulated ranks ([SP-concept] section "三、Ulysses 的 AllToAll 轉置", worked
example with N=4 devices and 4 heads; [CP-TE] section 2.3):
  sequence-split [N, S/N, H, d]  ->  head-split [N, S, H/N, d]
  out[rho, j*S_l + i, h', :] = in[j, i, rho*H/N + h', :]
Device rho receives every token (ordered by source rank j, then local index i)
of heads [rho*H/N, (rho+1)*H/N). The inverse is the transpose of that map.
H must be divisible by N ([How-to] section 5: sequence_parallel_size must
divide the head count).
"""
from __future__ import annotations

import numpy as np

from .partition import positions


def cp_reorder(x, cp: int, partition: str, inverse: bool = False, cu_seqlens=None, s_total=None):
    """Forward: x [S, ...] -> [CP, S_l, ...]. Inverse: [CP, S_l, ...] -> [S, ...].
    doc_zigzag (needs cu_seqlens; the inverse also s_total): padding rows of the
    forward output are zero, and the inverse drops them."""
    x = np.asarray(x)
    if not inverse:
        S = x.shape[0]
        rows = []
        for r in range(cp):
            pos = positions(partition, S, cp, r, cu_seqlens)
            g = x[np.maximum(pos, 0)].copy()
            g[pos < 0] = 0
            rows.append(g)
        return np.stack(rows)
    cpx, sl = x.shape[0], x.shape[1]
    if cpx != cp:
        raise ValueError("leading axis must equal CP")
    S = cp * sl if s_total is None else s_total
    out = np.empty((S,) + x.shape[2:], dtype=x.dtype)
    for r in range(cp):
        pos = positions(partition, S, cp, r, cu_seqlens)
        out[pos[pos >= 0]] = x[r][pos >= 0]
    return out


def ulysses_permute(x, n: int, inverse: bool = False):
    """Forward: [N, S/N, H, d] -> [N, S, H/N, d]. Inverse: [N, S, H/N, d] -> [N, S/N, H, d]."""
    x = np.asarray(x)
    if not inverse:
        N, sl, H, d = x.shape
        if N != n or H % n:
            raise ValueError("bad shape for ulysses_permute")
        hn = H // n
        out = np.empty((n, n * sl, hn, d), dtype=x.dtype)
        for rho in range(n):
            for j in range(n):
                out[rho, j * sl:(j + 1) * sl] = x[j, :, rho * hn:(rho + 1) * hn]
        return out
    N, S, hn, d = x.shape
    if N != n or S % n:
        raise ValueError("bad shape for inverse ulysses_permute")
    sl = S // n
    out = np.empty((n, sl, hn * n, d), dtype=x.dtype)
    for rho in range(n):
        for j in range(n):
            out[j, :, rho * hn:(rho + 1) * hn] = x[rho, j * sl:(j + 1) * sl]
    return out
