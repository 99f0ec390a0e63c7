"""Hybrid Ulysses x Ring sequence parallelism ("USP") for a U x R grid of
simulated devices (oracle; test infrastructure only).

The pages describe the hybrid without fixing its layout: inside a group of
devices the Ulysses all-to-all rearranges heads, across groups a ring passes the
sequence ([CP-TE] section 2.4, Ulysses head rearrangement inside the CP group
then Ring passing the sequence, and section 6, Ulysses inside the node and Ring
across nodes; [How-to] section 6, Ulysses all-to-all inside the NVLink domain
and Ring P2P across machines; [LongCtx] timeline, USP). Reading taken:

  * the ring partition (contiguous / zigzag / striped, CP = R) splits the global
    sequence over R ring groups; ring group r's tokens, in that partition's local
    order, are cut into U equal contiguous pieces, one per device (u, r) of the
    group: device inputs X[r][u] = [S/(R U), H, d];
  * Ulysses all-to-all inside group r (oracle.layouts.ulysses_permute, the
    [SP-concept] section 三 layout): device (u, r) gets ring group r's tokens for
    heads [u H/U, (u+1) H/U) (K and V with their own head count, so under GQA
    slice u holds KV heads [u hkv/U, (u+1) hkv/U));
  * ring attention across the R devices with the same u: at step t device (u, r)
    attends to the chunk of ring rank (r - t) mod R for its head slice, the steps
    merged through their LSE (oracle.attention: attention_rows + lse_merge), with
    the mask on global positions;
  * the inverse all-to-all returns to each device its own tokens for all heads.

Every step uses the oracle's own layout and attention functions in that order.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_rows, lse_merge, ring_chunk_order
from .layouts import ulysses_permute
from .partition import positions


def usp_device_shards(x, U: int, R: int, partition: str) -> np.ndarray:
    """Device inputs [R, U, S/(R U), H, d] from a global tensor [S, H, d]."""
    x = np.asarray(x)
    S = x.shape[0]
    sl = S // R
    if S % R or sl % U:
        raise ValueError("S must split into R ring shares of U equal pieces")
    out = np.empty((R, U, sl // U) + x.shape[1:], dtype=x.dtype)
    for r in range(R):
        pos = positions(partition, S, R, r)
        for u in range(U):
            out[r, u] = x[pos[u * (sl // U):(u + 1) * (sl // U)]]
    return out


def usp_forward(gq, gk, gv, cu_seqlens, U: int, R: int, partition: str, causal=True, scale=None):
    """Outputs of every device after the inverse all-to-all: O [R, U, S/(R U), hq, d]
    and the ring LSE of every device [R, U, hq/U, S/R] (before the inverse
    all-to-all, in ring group r's local token order), fp64."""
    S, hq, d = gq.shape
    hkv = gk.shape[1]
    if hq % U or hkv % U:
        raise ValueError("U must divide both head counts")
    sl = S // R
    # 1. device shards and the Ulysses all-to-all inside every ring group
    Yq = [ulysses_permute(s, U) for s in usp_device_shards(gq, U, R, partition)]   # each [U, S/R, hq/U, d]
    Yk = [ulysses_permute(s, U) for s in usp_device_shards(gk, U, R, partition)]
    Yv = [ulysses_permute(s, U) for s in usp_device_shards(gv, U, R, partition)]
    pos = [positions(partition, S, R, r) for r in range(R)]
    O = np.zeros((R, U, sl, hq // U, d))
    L = np.full((R, U, hq // U, sl), -np.inf)
    # 2. ring attention of device (u, r) over the R chunks of head slice u
    for r in range(R):
        for u in range(U):
            o = lse = None
            for s in ring_chunk_order(R, r):
                o_t, l_t = attention_rows(Yq[r][u], pos[r], Yk[s][u], Yv[s][u], pos[s], cu_seqlens, S, causal,
                                          scale)
                o, lse = (o_t, l_t) if o is None else lse_merge(o, lse, o_t, l_t)
            O[r, u], L[r, u] = o, lse
    # 3. inverse all-to-all inside every ring group
    out = np.stack([ulysses_permute(O[r], U, inverse=True) for r in range(R)])   # [R, U, S/(R U), hq, d]
    return out, L
