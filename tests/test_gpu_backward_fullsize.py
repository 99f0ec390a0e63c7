"""GPU parity of ra_backward at the full workload sizes, on what the oracle can
compute one element at a time.

The GPU runs the training chain on the whole share, in the launch
configuration the benchmark times: ra_forward (bf16 output, as a training step
stores it) then ra_backward on that output and LSE. The oracle then computes:
  * dQ of sampled rows (a row's dQ needs only that row's scores against all keys);
  * dK / dV of sampled keys that at most 48 of the rank's rows see (the exact
    gradient of such a key is the sum over those rows), and keys that no row of
    the rank sees (exactly 0).
Bounds as in the small backward tests (2^-8 of the absolute terms), plus the
error of D = dO . O from the forward: its P is rounded to bf16 (2^-8 of
sum_k P |v|) and O is stored in bf16 (2^-9 |O|), and its LSE is within the
forward's own 1e-3 bar (a relative 1e-3 of P).
"""
import numpy as np
import pytest
import torch

import oracle
import sequence_parallelism_amd as ra
import synth
from tests.bwd_common import SLACK, Ref, check_bound
from tests.gpu_common import rank_inputs, sample_rows, to_device

pytestmark = pytest.mark.gpu

REL = 2.0 ** -8 + 1e-3


def _viewers(pos_sorted, order, cu, S, keys):
    """Local rows of the rank that see each key (causal): positions in [p, end of p's document)."""
    out = []
    for p in keys:
        end = S if cu is None else int(cu[np.searchsorted(cu, p, side="right")])
        a, b = np.searchsorted(pos_sorted, p), np.searchsorted(pos_sorted, end)
        out.append(np.sort(order[a:b]))
    return out


def _sample_keys(pos, cu, S, seed, n_few=8, n_none=4, max_view=48):
    order = np.argsort(pos)
    ps = pos[order]
    keys = np.arange(S)
    end = np.full(S, S) if cu is None else cu[np.searchsorted(cu, keys, side="right")]
    n_view = np.searchsorted(ps, end) - np.searchsorted(ps, keys)
    rng = np.random.default_rng(seed)
    few = np.flatnonzero((n_view >= 1) & (n_view <= max_view))
    none = np.flatnonzero(n_view == 0)
    pick = list(rng.choice(few, min(n_few, len(few)), replace=False)) if len(few) else []
    pick += list(rng.choice(none, min(n_none, len(none)), replace=False)) if len(none) else []
    return np.array(sorted(int(x) for x in pick)), ps, order


def _fullsize(w, rank, rows, seed, input_seed=0):
    g = synth.make_global_inputs(w, input_seed)
    gdo = synth.make_global_dout(w, input_seed)
    cp, part, S = w.cp, w.partition, w.s_total
    qr, kr, vr = rank_inputs(g, cp, rank, part)
    out, lse = ra.ra_forward(qr, kr, vr, g.cu_seqlens, cp, rank, part, out_dtype=torch.bfloat16)
    do = ra.cp_reorder(to_device(gdo, g.dtype), cp, part)[rank].contiguous()
    dq, dk, dv = ra.ra_backward(qr, kr, vr, out, lse, do, g.cu_seqlens, cp, rank, part)
    torch.cuda.synchronize()
    del qr, kr, vr, do

    def d_bounds(ref):
        eD = (np.abs(ref.dout) * (2.0 ** -8 * ref.PV + 2.0 ** -9 * np.abs(ref.O))).sum(axis=2)
        return ref.d_error_bounds(eD)

    # dQ on sampled rows
    ref = Ref(g, gdo, cp, rank, part, rows=rows)
    xq, _ = d_bounds(ref)
    check_bound("dq", dq[torch.from_numpy(rows).cuda()].cpu().numpy(), ref.dq, REL * ref.A_dq + xq + SLACK)

    # dK / dV on sampled keys
    pos = oracle.positions(part, S, cp, rank)
    keys, ps, order = _sample_keys(pos, g.cu_seqlens, S, seed)
    views = _viewers(ps, order, g.cu_seqlens, S, keys)
    owner_local = {}
    for s in range(cp):
        for j, p in enumerate(oracle.positions(part, S, cp, s)):
            owner_local[int(p)] = (s, j)
    sel = [owner_local[int(p)] for p in keys]
    got_k = np.stack([dk[s, j].cpu().numpy() for s, j in sel])
    got_v = np.stack([dv[s, j].cpu().numpy() for s, j in sel])
    seen = [p for p, v in zip(keys, views) if len(v)]
    unseen = [i for i, v in enumerate(views) if len(v) == 0]
    for i in unseen:
        assert np.all(got_k[i] == 0) and np.all(got_v[i] == 0), f"key {keys[i]} is seen by no row but dK/dV != 0"
    if seen:
        vrows = np.unique(np.concatenate([v for v in views if len(v)]))
        ref = Ref(g, gdo, cp, rank, part, rows=vrows)
        _, xk = d_bounds(ref)
        idx = [i for i, v in enumerate(views) if len(v)]
        kp = np.array(seen)
        check_bound("dk", got_k[idx], ref.dk[kp], REL * ref.A_dk[kp] + xk[kp] + SLACK)
        check_bound("dv", got_v[idx], ref.dv[kp], REL * ref.A_dv[kp] + SLACK)
    assert np.all(np.isfinite(dq.cpu().numpy())) and np.all(np.isfinite(dk.cpu().numpy()))
    assert np.all(np.isfinite(dv.cpu().numpy()))
    return len(seen), len(unseen)


@pytest.mark.parametrize("rank", [0, 3])
def test_backward_llama7b_zigzag_sampled(rank):
    w = synth.LLAMA7B_ZIGZAG
    rows = sample_rows(w.s_total // w.cp, extra=(4095, 4096, 8191), n_random=12, seed=rank)
    n_seen, _ = _fullsize(w, rank, rows, seed=rank)
    assert n_seen > 0


def test_backward_gqa_striped_sampled():
    w = synth.GQA_STRIPED
    rows = sample_rows(w.s_total // w.cp, n_random=12, seed=3)
    n_seen, _ = _fullsize(w, 0, rows, seed=3)
    assert n_seen > 0


@pytest.mark.parametrize("input_seed", [0, 1])
def test_backward_packed_documents_sampled(input_seed):
    """Two document layouts (input seeds 0 and 1) of the packed workload."""
    w = synth.PACKED_ZIGZAG
    for rank in ((0, 5) if input_seed == 0 else (7,)):
        rows = sample_rows(w.s_total // w.cp, n_random=8, seed=10 + rank)
        print(f"packed backward input seed {input_seed} rank {rank}", flush=True)
        n_seen, _ = _fullsize(w, rank, rows, seed=10 + rank, input_seed=input_seed)
        assert n_seen > 0
