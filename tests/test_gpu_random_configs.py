"""GPU parity over seeded random configurations: the forward (and, for a subset,
the backward) of every partition at shapes the fixed cases do not reach.

Each configuration is drawn from a fixed generator: head_dim 64 or 128, 1-3 KV
heads with GQA ratio 1, 2 or 4, CP from 1 to 8 (odd sizes included), any
partition including per-document zigzag, packed documents or one sequence,
causal or document-only masks, a default or explicit softmax scale, fp32 or
bf16 output, and a few fp32-input cases. Local lengths are random, so tiles are
ragged. A second set of edge draws takes local lengths from a single row, CP up
to the 64-rank maximum (odd and prime sizes among them) and up to 64 query heads.
Ranks 0 and CP-1 are checked on every row against the fp64 oracle at the usual
bars (max-abs 1e-2 on O, after a bf16 output's store rounding, and 1e-3 on LSE for
bf16 inputs; 1e-4 for fp32 inputs; the backward's derived per-element bound).
Random Ulysses x Ring grids go through usp_forward against oracle.usp_forward, and
the per-step partials of ra_forward_steps, folded with ra_lse_merge, against the
oracle's step partials and whole-ring rows.
"""
import numpy as np
import pytest
import torch

import oracle
import sequence_parallelism_amd as ra
import synth
from oracle.partition import positions
from tests.bwd_common import check_rank as check_backward_rank
from tests.gpu_common import (TOL_LSE_BF16, TOL_LSE_F32, TOL_O_BF16, TOL_O_F32, max_abs, o_err, oracle_inputs,
                              rank_inputs, to_device)

pytestmark = pytest.mark.gpu

PARTS = ("contiguous", "zigzag", "striped", "doc_zigzag")


def _draw(i):
    rng = np.random.default_rng(20261204 + i)
    d = int(rng.choice([64, 128]))
    hkv = int(rng.integers(1, 4))
    hq = hkv * int(rng.choice([1, 2, 4]))
    cp = int(rng.choice([1, 2, 3, 4, 5, 8]))
    part = PARTS[int(rng.integers(0, 4))]
    unit = 2 * cp if part == "zigzag" else cp
    s_l = int(rng.integers(24, 420)) if rng.random() < 0.8 else int(rng.integers(420, 1100))
    S = max(unit, (s_l * cp // unit) * unit)
    docs = part == "doc_zigzag" or rng.random() < 0.5
    causal = bool(rng.random() < 0.75)
    scale = float(rng.uniform(0.04, 0.2)) if rng.random() < 0.3 else 0.0
    out_bf16 = bool(rng.random() < 0.3)
    dtype = "f32" if rng.random() < 0.15 else "bf16"
    return dict(d=d, hq=hq, hkv=hkv, cp=cp, part=part, S=S, docs=docs, causal=causal, scale=scale,
                out_bf16=out_bf16 and dtype == "bf16", dtype=dtype, seed=1000 + i)


def _draw_edge(i):
    """Edge draws: local lengths from 1 row, CP up to the 64-rank maximum (odd and
    prime sizes included), up to 64 query heads."""
    rng = np.random.default_rng(777000 + i)
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2, 3, 8, 16]))
    hq = min(hkv * int(rng.choice([1, 2, 4, 8])), 64)
    hkv = hq // max(1, hq // hkv)
    cp = int(rng.choice([1, 2, 6, 7, 12, 16, 31, 32, 64]))
    part = PARTS[int(rng.integers(0, 4))]
    unit = 2 * cp if part == "zigzag" else cp
    s_l = int(rng.integers(1, 40)) if rng.random() < 0.6 else int(rng.integers(40, 300))
    S = min(max(unit, (s_l * cp // unit) * unit), max(unit, (6000 // unit) * unit))
    docs = part == "doc_zigzag" or rng.random() < 0.5
    causal = bool(rng.random() < 0.75)
    scale = float(rng.uniform(0.04, 0.2)) if rng.random() < 0.3 else 0.0
    out_bf16 = bool(rng.random() < 0.3)
    dtype = "f32" if rng.random() < 0.1 else "bf16"
    return dict(d=d, hq=hq, hkv=hkv, cp=cp, part=part, S=S, docs=docs, causal=causal, scale=scale,
                out_bf16=out_bf16 and dtype == "bf16", dtype=dtype, seed=5000 + i)


CONFIGS = [_draw(i) for i in range(64)] + [_draw_edge(i) for i in range(48)]


def _inputs(c):
    w = synth.Workload("random", c["S"], c["hq"], c["hkv"], c["d"], 1, "contiguous", 0, c["dtype"],
                       docs="loguniform" if c["docs"] else None, doc_lo=8, doc_hi=max(9, c["S"] // 2))
    return synth.make_global_inputs(w, c["seed"])


def _label(c):
    return (f"{c['part']}-cp{c['cp']}-S{c['S']}-h{c['hq']}x{c['hkv']}-d{c['d']}-{c['dtype']}"
            f"{'-docs' if c['docs'] else ''}{'' if c['causal'] else '-noncausal'}"
            f"{'-scaled' if c['scale'] else ''}{'-bf16out' if c['out_bf16'] else ''}")


@pytest.mark.parametrize("c", CONFIGS, ids=_label)
def test_forward_random_config(c):
    g = _inputs(c)
    cp, part = c["cp"], c["part"]
    out_dtype = torch.bfloat16 if c["out_bf16"] else torch.float32
    tol_o, tol_l = (TOL_O_BF16, TOL_LSE_BF16) if c["dtype"] == "bf16" else (TOL_O_F32, TOL_LSE_F32)
    gq, gk, gv = oracle_inputs(g)
    for rank in sorted({0, cp - 1}):
        print(f"[random-config] {_label(c)} rank {rank}", flush=True)
        qr, kr, vr = rank_inputs(g, cp, rank, part)
        out, lse = ra.ra_forward(qr, kr, vr, g.cu_seqlens, cp, rank, part, causal=c["causal"], out_dtype=out_dtype,
                                 softmax_scale=c["scale"], s_total=c["S"] if part == "doc_zigzag" else None)
        torch.cuda.synchronize()
        O, L = oracle.attention_rank(gq, gk, gv, g.cu_seqlens, cp, rank, part, c["causal"], scale=c["scale"] or None)
        o, l = out.float().cpu().numpy(), lse.cpu().numpy()
        assert o.shape == O.shape and l.shape == L.shape
        eo, el = o_err(o, O, c["out_bf16"]), max_abs(l, L)
        assert eo <= tol_o and el <= tol_l, f"rank {rank}: max-abs O {eo:.3e} LSE {el:.3e}"
        if part == "doc_zigzag":
            pad = positions("doc_zigzag", c["S"], cp, rank, g.cu_seqlens) < 0
            assert np.all(o[pad] == 0) and np.all(np.isneginf(l[:, pad]))
        else:
            assert np.all(np.isfinite(o)) and not np.any(np.isnan(l))


BWD_CONFIGS = [c for c in CONFIGS[:64] if not c["scale"]][:20] + [c for c in CONFIGS[64:] if not c["scale"]][:16]


@pytest.mark.parametrize("c", BWD_CONFIGS, ids=_label)
def test_backward_random_config(c):
    w = synth.Workload("random", c["S"], c["hq"], c["hkv"], c["d"], 1, "contiguous", 0, c["dtype"],
                       docs="loguniform" if c["docs"] else None, doc_lo=8, doc_hi=max(9, c["S"] // 2))
    g, gdo = synth.make_global_inputs(w, c["seed"]), synth.make_global_dout(w, c["seed"])
    out_dtype = torch.bfloat16 if c["out_bf16"] else torch.float32
    kw = {} if c["dtype"] == "bf16" else {"rel": 2.0 ** -12, "slack": 1e-4}
    for rank in sorted({0, c["cp"] - 1}):
        print(f"[random-config backward] {_label(c)} rank {rank}", flush=True)
        check_backward_rank(g, gdo, c["cp"], rank, c["part"], causal=c["causal"], out_dtype=out_dtype, **kw)


def _draw_usp(i):
    rng = np.random.default_rng(884000 + i)
    U, R = int(rng.choice([1, 2, 3, 4, 8])), int(rng.choice([1, 2, 3, 4]))
    part = ("contiguous", "zigzag", "striped")[int(rng.integers(0, 3))]
    hkv = U * int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    unit = R * U * (2 if part == "zigzag" else 1)
    S = unit * int(rng.integers(1, max(2, 2400 // unit)))
    return dict(U=U, R=R, part=part, hq=hq, hkv=hkv, d=int(rng.choice([64, 128])), S=S,
                docs=bool(rng.random() < 0.5), dtype="f32" if rng.random() < 0.15 else "bf16",
                out_bf16=bool(rng.random() < 0.3), seed=6000 + i)


USP_CONFIGS = [_draw_usp(i) for i in range(24)]


def _usp_label(c):
    return (f"{c['part']}-u{c['U']}-r{c['R']}-S{c['S']}-h{c['hq']}x{c['hkv']}-d{c['d']}-{c['dtype']}"
            f"{'-docs' if c['docs'] else ''}{'-bf16out' if c['out_bf16'] and c['dtype'] == 'bf16' else ''}")


@pytest.mark.parametrize("c", USP_CONFIGS, ids=_usp_label)
def test_usp_random_config(c):
    """The Ulysses x Ring grid: every device's output and LSE against oracle.usp_forward."""
    w = synth.Workload("random_usp", c["S"], c["hq"], c["hkv"], c["d"], 1, "contiguous", 0, c["dtype"],
                       docs="loguniform" if c["docs"] else None, doc_lo=8, doc_hi=max(9, c["S"] // 2))
    g = synth.make_global_inputs(w, c["seed"])
    U, R, part, S = c["U"], c["R"], c["part"], c["S"]
    out_bf16 = c["out_bf16"] and c["dtype"] == "bf16"
    print(f"[random-config usp] {_usp_label(c)}", flush=True)
    q, k, v = (ra.cp_reorder(to_device(x, g.dtype), R, part).view(R, U, S // (R * U), x.shape[1], x.shape[2])
               for x in (g.q, g.k, g.v))
    out, lse = ra.usp_forward(q, k, v, g.cu_seqlens, U, R, part,
                              out_dtype=torch.bfloat16 if out_bf16 else torch.float32)
    torch.cuda.synchronize()
    gq, gk, gv = oracle_inputs(g)
    O, L = oracle.usp_forward(gq, gk, gv, g.cu_seqlens, U, R, part)
    tol_o, tol_l = (TOL_O_BF16, TOL_LSE_BF16) if c["dtype"] == "bf16" else (TOL_O_F32, TOL_LSE_F32)
    eo = o_err(out.float().cpu().numpy(), O, out_bf16)
    el = max_abs(np.transpose(lse.cpu().numpy(), (1, 0, 2, 3)), L)
    assert eo <= tol_o and el <= tol_l, f"max-abs O {eo:.3e} LSE {el:.3e}"


STEPS_CONFIGS = [c for c in CONFIGS if c["cp"] > 1][:24]


@pytest.mark.parametrize("c", STEPS_CONFIGS, ids=_label)
def test_steps_and_merge_random_config(c):
    """Per-step partials against the oracle's, and their LSE-merge fold against the
    oracle's whole-ring rows."""
    g = _inputs(c)
    cp, part = c["cp"], c["part"]
    rank = cp - 1
    tol_o, tol_l = (TOL_O_BF16, TOL_LSE_BF16) if c["dtype"] == "bf16" else (TOL_O_F32, TOL_LSE_F32)
    print(f"[random-config steps] {_label(c)} rank {rank}", flush=True)
    qr, kr, vr = rank_inputs(g, cp, rank, part)
    o_steps, lse_steps = ra.ra_forward_steps(qr, kr, vr, g.cu_seqlens, cp, rank, part, causal=c["causal"],
                                             softmax_scale=c["scale"],
                                             s_total=c["S"] if part == "doc_zigzag" else None)
    torch.cuda.synchronize()
    gq, gk, gv = oracle_inputs(g)
    for t, (_, O_t, L_t) in enumerate(oracle.step_partials(gq, gk, gv, g.cu_seqlens, cp, rank, part, c["causal"],
                                                           scale=c["scale"] or None)):
        eo, el = max_abs(o_steps[t].cpu().numpy(), O_t), max_abs(lse_steps[t].cpu().numpy(), L_t)
        assert eo <= tol_o and el <= tol_l, f"step {t}: max-abs O {eo:.3e} LSE {el:.3e}"
    o, l = o_steps[0].clone(), lse_steps[0].clone()
    for t in range(1, cp):
        o, l = ra.ra_lse_merge(o, l, o_steps[t], lse_steps[t], o_out=o, lse_out=l)
    O, L = oracle.attention_rank(gq, gk, gv, g.cu_seqlens, cp, rank, part, c["causal"], scale=c["scale"] or None)
    eo, el = max_abs(o.cpu().numpy(), O), max_abs(l.cpu().numpy(), L)
    assert eo <= tol_o and el <= tol_l, f"merged: max-abs O {eo:.3e} LSE {el:.3e}"
