"""Shared parts of the backward parity tests: the oracle reference of one rank
(forward, gradients, and per-element rounding bounds from the oracle's P and
dS), the bound check, and the GPU call. No attention arithmetic runs on the
GPU side here; expected values and bounds come from the oracle only."""
import math

import numpy as np
import torch

import oracle
import sequence_parallelism_amd as ra
import synth
from oracle import backward as obwd
from tests.gpu_common import oracle_inputs, rank_inputs, reorder, to_device

SLACK = 1e-5


def bwd_case(S, hq, hkv, d, dtype, seed, docs=None):
    w = synth.Workload("bwd_case", S, hq, hkv, d, 1, "contiguous", 0, dtype, docs=docs, doc_lo=16,
                       doc_hi=max(17, S // 3))
    return synth.make_global_inputs(w, seed), synth.make_global_dout(w, seed)


def bf16_round(x):
    return synth.bf16_bits_to_f64(synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


class Ref:
    """Oracle forward + gradients of one rank, and per-element rounding bounds."""

    def __init__(self, g, gdo, cp, rank, part, causal=True, scale=None, rows=None):
        S = g.q.shape[0]
        self.gq, self.gk, self.gv = oracle_inputs(g)
        pos = oracle.positions(part, S, cp, rank, g.cu_seqlens)
        self.rows = np.arange(len(pos)) if rows is None else np.asarray(rows)
        self.pos = pos[self.rows]
        self.dout = synth.to_f64(gdo, g.dtype)[np.maximum(self.pos, 0)] * (self.pos >= 0)[:, None, None]
        self.cu, self.S, self.causal = g.cu_seqlens, S, causal
        d = self.gq.shape[2]
        self.scale = 1.0 / math.sqrt(d) if scale is None else scale
        qr = self.gq[np.maximum(self.pos, 0)]
        keys = np.arange(S)
        self.O, self.L = oracle.attention_rows(qr, self.pos, self.gk, self.gv, keys, self.cu, S, causal, self.scale)
        self.dq, self.dk, self.dv = oracle.attention_rows_backward(qr, self.pos, self.gk, self.gv, keys, self.dout,
                                                                   self.cu, S, causal, self.scale)
        hq, hkv = qr.shape[1], self.gk.shape[1]
        G = hq // hkv
        R = len(self.pos)
        self.A_dq = np.zeros((R, hq, d))
        self.A_dk = np.zeros((S, hkv, d))
        self.A_dv = np.zeros((S, hkv, d))
        self.PK = np.zeros((R, hq, d))   # sum_k P_ik |k_k|
        self.PV = np.zeros((R, hq, d))   # sum_k P_ik |v_k|
        self._P = []
        for h in range(hq):
            gh = h // G
            P, _, dS = obwd.softmax_grad_terms(qr, self.pos, self.gk, self.gv, keys, self.dout, self.cu, S, h,
                                               causal, self.scale)
            self.A_dq[:, h] = self.scale * (np.abs(dS) @ np.abs(self.gk[:, gh]))
            self.A_dk[:, gh] += self.scale * (np.abs(dS).T @ np.abs(qr[:, h]))
            self.A_dv[:, gh] += P.T @ np.abs(self.dout[:, h])
            self.PK[:, h] = P @ np.abs(self.gk[:, gh])
            self.PV[:, h] = P @ np.abs(self.gv[:, gh])
            self._P.append(P)

    def d_error_bounds(self, eD):
        """Extra bounds on dQ [R,hq,d] and dK [S,hkv,d] from an error |dD_i| <= eD [R,hq]."""
        hq, hkv = self.dq.shape[1], self.dk.shape[1]
        G = hq // hkv
        xq = self.scale * eD[:, :, None] * self.PK
        xk = np.zeros_like(self.dk)
        qr = self.gq[np.maximum(self.pos, 0)]
        for h in range(hq):
            xk[:, h // G] += self.scale * (self._P[h].T @ (eD[:, h, None] * np.abs(qr[:, h])))
        return xq, xk

    def chunked(self, x, part, cp):
        """Global-order [S,hkv,d] -> rank-major chunks [cp,S_l,hkv,d] (padding slots 0)."""
        out = []
        for s in range(cp):
            p = oracle.positions(part, self.S, cp, s, self.cu)
            out.append(x[np.maximum(p, 0)] * (p >= 0)[:, None, None])
        return np.stack(out)


def check_bound(name, got, ref, bound):
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite"
    err = np.abs(got - ref)
    ratio = err / bound
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert ratio.max() <= 1.0, (f"{name}: error {err[worst]:.3e} > bound {bound[worst]:.3e} at {worst} "
                                f"(ref {ref[worst]:.4e}); max-abs err {err.max():.3e}")
    return float(err.max())


def run_backward(g, gdo, cp, rank, part, O, L, causal=True, out_dtype=torch.float32, scale=0.0):
    qr, kr, vr = rank_inputs(g, cp, rank, part)
    do = reorder(to_device(gdo, g.dtype), cp, part, g.cu_seqlens)[rank].contiguous()
    if out_dtype == torch.bfloat16:
        out = to_device(synth.f32_to_bf16_bits(np.asarray(O, dtype=np.float32)), "bf16")
    else:
        out = torch.from_numpy(np.asarray(O, dtype=np.float32)).cuda()
    lse = torch.from_numpy(np.asarray(L, dtype=np.float32)).cuda()
    dq, dk, dv = ra.ra_backward(qr, kr, vr, out, lse, do, g.cu_seqlens, cp, rank, part, causal=causal,
                                softmax_scale=scale)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()


def check_rank(g, gdo, cp, rank, part, causal=True, out_dtype=torch.float32, rel=2.0 ** -8, slack=SLACK):
    ref = Ref(g, gdo, cp, rank, part, causal)
    dq, dk, dv = run_backward(g, gdo, cp, rank, part, ref.O, ref.L, causal, out_dtype)
    bq = rel * ref.A_dq + slack
    bk = rel * ref.A_dk
    bv = rel * ref.A_dv
    if out_dtype == torch.bfloat16:
        # D is computed from O rounded to bf16: |dD_i| <= sum_c |dO_ic| |O_ic - bf16(O_ic)|
        eD = np.abs(ref.dout * (ref.O - bf16_round(ref.O))).sum(axis=2)
        xq, xk = ref.d_error_bounds(eD)
        bq, bk = bq + 2 * xq, bk + 2 * xk
    # (the slack is added after chunking: padding slots keep a non-zero bound)
    e = (check_bound("dq", dq, ref.dq, bq),
         check_bound("dk", dk, ref.chunked(ref.dk, part, cp), ref.chunked(bk, part, cp) + slack),
         check_bound("dv", dv, ref.chunked(ref.dv, part, cp), ref.chunked(bv, part, cp) + slack))
    return ref, e
