"""Helpers for the GPU parity tests: move seeded inputs to the device, run one
rank's hot path through the C ABI, and fetch results. No attention arithmetic
here: expected values come from the oracle, results from the HIP library."""
from __future__ import annotations

import numpy as np
import torch

import sequence_parallelism_amd as ra
import synth

# Parity bar for bf16 inputs: max-abs error on O and on the natural-log LSE.
TOL_O_BF16 = 1e-2
TOL_LSE_BF16 = 1e-3
# fp32 inputs (fp32 VALU path; v_exp_f32 and fp32 sums): far inside the bf16 bar.
TOL_O_F32 = 1e-4
TOL_LSE_F32 = 1e-4


def to_device(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def device_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bits of a device tensor on the host (uint16 for 2-byte types)."""
    if t.element_size() == 2:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def reorder(x: torch.Tensor, cp: int, partition: str, cu_seqlens=None) -> torch.Tensor:
    """Global [S,h,d] -> rank-major [cp,S_l,h,d] with the GPU reorder kernels."""
    if partition == "doc_zigzag":
        return ra.cp_reorder_docs(x, cp, cu_seqlens)
    return ra.cp_reorder(x, cp, partition)


def rank_inputs(g: synth.GlobalInputs, cp: int, rank: int, partition: str):
    """Global Q/K/V -> (q of `rank` [S_l,hq,d], k/v [cp,S_l,hkv,d]) with the GPU reorder kernels."""
    q = to_device(g.q, g.dtype)
    k = to_device(g.k, g.dtype)
    v = to_device(g.v, g.dtype)
    qr = reorder(q, cp, partition, g.cu_seqlens)[rank].contiguous()
    kr = reorder(k, cp, partition, g.cu_seqlens)
    vr = reorder(v, cp, partition, g.cu_seqlens)
    return qr, kr, vr


def oracle_inputs(g: synth.GlobalInputs):
    return synth.to_f64(g.q, g.dtype), synth.to_f64(g.k, g.dtype), synth.to_f64(g.v, g.dtype)


def max_abs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_ninf = np.isneginf(a) & np.isneginf(b)
    d = np.abs(np.where(both_ninf, 0.0, a) - np.where(both_ninf, 0.0, b))
    return float(np.max(d)) if d.size else 0.0


def bf16_half_ulp(x):
    """Half a unit in the last place of bf16 (8 significant bits) at |x|: the most
    that one round-to-nearest store to bf16 moves a value of that magnitude."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(x)  # |x| = m 2^e with m in [0.5, 1), so the bf16 ulp is 2^(e - 8)
    return np.where(x > 0, np.ldexp(1.0, e - 9), 0.0)


def o_err(o, O, out_bf16=False):
    """Max-abs error of an attention output against the oracle. The bar applies to
    the arithmetic; a bf16 output is that result rounded once more by the store,
    so up to half a bf16 ulp of the value is taken off each element's error first.
    An unwritten (NaN) element still fails."""
    o = np.asarray(o, dtype=np.float64)
    O = np.asarray(O, dtype=np.float64)
    d = np.abs(o - O)
    if out_bf16:
        d = np.maximum(d - bf16_half_ulp(np.maximum(np.abs(o), np.abs(O))), 0.0)
    return float(np.max(d)) if d.size else 0.0


def sample_rows(s_local: int, extra=(), n_random: int = 24, seed: int = 0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    rows = {0, 1, s_local // 2 - 1, s_local // 2, s_local - 2, s_local - 1}
    rows.update(int(x) for x in extra if 0 <= x < s_local)
    rows.update(int(x) for x in rng.integers(0, s_local, n_random))
    return np.array(sorted(r for r in rows if 0 <= r < s_local), dtype=np.int64)
