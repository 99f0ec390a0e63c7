"""Seeded synthetic inputs for the ring-attention workloads.

This module is shared by the CPU oracle tests, the GPU parity tests and the
benchmark. It holds only input recipes: shapes, seeded random tensors, the
bf16 rounding of those tensors and the packed-document boundaries. It holds
none of the attention arithmetic (no positions, masks, softmax or merges), so
that neither side of a parity comparison borrows code from the other.

Workload shapes follow the pages' Llama-2-7B-shaped training setup
(32 heads x head_dim 128, bf16, sequences of 32K-128K tokens; Context
Parallelism in Transformer Engine and Megatron page, section 4.1) and the
GQA / packed-document settings of the DeepSpeed-Ulysses vs Ring-Attention
how-to page (section 2) and the XTuner chapter (section 9.5, cu_seqlens).
"""
from __future__ import annotations

import concurrent.futures as _cf
import math
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# Tensor identifiers used to derive independent random streams.
TID_Q, TID_K, TID_V, TID_DOCS, TID_DOUT = 1, 2, 3, 4, 5

PARTITIONS = ("contiguous", "zigzag", "striped")


@dataclass(frozen=True)
class Workload:
    """One attention workload: global sequence, heads, partition and rank."""

    name: str
    s_total: int
    hq: int
    hkv: int
    d: int
    cp: int
    partition: str
    rank: int
    dtype: str  # "bf16" or "f32" for the Q/K/V inputs
    causal: bool = True
    docs: Optional[str] = None  # None or "loguniform"
    doc_lo: int = 512
    doc_hi: int = 32768
    prescale: float = 1.0  # multiply N(0,1) draws by this before rounding
    ulysses_n: int = 0  # >0: the Ulysses path with this many simulated ranks
    extra: dict = field(default_factory=dict)


# The five workloads. Names say what they are.
TINY_RING = Workload("tiny_ring_s512_cp4_contig_f32", 512, 1, 1, 64, 4, "contiguous", 2, "f32")
LLAMA7B_ZIGZAG = Workload("llama7b_s32k_h32_d128_cp4_zigzag", 32768, 32, 32, 128, 4, "zigzag", 0, "bf16")
ULYSSES_128K = Workload("ulysses_n4_s128k_h32to8_d128", 131072, 8, 8, 128, 1, "contiguous", 0, "bf16",
                        ulysses_n=4, extra={"h_full": 32})
GQA_STRIPED = Workload("gqa_s64k_h32kv8_d128_cp8_striped", 65536, 32, 8, 128, 8, "striped", 0, "bf16")
PACKED_ZIGZAG = Workload("packed_s128k_h32_d128_cp8_zigzag_docs", 131072, 32, 32, 128, 8, "zigzag", 0, "bf16",
                         docs="loguniform")

WORKLOADS = {w.name: w for w in (TINY_RING, LLAMA7B_ZIGZAG, ULYSSES_128K, GQA_STRIPED, PACKED_ZIGZAG)}


# ---------------------------------------------------------------------------
# bf16 encoding of inputs (round-to-nearest-even on the fp32 bit pattern)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns exactly to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns exactly to fp64."""
    return bf16_bits_to_f32(bits).astype(np.float64)


# ---------------------------------------------------------------------------
# Seeded tensors
# ---------------------------------------------------------------------------

_ROWS_PER_BLOCK = 1024


def _block_normals(seed: int, tid: int, block: int, n: int) -> np.ndarray:
    rng = np.random.default_rng(np.random.SeedSequence([seed, tid, block]))
    return rng.standard_normal(n, dtype=np.float32)


def normal_f32(seed: int, tid: int, shape: tuple, prescale: float = 1.0) -> np.ndarray:
    """N(0,1) fp32 tensor; rows (first axis) are drawn in independent blocks so
    that generation can run on several threads and is reproducible."""
    shape = tuple(int(s) for s in shape)
    rows = shape[0]
    row_elems = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    out = np.empty((rows, row_elems), dtype=np.float32)
    nblocks = (rows + _ROWS_PER_BLOCK - 1) // _ROWS_PER_BLOCK

    def work(b):
        r0 = b * _ROWS_PER_BLOCK
        r1 = min(rows, r0 + _ROWS_PER_BLOCK)
        blk = _block_normals(seed, tid, b, (r1 - r0) * row_elems).reshape(r1 - r0, row_elems)
        if prescale != 1.0:
            blk *= np.float32(prescale)
        out[r0:r1] = blk

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    if nblocks > 1 and workers > 1:
        with _cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(work, range(nblocks)))
    else:
        for b in range(nblocks):
            work(b)
    return out.reshape(shape)


def normal_bf16_bits(seed: int, tid: int, shape: tuple, prescale: float = 1.0) -> np.ndarray:
    """N(0,1) draws (times `prescale`) rounded to bf16; returns uint16 bit patterns."""
    x = normal_f32(seed, tid, shape, prescale)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    step = 1 << 24
    for i in range(0, flat.size, step):
        out[i:i + step] = f32_to_bf16_bits(flat[i:i + step])
    return out.reshape(x.shape)


def loguniform_cu_seqlens(seed: int, total: int, lo: int, hi: int) -> np.ndarray:
    """Packed-document boundaries: document lengths round(exp(U(ln lo, ln hi)))
    appended until the total is reached; the last document is truncated so the
    lengths sum to exactly `total`. Returns int32 [n_docs + 1], starting at 0."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, TID_DOCS]))
    lens = []
    acc = 0
    while acc < total:
        L = int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))
        L = max(1, min(L, total - acc))
        lens.append(L)
        acc += L
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


@dataclass
class GlobalInputs:
    """Global (unpartitioned) Q/K/V in sequence order, plus document bounds.

    For bf16 workloads `q`, `k`, `v` hold uint16 bit patterns; for f32
    workloads they hold float32 values. Shapes: q [S, hq, d], k/v [S, hkv, d].
    """

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    cu_seqlens: Optional[np.ndarray]
    dtype: str


def make_global_inputs(w: Workload, seed: int = 0, s_total: Optional[int] = None,
                       prescale: Optional[float] = None) -> GlobalInputs:
    """Seeded global Q/K/V for workload `w` (optionally at a reduced length)."""
    S = int(s_total or w.s_total)
    ps = w.prescale if prescale is None else prescale
    if w.dtype == "bf16":
        q = normal_bf16_bits(seed, TID_Q, (S, w.hq, w.d), ps)
        k = normal_bf16_bits(seed, TID_K, (S, w.hkv, w.d), ps)
        v = normal_bf16_bits(seed, TID_V, (S, w.hkv, w.d), ps)
    else:
        q = normal_f32(seed, TID_Q, (S, w.hq, w.d), ps)
        k = normal_f32(seed, TID_K, (S, w.hkv, w.d), ps)
        v = normal_f32(seed, TID_V, (S, w.hkv, w.d), ps)
    cu = loguniform_cu_seqlens(seed, S, w.doc_lo, w.doc_hi) if w.docs == "loguniform" else None
    return GlobalInputs(q, k, v, cu, w.dtype)


def make_global_dout(w: Workload, seed: int = 0, s_total: Optional[int] = None) -> np.ndarray:
    """Seeded upstream gradient dO [S, hq, d] in global order, N(0,1) (bf16 bits
    for bf16 workloads, fp32 values otherwise)."""
    S = int(s_total or w.s_total)
    if w.dtype == "bf16":
        return normal_bf16_bits(seed, TID_DOUT, (S, w.hq, w.d))
    return normal_f32(seed, TID_DOUT, (S, w.hq, w.d))


def make_ulysses_inputs(n: int, s_local: int, h: int, d: int, seed: int = 0, tid: int = TID_Q) -> np.ndarray:
    """Seeded bf16 bits of shape [n, s_local, h, d]: n simulated ranks' sequence shards."""
    return normal_bf16_bits(seed, tid, (n * s_local, h, d)).reshape(n, s_local, h, d)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 view of a generated tensor (bf16 bits or fp32 values)."""
    return bf16_bits_to_f64(x) if dtype == "bf16" else np.asarray(x, dtype=np.float64)
