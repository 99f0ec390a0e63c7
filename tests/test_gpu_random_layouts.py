"""GPU bit-exactness of the layout kernels over seeded random shapes.

Each draw comes from a fixed generator: CP from 1 to 64, local lengths from one
row, head counts and row sizes that are not powers of two, elements of 1, 2, 4 or
8 bytes (so rows of any byte length and alignment), and, for the per-document
zigzag, document lengths from a single token up. The reorders and the Ulysses
permute must equal the oracle's permutation bit for bit and invert exactly; the
tile classification must equal the oracle's brute-force count for every tile
(any tile size, and 16 to 128 slots under the per-document zigzag, which is what
the library accepts there).
"""
import numpy as np
import pytest
import torch

import oracle
import sequence_parallelism_amd as ra
from oracle.partition import local_length

pytestmark = pytest.mark.gpu

NP_OF = {1: np.uint8, 2: np.int16, 4: np.int32, 8: np.int64}
CPS = [1, 2, 3, 5, 7, 8, 12, 16, 31, 64]


def _bits(rng, shape, eb):
    raw = rng.integers(0, 256, size=tuple(shape) + (eb,), dtype=np.uint8)
    return np.ascontiguousarray(raw).view(NP_OF[eb]).reshape(shape)


def _host(t):
    return t.cpu().numpy()


def _docs(rng, S):
    """Random document boundaries: many single-token documents, some long ones."""
    cuts, at = [0], 0
    while at < S:
        n = int(rng.integers(1, 4)) if rng.random() < 0.4 else int(rng.integers(4, max(5, S // 2)))
        at = min(S, at + n)
        cuts.append(at)
    return np.array(cuts, dtype=np.int32)


def _reorder_case(i):
    rng = np.random.default_rng(880000 + i)
    part = ("contiguous", "zigzag", "striped")[i % 3]
    cp = int(rng.choice(CPS))
    unit = 2 * cp if part == "zigzag" else cp
    S = unit * int(rng.integers(1, 40))
    return rng, part, cp, S, int(rng.integers(1, 9)), int(rng.integers(1, 131)), int(rng.choice([1, 2, 4, 8]))


@pytest.mark.parametrize("i", range(36))
def test_cp_reorder_random_shapes(i):
    rng, part, cp, S, h, d, eb = _reorder_case(i)
    print(f"[cp_reorder] {part} cp {cp} S {S} h {h} d {d} elem {eb}", flush=True)
    x = _bits(rng, (S, h, d), eb)
    xt = torch.from_numpy(x).cuda()
    y = ra.cp_reorder(xt, cp, part)
    assert np.array_equal(_host(y), oracle.cp_reorder(x, cp, part))
    assert np.array_equal(_host(ra.cp_reorder(y, cp, part, inverse=True)), x)


@pytest.mark.parametrize("i", range(30))
def test_ulysses_permute_random_shapes(i):
    rng = np.random.default_rng(881000 + i)
    n = int(rng.choice([1, 2, 3, 4, 5, 8]))
    sl, h, d = int(rng.integers(1, 60)), n * int(rng.integers(1, 9)), int(rng.integers(1, 131))
    eb = int(rng.choice([1, 2, 4, 8]))
    print(f"[ulysses] n {n} s_l {sl} h {h} d {d} elem {eb}", flush=True)
    x = _bits(rng, (n, sl, h, d), eb)
    xt = torch.from_numpy(x).cuda()
    y = ra.ulysses_permute(xt, n)
    assert np.array_equal(_host(y), oracle.ulysses_permute(x, n))
    assert np.array_equal(_host(ra.ulysses_permute(y, n, inverse=True)), x)


@pytest.mark.parametrize("i", range(30))
def test_cp_reorder_docs_random_documents(i):
    rng = np.random.default_rng(882000 + i)
    cp = int(rng.choice([1, 2, 3, 4, 7, 8, 16]))
    S = int(rng.integers(1, 5000))
    cu = _docs(rng, S) if rng.random() < 0.8 else None
    h, d, eb = int(rng.integers(1, 5)), int(rng.integers(1, 131)), int(rng.choice([1, 2, 4, 8]))
    print(f"[cp_reorder_docs] cp {cp} S {S} docs {0 if cu is None else len(cu) - 1} h {h} d {d} elem {eb}",
          flush=True)
    sl = local_length("doc_zigzag", S, cp, cu)
    assert ra.ra_local_length(S, cp, "doc_zigzag", cu) == sl
    x = _bits(rng, (S, h, d), eb)
    xt = torch.from_numpy(x).cuda()
    y = ra.cp_reorder_docs(xt, cp, cu)
    assert tuple(y.shape) == (cp, sl, h, d)
    assert np.array_equal(_host(y), oracle.cp_reorder(x, cp, "doc_zigzag", cu_seqlens=cu))
    assert np.array_equal(_host(ra.cp_reorder_docs(y, cp, cu, inverse=True, s_total=S)), x)


@pytest.mark.parametrize("i", range(30))
def test_classify_random_tiles(i):
    rng = np.random.default_rng(883000 + i)
    part = ("contiguous", "zigzag", "striped", "doc_zigzag")[i % 4]
    cp = int(rng.choice([1, 2, 3, 4, 8, 16, 64]))
    unit = 2 * cp if part == "zigzag" else cp
    S = unit * int(rng.integers(1, max(2, 1200 // unit)))
    cu = _docs(rng, S) if (part == "doc_zigzag" or rng.random() < 0.5) else None
    causal = bool(rng.random() < 0.75)
    if part == "doc_zigzag":  # tiles of 16 to 128 slots, so that none spans more than two 64-slot blocks
        bm, bn = int(rng.choice([16, 32, 64, 128])), int(rng.choice([16, 32, 64, 128]))
    else:
        bm, bn = int(rng.choice([1, 7, 16, 64, 100, 128, 256])), int(rng.choice([1, 13, 32, 64, 128, 300]))
    rank = int(rng.integers(0, cp))
    print(f"[classify] {part} cp {cp} rank {rank} S {S} bm {bm} bn {bn} causal {causal}", flush=True)
    got = ra.ra_classify(S, cp, rank, part, bm, bn, cu, causal).cpu().numpy()
    assert np.array_equal(got, oracle.classify_tiles(S, cp, rank, part, cu, bm, bn, causal))
