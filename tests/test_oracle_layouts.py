"""Pins of the oracle's permutations and tile classification (CPU only)."""
import itertools
import os

import numpy as np
import pytest

import oracle
from oracle import brute
from oracle.partition import positions

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_ulysses_worked_layout_golden():
    """The N=4, 4-head worked example of the concept page's all-to-all section."""
    rows = []
    with open(os.path.join(GOLDEN, "ulysses_n4_h4_layout.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                ph, dev, t0, t1, h0, h1 = line.split()
                rows.append((ph, int(dev), int(t0), int(t1), int(h0), int(h1)))
    N, S, H = 4, 8, 4
    sl = S // N
    # tag every element with its (global token, head)
    x = np.zeros((N, sl, H, 2), dtype=np.int64)
    for j in range(N):
        for i in range(sl):
            for h in range(H):
                x[j, i, h] = (j * sl + i, h)
    for ph, dev, t0, t1, h0, h1 in rows:
        if ph == "before":
            assert set(x[dev, :, :, 0].ravel()) == set(range(t0, t1))
            assert set(x[dev, :, :, 1].ravel()) == set(range(h0, h1))
    y = oracle.ulysses_permute(x, N)
    assert y.shape == (N, S, H // N, 2)
    for ph, dev, t0, t1, h0, h1 in rows:
        if ph == "after":
            assert list(y[dev, :, 0, 0]) == list(range(t0, t1))  # all tokens, in order
            assert set(y[dev, :, :, 1].ravel()) == set(range(h0, h1))
    assert np.array_equal(oracle.ulysses_permute(y, N, inverse=True), x)


@pytest.mark.parametrize("n,sl,H,d", [(1, 5, 3, 2), (2, 3, 4, 1), (4, 6, 8, 3), (8, 2, 8, 2)])
def test_ulysses_inverse_roundtrip_and_indexing(n, sl, H, d):
    x = np.random.default_rng(n * 100 + sl).integers(0, 1 << 16, (n, sl, H, d)).astype(np.uint16)
    y = oracle.ulysses_permute(x, n)
    hn = H // n
    for rho, j, i, hp in itertools.product(range(n), range(n), range(sl), range(hn)):
        assert np.array_equal(y[rho, j * sl + i, hp], x[j, i, rho * hn + hp])
    assert np.array_equal(oracle.ulysses_permute(y, n, inverse=True), x)
    if n == 1:
        assert np.array_equal(y, x)


def test_ulysses_head_divisibility():
    with pytest.raises(ValueError):
        oracle.ulysses_permute(np.zeros((4, 2, 6, 1)), 4)


@pytest.mark.parametrize("part", ["contiguous", "zigzag", "striped"])
@pytest.mark.parametrize("cp", [1, 2, 4, 8])
def test_cp_reorder_against_brute_positions(part, cp):
    S = 16 * cp
    x = np.random.default_rng(cp).integers(0, 1 << 16, (S, 3, 2)).astype(np.uint16)
    y = oracle.cp_reorder(x, cp, part)
    for r in range(cp):
        bp = brute.brute_positions(part, S, cp, r)
        assert list(positions(part, S, cp, r)) == bp
        for i, p in enumerate(bp):
            assert np.array_equal(y[r, i], x[p])
    assert np.array_equal(oracle.cp_reorder(y, cp, part, inverse=True), x)
    if cp == 1:
        assert np.array_equal(y[0], x)


def test_partition_maps_cover_sequence_once():
    for part, S, cp in (("contiguous", 48, 4), ("zigzag", 48, 4), ("striped", 48, 4), ("zigzag", 64, 8)):
        allpos = np.concatenate([positions(part, S, cp, r) for r in range(cp)])
        assert sorted(allpos.tolist()) == list(range(S))


def test_zigzag_and_striped_divisibility():
    with pytest.raises(ValueError):
        positions("zigzag", 12, 4, 0)
    with pytest.raises(ValueError):
        positions("striped", 10, 4, 0)


CLS_CASES = list(itertools.product(["contiguous", "zigzag", "striped"], [1, 2, 4], [False, True],
                                   [(4, 4), (3, 5), (8, 2)], [True, False]))


@pytest.mark.parametrize("part,cp,docs,tile,causal", CLS_CASES)
def test_classify_matches_brute_force(part, cp, docs, tile, causal):
    S = 48 if cp != 4 else 64
    cu = [0, 7, 8, 30, S] if docs else None
    bm, bn = tile
    for r in range(cp):
        got = oracle.classify_tiles(S, cp, r, part, None if cu is None else np.array(cu), bm, bn, causal)
        exp = np.array(brute.brute_classify(S, cp, r, part, cu, bm, bn, causal), dtype=np.int8)
        assert np.array_equal(got, exp)


def test_classify_counts_sum_to_visible_totals():
    S, cp = 256, 4
    cu = np.array([0, 50, 51, 200, 256])
    for part in ("contiguous", "zigzag", "striped"):
        for r in range(cp):
            cls, cnt = oracle.classify_tiles(S, cp, r, part, cu, 32, 16, True, return_counts=True)
            tot = oracle.visible_counts(positions(part, S, cp, r), cu, S, True).sum()
            assert cnt.sum() == tot
            assert np.all(cnt[cls == oracle.SKIP] == 0)
