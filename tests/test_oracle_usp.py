"""Pins of the oracle's Ulysses x Ring hybrid (CPU only).

The hybrid splits the same attention over a U x R grid of devices, so its
outputs, gathered back to global positions, must equal plain attention of the
whole sequence (torch's fp64 scaled_dot_product_attention where there is one
document, and the pinned dense oracle with documents); its corner cases reduce
to the pure Ring (U = 1) and pure Ulysses (R = 1) paths.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.partition import positions


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _gather_back(out, S, U, R, partition):
    """Device outputs [R, U, S/(R U), h, d] -> global order [S, h, d]."""
    sl = S // R
    g = np.empty((S,) + out.shape[3:])
    for r in range(R):
        pos = positions(partition, S, R, r)
        g[pos] = out[r].reshape((sl,) + out.shape[3:])
    return g


CASES = list(itertools.product([1, 2, 4], [1, 2, 4], ["contiguous", "zigzag", "striped"], [False, True]))


@pytest.mark.parametrize("U,R,part,docs", CASES)
def test_usp_equals_global_attention(U, R, part, docs):
    S, hq, hkv, d = 32, 8, 4, 4
    seed = CASES.index((U, R, part, docs))
    gq, gk, gv = _rand((S, hq, d), seed), _rand((S, hkv, d), seed + 50), _rand((S, hkv, d), seed + 99)
    cu = np.array([0, 5, 17, 32], dtype=np.int32) if docs else None
    out, L = oracle.usp_forward(gq, gk, gv, cu, U, R, part)
    got = _gather_back(out, S, U, R, part)
    O, LSE = oracle.attention_rank(gq, gk, gv, cu, 1, 0, "contiguous")
    np.testing.assert_allclose(got, O, rtol=0, atol=1e-12)
    # device (u, r)'s LSE is the global LSE of ring rank r's rows for head slice u
    for r in range(R):
        pos = positions(part, S, R, r)
        for u in range(U):
            np.testing.assert_allclose(L[r, u], LSE[u * hq // U:(u + 1) * hq // U][:, pos], rtol=0, atol=1e-12)
    if not docs:
        t = lambda x: torch.from_numpy(x).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(t(gq), t(gk), t(gv), is_causal=True, enable_gqa=True)
        np.testing.assert_allclose(got, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_usp_corner_cases_reduce_to_ring_and_ulysses():
    S, hq, hkv, d = 48, 4, 4, 8
    gq, gk, gv = _rand((S, hq, d), 1), _rand((S, hkv, d), 2), _rand((S, hkv, d), 3)
    # U = 1: device (0, r) output is ring rank r's attention output
    out, _ = oracle.usp_forward(gq, gk, gv, None, 1, 4, "zigzag")
    for r in range(4):
        O, _ = oracle.attention_rank(gq, gk, gv, None, 4, r, "zigzag")
        np.testing.assert_allclose(out[r, 0], O, rtol=0, atol=1e-12)
    # R = 1: the Ulysses path -- shards are contiguous pieces of the sequence
    out, _ = oracle.usp_forward(gq, gk, gv, None, 4, 1, "contiguous")
    O, _ = oracle.attention_rank(gq, gk, gv, None, 1, 0, "contiguous")
    np.testing.assert_allclose(out[0].reshape(S, hq, d), O, rtol=0, atol=1e-12)


def test_usp_device_shards_layout():
    S, h, d, U, R = 16, 2, 1, 2, 2
    x = np.arange(S, dtype=np.float64)[:, None, None] * np.ones((1, h, d))
    sh = oracle.usp_device_shards(x, U, R, "zigzag")
    # zigzag R=2: rank 0 holds chunks 0 and 3 of 4 (positions 0-3, 12-15); rank 1 holds 4-7, 8-11
    assert sh[0, 0, :, 0, 0].tolist() == [0, 1, 2, 3]
    assert sh[0, 1, :, 0, 0].tolist() == [12, 13, 14, 15]
    assert sh[1, 0, :, 0, 0].tolist() == [4, 5, 6, 7]
    assert sh[1, 1, :, 0, 0].tolist() == [8, 9, 10, 11]
    with pytest.raises(ValueError):
        oracle.usp_device_shards(np.zeros((12, 1, 1)), 4, 2, "contiguous")
