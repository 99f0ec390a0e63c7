"""GPU bit-exactness of the permutation and classification kernels against the oracle."""
import itertools

import numpy as np
import pytest
import torch

import oracle
import sequence_parallelism_amd as ra
import synth
from tests.gpu_common import device_bits, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("part,cp", list(itertools.product(["contiguous", "zigzag", "striped"], [1, 2, 4, 8])))
def test_cp_reorder_small_bitexact(part, cp):
    S = 2 * cp * 37
    for h, d, eb in ((3, 5, 2), (2, 64, 2), (1, 7, 4), (4, 3, 1)):
        x = np.random.default_rng(cp + h).integers(0, 255, (S, h, d * eb)).astype(np.uint8)
        xt = torch.from_numpy(x).cuda()
        if eb == 2:
            xt = xt.view(torch.int16)
        elif eb == 4:
            xt = xt.view(torch.int32)
        y = ra.cp_reorder(xt, cp, part)
        exp = oracle.cp_reorder(x, cp, part)
        assert np.array_equal(y.view(torch.uint8).cpu().numpy().reshape(exp.shape), exp)
        z = ra.cp_reorder(y, cp, part, inverse=True)
        assert np.array_equal(z.view(torch.uint8).cpu().numpy().reshape(x.shape), x)


@pytest.mark.parametrize("w", [synth.LLAMA7B_ZIGZAG, synth.GQA_STRIPED])
def test_cp_reorder_full_size_bitexact(w):
    q = synth.normal_bf16_bits(0, synth.TID_K, (w.s_total, w.hkv, w.d))
    qt = to_device(q, "bf16")
    y = ra.cp_reorder(qt, w.cp, w.partition)
    assert np.array_equal(device_bits(y), oracle.cp_reorder(q, w.cp, w.partition))
    assert torch.equal(ra.cp_reorder(y, w.cp, w.partition, inverse=True), qt)


@pytest.mark.parametrize("n,sl,h,d", [(1, 5, 3, 2), (2, 7, 4, 3), (4, 9, 8, 64), (8, 3, 8, 5), (2, 5, 64, 128),
                                     (2, 3, 128, 128), (4, 37, 4, 128)])
def test_ulysses_small_bitexact(n, sl, h, d):
    x = np.random.default_rng(n).integers(0, 1 << 16, (n, sl, h, d)).astype(np.uint16)
    xt = to_device(x, "bf16")
    y = ra.ulysses_permute(xt, n)
    assert np.array_equal(device_bits(y), oracle.ulysses_permute(x, n))
    # compare bits: random patterns include NaNs, which never compare equal as values
    assert np.array_equal(device_bits(ra.ulysses_permute(y, n, inverse=True)), x)


def test_ulysses_full_size_bitexact():
    """[4, 32768, 32, 128] bf16 -> [4, 131072, 8, 128] and back."""
    x = synth.make_ulysses_inputs(4, 32768, 32, 128, seed=0)
    xt = to_device(x, "bf16")
    y = ra.ulysses_permute(xt, 4)
    assert np.array_equal(device_bits(y), oracle.ulysses_permute(x, 4))
    del x
    assert torch.equal(ra.ulysses_permute(y, 4, inverse=True), xt)


def test_ulysses_worked_layout():
    """The N=4, 4-head example: device r ends with every token and head r only."""
    N, S, H = 4, 8, 4
    tags = np.zeros((N, S // N, H, 2), dtype=np.uint16)
    for j in range(N):
        for i in range(S // N):
            for hh in range(H):
                tags[j, i, hh] = (j * (S // N) + i, hh)
    y = device_bits(ra.ulysses_permute(to_device(tags, "bf16"), N))
    for r in range(N):
        assert list(y[r, :, 0, 0]) == list(range(S)) and set(y[r, :, 0, 1]) == {r}


CLS = list(itertools.product(["contiguous", "zigzag", "striped"], [1, 2, 4, 8], [False, True], [True, False]))


@pytest.mark.parametrize("part,cp,docs,causal", CLS)
def test_classify_small_bitexact(part, cp, docs, causal):
    S = 2 * cp * 61
    cu = synth.loguniform_cu_seqlens(cp, S, 5, 90) if docs else None
    for rank in sorted({0, cp - 1}):
        for bm, bn in ((16, 16), (7, 13), (64, 32), (128, 64)):
            got = ra.ra_classify(S, cp, rank, part, bm, bn, cu, causal).cpu().numpy()
            exp = oracle.classify_tiles(S, cp, rank, part, cu, bm, bn, causal)
            assert np.array_equal(got, exp), (rank, bm, bn)


def test_classify_llama7b_zigzag_bitexact():
    w = synth.LLAMA7B_ZIGZAG
    for rank in (0, 3):
        got = ra.ra_classify(w.s_total, w.cp, rank, w.partition, 128, 128).cpu().numpy()
        exp = oracle.classify_tiles(w.s_total, w.cp, rank, w.partition, None, 128, 128)
        assert np.array_equal(got, exp)


def test_classify_packed_documents_bitexact():
    """131072 packed tokens, log-uniform documents, CP=8 zigzag, 256 x 256 tiles."""
    w = synth.PACKED_ZIGZAG
    cu = synth.loguniform_cu_seqlens(0, w.s_total, w.doc_lo, w.doc_hi)
    for rank in (0, 5):
        got = ra.ra_classify(w.s_total, w.cp, rank, w.partition, 256, 256, cu).cpu().numpy()
        exp = oracle.classify_tiles(w.s_total, w.cp, rank, w.partition, cu, 256, 256)
        assert np.array_equal(got, exp)
