"""GPU parity of the Ulysses x Ring hybrid (usp_forward) and of the strided
Ulysses permute it is built on, against the oracle.

The strided permute is a bit-exact copy: compared bit for bit with the oracle's
ulysses_permute placed into blocks, and the gaps between blocks must stay
untouched. usp_forward is attention: every device's output and LSE are
compared with oracle.usp_forward (which follows the hybrid's steps) at the
attention bar (max-abs 1e-2 on O, 1e-3 on LSE for bf16 inputs; 1e-4 for fp32),
and at a larger size on sampled tokens with the oracle's global attention (the
hybrid is the same attention redistributed, a pinned identity).
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
import sequence_parallelism_amd as ra
import synth
from oracle.partition import positions
from tests.gpu_common import (TOL_LSE_BF16, TOL_LSE_F32, TOL_O_BF16, TOL_O_F32, device_bits, max_abs, o_err, to_device)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,sl,h,d", [(4, 64, 8, 128), (2, 33, 4, 64), (4, 16, 12, 8)])
def test_ulysses_strided_bit_exact(n, sl, h, d):
    rng = np.random.default_rng(n * 100 + sl)
    x = rng.integers(0, 1 << 16, size=(n, sl, h, d), dtype=np.uint16)
    xd = to_device(x, "bf16")
    hn = h // n
    block = n * sl * hn * d * 2
    stride = 3 * block + hn * d * 2           # blocks apart, with a gap of 2 blocks and 1 run
    span = (n - 1) * stride + block
    sentinel = 0x7fc1
    buf = torch.full((span // 2,), 0, dtype=torch.int16, device="cuda")
    buf.fill_(sentinel)
    ra.ulysses_permute_strided(xd, n, buf.view(torch.bfloat16), stride)
    got = buf.cpu().numpy().view(np.uint16)
    ref = oracle.ulysses_permute(x, n)        # [n, n sl, hn, d]
    expect = np.full(span // 2, sentinel, dtype=np.uint16)
    for rho in range(n):
        o = rho * stride // 2
        expect[o:o + block // 2] = ref[rho].reshape(-1)
    assert np.array_equal(got, expect)
    # inverse from the strided blocks back to the packed sequence-split layout
    back = torch.empty_like(xd)
    ra.ulysses_permute_strided(buf.view(torch.bfloat16), n, back, stride, inverse=True)
    assert np.array_equal(device_bits(back), x)


def _usp_case(S, hq, hkv, d, dtype, seed, docs=None):
    w = synth.Workload("usp_case", S, hq, hkv, d, 1, "contiguous", 0, dtype, docs=docs, doc_lo=16,
                       doc_hi=max(17, S // 3))
    return synth.make_global_inputs(w, seed)


def _run_usp(g, U, R, part, out_dtype=torch.float32):
    """Device inputs from the GPU's own cp_reorder: ring group r's tokens in partition
    order, cut into U contiguous pieces."""
    S = g.q.shape[0]
    q, k, v = (ra.cp_reorder(to_device(x, g.dtype), R, part).view(R, U, S // (R * U), x.shape[1], x.shape[2])
               for x in (g.q, g.k, g.v))
    out, lse = ra.usp_forward(q, k, v, g.cu_seqlens, U, R, part, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


GRID = list(itertools.product([2, 4], [1, 2, 4], ["contiguous", "zigzag", "striped"]))


@pytest.mark.parametrize("U,R,part", GRID)
def test_usp_small_grids(U, R, part):
    """bf16, d=128, 8 query / 4 KV heads, S=2048 with documents: every device."""
    g = _usp_case(2048, 8, 4, 128, "bf16", seed=U * 10 + R, docs="loguniform")
    out, lse = _run_usp(g, U, R, part)
    gq, gk, gv = (synth.to_f64(x, g.dtype) for x in (g.q, g.k, g.v))
    O, L = oracle.usp_forward(gq, gk, gv, g.cu_seqlens, U, R, part)
    eo, el = max_abs(out, O), max_abs(np.transpose(lse, (1, 0, 2, 3)), L)
    assert eo <= TOL_O_BF16 and el <= TOL_LSE_BF16, f"max-abs O {eo:.3e} LSE {el:.3e}"


def test_usp_bf16_output_and_mha():
    g = _usp_case(1024, 4, 4, 64, "bf16", seed=5)
    out, lse = _run_usp(g, 4, 2, "zigzag", out_dtype=torch.bfloat16)
    gq, gk, gv = (synth.to_f64(x, g.dtype) for x in (g.q, g.k, g.v))
    O, L = oracle.usp_forward(gq, gk, gv, None, 4, 2, "zigzag")
    assert o_err(out, O, True) <= TOL_O_BF16 and max_abs(np.transpose(lse, (1, 0, 2, 3)), L) <= TOL_LSE_BF16


def test_usp_fp32_inputs():
    g = _usp_case(512, 4, 2, 64, "f32", seed=6, docs="loguniform")
    out, lse = _run_usp(g, 2, 2, "striped")
    gq, gk, gv = (synth.to_f64(x, g.dtype) for x in (g.q, g.k, g.v))
    O, L = oracle.usp_forward(gq, gk, gv, g.cu_seqlens, 2, 2, "striped")
    assert max_abs(out, O) <= TOL_O_F32 and max_abs(np.transpose(lse, (1, 0, 2, 3)), L) <= TOL_LSE_F32


def test_usp_u4_r2_s32k_sampled():
    """32 query / 8 KV heads, S=32768, a 4 x 2 grid (zigzag ring): sampled tokens of
    every device against the oracle's global attention (the hybrid redistributes it)."""
    S, hq, hkv, d, U, R, part = 32768, 32, 8, 128, 4, 2, "zigzag"
    w = synth.Workload("usp_s32k", S, hq, hkv, d, 1, "contiguous", 0, "bf16")
    g = synth.make_global_inputs(w, 7)
    out, _ = _run_usp(g, U, R, part)
    gq, gk, gv = (synth.to_f64(x, "bf16") for x in (g.q, g.k, g.v))
    sl, sh = S // R, S // (R * U)
    rng = np.random.default_rng(1)
    for r in range(R):
        pos = positions(part, S, R, r)
        for u in range(U):
            idx = np.unique(np.concatenate([[0, sh - 1], rng.integers(0, sh, 6)]))
            p = pos[u * sh + idx]
            O, _ = oracle.attention_rows(gq[p], p, gk, gv, np.arange(S), None, S, True)
            e = max_abs(out[r, u, idx], O)
            assert e <= TOL_O_BF16, f"device ({u},{r}): max-abs {e:.3e}"
