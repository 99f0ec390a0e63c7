"""GPU parity of the ring-attention backward (ra_backward) against the fp64 oracle.

Expected gradients come only from the oracle on the same seeded inputs. The
backward kernels round P (for dV) and dS (for dK and dQ) to bf16 before their
MFMA products, a relative error of at most 2^-9 per product term; everything
else is fp32. So each gradient element is checked against the bound

    |gpu - oracle| <= 2^-8 * sum_terms |term| + 1e-5

where the sum of absolute terms is computed from the oracle's P and dS
(dV_k: sum_i P_ik |dO_i|; dK_k: scale sum_i |dS_ik| |q_i|; dQ_i: scale
sum_k |dS_ik| |k_k|), i.e. twice the rounding bound. When the forward output
that enters D = dO . O is itself rounded (bf16 storage, or the GPU forward's
own bf16 P), the error of D is bounded the same way from oracle quantities and
propagated: dS moves by P_ik dD_i, so dQ_i moves by at most
scale |dD_i| sum_k P_ik |k_k| and dK_k by scale sum_i P_ik |dD_i| |q_i|.
fp32 inputs (VALU path, no bf16 rounding) use 2^-12 and 1e-4: fp32 sums over
up to ~1000 terms (n * 2^-24 relative) and fp32 dP - D cancellation are the
only error sources there.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
import sequence_parallelism_amd as ra
import synth
from tests.bwd_common import SLACK, Ref, bwd_case, check_bound, check_rank, run_backward
from tests.gpu_common import rank_inputs, reorder, to_device

pytestmark = pytest.mark.gpu

SMALL = list(itertools.product(["contiguous", "zigzag", "striped"], [1, 2, 4, 8], [False, True]))


@pytest.mark.parametrize("part,cp,docs", SMALL)
def test_backward_small_bf16_partitions(part, cp, docs):
    """bf16, d=128, GQA 4:2, S=2048: ranks 0, CP/2 and CP-1, every row and key."""
    g, gdo = bwd_case(2048, 4, 2, 128, "bf16", seed=100 + cp * 10 + docs, docs="loguniform" if docs else None)
    for rank in sorted({0, cp // 2, cp - 1}):
        check_rank(g, gdo, cp, rank, part)


@pytest.mark.parametrize("part", ["contiguous", "zigzag", "striped"])
def test_backward_ragged_and_noncausal(part):
    """S_l = 346 (not a multiple of the 64-row, 128-key or 64-key tiles), zigzag
    halves straddling tiles, documents, causal and document-only masks."""
    cp = 4
    g, gdo = bwd_case(2 * cp * 173, 2, 1, 128, "bf16", seed=107, docs="loguniform")
    for rank in range(cp):
        check_rank(g, gdo, cp, rank, part, causal=True)
        check_rank(g, gdo, cp, rank, part, causal=False)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("out_bf16", [False, True])
def test_backward_head_dims_and_output_dtypes(d, out_bf16):
    g, gdo = bwd_case(1024, 2, 2, d, "bf16", seed=111)
    check_rank(g, gdo, 2, 1, "zigzag", out_dtype=torch.bfloat16 if out_bf16 else torch.float32)


@pytest.mark.parametrize("S,cp,part", [(256, 16, "contiguous"), (384, 64, "zigzag"), (320, 64, "striped")])
def test_backward_large_cp_tiny_shares(S, cp, part):
    """CP up to its limit of 64 with a few rows per rank: the ring step reaches 63,
    and every tile of every chunk is ragged."""
    g, gdo = bwd_case(S, 2, 1, 128, "bf16", seed=S + cp)
    for rank in sorted({0, 1, cp // 2, cp - 1}):
        check_rank(g, gdo, cp, rank, part)


def test_backward_gqa_striped_cp8():
    g, gdo = bwd_case(4096, 8, 2, 128, "bf16", seed=113, docs="loguniform")
    for rank in (0, 5, 7):
        check_rank(g, gdo, 8, rank, "striped")


@pytest.mark.parametrize("d", [64, 128])
def test_backward_fp32_inputs(d):
    """fp32 inputs take the VALU kernels: no bf16 rounding anywhere."""
    g, gdo = bwd_case(768, 2, 1, d, "f32", seed=115, docs="loguniform")
    for rank in range(3):
        check_rank(g, gdo, 3, rank, "striped", rel=2.0 ** -12, slack=1e-4)


def test_backward_tiny_ring_fp32():
    """The tiny ring simulation's shape (S=512, H=1, d=64, fp32, CP=4 contiguous), every rank."""
    w = synth.TINY_RING
    g = synth.make_global_inputs(w, 0)
    gdo = synth.make_global_dout(w, 0)
    for rank in (2, 0, 1, 3):
        check_rank(g, gdo, 4, rank, "contiguous", rel=2.0 ** -12, slack=1e-4)


def test_backward_ranks_sum_to_whole_sequence_gradient():
    """A real ring adds every rank's dK / dV partial as the chunk travels: the sum
    over ranks equals the gradient of attention over the whole sequence (CP = 1)."""
    cp, part = 4, "zigzag"
    g, gdo = bwd_case(2048, 4, 2, 128, "bf16", seed=117, docs="loguniform")
    dk_sum = dv_sum = 0
    bk_sum = bv_sum = 0
    for rank in range(cp):
        ref = Ref(g, gdo, cp, rank, part)
        _, dk, dv = run_backward(g, gdo, cp, rank, part, ref.O, ref.L)
        dk_sum = dk_sum + dk
        dv_sum = dv_sum + dv
        bk_sum = bk_sum + ref.chunked(2.0 ** -8 * ref.A_dk, part, cp) + SLACK
        bv_sum = bv_sum + ref.chunked(2.0 ** -8 * ref.A_dv, part, cp) + SLACK
    full = Ref(g, gdo, 1, 0, "contiguous")
    check_bound("sum dk", dk_sum, full.chunked(full.dk, part, cp), bk_sum)
    check_bound("sum dv", dv_sum, full.chunked(full.dv, part, cp), bv_sum)


def test_backward_after_gpu_forward():
    """The chain a training step runs: ra_forward (fp32 output) then ra_backward on
    its O and LSE. The forward rounds P to bf16, so |O - O_exact| <= 2^-8 sum_k P|v|
    per element, which bounds the error of D = dO . O."""
    cp, rank, part = 4, 1, "zigzag"
    g, gdo = bwd_case(2048, 4, 4, 128, "bf16", seed=119, docs="loguniform")
    ref = Ref(g, gdo, cp, rank, part)
    qr, kr, vr = rank_inputs(g, cp, rank, part)
    out, lse = ra.ra_forward(qr, kr, vr, g.cu_seqlens, cp, rank, part, out_dtype=torch.float32)
    do = reorder(to_device(gdo, g.dtype), cp, part, g.cu_seqlens)[rank].contiguous()
    dq, dk, dv = ra.ra_backward(qr, kr, vr, out, lse, do, g.cu_seqlens, cp, rank, part)
    torch.cuda.synchronize()
    eD = (np.abs(ref.dout) * (2.0 ** -8 * ref.PV)).sum(axis=2)
    xq, xk = ref.d_error_bounds(eD)
    # The forward's LSE is within its own parity bar (1e-3), which scales a row's P
    # by at most e^(1e-3): a relative 1e-3 of every term of dS and P.
    r = 2.0 ** -8 + 1e-3
    check_bound("dq", dq.cpu().numpy(), ref.dq, r * ref.A_dq + xq + SLACK)
    check_bound("dk", dk.cpu().numpy(), ref.chunked(ref.dk, part, cp), ref.chunked(r * ref.A_dk + xk, part, cp) + SLACK)
    check_bound("dv", dv.cpu().numpy(), ref.chunked(ref.dv, part, cp), ref.chunked(r * ref.A_dv, part, cp) + SLACK)


def test_backward_invisible_keys_and_determinism():
    """Keys that no row of the rank sees get exactly zero dK / dV; changing K / V
    at those positions leaves dQ bit-identical; repeated calls are bit-identical."""
    cp, rank, part = 4, 1, "zigzag"
    g, gdo = bwd_case(2048, 2, 2, 128, "bf16", seed=121, docs="loguniform")
    ref = Ref(g, gdo, cp, rank, part)
    dq1, dk1, dv1 = run_backward(g, gdo, cp, rank, part, ref.O, ref.L)
    dq1b, dk1b, dv1b = run_backward(g, gdo, cp, rank, part, ref.O, ref.L)
    assert np.array_equal(dq1, dq1b) and np.array_equal(dk1, dk1b) and np.array_equal(dv1, dv1b)
    vis = oracle.visible_matrix(ref.pos, np.arange(2048), g.cu_seqlens, 2048, True).any(axis=0)
    inv_chunks = ref.chunked(~vis[:, None, None] & np.ones((2048, 2, 128), bool), part, cp)
    assert inv_chunks.any()
    assert np.all(dk1[inv_chunks] == 0) and np.all(dv1[inv_chunks] == 0)
    g2 = synth.GlobalInputs(g.q, g.k.copy(), g.v.copy(), g.cu_seqlens, g.dtype)
    noise = synth.normal_bf16_bits(99, 9, g.k.shape, 30.0)
    g2.k[~vis] = noise[~vis]
    g2.v[~vis] = noise[~vis][:, :, ::-1]
    dq2, dk2, dv2 = run_backward(g2, gdo, cp, rank, part, ref.O, ref.L)
    assert np.array_equal(dq1, dq2)
    vis_chunks = ~inv_chunks
    assert np.array_equal(dk1[vis_chunks], dk2[vis_chunks]) and np.array_equal(dv1[vis_chunks], dv2[vis_chunks])
