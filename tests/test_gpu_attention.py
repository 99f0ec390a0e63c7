"""GPU parity of the ring-attention path against the fp64 oracle.

Every case runs the product path through the C ABI: the global inputs are
reordered on the GPU (cp_reorder), then ra_forward / ra_forward_steps run one
rank's ring. Expected values come only from the oracle on the same seeded
inputs. Bar: max-abs <= 1e-2 on O and <= 1e-3 on LSE for bf16 inputs (fp32
outputs are the gate; bf16 outputs are checked at the same bar), 1e-4 for the
fp32-input path.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
import sequence_parallelism_amd as ra
import synth
from tests.gpu_common import (TOL_LSE_BF16, TOL_LSE_F32, TOL_O_BF16, TOL_O_F32, max_abs, o_err, oracle_inputs,
                              rank_inputs, sample_rows, to_device)

pytestmark = pytest.mark.gpu


def _case_inputs(S, hq, hkv, d, dtype, seed, docs=None, prescale=1.0):
    w = synth.Workload("case", S, hq, hkv, d, 1, "contiguous", 0, dtype, docs=docs, doc_lo=16, doc_hi=max(17, S // 3),
                       prescale=prescale)
    return synth.make_global_inputs(w, seed)


def _check_rank(g, cp, rank, part, causal=True, rows=None, out_dtype=torch.float32, tol_o=None, tol_l=None,
                scale=0.0):
    qr, kr, vr = rank_inputs(g, cp, rank, part)
    out, lse = ra.ra_forward(qr, kr, vr, g.cu_seqlens, cp, rank, part, causal=causal, out_dtype=out_dtype,
                             softmax_scale=scale)
    torch.cuda.synchronize()
    gq, gk, gv = oracle_inputs(g)
    O, L = oracle.attention_rank(gq, gk, gv, g.cu_seqlens, cp, rank, part, causal, scale=scale or None, rows=rows)
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    if rows is not None:
        o, l = o[rows], l[:, rows]
    if tol_o is None:
        tol_o = TOL_O_BF16 if g.dtype == "bf16" else TOL_O_F32
        tol_l = TOL_LSE_BF16 if g.dtype == "bf16" else TOL_LSE_F32
    eo, el = o_err(o, O, out_dtype == torch.bfloat16), max_abs(l, L)
    assert np.all(np.isfinite(o)), "non-finite output"
    assert eo <= tol_o and el <= tol_l, f"max-abs O {eo:.3e} LSE {el:.3e}"
    return eo, el


def test_tiny_ring_fp32_all_ranks():
    """S=512, H=1, d=64, fp32, CP=4 contiguous: the tiny ring simulation, rank 2 first."""
    g = synth.make_global_inputs(synth.TINY_RING, 0)
    for rank in (2, 0, 1, 3):
        _check_rank(g, 4, rank, "contiguous")


def test_tiny_ring_steps_and_classes():
    """Rank 2 visits chunks 2, 1, 0, 3: a diagonal step, two full steps, an empty step."""
    g = synth.make_global_inputs(synth.TINY_RING, 0)
    qr, kr, vr = rank_inputs(g, 4, 2, "contiguous")
    o_steps, lse_steps = ra.ra_forward_steps(qr, kr, vr, None, 4, 2, "contiguous")
    gq, gk, gv = oracle_inputs(g)
    parts = oracle.step_partials(gq, gk, gv, None, 4, 2, "contiguous")
    assert [p[0] for p in parts] == [2, 1, 0, 3]
    for t, (s, O_t, L_t) in enumerate(parts):
        assert max_abs(o_steps[t].cpu().numpy(), O_t) <= TOL_O_F32
        assert max_abs(lse_steps[t].cpu().numpy(), L_t) <= TOL_LSE_F32
    assert torch.all(o_steps[3] == 0) and torch.all(torch.isneginf(lse_steps[3]))
    cls = ra.ra_classify(512, 4, 2, "contiguous", 128, 128).cpu().numpy()
    assert cls.reshape(4).tolist() == [1, 2, 2, 0]  # partial(diagonal), full, full, skip


SMALL = list(itertools.product(["contiguous", "zigzag", "striped"], [1, 2, 4, 8], [False, True]))


@pytest.mark.parametrize("part,cp,docs", SMALL)
def test_small_bf16_partitions(part, cp, docs):
    """bf16, d=128, GQA 4:2, S=2048: every rank, every row."""
    g = _case_inputs(2048, 4, 2, 128, "bf16", seed=cp * 10 + docs, docs="loguniform" if docs else None)
    for rank in sorted({0, cp - 1, cp // 2}):
        _check_rank(g, cp, rank, part)


@pytest.mark.parametrize("part", ["contiguous", "zigzag", "striped"])
def test_ragged_tiles_and_noncausal(part):
    """S_l not a multiple of the 128-row / 64-key tiles, zigzag halves straddling a
    key tile, documents, and the non-causal (document-only) mask."""
    cp = 4
    S = 2 * cp * 173  # S_l = 346, zigzag half = 173
    g = _case_inputs(S, 2, 1, 128, "bf16", seed=7, docs="loguniform")
    for rank in range(cp):
        _check_rank(g, cp, rank, part, causal=True)
        _check_rank(g, cp, rank, part, causal=False)


@pytest.mark.parametrize("S,cp,part", [(16, 1, "contiguous"), (64, 1, "contiguous"), (100, 1, "contiguous"),
                                       (128, 2, "zigzag"), (200, 2, "striped"), (384, 3, "zigzag"),
                                       (256, 16, "contiguous"), (384, 64, "zigzag"), (320, 64, "striped")])
def test_short_work_lists(S, cp, part):
    """Query tiles whose work lists hold one or two entries (the head_dim-128 kernel
    still loads tiles two entries ahead, past the end of the list) and ragged key
    tiles, causal and not."""
    g = _case_inputs(S, 2, 1, 128, "bf16", seed=S + cp)
    for rank in range(cp):
        _check_rank(g, cp, rank, part, causal=True)
        _check_rank(g, cp, rank, part, causal=False)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("out_bf16", [False, True])
def test_head_dims_and_output_dtypes(d, out_bf16):
    g = _case_inputs(1024, 2, 2, d, "bf16", seed=11)
    _check_rank(g, 2, 1, "zigzag", out_dtype=torch.bfloat16 if out_bf16 else torch.float32)


def test_fp32_inputs_d128_and_docs():
    g = _case_inputs(768, 2, 1, 128, "f32", seed=12, docs="loguniform")
    for rank in range(3):
        _check_rank(g, 3, rank, "striped")


def test_steps_partials_and_merge_chain():
    """ra_forward_steps matches the oracle's per-step partials; folding them with
    ra_lse_merge reproduces ra_forward and the unchunked oracle."""
    cp, rank, part = 4, 1, "zigzag"
    g = _case_inputs(2048, 4, 4, 128, "bf16", seed=13, docs="loguniform")
    qr, kr, vr = rank_inputs(g, cp, rank, part)
    o_steps, lse_steps = ra.ra_forward_steps(qr, kr, vr, g.cu_seqlens, cp, rank, part)
    gq, gk, gv = oracle_inputs(g)
    parts = oracle.step_partials(gq, gk, gv, g.cu_seqlens, cp, rank, part)
    for t, (s, O_t, L_t) in enumerate(parts):
        assert max_abs(o_steps[t].cpu().numpy(), O_t) <= TOL_O_BF16
        assert max_abs(lse_steps[t].cpu().numpy(), L_t) <= TOL_LSE_BF16
    o, l = o_steps[0].clone(), lse_steps[0].clone()
    for t in range(1, cp):
        o, l = ra.ra_lse_merge(o, l, o_steps[t], lse_steps[t], o_out=o, lse_out=l)  # in place
    out, lse = ra.ra_forward(qr, kr, vr, g.cu_seqlens, cp, rank, part, out_dtype=torch.float32)
    O, L = oracle.attention_rank(gq, gk, gv, g.cu_seqlens, cp, rank, part)
    assert max_abs(o.cpu().numpy(), O) <= TOL_O_BF16 and max_abs(l.cpu().numpy(), L) <= TOL_LSE_BF16
    # The two paths round P to bf16 (relative 2^-9) against different running maxima
    # (per step vs carried across steps), so O may differ by about 2 * 2^-9 * max|O|.
    # LSE does not depend on the rounding of P.
    bound = 2 * 2.0 ** -9 * max(1.0, float(np.abs(O).max()))
    assert max_abs(o.cpu().numpy(), out.cpu().numpy()) <= bound
    assert max_abs(l.cpu().numpy(), lse.cpu().numpy()) <= 1e-4


def test_lse_merge_kernel_against_oracle():
    rng = np.random.default_rng(3)
    for rows, h, d in ((37, 3, 128), (5, 2, 6), (64, 4, 64), (1003, 8, 128)):
        oa, ob = rng.standard_normal((rows, h, d)), rng.standard_normal((rows, h, d))
        la, lb = rng.standard_normal((h, rows)) * 5, rng.standard_normal((h, rows)) * 5
        la[0, :3] = -np.inf
        lb[0, 1:4] = -np.inf
        la[1, 5 % rows] = lb[1, 5 % rows] = -np.inf
        t = lambda x: torch.from_numpy(x.astype(np.float32)).cuda()
        o, l = ra.ra_lse_merge(t(oa), t(la), t(ob), t(lb))
        O, L = oracle.lse_merge(oa.astype(np.float32), la.astype(np.float32), ob.astype(np.float32),
                                lb.astype(np.float32))
        assert max_abs(o.cpu().numpy(), O) <= 1e-5
        assert max_abs(l.cpu().numpy(), L) <= 1e-5
        assert np.array_equal(np.isneginf(l.cpu().numpy()), np.isneginf(L))
        # in place (outputs over the first operand) gives the same bits
        oi, li_ = t(oa), t(la)
        ra.ra_lse_merge(oi, li_, t(ob), t(lb), o_out=oi, lse_out=li_)
        assert torch.equal(oi, o) and torch.equal(li_, l)


def test_causality_perturbation_is_bit_identical():
    """Changing K/V at positions no row of the rank can see leaves O and LSE
    bit-identical: skipped tiles are never read and masked keys contribute 0."""
    cp, rank, part = 4, 1, "zigzag"
    g = _case_inputs(2048, 2, 2, 128, "bf16", seed=17, docs="loguniform")
    qr, kr, vr = rank_inputs(g, cp, rank, part)
    out1, lse1 = ra.ra_forward(qr, kr, vr, g.cu_seqlens, cp, rank, part, out_dtype=torch.float32)
    pos = oracle.positions(part, 2048, cp, rank)
    vis = oracle.visible_matrix(pos, np.arange(2048), g.cu_seqlens, 2048, True).any(axis=0)
    g2 = synth.GlobalInputs(g.q, g.k.copy(), g.v.copy(), g.cu_seqlens, g.dtype)
    noise = synth.normal_bf16_bits(99, 9, g.k.shape, 30.0)
    g2.k[~vis] = noise[~vis]
    g2.v[~vis] = noise[~vis][:, :, ::-1]
    qr2, kr2, vr2 = rank_inputs(g2, cp, rank, part)
    out2, lse2 = ra.ra_forward(qr2, kr2, vr2, g.cu_seqlens, cp, rank, part, out_dtype=torch.float32)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_repeat_runs_are_bit_identical():
    g = _case_inputs(4096, 4, 1, 128, "bf16", seed=19)
    qr, kr, vr = rank_inputs(g, 8, 3, "striped")
    a = ra.ra_forward(qr, kr, vr, None, 8, 3, "striped")
    b = ra.ra_forward(qr, kr, vr, None, 8, 3, "striped")
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_prescaled_input_reading():
    """The alternative reading of 'N(0,1)/sqrt(128) scale': inputs pre-scaled by 1/sqrt(128)."""
    g = _case_inputs(2048, 4, 4, 128, "bf16", seed=21, prescale=1 / np.sqrt(128))
    _check_rank(g, 4, 0, "zigzag")


def test_side_stream_launch_matches_the_current_stream():
    """A call on a non-current stream allocates its workspace and default outputs on
    that stream: the caching allocator may hand the freed workspace only to work
    ordered after the kernels. Right after the call, the current stream allocates and
    overwrites memory while the side stream may still read its plan; the side-stream
    result must equal a current-stream run bit for bit."""
    g = _case_inputs(8192, 8, 2, 128, "bf16", seed=23, docs="loguniform")
    cp, rank, part = 4, 2, "zigzag"
    qr, kr, vr = rank_inputs(g, cp, rank, part)
    ref_o, ref_l = ra.ra_forward(qr, kr, vr, g.cu_seqlens, cp, rank, part, out_dtype=torch.float32)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        o, l = ra.ra_forward(qr, kr, vr, g.cu_seqlens, cp, rank, part, out_dtype=torch.float32, stream=side)
        outs.append((o, l))
        junk = [torch.full((1 << 20,), -1, dtype=torch.int32, device="cuda") for _ in range(8)]
        del junk
    torch.cuda.synchronize()
    for o, l in outs:
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l)
    # a raw hipStream_t handle is accepted as well
    o, l = ra.ra_forward(qr, kr, vr, g.cu_seqlens, cp, rank, part, out_dtype=torch.float32,
                         stream=side.cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)


def test_plan_used_on_another_stream_after_it_is_dropped():
    """A plan built on the current stream, then executed on a side stream (after the
    side stream waits for the plan), then dropped while that launch may still read
    it: the plan's workspace is recorded on the side stream, so the allocator does
    not hand it to the current stream's next allocations before the launch ends."""
    g = _case_inputs(8192, 8, 2, 128, "bf16", seed=29)
    cp, rank, part = 4, 1, "zigzag"
    qr, kr, vr = rank_inputs(g, cp, rank, part)
    ref_o, ref_l = ra.ra_forward(qr, kr, vr, None, cp, rank, part, out_dtype=torch.float32)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    outs = []
    for _ in range(3):
        plan = ra.ra_plan(8192, 8, 2, 128, None, cp, rank, part, out_dtype=torch.float32)
        side.wait_stream(torch.cuda.current_stream())
        outs.append(ra.ra_forward_planned(qr, kr, vr, plan, stream=side))
        del plan
        junk = [torch.full((1 << 20,), -1, dtype=torch.int32, device="cuda") for _ in range(8)]
        del junk
    torch.cuda.synchronize()
    for o, l in outs:
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l)
