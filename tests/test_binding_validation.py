"""The Python binding checks every tensor a caller passes (shape, dtype,
contiguity, device, workspace size) against the call's shape or plan before
anything reaches the library, so that a mismatched tensor raises ValueError
instead of sending the kernels past the end of a buffer. CPU only: every case
raises before any GPU work (CPU tensors that pass the shape checks are refused
as not on a GPU)."""
import pytest
import torch

import sequence_parallelism_amd as ra

BF, F32 = torch.bfloat16, torch.float32


def _qkv(sl=256, hq=4, hkv=2, d=64, cp=4, dtype=BF):
    return (torch.zeros((sl, hq, d), dtype=dtype), torch.zeros((cp, sl, hkv, d), dtype=dtype),
            torch.zeros((cp, sl, hkv, d), dtype=dtype))


def _raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_forward_checks_every_tensor():
    q, k, v = _qkv()
    f = ra.ra_forward
    _raises("out must have shape", f, q, k, v, None, 4, 0, "zigzag", out=torch.zeros((255, 4, 64), dtype=BF))
    _raises("out must be", f, q, k, v, None, 4, 0, "zigzag", out=torch.zeros((256, 4, 64), dtype=F32),
            out_dtype=BF)
    # without out_dtype, a given out sets it (fp32 here): the call gets past the dtype check
    _raises("on a GPU", f, q, k, v, None, 4, 0, "zigzag", out=torch.zeros((256, 4, 64), dtype=F32))
    _raises("lse must have shape", f, q, k, v, None, 4, 0, "zigzag", lse=torch.zeros((256, 4), dtype=F32))
    _raises("lse must be", f, q, k, v, None, 4, 0, "zigzag", lse=torch.zeros((4, 256), dtype=BF))
    _raises("k has shape", f, q, k[:3], v[:3], None, 4, 0, "zigzag")
    _raises("v must have shape", f, q, k, v[:, :128], None, 4, 0, "zigzag")
    _raises("k must be", f, q, k.float(), v, None, 4, 0, "zigzag")
    _raises("q must be contiguous", f, q.transpose(0, 1).contiguous().transpose(0, 1), k, v, None, 4, 0, "zigzag")
    _raises("k must be contiguous", f, q, k.transpose(1, 2).contiguous().transpose(1, 2), v, None, 4, 0, "zigzag")
    _raises("s_total", f, q, k, v, None, 4, 0, "zigzag", s_total=2048)
    _raises("workspace holds", f, q, k, v, None, 4, 0, "zigzag", workspace=torch.zeros(16, dtype=torch.uint8))
    _raises("on a GPU", f, q, k, v, None, 4, 0, "zigzag")


def test_forward_doc_zigzag_checks_the_local_length():
    cu = [0, 100, 1000]
    S = 1000
    sl = ra.ra_local_length(S, 4, "doc_zigzag", cu)
    assert sl > S // 4
    q, k, v = _qkv(sl=S // 4)
    _raises("doc_zigzag", ra.ra_forward, q, k, v, cu, 4, 0, "doc_zigzag")
    q, k, v = _qkv(sl=sl)
    _raises("on a GPU", ra.ra_forward, q, k, v, cu, 4, 0, "doc_zigzag")


def test_planned_call_checks_tensors_against_the_plan():
    sh = ra.make_shape(1024, 4, 2, 64, True, 0.0, ra.RA_BF16, ra.RA_F32)
    plan = ra.Plan(sh, 0, 4, 0, 1, torch.zeros(ra.ra_workspace_size(sh, 4, 0), dtype=torch.uint8), 0, 256)
    q, k, v = _qkv()
    f = ra.ra_forward_planned
    _raises("q must be", f, q.float(), k, v, plan)
    _raises("q must have shape", f, q[:128], k, v, plan)
    _raises("k must have shape", f, q, torch.zeros((4, 256, 4, 64), dtype=BF), v, plan)
    _raises("v must have shape", f, q, k, torch.zeros((2, 256, 2, 64), dtype=BF), plan)
    _raises("out must be", f, q, k, v, plan, out=torch.zeros((256, 4, 64), dtype=BF))  # the plan says fp32
    _raises("lse must have shape", f, q, k, v, plan, lse=torch.zeros((4, 255), dtype=F32))
    _raises("on a GPU", f, q, k, v, plan)


def test_steps_and_backward_check_their_outputs():
    q, k, v = _qkv()
    _raises("o_steps must have shape", ra.ra_forward_steps, q, k, v, None, 4, 0, "zigzag",
            o_steps=torch.zeros((3, 256, 4, 64), dtype=F32))
    _raises("lse_steps must be", ra.ra_forward_steps, q, k, v, None, 4, 0, "zigzag",
            lse_steps=torch.zeros((4, 4, 256), dtype=BF))
    out, lse, do = torch.zeros_like(q), torch.zeros((4, 256), dtype=F32), torch.zeros_like(q)
    b = ra.ra_backward
    _raises("dout must be", b, q, k, v, out, lse, do.float(), None, 4, 0, "zigzag")
    _raises("lse must have shape", b, q, k, v, out, lse.t().contiguous(), do, None, 4, 0, "zigzag")
    _raises("out must have shape", b, q, k, v, out[:100], lse, do, None, 4, 0, "zigzag")
    _raises("dq must be", b, q, k, v, out, lse, do, None, 4, 0, "zigzag", dq=torch.zeros_like(q))
    _raises("dk must have shape", b, q, k, v, out, lse, do, None, 4, 0, "zigzag",
            dk=torch.zeros((4, 256, 4, 64), dtype=F32))
    _raises("dv must have shape", b, q, k, v, out, lse, do, None, 4, 0, "zigzag",
            dv=torch.zeros((3, 256, 2, 64), dtype=F32))
    _raises("workspace holds", b, q, k, v, out, lse, do, None, 4, 0, "zigzag",
            workspace=torch.zeros(64, dtype=torch.uint8))
    _raises("on a GPU", b, q, k, v, out, lse, do, None, 4, 0, "zigzag")


def test_merge_checks_both_partials_and_outputs():
    oa, la = torch.zeros((8, 2, 16)), torch.zeros((2, 8))
    m = ra.ra_lse_merge
    _raises("o_b must have shape", m, oa, la, torch.zeros((7, 2, 16)), la)
    _raises("lse_b must have shape", m, oa, la, oa, torch.zeros((2, 9)))
    _raises("o_b must be", m, oa, la, oa.to(BF), la)
    _raises("o_out must have shape", m, oa, la, oa, la, o_out=torch.zeros((8, 2, 15)))
    _raises("lse_out must be", m, oa, la, oa, la, lse_out=torch.zeros((2, 8), dtype=BF))
    _raises("o_a must be contiguous", m, oa.transpose(0, 2).contiguous().transpose(0, 2), la, oa, la)
    _raises("on a GPU", m, oa, la, oa, la)


def test_permutes_check_outputs_and_contiguity():
    x = torch.zeros((1024, 4, 64), dtype=BF)
    _raises("out must have shape", ra.cp_reorder, x, 4, "zigzag", out=torch.zeros((4, 255, 4, 64), dtype=BF))
    _raises("out must be", ra.cp_reorder, x, 4, "zigzag", out=torch.zeros((4, 256, 4, 64), dtype=F32))
    _raises("must divide", ra.cp_reorder, x[:1001], 4, "zigzag")
    _raises("input must be contiguous", ra.cp_reorder, x.transpose(0, 1).contiguous().transpose(0, 1), 4, "zigzag")
    _raises("leading dimension", ra.cp_reorder, torch.zeros((2, 512, 4, 64), dtype=BF), 4, "zigzag", inverse=True)
    _raises("on a GPU", ra.cp_reorder, x, 4, "zigzag")
    u = torch.zeros((4, 64, 8, 32), dtype=BF)
    _raises("out must have shape", ra.ulysses_permute, u, 4, out=torch.zeros((4, 256, 8, 32), dtype=BF))
    _raises("input must be contiguous", ra.ulysses_permute, u.transpose(2, 3).contiguous().transpose(2, 3), 4)
    _raises("must divide", ra.ulysses_permute, torch.zeros((4, 64, 6, 32), dtype=BF), 4)
    _raises("on a GPU", ra.ulysses_permute, u, 4)
    block = 4 * 64 * 2 * 32 * 2
    _raises("holds", ra.ulysses_permute_strided, u, 4, torch.zeros(4 * block // 2 - 1, dtype=BF), block)
    _raises("x must be contiguous", ra.ulysses_permute_strided, u.transpose(2, 3).contiguous().transpose(2, 3), 4,
            torch.zeros(4 * block // 2, dtype=BF), block)
    _raises("smaller than one block", ra.ulysses_permute_strided, u, 4, torch.zeros(4 * block, dtype=BF), block - 2)
    _raises("on a GPU", ra.ulysses_permute_strided, u, 4, torch.zeros(4 * block // 2, dtype=BF), block)


def test_doc_reorder_checks_the_local_layout():
    cu = [0, 100, 1000]
    sl = ra.ra_local_length(1000, 4, "doc_zigzag", cu)
    x = torch.zeros((1000, 2, 64), dtype=BF)
    _raises("out must have shape", ra.cp_reorder_docs, x, 4, cu, out=torch.zeros((4, 250, 2, 64), dtype=BF))
    _raises("input must have shape", ra.cp_reorder_docs, torch.zeros((4, 250, 2, 64), dtype=BF), 4, cu, inverse=True)
    _raises("workspace holds", ra.cp_reorder_docs, x, 4, cu, workspace=torch.zeros(8, dtype=torch.uint8))
    _raises("on a GPU", ra.cp_reorder_docs, x, 4, cu)
    _raises("on a GPU", ra.cp_reorder_docs, torch.zeros((4, sl, 2, 64), dtype=BF), 4, cu, inverse=True)


def test_usp_checks_outputs_and_workspace():
    q = torch.zeros((2, 4, 128, 8, 64), dtype=BF)
    k = torch.zeros((2, 4, 128, 4, 64), dtype=BF)
    f = ra.usp_forward
    _raises("out must have shape", f, q, k, k, None, 4, 2, "zigzag", out=torch.zeros((2, 4, 128, 8, 32), dtype=BF))
    _raises("lse must have shape", f, q, k, k, None, 4, 2, "zigzag", lse=torch.zeros((4, 2, 2, 511), dtype=F32))
    _raises("workspace holds", f, q, k, k, None, 4, 2, "zigzag", workspace=torch.zeros(64, dtype=torch.uint8))
    _raises("must divide by ulysses", f, torch.zeros((2, 3, 128, 8, 64), dtype=BF),
            torch.zeros((2, 3, 128, 4, 64), dtype=BF), torch.zeros((2, 3, 128, 4, 64), dtype=BF), None, 3, 2)
    _raises("v must be", f, q, k, k.float(), None, 4, 2, "zigzag")
    _raises("on a GPU", f, q, k, k, None, 4, 2, "zigzag")


def test_classify_refuses_a_cpu_device():
    _raises("on a GPU", ra.ra_classify, 1024, 4, 0, "zigzag", 64, 64, device="cpu")
    _raises("positive", ra.ra_classify, 1024, 4, 0, "zigzag", 0, 64, device="cuda")
