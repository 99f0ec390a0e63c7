"""ra_forward_noalloc, the entry point for callers that cannot allocate, against
ra_forward: the same kernels on the same plan, so the outputs must be
bit-identical. Two calls in a row on the library's fixed scratch, the second
with a smaller input (its plan overwrites only part of the first one's), plus a
per-document zigzag call. Outputs are filled with NaN first, so a row the call
leaves unwritten fails. Last, the call captured in a HIP graph: the graph holds
the plan kernels and the attention kernel (the library records no memset or
copy), so each replay rebuilds the plan in the fixed scratch and must reproduce
the eager result bit for bit, also after another call has overwritten that
scratch in between."""
import pytest
import torch

import sequence_parallelism_amd as ra
import synth
from tests.gpu_common import rank_inputs

pytestmark = pytest.mark.gpu


def _case(S, hq, hkv, d, cp, rank, part, docs, out_dtype, seed):
    w = synth.Workload("noalloc", S, hq, hkv, d, cp, part, rank, "bf16", docs=docs, doc_lo=64, doc_hi=S // 3)
    g = synth.make_global_inputs(w, seed)
    qr, kr, vr = rank_inputs(g, cp, rank, part)
    ref_o, ref_l = ra.ra_forward(qr, kr, vr, g.cu_seqlens, cp, rank, part, out_dtype=out_dtype)
    out = torch.full_like(ref_o, float("nan"))
    lse = torch.full_like(ref_l, float("nan"))
    got_o, got_l = ra.ra_forward_noalloc(qr, kr, vr, g.cu_seqlens, cp, rank, part, out=out, lse=lse)
    torch.cuda.synchronize()
    assert got_o.data_ptr() == out.data_ptr() and got_l.data_ptr() == lse.data_ptr()
    print(f"noalloc S={S} hq={hq} cp={cp} {part} rank {rank}", flush=True)
    assert torch.equal(got_o.view(torch.int16) if got_o.element_size() == 2 else got_o.view(torch.int32),
                       ref_o.view(torch.int16) if ref_o.element_size() == 2 else ref_o.view(torch.int32))
    assert torch.equal(got_l.view(torch.int32), ref_l.view(torch.int32))
    assert bool(torch.isfinite(got_o.float()).all())


def test_noalloc_matches_ra_forward_then_a_smaller_call():
    # first call: 8192 tokens, GQA 8/2, zigzag over 4 ranks, packed documents
    _case(8192, 8, 2, 128, 4, 1, "zigzag", "loguniform", torch.float32, seed=3)
    # second call, smaller: 2048 tokens striped over 2 ranks, one document, bf16 output
    _case(2048, 4, 4, 128, 2, 0, "striped", None, torch.bfloat16, seed=4)


def test_noalloc_doc_zigzag_and_head_dim_64():
    _case(4096, 4, 4, 128, 4, 2, "doc_zigzag", "loguniform", torch.float32, seed=5)
    _case(1024, 2, 1, 64, 2, 1, "contiguous", None, torch.float32, seed=6)


def test_noalloc_refuses_a_plan_beyond_the_fixed_scratch():
    # 2^20 tokens on one rank: the plan needs 256 MiB, above the 16 MiB scratch
    S = 1 << 20
    q = torch.empty((S, 1, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((1, S, 1, 64), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((1, S), dtype=torch.float32, device="cuda")
    with pytest.raises(ra.RAError) as e:
        ra.ra_forward_noalloc(q, k, k, None, 1, 0, "contiguous", out=out, lse=lse)
    assert e.value.status == ra.RA_ERR_SCRATCH


def _graph_inputs(S, hq, hkv, cp, rank, part, docs, seed):
    w = synth.Workload("graph", S, hq, hkv, 128, cp, part, rank, "bf16", docs=docs, doc_lo=64, doc_hi=S // 3)
    g = synth.make_global_inputs(w, seed)
    return g, rank_inputs(g, cp, rank, part)


def test_noalloc_replays_of_a_captured_graph_match_eager():
    cp, rank, part = 4, 1, "zigzag"
    g, (qr, kr, vr) = _graph_inputs(8192, 8, 2, cp, rank, part, "loguniform", seed=7)
    ref_o, ref_l = ra.ra_forward(qr, kr, vr, g.cu_seqlens, cp, rank, part, out_dtype=torch.float32)
    out = torch.empty_like(ref_o)
    lse = torch.empty_like(ref_l)
    ra.ra_forward_noalloc(qr, kr, vr, g.cu_seqlens, cp, rank, part, out=out, lse=lse)  # eager warm-up
    torch.cuda.synchronize()
    # another call's arguments, run between replays: it overwrites the fixed scratch
    g2, (q2, k2, v2) = _graph_inputs(2048, 4, 4, 2, 0, "striped", None, seed=8)
    o2 = torch.empty((q2.shape[0], 4, 128), dtype=torch.float32, device="cuda")
    l2 = torch.empty((4, q2.shape[0]), dtype=torch.float32, device="cuda")
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            ra.ra_forward_noalloc(qr, kr, vr, g.cu_seqlens, cp, rank, part, out=out, lse=lse)
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        ra.ra_forward_noalloc(q2, k2, v2, None, 2, 0, "striped", out=o2, lse=l2)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print(f"graph replay {i}", flush=True)
        assert torch.equal(out.view(torch.int32), ref_o.view(torch.int32)), f"replay {i}: O"
        assert torch.equal(lse.view(torch.int32), ref_l.view(torch.int32)), f"replay {i}: LSE"
