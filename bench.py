#!/usr/bin/env python3
"""Benchmark: one context-parallel rank's ring-attention hot path on one MI355X.

Headline workload: Llama-2-7B-shaped attention layer (S=32768, 32 heads,
head_dim 128, bf16, causal), CP=4 zigzag partition, rank 0's 8192-token share
against the 4 KV chunks. One step = the whole hot path over one batch:
  cp_reorder of the global Q, K and V into rank-major zigzag order
  -> ra_forward (work-list planning with tile classification, ring-step
     attention over the 4 chunks, steps combined, normalise + store).
Inputs are resident in HBM before the timed region. The metric is
causal-effective TFLOP/s: 4 * head_dim * heads * (visible query/key pairs of
the rank), i.e. masked or skipped work is not counted.

Also reported (extra "kernels" object): the attention kernel alone (HIP events
on the launch stream) with its roofline against the bf16 MFMA peak, the
backward of the same share (ra_backward, FLOPs counted as 2.5 x the forward's),
the permute / reorder / merge kernels in HBM GB/s, and the other workloads
(Ulysses path at 131072 tokens, a 4 x 2 Ulysses x Ring grid, GQA striped,
packed documents under the global zigzag and under per-document zigzag). The
CPU oracle is timed on a bounded row sample on the host cores (rank 0 only).

Runs on one GPU only: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "causal-effective attention TFLOP/s per CP-rank share (% bf16 MFMA peak); permute GB/s"
ATTN_KERNEL = "ring_attn_pp_kernel<true,false>"   # bf16 in and out, head_dim 128, fused steps
# sources whose hash ties a committed counter profile to the kernel it measured
KERNEL_SOURCES = ("ra_attn_pp.hip", "ra_common.h", "ra_device.h", "ra_internal.h")
PART_CODE = {"contiguous": 0, "zigzag": 1, "striped": 2}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# FLOP accounting: visible (query, key) pairs of one rank (plain counting)
# ---------------------------------------------------------------------------
def rank_positions(np, part, S, cp, r):
    sl = S // cp
    if part == "contiguous":
        return np.arange(r * sl, (r + 1) * sl, dtype=np.int64)
    if part == "striped":
        return np.arange(r, S, cp, dtype=np.int64)
    h = S // (2 * cp)
    return np.concatenate([np.arange(r * h, (r + 1) * h), np.arange((2 * cp - 1 - r) * h, (2 * cp - r) * h)])


def visible_pairs(np, part, S, cp, r, cu=None, causal=True):
    pos = rank_positions(np, part, S, cp, r)
    if cu is None:
        return int((pos + 1).sum()) if causal else int(len(pos) * S)
    cu = np.asarray(cu, dtype=np.int64)
    j = np.searchsorted(cu, pos, side="right") - 1
    if causal:
        return int((pos - cu[j] + 1).sum())
    return int((cu[j + 1] - cu[j]).sum())


# ---------------------------------------------------------------------------
# Timing helpers (HIP events on the stream the library launches on)
# ---------------------------------------------------------------------------
def time_events(torch, fn, reps, warm=2):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        times.append((a, b))
    torch.cuda.synchronize()
    ms = sorted(x.elapsed_time(y) for x, y in times)
    return {"avg_ms": sum(ms) / len(ms), "min_ms": ms[0], "median_ms": ms[len(ms) // 2]}


def traffic_from_profiles(kernel_src_sha):
    """HBM bytes per launch of the attention kernel from the committed counter
    summary, if it was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "ring_attn_llama7b_zigzag_counters.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_sha = re.search(r"[Kk]ernel source sha256[^:]*:\s*([0-9a-f]{64})", txt)
    m_b = re.search(r"HBM bytes per launch \(scaled\):\s*([0-9.eE+]+)", txt)
    if not m_sha or not m_b or m_sha.group(1) != kernel_src_sha:
        return None
    return float(m_b.group(1))


def kernel_source_sha():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, "sequence_parallelism_amd", "csrc", f), "rb").read())
    return h.hexdigest()


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of rank 0's rows
# ---------------------------------------------------------------------------
def cpu_baseline(np, w, g, rows_every):
    import oracle
    import synth
    gq, gk, gv = (synth.to_f64(x, g.dtype) for x in (g.q, g.k, g.v))
    sl = w.s_total // w.cp
    rows = np.arange(0, sl, rows_every, dtype=np.int64)
    t0 = time.perf_counter()
    oracle.attention_rank(gq, gk, gv, g.cu_seqlens, w.cp, w.rank, w.partition, rows=rows)
    dt = time.perf_counter() - t0
    pos = rank_positions(np, w.partition, w.s_total, w.cp, w.rank)[rows]
    pairs = int((pos + 1).sum())
    flops = 4.0 * w.d * w.hq * pairs
    cores = len(os.sched_getaffinity(0))
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = sum(i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas") or None
    except Exception:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads or cores,
            "kind": "oracle",
            "sample": f"{len(rows)} of rank {w.rank}'s {sl} rows (1 in every {rows_every}), all {w.hq} heads, "
                      f"fp64 dense masked scores against all {w.s_total} keys; {dt:.1f} s on {cores} host cores "
                      f"({threads} BLAS threads)",
            "seconds": dt}


# ---------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extras", action="store_true", help="headline only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows-every", type=int, default=4)
    ap.add_argument("--mode", default="full", choices=["full", "attn-only", "bwd-only", "copy-only"],
                    help="attn-only / copy-only: a few launches of one kernel, for counter runs")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU's share of the ring (the ring is simulated on one GPU); "
              f"--gpus {args.gpus} / WORLD_SIZE {world} is not supported: run with --gpus 1.", flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import sequence_parallelism_amd as ra
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", flush=True)
        sys.exit(1)
    ra.load_library()
    dev = torch.device("cuda:0")
    w = synth.LLAMA7B_ZIGZAG

    if args.mode == "copy-only":
        # plain copy of known size (CP=1 contiguous reorder = identity copy): counter calibration
        n = 1 << 29  # 1 GiB of bf16
        src = torch.randn(n, device=dev, dtype=torch.bfloat16).view(n // 8192, 64, 128)
        dst = torch.empty_like(src)
        for _ in range(3):
            ra.cp_reorder(src, 1, "contiguous", out=dst.view(1, *src.shape))
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy-only", "bytes_read": src.numel() * 2, "bytes_written": src.numel() * 2}))
        return

    log(f"generating seeded inputs for {w.name}")
    g = synth.make_global_inputs(w, seed=0)

    def dev_bits(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    q_g, k_g, v_g = dev_bits(g.q), dev_bits(g.k), dev_bits(g.v)
    S, cp, rank = w.s_total, w.cp, w.rank
    sl = S // cp
    q_p = torch.empty((cp, sl, w.hq, w.d), dtype=torch.bfloat16, device=dev)
    k_p = torch.empty((cp, sl, w.hkv, w.d), dtype=torch.bfloat16, device=dev)
    v_p = torch.empty_like(k_p)
    out = torch.empty((sl, w.hq, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.hq, sl), dtype=torch.float32, device=dev)
    shape = ra.make_shape(S, w.hq, w.hkv, w.d, True, 0.0, ra.RA_BF16, ra.RA_BF16)
    ws = torch.empty(ra.ra_workspace_size(shape, cp, 0), dtype=torch.uint8, device=dev)
    pairs = visible_pairs(np, w.partition, S, cp, rank)
    flops = 4.0 * w.d * w.hq * pairs

    if args.mode == "attn-only":
        plan = ra.ra_plan(S, w.hq, w.hkv, w.d, None, cp, rank, w.partition, workspace=ws)
        ra.cp_reorder(q_g, cp, w.partition, out=q_p)
        ra.cp_reorder(k_g, cp, w.partition, out=k_p)
        ra.cp_reorder(v_g, cp, w.partition, out=v_p)
        for _ in range(24):
            ra.ra_forward_planned(q_p[rank], k_p, v_p, plan, out=out, lse=lse)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "attn-only", "launches": 24, "flops_per_launch": flops}))
        return

    if args.mode == "bwd-only":
        ra.cp_reorder(q_g, cp, w.partition, out=q_p)
        ra.cp_reorder(k_g, cp, w.partition, out=k_p)
        ra.cp_reorder(v_g, cp, w.partition, out=v_p)
        ra.ra_forward(q_p[rank], k_p, v_p, None, cp, rank, w.partition, out=out, lse=lse, workspace=ws)
        bw = backward_buffers(torch, ra, w, dev)
        for _ in range(12):
            run_backward(ra, w, q_p[rank], k_p, v_p, out, lse, bw)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "bwd-only", "launches": 12, "flops_per_launch": 2.5 * flops}))
        return

    def step():
        ra.cp_reorder(q_g, cp, w.partition, out=q_p)
        ra.cp_reorder(k_g, cp, w.partition, out=k_p)
        ra.cp_reorder(v_g, cp, w.partition, out=v_p)
        ra.ra_forward(q_p[rank], k_p, v_p, None, cp, rank, w.partition, out=out, lse=lse, workspace=ws)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    log(f"step {ms_per_step:.3f} ms -> {value:.1f} causal-effective TFLOP/s")

    # the dominant kernel alone: ring attention on a prebuilt plan
    plan = ra.ra_plan(S, w.hq, w.hkv, w.d, None, cp, rank, w.partition, workspace=torch.empty_like(ws))
    attn = time_events(torch, lambda: ra.ra_forward_planned(q_p[rank], k_p, v_p, plan, out=out, lse=lse),
                       max(10, args.steps))
    attn_tflops = flops / (attn["avg_ms"] * 1e-3) / 1e12
    alg_bytes = (q_p[rank].numel() + k_p.numel() + v_p.numel() + out.numel()) * 2 + lse.numel() * 4
    kernels = {"ring_attn_llama7b_zigzag_rank0": {
        "avg_ms": attn["avg_ms"], "min_ms": attn["min_ms"], "tflops": attn_tflops,
        "frac_bf16_peak": attn_tflops / PEAK_BF16_TFLOPS, "flops": flops, "visible_pairs_per_head": pairs,
        "algorithmic_bytes": alg_bytes}}
    reo = time_events(torch, lambda: ra.cp_reorder(k_g, cp, w.partition, out=k_p), max(10, args.steps))
    nbytes = 2 * k_g.numel() * 2
    kernels["cp_reorder_k_s32k_h32_zigzag"] = {"avg_ms": reo["avg_ms"], "bytes": nbytes,
                                               "gbs": nbytes / (reo["avg_ms"] * 1e-3) / 1e9}
    kernels["cp_reorder_k_s32k_h32_zigzag"]["frac_hbm_peak"] = \
        kernels["cp_reorder_k_s32k_h32_zigzag"]["gbs"] / PEAK_HBM_GBS
    log(f"attention kernel {attn['avg_ms']:.3f} ms = {attn_tflops:.1f} TFLOP/s; "
        f"cp_reorder {kernels['cp_reorder_k_s32k_h32_zigzag']['gbs']:.0f} GB/s")

    # backward of the same share: dQ, and this rank's dK / dV partials of every chunk
    bw = backward_buffers(torch, ra, w, dev)
    tb = time_events(torch, lambda: run_backward(ra, w, q_p[rank], k_p, v_p, out, lse, bw), max(5, args.steps // 2))
    bflops = 2.5 * flops
    kernels["ring_attn_backward_llama7b_zigzag_rank0"] = {
        "avg_ms": tb["avg_ms"], "min_ms": tb["min_ms"], "flops": bflops,
        "tflops": bflops / (tb["avg_ms"] * 1e-3) / 1e12,
        "frac_bf16_peak": bflops / (tb["avg_ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "mfma_tflops_executed": 3.5 * flops / (tb["avg_ms"] * 1e-3) / 1e12,
        "note": "whole ra_backward call (plans, D = dO.O, dQ kernel, dK/dV kernel); FLOPs = 2.5 x forward"}
    log(f"backward {tb['avg_ms']:.3f} ms = {kernels['ring_attn_backward_llama7b_zigzag_rank0']['tflops']:.1f} "
        f"TFLOP/s (2.5 x forward FLOPs)")
    del bw

    if not args.no_extras:
        kernels.update(extras(np, torch, ra, synth, dev, max(5, args.steps // 2)))

    src_sha = kernel_source_sha()
    traffic = traffic_from_profiles(src_sha)
    roofline = {"bound": "mfma", "achieved": attn_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": attn_tflops / PEAK_BF16_TFLOPS, "traffic": traffic,
                "kernel": ATTN_KERNEL, "avg_launch_ms": attn["avg_ms"],
                "flops_per_launch": flops}

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a row sample")
        cpu = cpu_baseline(np, w, g, args.cpu_rows_every)
        log(f"oracle {cpu['value'] * 1e3:.2f} GFLOP/s causal-effective in {cpu['seconds']:.1f} s")

    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "s_total": S, "heads": w.hq, "kv_heads": w.hkv, "head_dim": w.d, "cp": cp,
                   "partition": w.partition, "rank": rank, "causal": True,
                   "step": "cp_reorder(q,k,v) + ra_forward(plan + ring attention), bf16 out"},
        "frac_bf16_peak": value / PEAK_BF16_TFLOPS,
        "roofline": roofline, "cpu_baseline": cpu, "kernels": kernels,
    }
    print(json.dumps(line), flush=True)


def backward_buffers(torch, ra, w, dev):
    """dO (seeded on the GPU), gradient outputs and workspace of one rank's backward."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    sl = w.s_total // w.cp
    shape = ra.make_shape(w.s_total, w.hq, w.hkv, w.d, True, 0.0, ra.RA_BF16, ra.RA_BF16)
    return {"dout": torch.randn((sl, w.hq, w.d), device=dev, dtype=torch.bfloat16, generator=gen),
            "dq": torch.empty((sl, w.hq, w.d), device=dev, dtype=torch.float32),
            "dk": torch.empty((w.cp, sl, w.hkv, w.d), device=dev, dtype=torch.float32),
            "dv": torch.empty((w.cp, sl, w.hkv, w.d), device=dev, dtype=torch.float32),
            "ws": torch.empty(ra.ra_backward_workspace_size(shape, w.cp, 0), device=dev, dtype=torch.uint8)}


def run_backward(ra, w, q, k, v, out, lse, bw, cu=None, rank=None):
    return ra.ra_backward(q, k, v, out, lse, bw["dout"], cu, w.cp, w.rank if rank is None else rank, w.partition,
                          dq=bw["dq"], dk=bw["dk"], dv=bw["dv"], workspace=bw["ws"])


def extras(np, torch, ra, synth, dev, reps):
    """Per-kernel figures for the other workloads (inputs drawn on the GPU)."""
    res = {}
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)

    def randn(*shape):
        return torch.randn(shape, device=dev, dtype=torch.bfloat16, generator=gen)

    # Ulysses path: [4, 32768, 32, 128] -> [4, 131072, 8, 128]; attention over 131072 tokens, 8 heads
    log("extras: Ulysses path")
    n, sl, H, d = 4, 32768, 32, 128
    xq, xk, xv = randn(n, sl, H, d), randn(n, sl, H, d), randn(n, sl, H, d)
    yq = torch.empty((n, n * sl, H // n, d), dtype=torch.bfloat16, device=dev)
    yk, yv, o_all = torch.empty_like(yq), torch.empty_like(yq), torch.zeros_like(yq)
    back = torch.empty_like(xq)
    t = time_events(torch, lambda: ra.ulysses_permute(xq, n, out=yq), reps)
    nbytes = 2 * xq.numel() * 2
    res["ulysses_permute_n4_s32k_h32"] = {"avg_ms": t["avg_ms"], "bytes": nbytes,
                                          "gbs": nbytes / (t["avg_ms"] * 1e-3) / 1e9}
    ti = time_events(torch, lambda: ra.ulysses_permute(o_all, n, inverse=True, out=back), reps)
    res["ulysses_permute_inverse_n4_s128k_h8"] = {"avg_ms": ti["avg_ms"], "bytes": nbytes,
                                                  "gbs": nbytes / (ti["avg_ms"] * 1e-3) / 1e9}
    ra.ulysses_permute(xk, n, out=yk)
    ra.ulysses_permute(xv, n, out=yv)
    S = n * sl
    plan = ra.ra_plan(S, H // n, H // n, d, None, 1, 0, "contiguous")
    ta = time_events(torch, lambda: ra.ra_forward_planned(yq[0], yk[0:1], yv[0:1], plan, out=o_all[0]),
                     max(3, reps // 2))
    fl = 4.0 * d * (H // n) * visible_pairs(np, "contiguous", S, 1, 0)
    res["ring_attn_ulysses_s128k_h8"] = {"avg_ms": ta["avg_ms"], "flops": fl,
                                         "tflops": fl / (ta["avg_ms"] * 1e-3) / 1e12}

    def pipeline():
        ra.ulysses_permute(xq, n, out=yq)
        ra.ulysses_permute(xk, n, out=yk)
        ra.ulysses_permute(xv, n, out=yv)
        ra.ra_forward(yq[0], yk[0:1], yv[0:1], None, 1, 0, "contiguous", out=o_all[0])
        ra.ulysses_permute(o_all, n, inverse=True, out=back)
    tp = time_events(torch, pipeline, max(3, reps // 2))
    res["ulysses_pipeline_s128k"] = {"avg_ms": tp["avg_ms"], "tflops": fl / (tp["avg_ms"] * 1e-3) / 1e12}
    del xq, xk, xv, yq, yk, yv, o_all, back

    # Ulysses x Ring hybrid: a 4 x 2 grid (Ulysses 4 inside, zigzag ring of 2 across), S=131072,
    # 32 heads; the whole grid's work on one GPU (all 8 devices' permutes and attention)
    log("extras: Ulysses x Ring grid")
    U, R, S = 4, 2, 131072
    sh = S // (U * R)
    gq, gk, gvv = randn(R, U, sh, H, d), randn(R, U, sh, H, d), randn(R, U, sh, H, d)
    ushape = ra.make_shape(S, H, H, d, True, 0.0, ra.RA_BF16, ra.RA_BF16)
    uws = torch.empty(ra.usp_workspace_size(ushape, U, R, 0), dtype=torch.uint8, device=dev)
    uout = torch.empty_like(gq)
    ulse = torch.empty((U, R, H // U, S // R), dtype=torch.float32, device=dev)
    tu = time_events(torch, lambda: ra.usp_forward(gq, gk, gvv, None, U, R, "zigzag", out=uout, lse=ulse,
                                                   workspace=uws), max(3, reps // 2))
    fl = 4.0 * d * H * visible_pairs(np, "contiguous", S, 1, 0)
    res["usp_grid_u4_r2_s128k_h32"] = {"avg_ms": tu["avg_ms"], "flops": fl,
                                       "tflops": fl / (tu["avg_ms"] * 1e-3) / 1e12,
                                       "per_device_ms": tu["avg_ms"] / (U * R),
                                       "note": "whole grid: 3 x R strided Ulysses permutes, U x R ring attentions "
                                               "(R steps each), R inverse permutes"}
    del gq, gk, gvv, uws, uout, ulse

    # GQA striped: 32 q heads / 8 kv heads, S=65536, CP=8, rank 0
    log("extras: GQA striped")
    w = synth.GQA_STRIPED
    slg = w.s_total // w.cp
    q = randn(slg, w.hq, w.d)
    k, v = randn(w.cp, slg, w.hkv, w.d), randn(w.cp, slg, w.hkv, w.d)
    plan = ra.ra_plan(w.s_total, w.hq, w.hkv, w.d, None, w.cp, 0, w.partition)
    tg = time_events(torch, lambda: ra.ra_forward_planned(q, k, v, plan), reps)
    fl = 4.0 * w.d * w.hq * visible_pairs(np, w.partition, w.s_total, w.cp, 0)
    res["ring_attn_gqa_striped_rank0"] = {"avg_ms": tg["avg_ms"], "flops": fl,
                                          "tflops": fl / (tg["avg_ms"] * 1e-3) / 1e12}
    del q, k, v

    # packed documents: 131072 tokens, log-uniform documents, CP=8 zigzag, every rank
    log("extras: packed documents")
    w = synth.PACKED_ZIGZAG
    cu = synth.loguniform_cu_seqlens(0, w.s_total, w.doc_lo, w.doc_hi)
    slp = w.s_total // w.cp
    q_all = randn(w.cp, slp, w.hq, w.d)
    k, v = randn(w.cp, slp, w.hkv, w.d), randn(w.cp, slp, w.hkv, w.d)
    per_rank = []
    for r in range(w.cp):
        plan = ra.ra_plan(w.s_total, w.hq, w.hkv, w.d, cu, w.cp, r, w.partition)
        tr = time_events(torch, lambda: ra.ra_forward_planned(q_all[r], k, v, plan), max(3, reps // 2))
        fl = 4.0 * w.d * w.hq * visible_pairs(np, w.partition, w.s_total, w.cp, r, cu)
        per_rank.append({"rank": r, "avg_ms": tr["avg_ms"], "flops": fl,
                         "tflops": fl / (tr["avg_ms"] * 1e-3) / 1e12})
    heavy = max(per_rank, key=lambda x: x["flops"])
    res["ring_attn_packed_docs_zigzag"] = {"n_docs": len(cu) - 1, "max_work_rank": heavy, "ranks": per_rank}
    del q_all, k, v

    # the same documents under per-document zigzag: every rank holds two pieces of every
    # document (padded to 64-slot blocks), so the ranks' work is even; timed with ra_forward
    # (plan included: the planned entry point does not take this partition)
    log("extras: packed documents, per-document zigzag")
    sld = ra.ra_local_length(w.s_total, w.cp, "doc_zigzag", cu)
    q_all = randn(w.cp, sld, w.hq, w.d)
    k, v = randn(w.cp, sld, w.hkv, w.d), randn(w.cp, sld, w.hkv, w.d)
    dshape = ra.make_shape(w.s_total, w.hq, w.hkv, w.d, True, 0.0, ra.RA_BF16, ra.RA_BF16)
    dws = torch.empty(ra.ra_workspace_size(dshape, w.cp, len(cu) - 1), dtype=torch.uint8, device=dev)
    dout = torch.empty((sld, w.hq, w.d), dtype=torch.bfloat16, device=dev)
    dlse = torch.empty((w.hq, sld), dtype=torch.float32, device=dev)
    per_rank_d = []
    for r in range(w.cp):
        tr = time_events(torch, lambda: ra.ra_forward(q_all[r], k, v, cu, w.cp, r, "doc_zigzag", out=dout, lse=dlse,
                                                      workspace=dws), max(3, reps // 2))
        per_rank_d.append({"rank": r, "avg_ms": tr["avg_ms"]})
    slowest = max(per_rank_d, key=lambda x: x["avg_ms"])
    total_fl = 4.0 * w.d * w.hq * visible_pairs(np, "contiguous", w.s_total, 1, 0, cu)
    res["ring_attn_packed_docs_doc_zigzag"] = {
        "n_docs": len(cu) - 1, "s_local": sld, "s_local_unpadded": slp, "slowest_rank": slowest, "ranks": per_rank_d,
        "slowest_rank_speedup_vs_global_zigzag": max(x["avg_ms"] for x in per_rank) / slowest["avg_ms"],
        "tflops_all_ranks": total_fl / (sum(x["avg_ms"] for x in per_rank_d) * 1e-3) / 1e12}

    # measured copy ceiling: torch's device-to-device copy of 1 GiB
    src = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    tc = time_events(torch, lambda: dst.copy_(src), reps)
    nbytes = 2 * src.numel() * 2
    res["reference_torch_copy_1GiB"] = {"avg_ms": tc["avg_ms"], "bytes": nbytes,
                                        "gbs": nbytes / (tc["avg_ms"] * 1e-3) / 1e9}
    del src, dst

    # fp32 LSE merge of two [8192, 32, 128] partials (HBM-bound)
    rows, h, dd = 8192, 32, 128
    oa = torch.randn((rows, h, dd), device=dev, generator=gen)
    ob, la, lb = torch.randn_like(oa), torch.randn((h, rows), device=dev), torch.randn((h, rows), device=dev)
    oo, lo = torch.empty_like(oa), torch.empty_like(la)
    tm = time_events(torch, lambda: ra.ra_lse_merge(oa, la, ob, lb, o_out=oo, lse_out=lo), reps)
    nbytes = 3 * oa.numel() * 4 + 3 * la.numel() * 4
    res["lse_merge_8192x32x128_f32"] = {"avg_ms": tm["avg_ms"], "bytes": nbytes,
                                        "gbs": nbytes / (tm["avg_ms"] * 1e-3) / 1e9}
    return res


if __name__ == "__main__":
    main()
