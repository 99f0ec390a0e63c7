#!/usr/bin/env python3
"""Benchmark: one context-parallel rank's ring-attention hot path on one MI355X.

Headline workload (the largest configuration that fits one GPU): the Ulysses
path. Four simulated ranks each hold [32768 tokens, 32 heads, head_dim 128]
bf16 Q, K and V; the Ulysses permute gives rank 0 every one of the 131072
tokens for heads 0-7 ([4, 32768, 32, 128] -> [4, 131072, 8, 128]); rank 0 runs
full causal attention over 131072 tokens for those 8 heads; the inverse
permute returns the output to the sequence-split layout. One step is that
whole path over one batch:
  ulysses_permute(Q), (K), (V)  ->  ra_forward(plan + attention, bf16 out)
  ->  ulysses_permute(O, inverse).
Inputs are the seeded synthetic tensors of the oracle's tests, resident in HBM
before the timed region. The metric is causal-effective TFLOP/s: 4 * head_dim
* heads * (visible query/key pairs), i.e. masked or skipped work is not
counted.

Also reported (the "kernels" object): the attention kernel alone (HIP events
on the launch stream) with its roofline against the bf16 MFMA peak; the other
workloads (Llama-2-7B-shaped zigzag share, GQA striped, packed documents under
the global zigzag and under per-document zigzag, a 4 x 2 Ulysses x Ring grid);
the backward of the zigzag share; the permute / reorder / merge kernels in HBM
GB/s; measured ceilings (a register-only bf16 MFMA loop, torch's device copy).
The CPU oracle is timed on a bounded row sample on the host cores.

--mode picks a short run of one kernel for rocprofv3 (kernel traces and
counters); see --help. Runs on one GPU only: --gpus above 1 exits with a
message.
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
COUNTERS_PROFILE = "ring_attn_ulysses_s128k_h8_counters.md"

# Ulysses path: 4 simulated ranks of [32768, 32, 128] -> rank 0's [131072, 8, 128]
U_N, U_SL, U_H, U_D = 4, 32768, 32, 128


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
def time_events(torch, fn, reps, warm=2, flush=None):
    """HIP-event times of `reps` calls of fn on the current stream (after `warm`
    untimed ones); flush, when given, runs before each timed call, outside the events."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        if flush is not None:
            flush()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        times.append((a, b))
    torch.cuda.synchronize()
    ms = sorted(x.elapsed_time(y) for x, y in times)
    return {"avg_ms": sum(ms) / len(ms), "min_ms": ms[0], "median_ms": ms[len(ms) // 2]}


_FLUSH = []


def mall_flush(torch):
    """Reads a 1 GiB scratch buffer, so that nothing of the previous repetition is
    still in the 256 MB last-level cache (MALL) when the next one starts: its
    inputs are gone, and its dirty output lines are written back during the flush
    (a flush by writing would leave its own dirty lines to drain during the timed
    kernel)."""
    if not _FLUSH:
        _FLUSH.append(torch.ones(1 << 28, dtype=torch.int32, device="cuda"))
    _FLUSH[0].sum()


ROTATE_BYTES = 2 << 30


def rotating_sets(nbytes):
    """Buffer sets for time_hbm: enough that the launches between two uses of one
    set move at least 2 GiB, eight times the 256 MB last-level cache."""
    return max(1, min(8, -(-ROTATE_BYTES // nbytes)))


def time_hbm(torch, fns, reps, nbytes):
    """An HBM-bound kernel timed cold. `fns` holds one call per buffer set (see
    rotating_sets). Each repetition flushes the cache, then runs every set once,
    back to back, between two events: no launch finds its data in the cache, and
    the events' own latency is shared by the launches of the stream, as in a run of
    reorders of Q, K and V. avg/min/median are per launch. The `single_launch`
    figures time the first set alone after each flush, event latency included."""
    if callable(fns):
        fns = [fns]

    def stream():
        for f in fns:
            f()

    t = time_events(torch, stream, reps, flush=lambda: mall_flush(torch))
    n = len(fns)
    one = time_events(torch, fns[0], reps, flush=lambda: mall_flush(torch))
    return {"avg_ms": t["avg_ms"] / n, "min_ms": t["min_ms"] / n, "median_ms": t["median_ms"] / n, "bytes": nbytes,
            "gbs": gbs(nbytes, t["avg_ms"] / n), "gbs_best": gbs(nbytes, t["min_ms"] / n),
            "frac_hbm_peak": gbs(nbytes, t["avg_ms"] / n) / PEAK_HBM_GBS, "buffer_sets": n,
            "single_launch": {"avg_ms": one["avg_ms"], "gbs": gbs(nbytes, one["avg_ms"]),
                              "frac_hbm_peak": gbs(nbytes, one["avg_ms"]) / PEAK_HBM_GBS}}


def traffic_from_profiles(kernel_src_sha):
    """HBM bytes per launch of the headline attention kernel from the committed
    counter summary, if it was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", COUNTERS_PROFILE)
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


def reorder_call(torch, ra, like, cp, partition):
    """cp_reorder of a fresh copy of `like` into a fresh output: one more buffer set for time_hbm."""
    x = like.clone()
    y = torch.empty((cp, like.shape[0] // cp) + tuple(like.shape[1:]), dtype=like.dtype, device=like.device)
    return lambda: ra.cp_reorder(x, cp, partition, out=y)


def gbs(nbytes, ms):
    return nbytes / (ms * 1e-3) / 1e9


# ---------------------------------------------------------------------------
# Headline inputs: the seeded Ulysses-path tensors (same bits as the oracle's tests)
# ---------------------------------------------------------------------------
def ulysses_inputs(np, torch, synth, dev):
    xs = [synth.make_ulysses_inputs(U_N, U_SL, U_H, U_D, seed=0, tid=t) for t in (synth.TID_Q, synth.TID_K,
                                                                              synth.TID_V)]
    dts = [torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev) for x in xs]
    return xs, dts


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of rank 0's rows
# ---------------------------------------------------------------------------
def cpu_baseline(np, xs, rows_every):
    import oracle
    import synth
    S = U_N * U_SL
    hq = U_H // U_N
    # device 0 of the Ulysses layout holds every token of heads 0..7 (the oracle's own permute)
    gq, gk, gv = (synth.bf16_bits_to_f64(oracle.ulysses_permute(x, U_N)[0]) for x in xs)
    rows = np.arange(rows_every // 2, S, rows_every, dtype=np.int64)
    t0 = time.perf_counter()
    oracle.attention_rank(gq, gk, gv, None, 1, 0, "contiguous", rows=rows)
    dt = time.perf_counter() - t0
    flops = 4.0 * U_D * hq * float((rows + 1).sum())
    cores = len(os.sched_getaffinity(0))
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = sum(i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas") or None
    except Exception:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads or cores,
            "kind": "oracle",
            "sample": f"{len(rows)} of rank 0's {S} query rows (1 in every {rows_every}, spread over the whole "
                      f"sequence), all {hq} heads, fp64 dense masked scores against all {S} keys; causal-effective "
                      f"FLOPs of those rows; {dt:.1f} s on {cores} host cores ({threads} BLAS threads)",
            "seconds": dt}


# ---------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extras", action="store_true", help="headline only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows-every", type=int, default=64)
    ap.add_argument("--mode", default="full",
                    choices=["full", "steps-only", "attn-only", "bwd-only", "permute-only", "copy-only",
                             "mfma-only"],
                    help="steps-only: the headline steps alone; attn-only: launches of one workload's attention "
                         "kernel (--workload, --rank); permute-only: one permute (--which); copy-only: torch's "
                         "1 GiB device copy (counter calibration); mfma-only: the register-only MFMA loop; "
                         "bwd-only: the backward of the Llama-2-7B-shaped share")
    ap.add_argument("--workload", default="ulysses", choices=["ulysses", "llama7b", "gqa", "packed", "packed_doc"])
    ap.add_argument("--rank", type=int, default=None, help="attn-only: the rank (default: the headline rank; -1: every rank in turn)")
    ap.add_argument("--which", default="ulysses_fwd",
                    choices=["ulysses_fwd", "ulysses_inv", "reorder_llama7b", "reorder_gqa_q", "reorder_gqa_kv",
                             "reorder_packed", "reorder_docs", "merge"])
    ap.add_argument("--launches", type=int, default=12, help="launches in the single-kernel modes")
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

    if args.mode == "copy-only":
        # a copy of known size that this library did not write: torch's device-to-device copy
        n = 1 << 29  # 1 GiB of bf16
        src = torch.randn(n, device=dev, dtype=torch.bfloat16)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy-only", "bytes_read": n * 2, "bytes_written": n * 2}), flush=True)
        return
    if args.mode == "mfma-only":
        r = mfma_ceiling(torch, ra, reps=3)
        print(json.dumps({"mode": "mfma-only", **r}), flush=True)
        return
    if args.mode == "attn-only":
        attn_only(np, torch, ra, synth, dev, args.workload, args.rank, args.launches)
        return
    if args.mode == "permute-only":
        permute_only(np, torch, ra, synth, dev, args.which, args.launches)
        return
    if args.mode == "bwd-only":
        bwd_only(np, torch, ra, synth, dev, args.launches)
        return

    # ---------------- headline: the Ulysses path over 131072 tokens ----------------
    log("generating the seeded Ulysses-path inputs ([4, 32768, 32, 128] bf16 x 3)")
    xs, (xq, xk, xv) = ulysses_inputs(np, torch, synth, dev)
    S, hq = U_N * U_SL, U_H // U_N
    yq = torch.empty((U_N, S, hq, U_D), dtype=torch.bfloat16, device=dev)
    yk, yv = torch.empty_like(yq), torch.empty_like(yq)
    o_all = torch.zeros_like(yq)  # rank 0's output lands in o_all[0]; the other ranks' slices stay zero
    back = torch.empty_like(xq)
    lse = torch.empty((hq, S), dtype=torch.float32, device=dev)
    shape = ra.make_shape(S, hq, hq, U_D, True, 0.0, ra.RA_BF16, ra.RA_BF16)
    ws = torch.empty(ra.ra_workspace_size(shape, 1, 0), dtype=torch.uint8, device=dev)
    pairs = visible_pairs(np, "contiguous", S, 1, 0)
    flops = 4.0 * U_D * hq * pairs

    def step():
        ra.ulysses_permute(xq, U_N, out=yq)
        ra.ulysses_permute(xk, U_N, out=yk)
        ra.ulysses_permute(xv, U_N, out=yv)
        ra.ra_forward(yq[0], yk[0:1], yv[0:1], None, 1, 0, "contiguous", out=o_all[0], lse=lse, workspace=ws)
        ra.ulysses_permute(o_all, U_N, inverse=True, out=back)

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
    if args.mode == "steps-only":
        print(json.dumps({"mode": "steps-only", "ms_per_step": ms_per_step, "tflops": value}), flush=True)
        return

    # the dominant kernel alone: ring attention on a prebuilt plan
    plan = ra.ra_plan(S, hq, hq, U_D, None, 1, 0, "contiguous", workspace=torch.empty_like(ws))
    attn = time_events(torch, lambda: ra.ra_forward_planned(yq[0], yk[0:1], yv[0:1], plan, out=o_all[0], lse=lse),
                       max(10, args.steps))
    attn_tflops = flops / (attn["avg_ms"] * 1e-3) / 1e12
    alg_bytes = 4 * yq[0].numel() * 2 + lse.numel() * 4  # Q, K, V, O bf16 + LSE fp32
    kernels = {"ring_attn_ulysses_s128k_h8": {
        "avg_ms": attn["avg_ms"], "min_ms": attn["min_ms"], "median_ms": attn["median_ms"], "tflops": attn_tflops,
        "frac_bf16_peak": attn_tflops / PEAK_BF16_TFLOPS, "flops": flops, "visible_pairs_per_head": pairs,
        "algorithmic_bytes": alg_bytes}}
    nbytes = 2 * xq.numel() * 2
    kernels["ulysses_permute_n4_s32k_h32"] = time_hbm(torch, lambda: ra.ulysses_permute(xq, U_N, out=yq),
                                                      args.steps, nbytes)
    kernels["ulysses_permute_inverse_n4_s128k_h8"] = time_hbm(
        torch, lambda: ra.ulysses_permute(o_all, U_N, inverse=True, out=back), args.steps, nbytes)
    log(f"attention kernel {attn['avg_ms']:.3f} ms = {attn_tflops:.1f} TFLOP/s; Ulysses permute "
        f"{kernels['ulysses_permute_n4_s32k_h32']['gbs']:.0f} / inverse "
        f"{kernels['ulysses_permute_inverse_n4_s128k_h8']['gbs']:.0f} GB/s")
    del yq, yk, yv, o_all, back, xq, xk, xv, ws, plan
    torch.cuda.empty_cache()

    if not args.no_extras:
        kernels.update(extras(np, torch, ra, synth, dev, max(10, args.steps), max(5, args.steps // 2)))

    src_sha = kernel_source_sha()
    traffic = traffic_from_profiles(src_sha)
    roofline = {"bound": "mfma", "achieved": attn_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": attn_tflops / PEAK_BF16_TFLOPS, "traffic": traffic,
                "kernel": ATTN_KERNEL, "avg_launch_ms": attn["avg_ms"], "flops_per_launch": flops}

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a row sample")
        cpu = cpu_baseline(np, xs, args.cpu_rows_every)
        log(f"oracle {cpu['value'] * 1e3:.2f} GFLOP/s causal-effective in {cpu['seconds']:.1f} s")

    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": synth.ULYSSES_128K.name, "ulysses_ranks": U_N, "tokens_per_rank": U_SL,
                   "s_total": S, "heads_total": U_H, "heads_per_rank": hq, "head_dim": U_D, "causal": True,
                   "rank": 0,
                   "step": "ulysses_permute(q,k,v) + ra_forward(plan + attention over 131072 tokens, 8 heads, "
                           "bf16 out) + inverse ulysses_permute(o)"},
        "frac_bf16_peak": value / PEAK_BF16_TFLOPS,
        "roofline": roofline, "cpu_baseline": cpu, "kernels": kernels,
    }
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------------------
# Other workloads and kernels
# ---------------------------------------------------------------------------
def mfma_ceiling(torch, ra, reps=5):
    """The register-only bf16 MFMA loop on the whole chip (1024 workgroups, 2 waves per SIMD)."""
    wg, waves, iters = 1024, 8, 20000
    sink = torch.empty(wg * waves * 64, dtype=torch.float32, device="cuda")
    t = time_events(torch, lambda: ra.ra_probe_mfma(iters, wg, waves, sink=sink), reps, warm=1)
    fl = wg * waves * iters * 4 * 32768.0
    return {"avg_ms": t["avg_ms"], "min_ms": t["min_ms"], "flops": fl,
            "tflops": fl / (t["avg_ms"] * 1e-3) / 1e12, "tflops_best": fl / (t["min_ms"] * 1e-3) / 1e12,
            "note": "v_mfma_f32_32x32x16_bf16 from registers, 4 independent accumulators per wave, "
                    f"{wg} workgroups x {waves} waves x {iters} iterations"}


def _randn(torch, gen, dev, *shape):
    return torch.randn(shape, device=dev, dtype=torch.bfloat16, generator=gen)


def _workload_tensors(np, torch, ra, synth, dev, name, gen):
    """Random inputs (drawn on the GPU) of one attention workload: (w, cu, s_local, q_all, k, v)."""
    if name == "llama7b":
        w, cu = synth.LLAMA7B_ZIGZAG, None
    elif name == "gqa":
        w, cu = synth.GQA_STRIPED, None
    else:
        w = synth.PACKED_ZIGZAG
        cu = synth.loguniform_cu_seqlens(0, w.s_total, w.doc_lo, w.doc_hi)
    part = "doc_zigzag" if name == "packed_doc" else w.partition
    sl = ra.ra_local_length(w.s_total, w.cp, part, cu)
    q_all = _randn(torch, gen, dev, w.cp, sl, w.hq, w.d)
    k, v = _randn(torch, gen, dev, w.cp, sl, w.hkv, w.d), _randn(torch, gen, dev, w.cp, sl, w.hkv, w.d)
    return w, part, cu, sl, q_all, k, v


def attn_only(np, torch, ra, synth, dev, workload, rank, launches):
    """A few launches of one workload's attention kernel, for rocprofv3."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    if workload == "ulysses":
        S, hq = U_N * U_SL, U_H // U_N
        q, k, v = (_randn(torch, gen, dev, S, hq, U_D), _randn(torch, gen, dev, 1, S, hq, U_D),
                   _randn(torch, gen, dev, 1, S, hq, U_D))
        plan = ra.ra_plan(S, hq, hq, U_D, None, 1, 0, "contiguous")
        out = torch.empty_like(q)
        for _ in range(launches):
            ra.ra_forward_planned(q, k, v, plan, out=out)
        fl = 4.0 * U_D * hq * visible_pairs(np, "contiguous", S, 1, 0)
    else:
        w, part, cu, sl, q_all, k, v = _workload_tensors(np, torch, ra, synth, dev, workload, gen)
        ranks = range(w.cp) if rank == -1 else [w.rank if rank is None else rank]  # -1: every rank in turn
        fl = 0.0
        for r in ranks:
            if part == "doc_zigzag":
                shape = ra.make_shape(w.s_total, w.hq, w.hkv, w.d, True, 0.0, ra.RA_BF16, ra.RA_BF16)
                ws = torch.empty(ra.ra_workspace_size(shape, w.cp, len(cu) - 1), dtype=torch.uint8, device=dev)
                for _ in range(launches):
                    ra.ra_forward(q_all[r], k, v, cu, w.cp, r, part, workspace=ws)
                # the ranks' shares of the documents' causal work are within a few percent
                fl += 4.0 * w.d * w.hq * visible_pairs(np, "contiguous", w.s_total, 1, 0, cu) / w.cp
            else:
                plan = ra.ra_plan(w.s_total, w.hq, w.hkv, w.d, cu, w.cp, r, part)
                out = torch.empty_like(q_all[r])
                for _ in range(launches):
                    ra.ra_forward_planned(q_all[r], k, v, plan, out=out)
                fl += 4.0 * w.d * w.hq * visible_pairs(np, part, w.s_total, w.cp, r, cu)
        fl /= len(ranks)
    torch.cuda.synchronize()
    print(json.dumps({"mode": "attn-only", "workload": workload, "rank": rank, "launches": launches,
                      "flops_per_launch": fl}), flush=True)


def permute_only(np, torch, ra, synth, dev, which, launches):
    """A few launches of one permute / reorder kernel at its workload size, for rocprofv3."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    if which in ("ulysses_fwd", "ulysses_inv"):
        x = _randn(torch, gen, dev, U_N, U_SL, U_H, U_D)
        y = ra.ulysses_permute(x, U_N)
        if which == "ulysses_fwd":
            fn = lambda: ra.ulysses_permute(x, U_N, out=y)  # noqa: E731
        else:
            fn = lambda: ra.ulysses_permute(y, U_N, inverse=True, out=x)  # noqa: E731
        nbytes = 2 * x.numel() * 2
    elif which == "merge":
        oa = torch.randn((8192, 32, 128), device=dev, generator=gen)
        ob, oo = torch.randn_like(oa), torch.empty_like(oa)
        la, lb = torch.randn((32, 8192), device=dev, generator=gen), torch.randn((32, 8192), device=dev, generator=gen)
        lo = torch.empty_like(la)
        fn = lambda: ra.ra_lse_merge(oa, la, ob, lb, o_out=oo, lse_out=lo)  # noqa: E731
        nbytes = 3 * oa.numel() * 4 + 3 * la.numel() * 4
    elif which == "reorder_docs":
        w = synth.PACKED_ZIGZAG
        cu = synth.loguniform_cu_seqlens(0, w.s_total, w.doc_lo, w.doc_hi)
        x = _randn(torch, gen, dev, w.s_total, w.hq, w.d)
        sld = ra.ra_local_length(w.s_total, w.cp, "doc_zigzag", cu)
        y = torch.empty((w.cp, sld, w.hq, w.d), dtype=torch.bfloat16, device=dev)
        fn = lambda: ra.cp_reorder_docs(x, w.cp, cu, out=y)  # noqa: E731
        nbytes = (w.s_total + w.cp * sld) * w.hq * w.d * 2
    else:
        w, h = {"reorder_llama7b": (synth.LLAMA7B_ZIGZAG, 32), "reorder_gqa_q": (synth.GQA_STRIPED, 32),
                "reorder_gqa_kv": (synth.GQA_STRIPED, 8), "reorder_packed": (synth.PACKED_ZIGZAG, 32)}[which]
        x = _randn(torch, gen, dev, w.s_total, h, w.d)
        y = torch.empty((w.cp, w.s_total // w.cp, h, w.d), dtype=torch.bfloat16, device=dev)
        fn = lambda: ra.cp_reorder(x, w.cp, w.partition, out=y)  # noqa: E731
        nbytes = 2 * x.numel() * 2
    for _ in range(launches):
        fn()
    torch.cuda.synchronize()
    print(json.dumps({"mode": "permute-only", "which": which, "launches": launches, "bytes_per_launch": nbytes}),
          flush=True)


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


def bwd_only(np, torch, ra, synth, dev, launches):
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    w, part, cu, sl, q_all, k, v = _workload_tensors(np, torch, ra, synth, dev, "llama7b", gen)
    out, lse = ra.ra_forward(q_all[w.rank], k, v, None, w.cp, w.rank, w.partition)
    bw = backward_buffers(torch, ra, w, dev)
    for _ in range(launches):
        run_backward(ra, w, q_all[w.rank], k, v, out, lse, bw)
    torch.cuda.synchronize()
    fl = 2.5 * 4.0 * w.d * w.hq * visible_pairs(np, w.partition, w.s_total, w.cp, w.rank)
    print(json.dumps({"mode": "bwd-only", "launches": launches, "flops_per_launch": fl}), flush=True)


def extras(np, torch, ra, synth, dev, reps, reps_long):
    """Per-kernel figures for the other workloads (inputs drawn on the GPU with a seeded generator)."""
    res = {}
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)

    # Llama-2-7B-shaped zigzag share: the whole step (3 reorders + ra_forward) and the kernel alone
    log("extras: Llama-2-7B-shaped zigzag share")
    w = synth.LLAMA7B_ZIGZAG
    S, cp, rank = w.s_total, w.cp, w.rank
    sl = S // cp
    q_g, k_g, v_g = (_randn(torch, gen, dev, S, w.hq, w.d) for _ in range(3))
    q_p = torch.empty((cp, sl, w.hq, w.d), dtype=torch.bfloat16, device=dev)
    k_p, v_p = torch.empty_like(q_p), torch.empty_like(q_p)
    out = torch.empty((sl, w.hq, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.hq, sl), dtype=torch.float32, device=dev)
    shape = ra.make_shape(S, w.hq, w.hkv, w.d, True, 0.0, ra.RA_BF16, ra.RA_BF16)
    ws = torch.empty(ra.ra_workspace_size(shape, cp, 0), dtype=torch.uint8, device=dev)
    fl = 4.0 * w.d * w.hq * visible_pairs(np, w.partition, S, cp, rank)

    def step():
        ra.cp_reorder(q_g, cp, w.partition, out=q_p)
        ra.cp_reorder(k_g, cp, w.partition, out=k_p)
        ra.cp_reorder(v_g, cp, w.partition, out=v_p)
        ra.ra_forward(q_p[rank], k_p, v_p, None, cp, rank, w.partition, out=out, lse=lse, workspace=ws)

    ts = time_events(torch, step, reps)
    plan = ra.ra_plan(S, w.hq, w.hkv, w.d, None, cp, rank, w.partition)
    ta = time_events(torch, lambda: ra.ra_forward_planned(q_p[rank], k_p, v_p, plan, out=out, lse=lse), reps)
    res["llama7b_zigzag_step"] = {"avg_ms": ts["avg_ms"], "tflops": fl / (ts["avg_ms"] * 1e-3) / 1e12,
                                  "step": "cp_reorder(q,k,v) + ra_forward (plan + attention), bf16 out"}
    res["ring_attn_llama7b_zigzag_rank0"] = {"avg_ms": ta["avg_ms"], "min_ms": ta["min_ms"], "flops": fl,
                                             "tflops": fl / (ta["avg_ms"] * 1e-3) / 1e12,
                                             "frac_bf16_peak": fl / (ta["avg_ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    nbytes = 2 * k_g.numel() * 2
    res["cp_reorder_s32k_h32_zigzag"] = time_hbm(
        torch, [lambda: ra.cp_reorder(k_g, cp, w.partition, out=k_p)] +
        [reorder_call(torch, ra, k_g, cp, w.partition) for _ in range(rotating_sets(nbytes) - 1)], reps, nbytes)

    # backward of the same share: dQ, and this rank's dK / dV partials of every chunk
    log("extras: backward of the zigzag share")
    bw = backward_buffers(torch, ra, w, dev)
    tb = time_events(torch, lambda: run_backward(ra, w, q_p[rank], k_p, v_p, out, lse, bw), reps_long)
    bfl = 2.5 * fl
    res["ring_attn_backward_llama7b_zigzag_rank0"] = {
        "avg_ms": tb["avg_ms"], "min_ms": tb["min_ms"], "flops": bfl,
        "tflops": bfl / (tb["avg_ms"] * 1e-3) / 1e12,
        "frac_bf16_peak": bfl / (tb["avg_ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "mfma_tflops_executed": 3.5 * fl / (tb["avg_ms"] * 1e-3) / 1e12,
        "note": "whole ra_backward call (plans, D = dO.O, dQ kernel, dK/dV kernel); FLOPs = 2.5 x forward"}
    del bw, q_g, k_g, v_g, q_p, k_p, v_p, out, lse, ws, plan

    # GQA striped: 32 q heads / 8 kv heads, S=65536, CP=8, rank 0, and its Q / K reorders
    log("extras: GQA striped")
    w = synth.GQA_STRIPED
    slg = w.s_total // w.cp
    q = _randn(torch, gen, dev, slg, w.hq, w.d)
    k, v = _randn(torch, gen, dev, w.cp, slg, w.hkv, w.d), _randn(torch, gen, dev, w.cp, slg, w.hkv, w.d)
    plan = ra.ra_plan(w.s_total, w.hq, w.hkv, w.d, None, w.cp, 0, w.partition)
    tg = time_events(torch, lambda: ra.ra_forward_planned(q, k, v, plan), reps)
    fl = 4.0 * w.d * w.hq * visible_pairs(np, w.partition, w.s_total, w.cp, 0)
    res["ring_attn_gqa_striped_rank0"] = {"avg_ms": tg["avg_ms"], "flops": fl,
                                          "tflops": fl / (tg["avg_ms"] * 1e-3) / 1e12}
    for h, tag in ((w.hq, "q"), (w.hkv, "kv")):
        x = _randn(torch, gen, dev, w.s_total, h, w.d)
        y = torch.empty((w.cp, slg, h, w.d), dtype=torch.bfloat16, device=dev)
        nbytes = 2 * x.numel() * 2
        res[f"cp_reorder_s64k_h{h}_striped_{tag}"] = time_hbm(
            torch, [lambda: ra.cp_reorder(x, w.cp, w.partition, out=y)] +
            [reorder_call(torch, ra, x, w.cp, w.partition) for _ in range(rotating_sets(nbytes) - 1)], reps, nbytes)
        del x, y
    del q, k, v

    # packed documents: 131072 tokens, log-uniform documents, CP=8 zigzag, every rank
    log("extras: packed documents, global zigzag")
    w = synth.PACKED_ZIGZAG
    cu = synth.loguniform_cu_seqlens(0, w.s_total, w.doc_lo, w.doc_hi)
    slp = w.s_total // w.cp
    q_all = _randn(torch, gen, dev, w.cp, slp, w.hq, w.d)
    k, v = _randn(torch, gen, dev, w.cp, slp, w.hkv, w.d), _randn(torch, gen, dev, w.cp, slp, w.hkv, w.d)
    per_rank = []
    for r in range(w.cp):
        plan = ra.ra_plan(w.s_total, w.hq, w.hkv, w.d, cu, w.cp, r, w.partition)
        tr = time_events(torch, lambda: ra.ra_forward_planned(q_all[r], k, v, plan), reps_long)
        fl = 4.0 * w.d * w.hq * visible_pairs(np, w.partition, w.s_total, w.cp, r, cu)
        per_rank.append({"rank": r, "avg_ms": tr["avg_ms"], "flops": fl,
                         "tflops": fl / (tr["avg_ms"] * 1e-3) / 1e12})
    heavy = max(per_rank, key=lambda x: x["flops"])
    total_fl = 4.0 * w.d * w.hq * visible_pairs(np, "contiguous", w.s_total, 1, 0, cu)
    sum_ms = sum(x["avg_ms"] for x in per_rank)
    res["ring_attn_packed_docs_zigzag"] = {"n_docs": len(cu) - 1, "max_work_rank": heavy, "ranks": per_rank,
                                           "sum_ms_all_ranks": sum_ms,
                                           "tflops_all_ranks": total_fl / (sum_ms * 1e-3) / 1e12}
    x = _randn(torch, gen, dev, w.s_total, w.hq, w.d)
    y = torch.empty((w.cp, slp, w.hq, w.d), dtype=torch.bfloat16, device=dev)
    nbytes = 2 * x.numel() * 2
    res["cp_reorder_s128k_h32_zigzag"] = time_hbm(torch, lambda: ra.cp_reorder(x, w.cp, w.partition, out=y), reps,
                                                  nbytes)
    del q_all, k, v, x, y

    # the same documents under per-document zigzag: every rank holds two pieces of every
    # document, so the ranks' work is even
    log("extras: packed documents, per-document zigzag")
    sld = ra.ra_local_length(w.s_total, w.cp, "doc_zigzag", cu)
    q_all = _randn(torch, gen, dev, w.cp, sld, w.hq, w.d)
    k, v = _randn(torch, gen, dev, w.cp, sld, w.hkv, w.d), _randn(torch, gen, dev, w.cp, sld, w.hkv, w.d)
    dshape = ra.make_shape(w.s_total, w.hq, w.hkv, w.d, True, 0.0, ra.RA_BF16, ra.RA_BF16)
    dws = torch.empty(ra.ra_workspace_size(dshape, w.cp, len(cu) - 1), dtype=torch.uint8, device=dev)
    dout = torch.empty((sld, w.hq, w.d), dtype=torch.bfloat16, device=dev)
    dlse = torch.empty((w.hq, sld), dtype=torch.float32, device=dev)
    per_rank_d = []
    for r in range(w.cp):
        # on a prebuilt plan, as the global zigzag ranks above; and ra_forward with its plan
        plan = ra.ra_plan(w.s_total, w.hq, w.hkv, w.d, cu, w.cp, r, "doc_zigzag")
        tr = time_events(torch, lambda: ra.ra_forward_planned(q_all[r], k, v, plan, out=dout, lse=dlse), reps_long)
        tp = time_events(torch, lambda: ra.ra_forward(q_all[r], k, v, cu, w.cp, r, "doc_zigzag", out=dout, lse=dlse,
                                                      workspace=dws), reps_long)
        per_rank_d.append({"rank": r, "avg_ms": tr["avg_ms"], "avg_ms_with_plan": tp["avg_ms"]})
        del plan
    slowest = max(per_rank_d, key=lambda x: x["avg_ms"])
    sum_d = sum(x["avg_ms"] for x in per_rank_d)
    sum_dp = sum(x["avg_ms_with_plan"] for x in per_rank_d)
    res["ring_attn_packed_docs_doc_zigzag"] = {
        "n_docs": len(cu) - 1, "s_local": sld, "s_local_unpadded": slp, "slowest_rank": slowest, "ranks": per_rank_d,
        "slowest_rank_speedup_vs_global_zigzag": max(x["avg_ms"] for x in per_rank) / slowest["avg_ms"],
        "sum_ms_all_ranks": sum_d, "sum_ratio_vs_global_zigzag": sum_d / sum_ms,
        "tflops_all_ranks": total_fl / (sum_d * 1e-3) / 1e12,
        "sum_ms_all_ranks_with_plan": sum_dp, "sum_ratio_vs_global_zigzag_with_plan": sum_dp / sum_ms,
        "note": "avg_ms: ra_forward_planned on a prebuilt plan per rank (as the global zigzag ranks); "
                "avg_ms_with_plan: ra_forward per rank (plan included)"}
    del q_all, k, v, dws, dout, dlse
    # the per-document zigzag reorder of a global [131072, 32, 128] tensor into the 8
    # ranks' padded shares (padding slots are written as zeros, so they count as bytes)
    xg = _randn(torch, gen, dev, w.s_total, w.hq, w.d)
    row_bytes = w.hq * w.d * 2
    nbytes = (w.s_total + w.cp * sld) * row_bytes

    def docs_call():
        x, y = xg.clone(), torch.empty((w.cp, sld, w.hq, w.d), dtype=torch.bfloat16, device=dev)
        return lambda: ra.cp_reorder_docs(x, w.cp, cu, out=y)

    res["cp_reorder_docs_s128k_h32"] = time_hbm(
        torch, [docs_call() for _ in range(rotating_sets(nbytes))], reps, nbytes)
    del xg

    # Ulysses x Ring hybrid: a 4 x 2 grid (Ulysses 4 inside, zigzag ring of 2 across), S=131072,
    # 32 heads; the whole grid's work on one GPU (all 8 devices' permutes and attention)
    log("extras: Ulysses x Ring grid")
    U, R, S, H, d = 4, 2, 131072, 32, 128
    sh = S // (U * R)
    gq, gk, gvv = (_randn(torch, gen, dev, R, U, sh, H, d) for _ in range(3))
    ushape = ra.make_shape(S, H, H, d, True, 0.0, ra.RA_BF16, ra.RA_BF16)
    uws = torch.empty(ra.usp_workspace_size(ushape, U, R, 0), dtype=torch.uint8, device=dev)
    uout = torch.empty_like(gq)
    ulse = torch.empty((U, R, H // U, S // R), dtype=torch.float32, device=dev)
    tu = time_events(torch, lambda: ra.usp_forward(gq, gk, gvv, None, U, R, "zigzag", out=uout, lse=ulse,
                                                   workspace=uws), max(3, reps_long // 2))
    fl = 4.0 * d * H * visible_pairs(np, "contiguous", S, 1, 0)
    res["usp_grid_u4_r2_s128k_h32"] = {"avg_ms": tu["avg_ms"], "flops": fl,
                                       "tflops": fl / (tu["avg_ms"] * 1e-3) / 1e12,
                                       "per_device_ms": tu["avg_ms"] / (U * R),
                                       "note": "whole grid: 3 x R strided Ulysses permutes, U x R ring attentions "
                                               "(R steps each), R inverse permutes"}
    del gq, gk, gvv, uws, uout, ulse

    # fp32 LSE merge of two [8192, 32, 128] partials (HBM-bound)
    rows, h, dd = 8192, 32, 128
    oa = torch.randn((rows, h, dd), device=dev, generator=gen)
    ob, la, lb = torch.randn_like(oa), torch.randn((h, rows), device=dev), torch.randn((h, rows), device=dev)
    oo, lo = torch.empty_like(oa), torch.empty_like(la)
    nbytes = 3 * oa.numel() * 4 + 3 * la.numel() * 4

    def merge_call():
        a, b, o = torch.randn_like(oa), torch.randn_like(oa), torch.empty_like(oa)
        sa, sb, so = torch.randn_like(la), torch.randn_like(la), torch.empty_like(la)
        return lambda: ra.ra_lse_merge(a, sa, b, sb, o_out=o, lse_out=so)

    res["lse_merge_8192x32x128_f32"] = time_hbm(
        torch, [lambda: ra.ra_lse_merge(oa, la, ob, lb, o_out=oo, lse_out=lo)] +
        [merge_call() for _ in range(rotating_sets(nbytes) - 1)], reps, nbytes)
    del oa, ob, la, lb, oo, lo

    # measured ceilings: torch's device-to-device copy of 1 GiB, and the register-only MFMA loop
    src = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    nbytes = 2 * src.numel() * 2
    res["ceiling_torch_copy_1GiB"] = time_hbm(torch, lambda: dst.copy_(src), reps, nbytes)
    del src, dst
    res["ceiling_mfma_bf16_loop"] = mfma_ceiling(torch, ra)
    log(f"ceilings: copy {res['ceiling_torch_copy_1GiB']['gbs']:.0f} GB/s, "
        f"MFMA loop {res['ceiling_mfma_bf16_loop']['tflops']:.0f} TFLOP/s")
    return res


if __name__ == "__main__":
    main()
