"""bench.py command line: one GPU only (the ring is simulated on one device)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "--gpus 2" in (r.stdout + r.stderr) and "one GPU" in (r.stdout + r.stderr)
    assert r.stdout.strip() == "" or not r.stdout.strip().startswith("{")


def test_bench_flop_count_matches_the_oracle_visible_pairs():
    """bench.py counts causal-effective FLOPs from its own visible-pair count; it must
    equal the oracle's (itself pinned by brute force and the closed forms) for every
    partition, with and without packed documents, at the workloads' sizes."""
    import numpy as np

    import bench
    import oracle
    import synth

    cu5 = synth.loguniform_cu_seqlens(0, 131072, 512, 32768)
    cases = [("zigzag", 32768, 4, None), ("striped", 65536, 8, None), ("contiguous", 131072, 1, None),
             ("zigzag", 131072, 8, cu5), ("striped", 4096, 8, [0, 5, 1000, 4096]),
             ("contiguous", 4096, 4, [0, 1, 2, 3000, 4096])]
    for part, S, cp, cu in cases:
        for r in range(cp):
            pos = oracle.positions(part, S, cp, r)
            want = int(oracle.visible_counts(pos, cu, S, True).sum())
            assert bench.visible_pairs(np, part, S, cp, r, cu) == want, (part, S, cp, r)
    # and against brute force on a small packed case
    S, cp, cu = 256, 4, [0, 17, 100, 256]
    for part in ("zigzag", "striped", "contiguous"):
        for r in range(cp):
            pos = oracle.positions(part, S, cp, r)
            vis = oracle.visible_matrix(pos, np.arange(S), cu, S, True)
            assert bench.visible_pairs(np, part, S, cp, r, cu) == int(vis.sum())
