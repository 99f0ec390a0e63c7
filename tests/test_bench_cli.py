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
