"""The benchmark's command line on a host without a GPU: it measures one GPU only and
says so for any other count before it touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2, (r.returncode, r.stderr[-2000:])
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line for a count it does not measure


def test_bench_lists_its_legs():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0
    for leg in ("configs", "sweep", "delta", "tree", "sampling", "adaptive"):
        assert leg in r.stdout
