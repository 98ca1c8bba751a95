"""bench.py's command line on a machine without a GPU: only the single-GPU run is
built, so any other GPU count ends at once with a message (nothing touches a GPU)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_unknown_workload_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "nope"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "invalid choice" in r.stderr
