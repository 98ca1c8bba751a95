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


def _bench_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_kernel_stats_order_statistics():
    b = _bench_module()
    ks = b.kernel_stats([5.0, 1.0, 3.0, 2.0, 4.0])
    assert ks["median"] == 3.0 and ks["min"] == 1.0 and ks["mean"] == 3.0 and ks["n"] == 5
    assert 4.0 <= ks["p90"] <= 5.0


def test_valu_floor_scales_with_the_mix():
    # the ALU ceiling is linear in the work: twice the tokens, twice the time; a mix with
    # no transcendentals per (t, d, n) costs less than one with them
    b = _bench_module()
    t1 = b.valu_floor_s(1 << 20, 16, b.FWD_MIX["general"])
    assert abs(b.valu_floor_s(2 << 20, 16, b.FWD_MIX["general"]) - 2 * t1) < 1e-15
    assert b.valu_floor_s(1 << 20, 16, b.FWD_MIX["structured"]) < t1
    # one exp and four VOP2 per (t, d, n) at 8.1 and 2.3 cycles dominate the 2.8B layer:
    # 41,943,040 token-channels take between 80 and 100 us on 1024 SIMDs at 2.4 GHz
    t = b.valu_floor_s(4 * 2048 * 5120, 16, b.FWD_MIX["general"])
    assert 80e-6 < t < 100e-6
