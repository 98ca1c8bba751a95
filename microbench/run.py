"""Hardware probes behind the figures in the design doc (section 4.1): HBM copy bandwidth,
FP32 VALU and v_exp_f32 issue rates by instruction form, single-wave issue latency, LDS
bandwidth, and the scan's exact global access pattern without compute.

    python microbench/run.py            # build (hipcc, gfx950) and run every probe
    python microbench/run.py --build-only

Each probe is a standalone HIP program; bounds are fixed in the sources.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PROBES = ["copy_and_alu", "issue_latency", "valu_forms", "dual_issue", "lds_bandwidth",
          "scan_access_pattern", "core_mix"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def main():
    out_dir = os.path.join(HERE, "_bin")
    os.makedirs(out_dir, exist_ok=True)
    for p in PROBES:
        exe = os.path.join(out_dir, p)
        subprocess.run(["hipcc", *FLAGS, os.path.join(HERE, p + ".hip"), "-o", exe], check=True,
                       stderr=subprocess.DEVNULL)
    if "--build-only" in sys.argv:
        return
    for p in PROBES:
        print(f"== {p}", flush=True)
        subprocess.run(["timeout", "-k", "10", "120", os.path.join(out_dir, p)], check=True)


if __name__ == "__main__":
    main()
