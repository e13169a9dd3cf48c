"""bench.py's command-line contract, checked on the CPU: a run on more than one
GPU is refused with one JSON line and exit status 2 before anything touches a
device, and the committed LM-head traffic summary parses to a figure at or
above the kernel's algorithmic bytes (or to None once its sources changed)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_several_gpus_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "error" in line


def test_traffic_summary_parses():
    sys.path.insert(0, ROOT)
    import bench
    t = bench.measured_traffic()
    algorithmic = 151936 * 4096 * 2 + 15 * 4096 * 2 + 15 * 8
    assert t is None or algorithmic <= t <= 1.05 * algorithmic
