"""bench.py's command line on the CPU: more than one GPU is refused with a
message (this build runs on one GPU), before any GPU library is touched."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"] and msg["n_gpus_requested"] == 2


def test_traffic_summary_lookup():
    sys.path.insert(0, ROOT)
    import bench

    # a kernel the summary does not list has no traffic figure
    assert bench.read_traffic_summary("no_such_kernel") is None
