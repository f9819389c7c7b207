"""bench.py's host-side contract checks that need no GPU."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""                     # no JSON line for a run that did not happen


def test_committed_traffic_record_is_well_formed():
    with open(os.path.join(ROOT, "profiles", "traffic_route_100M.json")) as f:
        tr = json.load(f)
    for key in ("bytes_per_launch", "algorithmic_bytes_per_launch", "source_hash"):
        assert key in tr
    # measured HBM traffic of one scan launch against its algorithmic bytes: no large re-reads
    assert 1.0 <= tr["bytes_per_launch"] / tr["algorithmic_bytes_per_launch"] < 1.1
