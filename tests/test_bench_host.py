"""Host-side logic of bench.py, without a GPU: the one-GPU refusal and the
validity rule of the committed HBM counter record."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_counter_record_is_used_only_for_the_sources_it_was_taken_on():
    # traffic comes from the committed record while the headline kernel's sources hash to the
    # recorded value, and is null (None) otherwise or for another kernel
    with open(os.path.join(ROOT, "profiles", "counters_square_bf16.json")) as f:
        rec = json.load(f)
    want = rec["bytes_per_launch"] if rec["source_hash"] == bench.kernel_source_hash() else None
    assert bench.traffic_for(rec["kernel"]) == want
    assert bench.traffic_for("some_other_kernel") is None
    assert len(bench.kernel_source_hash()) == 16
