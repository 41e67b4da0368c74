"""bench.py's command line without a GPU: more than one GPU is refused with
a message, and the counter traffic is reported only for the kernels and the
workload variant it was measured on."""
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_committed_counters_match_the_kernels_they_describe():
    digest = bench.kernel_source_digest()
    for w in ("7b", "70b", "long", "shared", "mixed"):
        with open(os.path.join(ROOT, "profiles", "traffic_%s_ps-1.json" % w)) as f:
            t = json.load(f)
        if t["kernel_source_digest"] != digest:
            # The bench then reports no traffic (null) until they are re-taken.
            assert bench.counter_traffic(w, -1) is None
            pytest.skip("counters for %s predate the current kernels" % w)
        assert bench.counter_traffic(w, -1) == t["hbm_bytes_per_launch"]
        # HBM bytes within a few percent of the algorithmic bytes (no re-reads),
        # except the shared prefix, whose blocks are read once per row block.
        assert 1.0 <= t["traffic_over_algorithmic"] < (1.3 if w == "shared" else 1.03), w
    assert bench.counter_traffic("7b", 0) is None       # never profiled: fixed partitions off
