"""Host-side parts of bench.py that need no GPU: the one-GPU refusal and the traffic records."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (imports no GPU module at import time)


@pytest.mark.parametrize("n", [0, 2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("config", ["full_heads", "tp_share"])
def test_traffic_record_matches_the_kernel_sources(config):
    """The counter record under profiles/ was taken from the current decode sources: when a kernel
    source changes, the counters must be taken again (bench.py then reports null, not a stale value)."""
    got = bench.recorded_traffic(config)
    assert isinstance(got, int) and got > 0, f"profiles/mla_decode_{config}.md: record missing or stale"


def test_traffic_record_absent_for_unprofiled_workload():
    assert bench.recorded_traffic("no_such_workload") is None
