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


def _work(b, s_q, h, seqlens, causal):
    import types

    import numpy as np
    inp = types.SimpleNamespace(b=b, s_q=s_q, h=h, causal=causal, seqlens=np.asarray(seqlens, dtype=np.int32))
    return bench.algorithmic_work(inp)


@pytest.mark.parametrize("b,s_q,h,L,causal,bound", [
    (128, 1, 32, 512, False, "hbm"),     # one tensor-parallel share of the heads
    (128, 1, 128, 2176, False, "hbm"),   # all heads, the mean length of the uniform 256..4096 draw
    (128, 2, 128, 4096, True, "mfma"),   # two causal query tokens
    (32, 8, 128, 2280, True, "mfma"),    # eight-token speculative verify
])
def test_roofline_bound_follows_arithmetic_intensity(b, s_q, h, L, causal, bound):
    """The decode call is priced against HBM below the chip's balance point (2.5 PF/s / 8 TB/s, about
    312 flop per byte) and against the bf16 matrix peak above it; achieved/peak/unit follow the bound."""
    work = _work(b, s_q, h, [L] * b, causal)
    assert bench.roofline_bound(work) == bound
    r = bench.roofline_entry(work, 1e-4, None)
    assert r["bound"] == bound and r["unit"] == ("TFLOP/s" if bound == "mfma" else "GB/s")
    expect = work["flops"] / 1e-4 / 1e12 if bound == "mfma" else work["bytes"] / 1e-4 / 1e9
    assert abs(r["achieved"] - expect) <= 0.05 and abs(r["frac"] - expect / r["peak"]) <= 1e-4
