"""The whole HIP path (plan, absorb, paged decode, combine, up-projection)
against the CPU oracle on the same seeded inputs.

Small cases compare every output element; the four full-size workloads are
run in the launch configuration the benchmark times and compared on sampled
sequences and heads that the oracle computes one by one.
"""
import numpy as np
import pytest

from gpu_path import DevInputs, compare, host, run_path, say
from mla_inputs import make_inputs
from oracle import mla_oracle as O

pytestmark = pytest.mark.gpu


def _check_all(mla, inp, **kw):
    res = host(run_path(mla, DevInputs(inp), **kw))
    ref = O.decode_naive_inputs(inp)
    stats = compare(res, ref, list(range(inp.b)), list(range(inp.h)), label=f"{inp.name} {kw}")
    assert mla.take_device_error() == 0
    return res, stats


def test_tiny_config(gpu_lib):
    _check_all(gpu_lib, make_inputs("tiny", seed=0))


def test_tiny_config_poisoned(gpu_lib):
    """NaN page tails and NaN trap pages behind unused block-table entries never leak."""
    _check_all(gpu_lib, make_inputs("tiny", seed=0, trap=True))


@pytest.mark.parametrize("seqlens,s_q,h,causal", [
    ([1, 2, 63, 64, 65, 127, 128, 129], 1, 16, False),
    ([1, 2, 3, 64, 65, 200], 2, 16, True),        # causal rows with 0 .. L - 1 keys
    ([0, 7, 0, 100], 1, 32, False),                # empty sequences
    ([300, 1500, 2100], 3, 16, True),              # 48 rows: two-wave workgroups
    ([130, 1100, 1030], 1, 64, False),
    ([1025, 1024, 5], 2, 64, True),
    ([700, 90], 4, 32, True),                      # 128 rows
    ([333, 2000], 4, 128, True),                   # 512 rows: four row blocks
    ([8, 100, 1031], 8, 128, True),                # 1024 rows: eight row blocks, the longest draft
    ([9, 64, 700], 8, 16, True),                   # 128 rows of 8 query tokens
])
def test_edge_shapes(gpu_lib, seqlens, s_q, h, causal):
    inp = make_inputs("tiny", seed=5, seqlens=seqlens, s_q=s_q, h=h, causal=causal, trap=True)
    say("edge", seqlens, "s_q", s_q, "h", h, "causal", causal)
    _check_all(gpu_lib, inp)


@pytest.mark.parametrize("slots", [1, 3, 7, 64, 1000])
def test_forced_split_counts(gpu_lib, slots):
    """From one workgroup for everything to one page per split."""
    inp = make_inputs("tiny", seed=6, seqlens=[1, 640, 64, 3000, 77], h=32, trap=True)
    say("slots", slots)
    res, _ = _check_all(gpu_lib, inp, slots=slots)


@pytest.mark.parametrize("b", [84, 86])
def test_combine_layout_switch(gpu_lib, b):
    """With 256 slots the plan cuts b sequences into at most b + 255 pieces: 84 sequences average
    more than four (the combine merges one row per wave) and 86 do not (four rows per wave). Both
    sides of the switch, with empty and poisoned sequences, every element against the oracle."""
    rng = np.random.default_rng(30 + b)
    seqlens = rng.integers(1, 200, b)
    seqlens[[3, b - 1]] = 0
    inp = make_inputs("tiny", seed=30 + b, seqlens=seqlens.tolist(), h=16, trap=True)
    say("combine layout switch: b", b, "slots 256")
    _check_all(gpu_lib, inp, slots=256)


def test_without_lo_plane_long_rows(gpu_lib):
    """On long caches with spread-out attention bf16 q_lat alone meets the bar."""
    inp = make_inputs("full_heads", seed=8, seqlens=[1100, 2500, 4096, 3000])
    _check_all(gpu_lib, inp, lo=False)


FULL = {
    # config: (sampled sequences, sampled heads)
    "tp_share": ([0, 17, 64, 127], [0, 13, 31]),
    "full_heads": ([0, 5, 42, 77, 127], [0, 64, 127]),
    "long_context": (None, [0, 100]),
    "multi_token": ([0, 63, 127], [0, 127]),
    "spec_verify": ([0, 17, 31], [0, 77, 127]),
}


@pytest.mark.parametrize("cfg", list(FULL))
def test_full_size_sampled(gpu_lib, cfg):
    inp = make_inputs(cfg, seed=0)
    seqs, heads = FULL[cfg]
    if seqs is None:  # long context: the shortest, the longest and a middle one
        order = np.argsort(inp.seqlens)
        seqs = sorted({int(order[0]), int(order[len(order) // 2]), int(order[-1])})
    say("full", cfg, "b", inp.b, "h", inp.h, "s_q", inp.s_q, "sum L", int(inp.seqlens.sum()), "seqs", seqs)
    res = host(run_path(gpu_lib, DevInputs(inp)))
    ref = O.decode_naive_inputs(inp, seqs=seqs, heads=heads)
    compare(res, ref, seqs, heads, label=cfg)
    assert np.isfinite(res["o_lat"]).all() and np.isfinite(res["lse"]).all()
    assert gpu_lib.take_device_error() == 0


@pytest.mark.parametrize("h", [16, 128])
def test_maximum_batch(gpu_lib, h):
    """b = MLA_MAX_BATCH (8192) short sequences, some empty: row and page offsets at the far end of
    every tensor, and 64 row blocks in the projections. Sampled sequences include both ends."""
    rng = np.random.default_rng(21)
    seqlens = rng.integers(0, 151, 8192)
    seqlens[[1, 4097, 8190]] = 0
    inp = make_inputs("tiny", seed=21, seqlens=seqlens.tolist(), h=h)
    seqs = sorted({0, 1, 2, 4096, 4097, 8189, 8190, 8191} | set(rng.integers(0, 8192, 4).tolist()))
    heads = [0, h // 2 + 1, h - 1]
    say("max batch h", h, "sum L", int(inp.seqlens.sum()), "seqs", seqs)
    res = host(run_path(gpu_lib, DevInputs(inp)))
    ref = O.decode_naive_inputs(inp, seqs=seqs, heads=heads)
    compare(res, ref, seqs, heads, label=f"max batch h={h}")
    empty = inp.seqlens <= 0
    assert (res["lse"][empty] == -np.inf).all() and not res["o_lat"][empty].any()
    assert gpu_lib.take_device_error() == 0
