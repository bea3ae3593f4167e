"""Seeded sweep over valid shapes: every output element of the HIP path against
the CPU oracle (indexing through poisoned pages and tails, ragged and empty
sequences, causal and not, planner slot counts from 1 to many)."""
import numpy as np
import pytest

from gpu_path import DevInputs, compare, host, run_path, say
from mla_inputs import make_inputs
from oracle import mla_oracle as O

pytestmark = pytest.mark.gpu


def _case(k: int):
    rng = np.random.default_rng(1000 + k)
    h = int(rng.choice([16, 32, 64, 128]))
    s_q = int(rng.integers(1, 5))
    b = int(rng.integers(1, 6))
    L = rng.integers(0, 1500, size=b)
    L[rng.random(b) < 0.15] = 0               # some empty sequences
    L[rng.random(b) < 0.25] = rng.integers(1, 70)  # some short ones around a page
    causal = bool(rng.random() < 0.5)
    slots = [None, 1, 7, 64, 300][int(rng.integers(0, 5))]
    return dict(seqlens=[int(x) for x in L], s_q=s_q, h=h, causal=causal), slots


@pytest.mark.parametrize("k", range(16))
def test_random_shape(gpu_lib, k):
    kw, slots = _case(k)
    inp = make_inputs("tiny", seed=2000 + k, trap=True, **kw)
    say("random case", k, kw, "slots", slots)
    res = host(run_path(gpu_lib, DevInputs(inp), slots=slots))
    ref = O.decode_naive_inputs(inp)
    compare(res, ref, list(range(inp.b)), list(range(inp.h)), label=f"random {k}")
    assert gpu_lib.take_device_error() == 0
