"""The whole step captured in a HIP graph (through torch's graph capture on the
library's stream) replays to exactly the eager result, replay after replay,
with other eager work and synchronisations between the replays.
"""
import numpy as np
import pytest
import torch

from gpu_path import DevInputs, say
from mla_inputs import make_inputs

pytestmark = pytest.mark.gpu


def _alloc(inp):
    shape = (inp.b, inp.s_q, inp.h)
    bf = dict(dtype=torch.bfloat16, device="cuda")
    return dict(q_lat=torch.empty(shape + (512,), **bf), q_lo=torch.empty(shape + (512,), **bf),
                o_lat=torch.empty(shape + (512,), **bf), o=torch.empty(shape + (128,), **bf),
                lse=torch.empty(shape, dtype=torch.float32, device="cuda"))


def _step(mla, d, bufs, ws, slots):
    inp = d.inp
    meta, ns = mla.get_metadata(d.sl, slots, s_q=inp.s_q, h=inp.h)
    mla.absorb_q(d.q_nope, d.w_uk, out=(bufs["q_lat"], bufs["q_lo"]))
    mla.decode_paged(bufs["q_lat"], d.q_pe, d.kv, d.bt, d.sl, meta, ns, inp.scale, inp.causal,
                     q_lat_lo=bufs["q_lo"], workspace=ws, out=(bufs["o_lat"], bufs["lse"]))
    mla.up_v(bufs["o_lat"], d.w_uv, out=bufs["o"])


def _bits(bufs):
    return {k: bufs[k].view(torch.int32 if bufs[k].dtype == torch.float32 else torch.int16).cpu().numpy().copy()
            for k in ("q_lat", "o_lat", "lse", "o")}


@pytest.mark.parametrize("cfg,kw", [
    ("tiny", dict(trap=True)),
    ("tiny", dict(seqlens=[3000, 64, 700, 1], h=128, trap=True)),            # split pieces and the combine
    ("tiny", dict(seqlens=[600, 900, 65], s_q=2, h=32, causal=True)),         # the token-split kernel
])
def test_graph_replays_match_eager(gpu_lib, cfg, kw):
    mla = gpu_lib
    inp = make_inputs(cfg, seed=15, **kw)
    d = DevInputs(inp)
    slots = mla.num_slots(inp.b, inp.s_q, inp.h)
    ws = torch.empty((mla.workspace_bytes(inp.b, inp.s_q, inp.h, slots),), dtype=torch.uint8, device="cuda")
    bufs = _alloc(inp)
    _step(mla, d, bufs, ws, slots)
    torch.cuda.synchronize()
    want = _bits(bufs)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(mla, d, bufs, ws, slots)
    other = DevInputs(make_inputs(cfg, seed=16, **kw))
    other_bufs = _alloc(inp)
    for rep in range(3):
        for k in bufs:
            bufs[k].fill_(0)  # eager work between replays; every output is rewritten by the replay
        _step(mla, other, other_bufs, ws, slots)  # eager call sharing the workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _bits(bufs)
        say("graph replay", rep, cfg, kw)
        for k in want:
            assert np.array_equal(got[k], want[k]), (rep, k)
    assert mla.take_device_error() == 0
