"""mla_decode_paged_noalloc (the decode entry point that allocates nothing: its
split partials live in a fixed per-GPU array inside the library) against
mla_decode_paged with a caller-provided workspace, called through the C ABI.

Two calls in a row on one GPU share that array: a larger shape first (128
heads, two draft tokens, sequences cut into many pieces), then a smaller one,
then the larger one again. Each result must be bit-identical to the workspace
call's and within the whole-path bar of the CPU oracle.
"""
import numpy as np
import pytest
import torch

from gpu_path import DevInputs, compare, say
from mla_inputs import f32, make_inputs
from oracle import mla_oracle as O

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu().numpy()


def _host(o_lat, lse):
    return f32(o_lat.view(torch.int16).cpu().numpy().view(np.uint16)), lse.cpu().numpy()


def _one(mla, inp, slots):
    d = DevInputs(inp)
    meta, ns = mla.get_metadata(d.sl, slots, s_q=inp.s_q, h=inp.h)
    q_lat, q_lo = mla.absorb_q(d.q_nope, d.w_uk)
    # outputs allocated before the calls, so the no-alloc call itself allocates nothing
    out_ws = (torch.empty((inp.b, inp.s_q, inp.h, 512), dtype=torch.bfloat16, device="cuda"),
              torch.empty((inp.b, inp.s_q, inp.h), dtype=torch.float32, device="cuda"))
    out_na = (torch.full((inp.b, inp.s_q, inp.h, 512), float("nan"), dtype=torch.bfloat16, device="cuda"),
              torch.full((inp.b, inp.s_q, inp.h), float("nan"), dtype=torch.float32, device="cuda"))
    mla.decode_paged(q_lat, d.q_pe, d.kv, d.bt, d.sl, meta, ns, inp.scale, inp.causal, q_lat_lo=q_lo, out=out_ws)
    torch.cuda.synchronize()
    mla.decode_paged_noalloc(q_lat, d.q_pe, d.kv, d.bt, d.sl, meta, ns, inp.scale, inp.causal, q_lat_lo=q_lo,
                             out=out_na)
    torch.cuda.synchronize()
    assert mla.take_device_error() == 0
    for a, b in zip(out_ws, out_na):
        assert np.array_equal(_bits(a), _bits(b))
    o_lat, lse = _host(*out_na)
    o = mla.up_v(out_na[0], d.w_uv)
    torch.cuda.synchronize()
    got = dict(o_lat=o_lat, lse=lse, o=f32(o.view(torch.int16).cpu().numpy().view(np.uint16)))
    ref = O.decode_naive_inputs(inp)
    compare(got, ref, list(range(inp.b)), list(range(inp.h)), label=f"noalloc {inp.name} h={inp.h} s_q={inp.s_q}")


def test_noalloc_matches_workspace_call(gpu_lib):
    big = make_inputs("tiny", seed=50, seqlens=[3000, 77, 1500, 640, 2], h=128, s_q=2, causal=True, trap=True)
    small = make_inputs("tiny", seed=51, seqlens=[37, 100], h=16, trap=True)
    need = gpu_lib.workspace_bytes(big.b, big.s_q, big.h, 200)
    assert need <= gpu_lib.NOALLOC_SCRATCH_BYTES
    for inp, slots in ((big, 200), (small, 7), (big, 200)):
        say("noalloc: b", inp.b, "h", inp.h, "s_q", inp.s_q, "slots", slots)
        _one(gpu_lib, inp, slots)


def test_noalloc_rejects_shapes_beyond_scratch(gpu_lib):
    inp = make_inputs("tiny", seed=52, seqlens=[10] * 2, h=128, s_q=8)
    d = DevInputs(inp)
    slots = 64 << 10  # about 69 GB of partials: far beyond the scratch
    assert gpu_lib.workspace_bytes(inp.b, inp.s_q, inp.h, slots) > gpu_lib.NOALLOC_SCRATCH_BYTES
    meta, ns = gpu_lib.get_metadata(d.sl, slots, s_q=inp.s_q, h=inp.h)
    q_lat, q_lo = gpu_lib.absorb_q(d.q_nope, d.w_uk)
    with pytest.raises(gpu_lib.MLAError, match="built-in scratch"):
        gpu_lib.decode_paged_noalloc(q_lat, d.q_pe, d.kv, d.bt, d.sl, meta, ns, inp.scale, inp.causal,
                                     q_lat_lo=q_lo)
