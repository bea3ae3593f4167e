"""mla_absorb_q and mla_up_v against the oracle's closed-form products."""
import numpy as np
import pytest
import torch

from gpu_path import from_dev_bf16, say, to_dev_bf16
from mla_inputs import make_inputs
from oracle import mla_oracle as O

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg,s_q,b", [("tiny", 1, 2), ("tiny", 3, 50), ("full_heads", 1, 128),
                                       ("full_heads", 2, 129), ("tp_share", 1, 128)])
def test_absorb_q(gpu_lib, cfg, s_q, b):
    mla = gpu_lib
    inp = make_inputs(cfg, seed=11, s_q=s_q, seqlens=[5] * b)
    say("absorb", cfg, "b", b, "s_q", s_q, "h", inp.h)
    q_lat, q_lo = mla.absorb_q(to_dev_bf16(inp.q_nope), to_dev_bf16(inp.w_uk), lo=True)
    torch.cuda.synchronize()
    hi, lo = from_dev_bf16(q_lat).astype(np.float64), from_dev_bf16(q_lo).astype(np.float64)
    ref = O.absorb_q(inp_f(inp.q_nope), inp_f(inp.w_uk))
    # bf16 rounding of an fp32 sum: half an ulp (2^-9 relative) plus accumulation noise
    assert (np.abs(hi - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6).all()
    # the lo plane carries the rounding residue: hi + lo is good to ~2^-16
    assert (np.abs(hi + lo - ref) <= 2.0 ** -15 * np.abs(ref) + 2e-6).all()
    # and hi is never worse than the nearest bf16 of the exact product by more than one ulp
    q_lat2, none = mla.absorb_q(to_dev_bf16(inp.q_nope), to_dev_bf16(inp.w_uk), lo=False)
    torch.cuda.synchronize()
    assert none is None and torch.equal(q_lat2.view(torch.int16), q_lat.view(torch.int16))


def inp_f(bits):
    from mla_inputs import f32
    return f32(bits).astype(np.float64)


@pytest.mark.parametrize("cfg,s_q,b", [("tiny", 1, 2), ("full_heads", 1, 128), ("full_heads", 2, 130),
                                       ("tp_share", 1, 64)])
def test_up_v(gpu_lib, cfg, s_q, b):
    mla = gpu_lib
    inp = make_inputs(cfg, seed=12, s_q=s_q, seqlens=[5] * b)
    say("up_v", cfg, "b", b, "s_q", s_q, "h", inp.h)
    rng = np.random.default_rng(3)
    from mla_inputs import bf16_bits
    o_lat_bits = bf16_bits(rng.standard_normal((b, s_q, inp.h, 512)).astype(np.float32) * 0.3)
    o = mla.up_v(to_dev_bf16(o_lat_bits), to_dev_bf16(inp.w_uv))
    torch.cuda.synchronize()
    got = from_dev_bf16(o).astype(np.float64)
    ref = O.up_v(inp_f(o_lat_bits), inp_f(inp.w_uv))
    assert (np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5).all()
