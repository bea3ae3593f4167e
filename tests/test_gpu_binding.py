"""The Python binding rejects mis-shaped device tensors before anything is launched.

The kernels address q_lat, block_table and tile_meta from the shapes passed
through the C ABI, so a tensor of another shape must raise MLAError on the
host instead of reaching the GPU.
"""
import pytest
import torch

from gpu_path import DevInputs
from mla_inputs import make_inputs

pytestmark = pytest.mark.gpu


def _call(mla, d, **over):
    inp = d.inp
    meta, ns = mla.get_metadata(d.sl, s_q=inp.s_q, h=inp.h)
    q_lat, q_lo = mla.absorb_q(d.q_nope, d.w_uk)
    args = dict(q_lat=q_lat, q_pe=d.q_pe, kv_cache=d.kv, block_table=d.bt, cache_seqlens=d.sl, tile_meta=meta,
                num_splits=ns, softmax_scale=inp.scale, causal=inp.causal, q_lat_lo=q_lo)
    args.update(over)
    return mla.decode_paged(**args)


@pytest.mark.parametrize("what", ["q_lat_width", "q_lat_rank", "block_table_rows", "block_table_rank",
                                  "tile_meta_words", "q_pe_heads"])
def test_decode_rejects_misshaped(gpu_lib, what):
    d = DevInputs(make_inputs("tiny", seed=0))
    inp = d.inp
    torch.cuda.synchronize()
    bad = {
        "q_lat_width": lambda: dict(q_lat=torch.zeros((inp.b, 1, inp.h, 256), dtype=torch.bfloat16, device="cuda")),
        "q_lat_rank": lambda: dict(q_lat=torch.zeros((inp.b, inp.h, 512), dtype=torch.bfloat16, device="cuda")),
        "block_table_rows": lambda: dict(block_table=d.bt[:1].contiguous()),
        "block_table_rank": lambda: dict(block_table=d.bt.reshape(-1)),
        "tile_meta_words": lambda: dict(tile_meta=torch.zeros((8, 4), dtype=torch.int32, device="cuda")),
        "q_pe_heads": lambda: dict(q_pe=d.q_pe[:, :, :8].contiguous()),
    }[what]()
    with pytest.raises(gpu_lib.MLAError):
        _call(gpu_lib, d, **bad)
    o_lat, lse = _call(gpu_lib, d)  # the well-formed call still runs
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all()
