"""Cache data that break the decode's contract, through the C ABI.

include/mla.h promises that a block-table entry outside [0, num_pages) and a
cache length past the block table (L_b > max_blocks * 64) are read as zero rows
and raise a device error bit (MLA_DEVERR_PAGE_ID, MLA_DEVERR_SEQ_TOO_LONG),
with no out-of-bounds access. Each case runs the row-block kernel (128 and 48
query rows), the token-split kernel (32 rows) and the quantised-cache kernel,
and compares every output element with the CPU oracle run on the same cache
with those pages replaced by a page of zeros, at the whole-path tolerances.
"""
import numpy as np
import pytest
import torch

from gpu_path import DevInputs, compare, from_dev_bf16, say, to_dev_i32
from mla_inputs import f32, make_inputs
from oracle import kv_quant as Q
from oracle import mla_oracle as O

pytestmark = pytest.mark.gpu


def _broken(inp, kind):
    """(block table, lengths) that break the contract, the oracle's table and lengths over a cache with one
    more page of zeros (id num_pages), and the device error bit the decode must raise."""
    bt, sl = inp.block_table.copy(), inp.seqlens.copy()
    zero = inp.num_pages
    if kind == "page_id":      # an id past the cache, inside sequence 1's pages
        bt[1, 3] = inp.num_pages + 5
        ref_bt = bt.copy()
        ref_bt[1, 3] = zero
        return bt, sl, ref_bt, sl, 1
    if kind == "negative_page_id":
        bt[0, 1] = -3
        ref_bt = bt.copy()
        ref_bt[0, 1] = zero
        return bt, sl, ref_bt, sl, 1
    # a length past the table: sequence 1 (whose table row is full) runs 30 tokens beyond it
    mb = bt.shape[1]
    assert int(inp.seqlens[1]) > (mb - 1) * 64
    sl[1] = mb * 64 + 30
    ref_bt = np.concatenate([bt, np.full((bt.shape[0], 1), zero, dtype=bt.dtype)], axis=1)
    return bt, sl, ref_bt, sl, 2


def _oracle(inp, kv_pages_f32, ref_bt, ref_sl):
    kv_ext = np.concatenate([kv_pages_f32, np.zeros((1,) + kv_pages_f32.shape[1:], kv_pages_f32.dtype)])
    return O.decode_naive(kv_ext, ref_bt, ref_sl, f32(inp.q_nope), f32(inp.q_pe), f32(inp.w_uk), f32(inp.w_uv),
                          inp.scale, inp.causal)


def _run(mla, inp, d, bt, sl, kv, fp8):
    bt_d, sl_d = to_dev_i32(bt), to_dev_i32(sl)
    meta, ns = mla.get_metadata(sl_d, 7, s_q=inp.s_q, h=inp.h)  # several pieces per sequence
    q_lat, q_lo = mla.absorb_q(d.q_nope, d.w_uk)
    dec = mla.decode_paged_fp8 if fp8 else mla.decode_paged
    o_lat, lse = dec(q_lat, d.q_pe, kv, bt_d, sl_d, meta, ns, inp.scale, inp.causal, q_lat_lo=q_lo)
    o = mla.up_v(o_lat, d.w_uv)
    torch.cuda.synchronize()
    return dict(o_lat=from_dev_bf16(o_lat), o=from_dev_bf16(o), lse=lse.cpu().numpy())


@pytest.mark.parametrize("kind", ["page_id", "negative_page_id", "too_long"])
@pytest.mark.parametrize("h,s_q,fp8", [(128, 1, False), (16, 3, False), (32, 1, False), (32, 1, True)])
def test_broken_cache_reads_zero_rows(gpu_lib, kind, h, s_q, fp8):
    mla = gpu_lib
    inp = make_inputs("tiny", seed=40, seqlens=[200, 700, 90], h=h, s_q=s_q, causal=s_q > 1)
    bt, sl, ref_bt, ref_sl, bit = _broken(inp, kind)
    say("contract", kind, "h", h, "s_q", s_q, "fp8", fp8)
    d = DevInputs(inp)
    assert mla.take_device_error() == 0
    if fp8:
        kv8 = mla.quantize_pages(d.kv)
        torch.cuda.synchronize()
        pages = Q.dequantize_cache(kv8.cpu().numpy())
        got = _run(mla, inp, d, bt, sl, kv8, True)
    else:
        pages = f32(inp.kv_cache)
        got = _run(mla, inp, d, bt, sl, d.kv, False)
    assert mla.take_device_error() == bit
    ref = _oracle(inp, pages, ref_bt, ref_sl)
    compare(got, ref, list(range(inp.b)), list(range(inp.h)), label=f"contract {kind} h={h} s_q={s_q} fp8={fp8}")
    assert mla.take_device_error() == 0
