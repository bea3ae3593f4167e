"""Cache append (mla_append_kv) against the CPU oracle: the whole cache bit-exact.

The new rows of a decode step go into their pages through the block table;
the lengths count the new tokens, so new row j of sequence b is token
L_b - s_q + j. Rows that break the contract (token index negative or past the
block table, page id outside the cache) are skipped and flagged.
"""
import numpy as np
import pytest
import torch

from gpu_path import DevInputs, compare, host, run_path, say, to_dev_bf16, to_dev_i32
from mla_inputs import MLAInputs, make_inputs, make_new_rows
from oracle import mla_oracle as O

pytestmark = pytest.mark.gpu


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _append_both(mla, inp, new, bt=None, sl=None):
    bt = inp.block_table if bt is None else bt
    sl = inp.seqlens if sl is None else sl
    kv = to_dev_bf16(inp.kv_cache)
    mla.append_kv(to_dev_bf16(new), kv, to_dev_i32(bt), to_dev_i32(sl))
    torch.cuda.synchronize()
    want = O.append_rows(inp.kv_cache, bt, sl, new)
    return kv, want


@pytest.mark.parametrize("seqlens,s_q", [
    ([1, 37, 100], 1),
    ([2, 63, 64, 65, 128, 129], 2),    # new rows on both sides of a page boundary
    ([4, 300, 1025, 64], 4),
    ([8, 9, 700], 8),
])
def test_append_bit_exact(gpu_lib, seqlens, s_q):
    inp = make_inputs("tiny", seed=12, seqlens=seqlens, s_q=s_q, trap=True)
    new = make_new_rows(inp, seed=3)
    say("append", seqlens, "s_q", s_q)
    kv, want = _append_both(gpu_lib, inp, new)
    assert np.array_equal(_bits(kv), want)
    assert gpu_lib.take_device_error() == 0


def test_append_flags_and_skips_bad_rows(gpu_lib):
    inp = make_inputs("tiny", seed=13, seqlens=[130, 70, 3, 64], s_q=2)
    new = make_new_rows(inp, seed=4)
    bt = inp.block_table.copy()
    sl = inp.seqlens.copy()
    sl[2] = 1                          # L < s_q: token -1 is skipped, token 0 is written
    bt[1, 1] = inp.num_pages + 5       # page id past the cache
    sl[3] = 64 * inp.max_blocks + 1    # second new token past the block table
    say("bad rows", sl.tolist())
    kv, want = _append_both(gpu_lib, inp, new, bt=bt, sl=sl)
    assert np.array_equal(_bits(kv), want)
    bits = gpu_lib.take_device_error()
    assert bits == (gpu_lib.MLA_DEVERR_PAGE_ID | gpu_lib.MLA_DEVERR_SEQ_TOO_LONG | gpu_lib.MLA_DEVERR_SHORT_SEQ), bits


@pytest.mark.parametrize("s_q,causal,h", [(1, False, 16), (2, True, 32), (4, True, 128)])
def test_append_then_decode(gpu_lib, s_q, causal, h):
    """A decode step: append the new rows, then attend over the updated cache."""
    inp = make_inputs("tiny", seed=14, seqlens=[5, 64, 130, 1000], s_q=s_q, h=h, causal=causal, trap=True)
    new = make_new_rows(inp, seed=5)
    d = DevInputs(inp)
    gpu_lib.append_kv(to_dev_bf16(new), d.kv, d.bt, d.sl)
    res = host(run_path(gpu_lib, d))
    upd = MLAInputs(**{**inp.__dict__, "kv_cache": O.append_rows(inp.kv_cache, inp.block_table, inp.seqlens, new)})
    ref = O.decode_naive_inputs(upd)
    say("append+decode s_q", s_q, "h", h)
    compare(res, ref, list(range(inp.b)), list(range(inp.h)), label="append+decode")
    assert gpu_lib.take_device_error() == 0


@pytest.mark.parametrize("cfg", ["full_heads", "multi_token"])
def test_append_full_size(gpu_lib, cfg):
    inp = make_inputs(cfg, seed=0)
    new = make_new_rows(inp, seed=6)
    say("append full", cfg, "b", inp.b, "s_q", inp.s_q, "pages", inp.num_pages)
    kv = to_dev_bf16(inp.kv_cache)
    gpu_lib.append_kv(to_dev_bf16(new), kv, to_dev_i32(inp.block_table), to_dev_i32(inp.seqlens))
    want = to_dev_bf16(O.append_rows(inp.kv_cache, inp.block_table, inp.seqlens, new))
    assert torch.equal(kv.view(torch.int16), want.view(torch.int16))
    assert gpu_lib.take_device_error() == 0
