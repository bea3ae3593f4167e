"""The quantised latent cache on the GPU, through the C ABI.

The MLA engineering page's quantised-MLA section stores the latent c^KV in 8
bits; the format is the library's reading (e4m3 codes and a power-of-two scale
per token, bf16 positional key). Checked here:
  * mla_quantize_pages and mla_append_kv_fp8 write exactly the bytes the CPU
    oracle's quantisation gives (bit for bit, whole caches);
  * mla_decode_paged_fp8 matches the CPU oracle run on the cache the pages
    stand for (the dequantised values), at the whole-path tolerances;
  * since the scales are powers of two and every dequantised value is a bf16
    value, the quantised decode is, rounding step for rounding step, the bf16
    decode on the dequantised cache: both kernels must agree bit for bit;
  * NaN in unused pages, in page tails and in their scale slots never leaks.
"""
import numpy as np
import pytest
import torch

from gpu_path import DevInputs, compare, say, to_dev_bf16, to_dev_i32
from mla_inputs import MLAInputs, bf16_bits, f32, make_inputs, make_new_rows
from oracle import kv_quant as Q
from oracle import mla_oracle as O

pytestmark = pytest.mark.gpu


def _u8(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy()


def _dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def _special_rows(inp):
    """Rows that exercise the format's corners, written into the first page of a cache."""
    kv = f32(inp.kv_cache).copy()
    rng = np.random.default_rng(7)
    kv[0, 0] = 0.0                                               # all-zero row: scale 1
    kv[0, 1, :5] = [1.0, -0.5, 3.0, 1.0625, 1.1875]              # ties after scaling by 128
    kv[0, 1, 5:512] = 0.0
    kv[0, 2, :512] = rng.standard_normal(512) * 2.0 ** -100      # tiny values: small exponents
    kv[0, 3, :512] = rng.standard_normal(512) * 2.0 ** 30        # huge values
    kv[0, 4, :512:3] = -0.0                                      # negative zeros
    kv[0, 5, :512] = 448.0 * np.sign(rng.standard_normal(512))   # every value at the top code
    kv[0, 6, :512] = rng.standard_normal(512) * 2.0 ** -130      # amax below 2^-126: the floor
    return MLAInputs(**{**inp.__dict__, "kv_cache": bf16_bits(kv)})


@pytest.mark.parametrize("name,seed", [("tiny", 0), ("tiny", 1), ("tp_share", 0)])
def test_quantize_pages_bit_exact(gpu_lib, name, seed):
    inp = make_inputs(name, seed=seed)
    if name == "tiny":
        inp = _special_rows(inp)
    say("quantize", name, "pages", inp.num_pages)
    got = _u8(gpu_lib.quantize_pages(to_dev_bf16(inp.kv_cache)))
    want = Q.quantize_cache(inp.kv_cache)
    assert np.array_equal(got, want), np.argwhere(got != want)[:10]


@pytest.mark.parametrize("seqlens,s_q", [([1, 37, 100], 1), ([2, 63, 64, 65, 128, 129], 2), ([8, 9, 700], 8)])
def test_append_fp8_bit_exact(gpu_lib, seqlens, s_q):
    inp = make_inputs("tiny", seed=22, seqlens=seqlens, s_q=s_q)
    new = make_new_rows(inp, seed=8)
    pages = Q.quantize_cache(inp.kv_cache)
    kv8 = _dev_u8(pages)
    say("append fp8", seqlens, "s_q", s_q)
    gpu_lib.append_kv_fp8(to_dev_bf16(new), kv8, to_dev_i32(inp.block_table), to_dev_i32(inp.seqlens))
    torch.cuda.synchronize()
    want = Q.append_rows_fp8(pages, inp.block_table, inp.seqlens, new)
    assert np.array_equal(_u8(kv8), want)
    assert gpu_lib.take_device_error() == 0


def test_append_fp8_flags_and_skips_bad_rows(gpu_lib):
    inp = make_inputs("tiny", seed=23, seqlens=[130, 70, 3, 64], s_q=2)
    new = make_new_rows(inp, seed=9)
    bt, sl = inp.block_table.copy(), inp.seqlens.copy()
    sl[2] = 1                          # L < s_q: token -1 skipped, token 0 written
    bt[1, 1] = inp.num_pages + 5       # page id past the cache
    sl[3] = 64 * inp.max_blocks + 1    # second new token past the block table
    pages = Q.quantize_cache(inp.kv_cache)
    kv8 = _dev_u8(pages)
    gpu_lib.append_kv_fp8(to_dev_bf16(new), kv8, to_dev_i32(bt), to_dev_i32(sl))
    torch.cuda.synchronize()
    assert np.array_equal(_u8(kv8), Q.append_rows_fp8(pages, bt, sl, new))
    bits = gpu_lib.take_device_error()
    assert bits == (gpu_lib.MLA_DEVERR_PAGE_ID | gpu_lib.MLA_DEVERR_SEQ_TOO_LONG | gpu_lib.MLA_DEVERR_SHORT_SEQ), bits


def _poison(pages: np.ndarray, inp) -> np.ndarray:
    """NaN everywhere a decode must not look: unused pages, and the rows and scale slots past each
    sequence's length in its last page."""
    out = pages.copy()
    used = set()
    for b in range(inp.b):
        n = (int(inp.seqlens[b]) + 63) // 64 if inp.seqlens[b] > 0 else 0
        used.update(int(p) for p in inp.block_table[b, :n])
        if n:
            last, tail = int(inp.block_table[b, n - 1]), int(inp.seqlens[b]) - (n - 1) * 64
            if tail < 64:
                out[last, tail * 640:64 * 640] = 0xFF                      # NaN codes and NaN keys
                out[last, Q.SCALES_OFFSET + 4 * tail:] = 0xFF              # NaN scales
    for p in range(inp.num_pages):
        if p not in used:
            out[p] = 0xFF
    return out


def _run_both(mla, inp, pages, poisoned=None, slots=None):
    """The quantised decode (on ``poisoned`` pages if given) and the bf16 decode on the dequantised
    cache, with the same plan and queries; returns host arrays of both."""
    d = DevInputs(inp)
    deq = Q.dequantize_cache(pages)
    kv_deq = to_dev_bf16(bf16_bits(deq.astype(np.float32)))
    kv8 = _dev_u8(pages if poisoned is None else poisoned)
    meta, ns = mla.get_metadata(d.sl, slots, s_q=inp.s_q, h=inp.h)
    q_lat, q_lo = mla.absorb_q(d.q_nope, d.w_uk)
    o8, l8 = mla.decode_paged_fp8(q_lat, d.q_pe, kv8, d.bt, d.sl, meta, ns, inp.scale, inp.causal, q_lat_lo=q_lo)
    o16, l16 = mla.decode_paged(q_lat, d.q_pe, kv_deq, d.bt, d.sl, meta, ns, inp.scale, inp.causal, q_lat_lo=q_lo)
    o = mla.up_v(o8, d.w_uv)
    torch.cuda.synchronize()
    assert mla.take_device_error() == 0
    h = lambda t: f32(t.view(torch.int16).cpu().numpy().view(np.uint16))  # noqa: E731
    return dict(o_lat=h(o8), lse=l8.cpu().numpy(), o=h(o)), dict(o_lat=h(o16), lse=l16.cpu().numpy()), deq


SHAPES = [
    ([1, 2, 63, 64, 65, 127, 128, 129], 1, 16, False),
    ([1, 2, 3, 64, 65, 200], 2, 16, True),        # causal rows with 0 .. L - 1 keys
    ([0, 7, 0, 100, 1500], 1, 32, False),          # empty sequences
    ([333, 2000, 77], 1, 32, False),
]


@pytest.mark.parametrize("slots", [None, 1, 7, 300])
@pytest.mark.parametrize("seqlens,s_q,h,causal", SHAPES)
def test_decode_fp8_matches_oracle_and_bf16_path(gpu_lib, seqlens, s_q, h, causal, slots):
    inp = make_inputs("tiny", seed=31, seqlens=seqlens, s_q=s_q, h=h, causal=causal)
    pages = Q.quantize_cache(inp.kv_cache)
    say("fp8 decode", seqlens, "s_q", s_q, "h", h, "causal", causal, "slots", slots)
    got, bf, deq = _run_both(gpu_lib, inp, pages, poisoned=_poison(pages, inp), slots=slots)
    ref = O.decode_naive(deq, inp.block_table, inp.seqlens, f32(inp.q_nope), f32(inp.q_pe), f32(inp.w_uk),
                         f32(inp.w_uv), inp.scale, inp.causal)
    compare(got, ref, list(range(inp.b)), list(range(inp.h)), label="fp8")
    _assert_same_bits(got, bf)


def _assert_same_bits(got, bf):
    d_o = float(np.nanmax(np.abs(got["o_lat"] - bf["o_lat"])))
    both_inf = np.isneginf(got["lse"]) & np.isneginf(bf["lse"])
    d_l = float(np.nanmax(np.abs(np.where(both_inf, 0, got["lse"]) - np.where(both_inf, 0, bf["lse"]))))
    assert np.array_equal(got["o_lat"], bf["o_lat"]) and np.array_equal(got["lse"], bf["lse"]), \
        f"the quantised decode differs from the bf16 decode of the dequantised cache (o_lat {d_o:.3e}, lse {d_l:.3e})"


def test_decode_fp8_restart(gpu_lib):
    """A key scoring far above the first tile's maximum forces the recompute in the quantised kernel."""
    inp = make_inputs("tiny", seed=9, seqlens=[300, 2100], h=16)
    kv = f32(inp.kv_cache)
    for b, t in ((0, 250), (1, 2000)):
        kv[inp.block_table[b, t // 64], t % 64, 512:] *= 80.0
    inp = MLAInputs(**{**inp.__dict__, "kv_cache": bf16_bits(kv)})
    pages = Q.quantize_cache(inp.kv_cache)
    got, bf, deq = _run_both(gpu_lib, inp, pages)
    ref = O.decode_naive(deq, inp.block_table, inp.seqlens, f32(inp.q_nope), f32(inp.q_pe), f32(inp.w_uk),
                         f32(inp.w_uv), inp.scale, inp.causal)
    assert (ref["lse"] > 60).any()
    compare(got, ref, [0, 1], list(range(inp.h)), label="fp8 restart")
    _assert_same_bits(got, bf)


def test_decode_fp8_full_size_sampled(gpu_lib):
    """The 32-head tensor-parallel share at full size, quantised on the GPU, in the bench's launch
    configuration; sampled sequences and heads against the oracle on the dequantised cache."""
    inp = make_inputs("tp_share", seed=0)
    d = DevInputs(inp)
    kv8 = gpu_lib.quantize_pages(d.kv)
    meta, ns = gpu_lib.get_metadata(d.sl, s_q=inp.s_q, h=inp.h)
    q_lat, q_lo = gpu_lib.absorb_q(d.q_nope, d.w_uk)
    o8, l8 = gpu_lib.decode_paged_fp8(q_lat, d.q_pe, kv8, d.bt, d.sl, meta, ns, inp.scale, inp.causal, q_lat_lo=q_lo)
    o = gpu_lib.up_v(o8, d.w_uv)
    torch.cuda.synchronize()
    h = lambda t: f32(t.view(torch.int16).cpu().numpy().view(np.uint16))  # noqa: E731
    got = dict(o_lat=h(o8), lse=l8.cpu().numpy(), o=h(o))
    deq = Q.dequantize_cache(_u8(kv8))
    seqs, heads = [0, 17, 64, 127], [0, 13, 31]
    ref = O.decode_naive(deq, inp.block_table, inp.seqlens, f32(inp.q_nope), f32(inp.q_pe), f32(inp.w_uk),
                         f32(inp.w_uv), inp.scale, inp.causal, seqs=seqs, heads=heads)
    compare(got, ref, seqs, heads, label="fp8 tp_share")
    assert gpu_lib.take_device_error() == 0


def test_decode_fp8_rejects_more_than_32_rows(gpu_lib):
    inp = make_inputs("tiny", seed=2, seqlens=[10, 20], h=64)
    d = DevInputs(inp)
    kv8 = gpu_lib.quantize_pages(d.kv)
    meta, ns = gpu_lib.get_metadata(d.sl, s_q=inp.s_q, h=inp.h)
    q_lat, q_lo = gpu_lib.absorb_q(d.q_nope, d.w_uk)
    with pytest.raises(gpu_lib.MLAError, match="at most 32 query rows"):
        gpu_lib.decode_paged_fp8(q_lat, d.q_pe, kv8, d.bt, d.sl, meta, ns, inp.scale, inp.causal, q_lat_lo=q_lo)
