"""Bit-exact integer and byte work on the GPU: the page loader and the split plan."""
import numpy as np
import pytest
import torch

from gpu_path import say, to_dev_bf16, to_dev_i32
from mla_inputs import make_inputs
from oracle import split_plan as SP

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seqlens,seed", [
    ([37, 100], 0), ([1, 64, 65, 127, 128, 129], 1), ([0, 5, 0, 300], 2), ([4096, 3, 700], 3),
])
def test_gather_pages_bit_exact(gpu_lib, seqlens, seed):
    mla = gpu_lib
    inp = make_inputs("tiny", seed=seed, seqlens=seqlens, trap=True)
    say("gather", seqlens, "pages", inp.num_pages)
    L = inp.seqlens.astype(np.int64)
    offs = np.concatenate([[0], np.cumsum(np.maximum(L, 0))[:-1]])
    total = int(np.maximum(L, 0).sum())
    out = mla.gather_pages(to_dev_bf16(inp.kv_cache), to_dev_i32(inp.block_table), to_dev_i32(inp.seqlens),
                           torch.from_numpy(offs).cuda(), total)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    for b in range(inp.b):
        t = np.arange(max(int(L[b]), 0))
        ref = inp.kv_cache[inp.block_table[b, t // 64], t % 64]  # fancy indexing: the closed form
        assert np.array_equal(got[offs[b]:offs[b] + t.size], ref), b
    assert mla.take_device_error() == 0


def test_gather_flags_bad_page_ids(gpu_lib):
    """An out-of-range page id reads as zeros and raises the device error bit."""
    mla = gpu_lib
    inp = make_inputs("tiny", seed=4, seqlens=[70, 10])
    bt = inp.block_table.copy()
    bt[0, 1] = inp.num_pages + 5
    out = mla.gather_pages(to_dev_bf16(inp.kv_cache), to_dev_i32(bt), to_dev_i32(inp.seqlens),
                           torch.tensor([0, 70], dtype=torch.int64, device="cuda"), 80)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert not got[64:70].any()
    assert np.array_equal(got[:64], inp.kv_cache[bt[0, 0]])
    assert mla.take_device_error() & 1
    assert mla.take_device_error() == 0


def _plan_cases():
    rng = np.random.default_rng(7)
    cases = [([37, 100], 4, 2), ([512] * 128, 256, 2), ([0, 5, 0, 64, 65, 1], 3, 1), ([0, 0, 0], 5, 2),
             ([65536, 1, 1, 8000], 256, 3), (list(rng.integers(256, 4097, 128)), 256, 2),
             (list(rng.integers(0, 70000, 16)), 256, 0), (list(rng.integers(1, 100, 8192)), 1000, 4)]
    for _ in range(10):
        b = int(rng.integers(1, 3000))
        cases.append((list(rng.integers(0, 5000, b)), int(rng.integers(1, 2000)), int(rng.integers(0, 6))))
    return cases


@pytest.mark.parametrize("seqlens,slots,F", _plan_cases())
def test_plan_bit_exact(gpu_lib, seqlens, slots, F):
    mla = gpu_lib
    say("plan b", len(seqlens), "slots", slots, "F", F)
    sl = torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    meta, ns = mla.get_metadata(sl, slots, split_overhead=F)
    torch.cuda.synchronize()
    ref_meta, ref_ns, _ = SP.plan(seqlens, slots, F)
    assert np.array_equal(ns.cpu().numpy(), ref_ns)
    assert np.array_equal(meta.cpu().numpy(), ref_meta)


def test_plan_into_given_buffers(gpu_lib):
    """get_metadata(out=...) writes the same plan into caller buffers (overwriting what they held)
    and rejects buffers of the wrong shape or dtype before any launch."""
    mla = gpu_lib
    seqlens = [3000, 0, 64, 700, 1]
    slots = 9
    sl = torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    meta = torch.full((slots, mla.META_WORDS), -7, dtype=torch.int32, device="cuda")
    ns = torch.full((len(seqlens) + 1,), -7, dtype=torch.int32, device="cuda")
    got_meta, got_ns = mla.get_metadata(sl, slots, split_overhead=2, out=(meta, ns))
    assert got_meta.data_ptr() == meta.data_ptr() and got_ns.data_ptr() == ns.data_ptr()
    ref_meta, ref_ns, _ = SP.plan(seqlens, slots, 2)
    torch.cuda.synchronize()
    assert np.array_equal(meta.cpu().numpy(), ref_meta)
    assert np.array_equal(ns.cpu().numpy(), ref_ns)
    bad = [(torch.empty((slots, 4), dtype=torch.int32, device="cuda"), ns),
           (meta, torch.empty((len(seqlens),), dtype=torch.int32, device="cuda")),
           (meta.to(torch.int64), ns)]
    for out in bad:
        with pytest.raises(mla.MLAError):
            mla.get_metadata(sl, slots, split_overhead=2, out=out)


@pytest.mark.parametrize("b,s_q,h,slots,F", [
    (2, 1, 16, 4, 2), (128, 1, 128, 256, 6), (128, 1, 32, 256, 2), (32, 8, 128, 32, 4),
    (300, 2, 64, 97, 3), (8192, 1, 16, 1000, 4),
])
def test_absorb_with_plan_matches_separate_calls(gpu_lib, b, s_q, h, slots, F):
    """mla_absorb_q_with_plan gives bit for bit the q_lat, q_lat_lo, tile_meta and num_splits of
    mla_absorb_q and mla_get_metadata (the plan by a 256-thread workgroup inside the GEMM launch)."""
    mla = gpu_lib
    rng = np.random.default_rng(40 + b)
    seqlens = rng.integers(0, 5000, b).astype(np.int32)
    seqlens[0] = 0
    say("absorb+plan b", b, "s_q", s_q, "h", h, "slots", slots, "F", F)
    sl = torch.tensor(seqlens, device="cuda")
    q_nope = torch.from_numpy(rng.standard_normal((b, s_q, h, 128)).astype(np.float32)).to(torch.bfloat16).cuda()
    w_uk = torch.from_numpy((rng.standard_normal((h, 128, 512)) / np.sqrt(512)).astype(np.float32)).to(torch.bfloat16).cuda()
    (ql, qlo), (meta, ns) = mla.absorb_q_with_plan(q_nope, w_uk, sl, slots, split_overhead=F)
    ql2, qlo2 = mla.absorb_q(q_nope, w_uk)
    meta2, ns2 = mla.get_metadata(sl, slots, split_overhead=F)
    torch.cuda.synchronize()
    assert torch.equal(ql.view(torch.int16), ql2.view(torch.int16))
    assert torch.equal(qlo.view(torch.int16), qlo2.view(torch.int16))
    assert torch.equal(meta, meta2) and torch.equal(ns, ns2)
    ref_meta, ref_ns, _ = SP.plan(seqlens.tolist(), slots, F)
    assert np.array_equal(meta.cpu().numpy(), ref_meta) and np.array_equal(ns.cpu().numpy(), ref_ns)
