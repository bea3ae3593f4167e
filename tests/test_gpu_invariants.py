"""Properties of the HIP path that hold at any size."""
import numpy as np
import pytest
import torch

from gpu_path import DevInputs, compare, host, run_path, say, to_dev_bf16
from mla_inputs import make_inputs, repage
from oracle import mla_oracle as O

pytestmark = pytest.mark.gpu


def _bits(res):
    return {k: res[k].contiguous().view(torch.int32 if res[k].dtype == torch.float32 else torch.int16).cpu().numpy()
            for k in ("o_lat", "lse", "o")}


def test_page_permutation_bit_identical(gpu_lib):
    inp = make_inputs("tiny", seed=1, seqlens=[900, 65, 3000, 1], h=64, trap=True)
    a = _bits(run_path(gpu_lib, DevInputs(inp)))
    for s in (1, 2):
        b = _bits(run_path(gpu_lib, DevInputs(repage(inp, s))))
        for k in a:
            assert np.array_equal(a[k], b[k]), k


def test_run_to_run_bit_identical(gpu_lib):
    inp = make_inputs("full_heads", seed=2, seqlens=[4000, 300, 2048, 64, 1500, 777, 1, 5000])
    d = DevInputs(inp)
    a = _bits(run_path(gpu_lib, d))
    for _ in range(2):
        b = _bits(run_path(gpu_lib, d))
        for k in a:
            assert np.array_equal(a[k], b[k]), k


def test_split_count_invariance(gpu_lib):
    """Different plans agree within rounding (splits change the summation order only)."""
    inp = make_inputs("tiny", seed=3, seqlens=[3000, 2000, 64, 129], h=32)
    d = DevInputs(inp)
    outs = [host(run_path(gpu_lib, d, slots=s)) for s in (1, 5, 40, 200)]
    for o in outs[1:]:
        assert np.abs(o["lse"] - outs[0]["lse"]).max() < 2e-5
        assert np.abs(o["o_lat"] - outs[0]["o_lat"]).max() < 2e-2


def test_causal_row0_equals_shorter_decode(gpu_lib):
    """Row j = 0 of a causal 2-token decode is a 1-token decode over L - 1 keys."""
    inp2 = make_inputs("tiny", seed=4, seqlens=[100, 1025, 64], s_q=2, causal=True, h=16)
    r2 = host(run_path(gpu_lib, DevInputs(inp2)))
    inp1 = make_inputs("tiny", seed=4, seqlens=[100, 1025, 64], s_q=2, causal=True, h=16)
    inp1.s_q = 1
    inp1.causal = False
    inp1.q_nope = np.ascontiguousarray(inp2.q_nope[:, :1])
    inp1.q_pe = np.ascontiguousarray(inp2.q_pe[:, :1])
    inp1.seqlens = inp2.seqlens - 1
    r1 = host(run_path(gpu_lib, DevInputs(inp1)))
    # both plans cut the same pages, so row 0 is computed in the same order: bit-identical
    assert np.array_equal(r2["lse"][:, 0], r1["lse"][:, 0])
    assert np.array_equal(r2["o_lat"][:, 0], r1["o_lat"][:, 0])


def test_large_score_growth_restarts_exactly(gpu_lib):
    """A key scoring far above the first tile's max forces a recompute with a
    larger softmax reference; the result still matches the oracle (with the
    attention on one token, lse carries that one score's error: the lo-plane
    correction removes it)."""
    inp = make_inputs("tiny", seed=9, seqlens=[300, 2100], h=16)
    # make one late token of each sequence dominate: scale its positional key
    # up (its latent values, which form the output, stay ordinary)
    from mla_inputs import bf16_bits, f32
    kv = f32(inp.kv_cache)
    for b, t in ((0, 250), (1, 2000)):
        pg, sl = inp.block_table[b, t // 64], t % 64
        kv[pg, sl, 512:] *= 80.0
    inp.kv_cache = bf16_bits(kv)
    ref = O.decode_naive_inputs(inp)
    assert (ref["lse"] > 60).any()  # the growth really is past the restart threshold
    res = host(run_path(gpu_lib, DevInputs(inp)))
    say("lse range", float(ref["lse"].min()), float(ref["lse"].max()))
    compare(res, ref, [0, 1], list(range(inp.h)), label="restart")


def _dominant_key_inputs(h, s_q, targets, seed=11):
    """Two sequences whose keys at ``targets`` [(b, t)] score far above everything before them in
    their piece: the positional key of those rows is scaled up (their latent values, which form the
    output, stay ordinary)."""
    from mla_inputs import bf16_bits, f32
    inp = make_inputs("tiny", seed=seed, seqlens=[3000, 700], h=h, s_q=s_q, causal=s_q > 1)
    kv = f32(inp.kv_cache)
    for b, t in targets:
        kv[inp.block_table[b, t // 64], t % 64, 512:] *= 80.0
    inp.kv_cache = bf16_bits(kv)
    return inp


def _largest_growth(inp, b, lo, t):
    """Largest growth, in log2 units, of a row's score at key t over its maxima on keys [lo, lo + 32):
    the first 32-token tile of the piece that starts at token lo."""
    from mla_inputs import f32
    rows = f32(inp.kv_cache)[inp.block_table[b, np.arange(lo, t + 1) // 64], np.arange(lo, t + 1) % 64]
    rows = rows.astype(np.float64)
    q_lat = O.absorb_q(f32(inp.q_nope[b:b + 1]), f32(inp.w_uk))[0]  # [s_q, h, 512]
    s = inp.scale * (np.einsum("tc,jhc->jht", rows[:, :512], q_lat)
                     + np.einsum("tc,jhc->jht", rows[:, 512:], f32(inp.q_pe[b]).astype(np.float64)))
    first = s[:, :, :32].max(axis=2)
    return float(((s[:, :, -1] - first) / np.log(2.0)).max())


@pytest.mark.parametrize("s_q", [1, 2])
@pytest.mark.parametrize("h", [64, 128])
@pytest.mark.parametrize("mode", ["whole", "split"])
def test_restart_in_row_block_kernel(gpu_lib, mode, h, s_q):
    """The recompute of a piece whose scores outgrow the softmax reference (the row's first tile max)
    in the row-block kernel (M = 64, 128, 256 rows), with the dominant key past the piece's first
    tile: in a sequence held whole by one slot (finalised in place) and in one piece of a split
    sequence (its partial then goes through the split merge). Every element against the oracle."""
    from oracle import split_plan
    F = gpu_lib.default_split_overhead(s_q, h)
    if mode == "whole":
        slots = 1
        targets = [(0, 1000), (1, 500)]
        starts = {0: 0, 1: 0}
    else:
        slots = 40
        _, ns, pieces = split_plan.plan([3000, 700], slots, F)
        targets, starts = [], {}
        for b in (0, 1):
            mine = [p for p in pieces if p[1] == b]
            assert len(mine) >= 3
            _, _, plo, phi, _ = mine[1]  # the second piece of the sequence
            targets.append((b, plo * 64 + 40))  # in the piece's second tile
            starts[b] = plo * 64
    inp = _dominant_key_inputs(h, s_q, targets)
    for b, t in targets:  # the premise: some row's growth passes the 64 (log2) slack
        g = _largest_growth(inp, b, starts[b], t)
        say("mode", mode, "h", h, "s_q", s_q, "seq", b, "key", t, "largest growth (log2)", round(g, 1))
        assert g > 70.0
    ref = O.decode_naive_inputs(inp)
    res = host(run_path(gpu_lib, DevInputs(inp), slots=slots))
    compare(res, ref, [0, 1], list(range(inp.h)), label=f"restart {mode} h={h} s_q={s_q}")
    assert gpu_lib.take_device_error() == 0
