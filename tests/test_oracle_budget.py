"""Precision budget of the decode path, simulated on the CPU.

The kernel scores bf16 operands on the matrix cores. Rounding the absorbed
query q_lat = W_UK^T q_nope to bf16 perturbs every score by about 1e-3 (about
2^-9 relative error summed over 512 terms, times the 1/sqrt(192) scale). lse
is a softmax-weighted mean of those score errors, so it averages down only
when attention is spread over many keys: short caches break the 1e-3 lse bar.
Carrying q_lat as bf16 hi + bf16 lo (lo = bf16(q_lat - hi)) and scoring both
removes the error. This test fixes the length below which the kernel adds the
lo pass (LO_PASS_MAX_LEN) and shows both sides of that choice.
"""
import numpy as np

from mla_inputs import bf16_bits, f32, make_inputs
from oracle import mla_oracle as O

LO_PASS_MAX_LEN = 1024  # the library uses the same constant (MLA_LO_PASS_MAX_LEN)


def _bf16(x):
    return f32(bf16_bits(np.asarray(x, dtype=np.float32))).astype(np.float64)


def lse_error(inp, lo_pass):
    kv = f32(inp.kv_cache).astype(np.float64)
    qp = f32(inp.q_pe).astype(np.float64)
    q_lat = O.absorb_q(f32(inp.q_nope), f32(inp.w_uk))
    hi = _bf16(q_lat)
    q_used = hi + _bf16(q_lat - hi) if lo_pass else hi
    worst = 0.0
    for b in range(inp.b):
        L = int(inp.seqlens[b])
        rows = O.token_rows(kv, inp.block_table, b, L)
        c, kpe = rows[:, :512], rows[:, 512:]
        for j in range(inp.s_q):
            s = (c @ q_used[b, j].T + kpe @ qp[b, j].T) * inp.scale
            s = s.astype(np.float32).astype(np.float64)  # fp32 accumulators
            lse = s.max(0) + np.log(np.exp(s - s.max(0)).sum(0))
            x = (c @ q_lat[b, j].T + kpe @ qp[b, j].T) * inp.scale
            lse_x = x.max(0) + np.log(np.exp(x - x.max(0)).sum(0))
            worst = max(worst, float(np.abs(lse - lse_x).max()))
    return worst


def test_bf16_query_breaks_lse_on_short_caches():
    inp = make_inputs("full_heads", seed=0, seqlens=[1, 4, 16, 64])
    assert lse_error(inp, lo_pass=False) > 1e-3


def test_hi_lo_query_meets_lse_on_short_caches():
    for seed in range(2):
        inp = make_inputs("full_heads", seed=seed, seqlens=[1, 2, 4, 16, 64, 300, LO_PASS_MAX_LEN])
        assert lse_error(inp, lo_pass=True) < 2e-5


def test_bf16_query_is_enough_past_threshold():
    for seed in range(2):
        inp = make_inputs("full_heads", seed=seed, seqlens=[LO_PASS_MAX_LEN + 1, 1500, 2500, 4096])
        assert lse_error(inp, lo_pass=False) < 0.7e-3
