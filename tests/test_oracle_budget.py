"""Precision budget of the decode path, simulated on the CPU.

The kernel scores bf16 operands on the matrix cores. Rounding the absorbed
query q_lat = W_UK^T q_nope to bf16 perturbs every score by about 1e-3 (about
2^-9 relative error summed over 512 terms, times the 1/sqrt(192) scale). lse
is a softmax-weighted mean of those score errors, so it averages down only
when attention is spread over many keys: short caches break the 1e-3 lse bar.

The rounding residue q_lo = q_lat - bf16(q_lat) is known exactly, and lse is
smooth in the scores with d lse / d s_t = p_t. So the first-order effect of the
residue on lse is scale * sum_t p_t (q_lo . c_t) = scale * (q_lo . o_lat), one
dot product with the latent output the kernel already holds. The second-order
remainder is at most half the square of the largest score shift, ~1e-5.
This test shows the bf16-only error, and that the corrected lse (computed the
way the kernel does it: fp32 scores, bf16 probabilities in o_lat) meets the bar
at every length.
"""
import numpy as np

from mla_inputs import bf16_bits, f32, make_inputs
from oracle import mla_oracle as O


def _bf16(x):
    return f32(bf16_bits(np.asarray(x, dtype=np.float32))).astype(np.float64)


def lse_errors(inp):
    """(max |lse error| with bf16 q_lat only, max |error| after the q_lo . o_lat correction)."""
    kv = f32(inp.kv_cache).astype(np.float64)
    qp = f32(inp.q_pe).astype(np.float64)
    q_lat = O.absorb_q(f32(inp.q_nope), f32(inp.w_uk))
    hi = _bf16(q_lat)
    lo = _bf16(q_lat - hi)
    worst_hi = worst_corr = 0.0
    for b in range(inp.b):
        L = int(inp.seqlens[b])
        rows = O.token_rows(kv, inp.block_table, b, L)
        c, kpe = rows[:, :512], rows[:, 512:]
        for j in range(inp.s_q):
            s = (c @ hi[b, j].T + kpe @ qp[b, j].T) * inp.scale
            s = s.astype(np.float32).astype(np.float64)  # fp32 accumulators
            m = s.max(0)
            p = np.exp(s - m)
            l = p.sum(0)
            lse_hi = m + np.log(l)
            o_lat = (_bf16(p).T @ c) / l[:, None]  # bf16 probabilities feed the PV product
            lse_corr = lse_hi + inp.scale * np.einsum("hd,hd->h", lo[b, j], o_lat)
            x = (c @ q_lat[b, j].T + kpe @ qp[b, j].T) * inp.scale
            lse_x = x.max(0) + np.log(np.exp(x - x.max(0)).sum(0))
            worst_hi = max(worst_hi, float(np.abs(lse_hi - lse_x).max()))
            worst_corr = max(worst_corr, float(np.abs(lse_corr - lse_x).max()))
    return worst_hi, worst_corr


def test_bf16_query_breaks_lse_on_short_caches():
    hi, _ = lse_errors(make_inputs("full_heads", seed=0, seqlens=[1, 4, 16, 64]))
    assert hi > 1e-3


def test_first_order_correction_meets_lse_everywhere():
    for seed in range(2):
        for lens in ([1, 2, 3, 4, 16, 64, 300], [1025, 2500, 4096]):
            hi, corr = lse_errors(make_inputs("full_heads", seed=seed, seqlens=lens))
            assert corr < 2e-5, (lens, corr)


def test_tiny_config_budget():
    for seed in range(3):
        _, corr = lse_errors(make_inputs("tiny", seed=seed))
        assert corr < 2e-5


def _merged_o_lat(inp, pieces: int, partial: str):
    """o_lat the way the split path computes it: bf16 q_lat scores, bf16 probabilities into
    PV, each piece normalised and stored as `partial`, merged by lse weights, bf16 out."""
    kv = f32(inp.kv_cache).astype(np.float64)
    qp = f32(inp.q_pe).astype(np.float64)
    q_lat = O.absorb_q(f32(inp.q_nope), f32(inp.w_uk))
    hi = _bf16(q_lat)
    out, ref = [], []
    for b in range(inp.b):
        L = int(inp.seqlens[b])
        rows = O.token_rows(kv, inp.block_table, b, L)
        c, kpe = rows[:, :512], rows[:, 512:]
        s = (c @ hi[b, 0].T + kpe @ qp[b, 0].T) * inp.scale
        x = (c @ q_lat[b, 0].T + kpe @ qp[b, 0].T) * inp.scale
        p = np.exp(x - x.max(0))
        ref.append((p / p.sum(0)).T @ c)
        parts = []
        cuts = np.linspace(0, L, pieces + 1).astype(int)
        for a, e in zip(cuts[:-1], cuts[1:]):
            ss = s[a:e].astype(np.float32).astype(np.float64)
            m = ss.max(0)
            pe = np.exp(ss - m)
            l = pe.sum(0)
            o = (_bf16(pe).T @ c[a:e]) / l[:, None]
            if partial == "fp32":
                o = o.astype(np.float32).astype(np.float64)
            else:  # fp16 rows divided by their largest magnitude, scale kept in fp32
                sc = np.abs(o).max(1, keepdims=True).astype(np.float32).astype(np.float64)
                sc[sc == 0] = 1.0
                o = (o / sc).astype(np.float16).astype(np.float64) * sc
            parts.append((o, m + np.log(l)))
        top = max(pp[1].max() for pp in parts)
        lse = np.log(sum(np.exp(pp[1] - top) for pp in parts)) + top
        out.append(_bf16(sum(np.exp(pp[1] - lse)[:, None] * pp[0] for pp in parts)))
    out, ref = np.stack(out), np.stack(ref)
    return float(np.abs(out - ref).max()), float(np.abs(out - ref).sum() / np.abs(ref).sum())


def test_scaled_fp16_partials_match_fp32_partials():
    """Split pieces hand their rows to the merge as fp16 scaled by the row's largest
    magnitude: the merged o_lat is as close to the exact result as with fp32 partials."""
    inp = make_inputs("full_heads", seed=3, seqlens=[300, 1100, 2500])
    mx32, l1_32 = _merged_o_lat(inp, 3, "fp32")
    mx16, l1_16 = _merged_o_lat(inp, 3, "fp16s")
    assert l1_16 < 5e-3 and mx16 < 2e-2
    assert l1_16 < l1_32 * 1.02 and mx16 < mx32 * 1.1
