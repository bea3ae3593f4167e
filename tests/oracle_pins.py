"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each pin raises AssertionError (or any exception) when the oracle is wrong.
tests/test_oracle_pins.py runs them; tests/test_oracle_mutations.py plants
plausible mistakes in the oracle and checks that some pin catches each one.

What pins what:
  brute_force_*     scalar loops over the definition (page lookup, per-head
                    expansion, concatenated scores, exact softmax) on tiny inputs
  sdpa_library      torch's CPU scaled_dot_product_attention / logsumexp on the
                    expanded keys and values
  absorb_identity   the absorbed form (q_lat = W_UK^T q_nope scored against the
                    latent) equals the naive form
  up_v_identity     o_lat @ W_UV[i] equals the naive output o
  rows_sum_to_one   a cache column fixed at 1 comes out as exactly 1
  page_permutation  moving physical pages (and the block table with them)
                    changes nothing, bit for bit
  gather_indexing   token rows come from block_table[b, t // page], slot t % page
  zero_query        q = 0 gives the mean row and lse = ln n
  single_token      L = 1 gives the token's own row
  identical_rows    identical rows give that row, and lse grows by ln(L2/L1)
  causal_reduction  causal row 0 of a 2-token decode equals a 1-token decode
                    over L - 1 keys
  split_merge       merged range partials equal the unsplit result
  streaming         the pages' key-by-key recurrence equals exact softmax
"""
from __future__ import annotations

import math

import numpy as np

from mla_inputs import f32, make_inputs, repage
from oracle import mla_oracle as O

TOL = 1e-11


def tiny_problem(seed, *, b=2, s_q=2, h=3, page=4, d_c=8, d_r=2, d_h=4, lens=(5, 11), causal=True):
    """A small float64 problem with arbitrary dimensions and a shuffled block table."""
    rng = np.random.default_rng(seed)
    lens = list(lens)[:b]
    pages = [-(-L // page) if L > 0 else 0 for L in lens]
    P = sum(pages) + 1
    perm = rng.permutation(P)
    mb = max(1, max(pages))
    bt = np.full((b, mb), perm[-1], dtype=np.int64)
    off = 0
    for i, n in enumerate(pages):
        bt[i, :n] = perm[off:off + n]
        off += n
    return dict(kv=rng.standard_normal((P, page, d_c + d_r)), bt=bt, lens=np.array(lens),
                q_nope=rng.standard_normal((b, s_q, h, d_h)), q_pe=rng.standard_normal((b, s_q, h, d_r)),
                w_uk=rng.standard_normal((h, d_h, d_c)) / math.sqrt(d_c),
                w_uv=rng.standard_normal((h, d_c, d_h)) / math.sqrt(d_c),
                scale=1.0 / math.sqrt(d_h + d_r), causal=causal)


def run_oracle(p, seqs=None, heads=None):
    return O.decode_naive(p["kv"], p["bt"], p["lens"], p["q_nope"], p["q_pe"], p["w_uk"], p["w_uv"],
                          p["scale"], p["causal"], seqs=seqs, heads=heads)


def brute(p, seqs=None, heads=None):
    """Scalar loops over the definition; plain Python floats and math.exp."""
    kv, bt, lens = p["kv"], p["bt"], p["lens"]
    qn, qp, wk, wv = p["q_nope"], p["q_pe"], p["w_uk"], p["w_uv"]
    B, s_q, H, d_h = qn.shape
    d_c = wk.shape[2]
    d_r = qp.shape[3]
    page = kv.shape[1]
    seqs = range(B) if seqs is None else seqs
    heads = range(H) if heads is None else heads
    res = {}
    for b in seqs:
        for j in range(s_q):
            L = int(lens[b])
            n = max(L - s_q + 1 + j, 0) if p["causal"] else max(L, 0)
            rows = [[float(x) for x in kv[bt[b][t // page]][t % page]] for t in range(n)]
            for i in heads:
                scores = []
                for t in range(n):
                    r = rows[t]
                    acc = 0.0
                    for d in range(d_h):
                        kd = 0.0
                        for c in range(d_c):
                            kd += float(wk[i][d][c]) * r[c]
                        acc += float(qn[b][j][i][d]) * kd
                    for e in range(d_r):
                        acc += float(qp[b][j][i][e]) * r[d_c + e]
                    scores.append(p["scale"] * acc)
                if n == 0:
                    res[(b, j, i)] = ([0.0] * d_c, [0.0] * d_h, -math.inf)
                    continue
                mx = max(scores)
                ws = [math.exp(s - mx) for s in scores]
                tot = sum(ws)
                probs = [w / tot for w in ws]
                o_lat = [sum(probs[t] * rows[t][c] for t in range(n)) for c in range(d_c)]
                o = []
                for d in range(d_h):
                    acc = 0.0
                    for t in range(n):
                        vd = 0.0
                        for c in range(d_c):
                            vd += float(wv[i][c][d]) * rows[t][c]
                        acc += probs[t] * vd
                    o.append(acc)
                res[(b, j, i)] = (o_lat, o, mx + math.log(tot))
    return res


def _compare_brute(p, seqs=None, heads=None):
    got = run_oracle(p, seqs, heads)
    ref = brute(p, seqs, heads)
    for (b, j, i), (o_lat, o, lse) in ref.items():
        si = got["seqs"].index(b)
        hi = got["heads"].index(i)
        if math.isinf(lse):
            assert np.isneginf(got["lse"][si, j, hi])
        else:
            assert abs(got["lse"][si, j, hi] - lse) <= TOL * max(1.0, abs(lse)), (b, j, i)
        np.testing.assert_allclose(got["o_lat"][si, j, hi], o_lat, rtol=0, atol=TOL)
        np.testing.assert_allclose(got["o"][si, j, hi], o, rtol=0, atol=TOL)


def brute_force_tiny():
    for seed, causal in ((1, True), (2, False)):
        _compare_brute(tiny_problem(seed, causal=causal))
    # square widths, so that a transposed weight would still run
    _compare_brute(tiny_problem(3, d_c=6, d_h=6, lens=(9, 3), causal=True))
    # a sequence too short for its causal rows
    _compare_brute(tiny_problem(4, lens=(1, 6), s_q=2, causal=True))


def brute_force_real_dims():
    inp = make_inputs("tiny", seed=0, seqlens=[3, 2])
    p = dict(kv=f32(inp.kv_cache).astype(np.float64), bt=inp.block_table, lens=inp.seqlens,
             q_nope=f32(inp.q_nope).astype(np.float64), q_pe=f32(inp.q_pe).astype(np.float64),
             w_uk=f32(inp.w_uk).astype(np.float64), w_uv=f32(inp.w_uv).astype(np.float64),
             scale=inp.scale, causal=False)
    _compare_brute(p, seqs=[0, 1], heads=[0, 11])


def sdpa_library():
    import torch
    import torch.nn.functional as F
    for seed, causal in ((5, True), (6, False)):
        p = tiny_problem(seed, b=2, s_q=2, h=2, page=4, d_c=16, d_r=4, d_h=8, lens=(13, 7), causal=causal)
        got = run_oracle(p)
        kv = torch.from_numpy(p["kv"])
        for b in range(2):
            L = int(p["lens"][b])
            rows = torch.stack([kv[int(p["bt"][b, t // 4]), t % 4] for t in range(L)])
            c, kpe = rows[:, :16], rows[:, 16:]
            for i in range(2):
                K = torch.cat([c @ torch.from_numpy(p["w_uk"][i]).T, kpe], dim=1)
                V = c @ torch.from_numpy(p["w_uv"][i])
                for j in range(2):
                    n = L - 2 + 1 + j if causal else L
                    q = torch.cat([torch.from_numpy(p["q_nope"][b, j, i]), torch.from_numpy(p["q_pe"][b, j, i])])
                    o = F.scaled_dot_product_attention(q.view(1, 1, 1, -1), K[:n].view(1, 1, n, -1),
                                                       V[:n].view(1, 1, n, -1), scale=p["scale"]).view(-1)
                    o_lat = F.scaled_dot_product_attention(q.view(1, 1, 1, -1), K[:n].view(1, 1, n, -1),
                                                           c[:n].view(1, 1, n, -1), scale=p["scale"]).view(-1)
                    lse = torch.logsumexp(p["scale"] * (K[:n] @ q), dim=0)
                    np.testing.assert_allclose(got["o"][b, j, i], o.numpy(), rtol=0, atol=1e-10)
                    np.testing.assert_allclose(got["o_lat"][b, j, i], o_lat.numpy(), rtol=0, atol=1e-10)
                    assert abs(got["lse"][b, j, i] - float(lse)) < 1e-10


def absorb_identity():
    for causal in (True, False):
        p = tiny_problem(7, causal=causal, lens=(6, 10))
        ref = run_oracle(p)
        q_lat = O.absorb_q(p["q_nope"], p["w_uk"])
        got = O.decode_absorbed(p["kv"], p["bt"], p["lens"], q_lat, p["q_pe"], p["w_uv"], p["scale"], p["causal"])
        for k in ("o_lat", "o", "lse"):
            np.testing.assert_allclose(got[k], ref[k], rtol=1e-12, atol=1e-12)
    # and the identity q^T (W c) = (W^T q)^T c itself, on real widths
    inp = make_inputs("tiny", seed=1)
    qn, wk = f32(inp.q_nope).astype(np.float64), f32(inp.w_uk).astype(np.float64)
    c = f32(inp.kv_cache[0, :8, :512]).astype(np.float64)
    q_lat = O.absorb_q(qn, wk)
    for i in (0, 9):
        lhs = (c @ wk[i].T) @ qn[1, 0, i]
        rhs = c @ q_lat[1, 0, i]
        np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def up_v_identity():
    p = tiny_problem(8, lens=(7, 12))
    ref = run_oracle(p)
    o = O.up_v(ref["o_lat"], p["w_uv"])
    np.testing.assert_allclose(o, ref["o"], rtol=1e-12, atol=1e-12)


def rows_sum_to_one():
    p = tiny_problem(9, lens=(5, 14))
    p["kv"][:, :, 0] = 1.0
    got = run_oracle(p)
    np.testing.assert_allclose(got["o_lat"][..., 0], 1.0, rtol=0, atol=1e-13)


def page_permutation():
    inp = make_inputs("tiny", seed=0)
    a = O.decode_naive_inputs(inp, heads=[0, 5, 15])
    for s in (1, 2):
        b = O.decode_naive_inputs(repage(inp, s), heads=[0, 5, 15])
        for k in ("o_lat", "o", "lse"):
            assert np.array_equal(a[k], b[k]), k


def gather_indexing():
    rng = np.random.default_rng(10)
    page, P = 64, 9
    kv = np.zeros((P, page, 576))
    for pg in range(P):
        kv[pg, :, 0] = pg
        kv[pg, :, 1] = np.arange(page)
    bt = rng.permutation(P).reshape(3, 3)
    for b in range(3):
        rows = O.token_rows(kv, bt, b, 150)
        for t in range(150):
            assert rows[t, 0] == bt[b][t // page] and rows[t, 1] == t % page


def zero_query():
    p = tiny_problem(11, lens=(6, 9), causal=True)
    p["q_nope"][:] = 0.0
    p["q_pe"][:] = 0.0
    got = run_oracle(p)
    d_c = p["w_uk"].shape[2]
    for b in range(2):
        for j in range(2):
            n = int(p["lens"][b]) - 2 + 1 + j
            rows = np.array([p["kv"][p["bt"][b][t // 4]][t % 4] for t in range(n)])
            mean_c = rows[:, :d_c].mean(axis=0)
            for i in range(3):
                np.testing.assert_allclose(got["o_lat"][b, j, i], mean_c, rtol=0, atol=1e-13)
                np.testing.assert_allclose(got["o"][b, j, i], mean_c @ p["w_uv"][i], rtol=0, atol=1e-13)
                assert abs(got["lse"][b, j, i] - math.log(n)) < 1e-13


def single_token():
    p = tiny_problem(12, lens=(1, 1), s_q=1, causal=False)
    got = run_oracle(p)
    d_c = p["w_uk"].shape[2]
    for b in range(2):
        r = p["kv"][p["bt"][b][0]][0]
        for i in range(3):
            np.testing.assert_allclose(got["o_lat"][b, 0, i], r[:d_c], rtol=0, atol=1e-14)
            np.testing.assert_allclose(got["o"][b, 0, i], r[:d_c] @ p["w_uv"][i], rtol=0, atol=1e-13)


def identical_rows():
    p = tiny_problem(13, lens=(5, 13), s_q=1, causal=False)
    r = p["kv"][0, 0].copy()
    p["kv"][:] = r
    got = run_oracle(p)
    d_c = p["w_uk"].shape[2]
    np.testing.assert_allclose(got["o_lat"], np.broadcast_to(r[:d_c], got["o_lat"].shape), rtol=0, atol=1e-13)
    # same query in both sequences -> lse differs by ln(13/5)
    p["q_nope"][1] = p["q_nope"][0]
    p["q_pe"][1] = p["q_pe"][0]
    got = run_oracle(p)
    np.testing.assert_allclose(got["lse"][1] - got["lse"][0], math.log(13 / 5), rtol=0, atol=1e-12)


def causal_reduction():
    p2 = tiny_problem(14, lens=(9, 12), s_q=2, causal=True)
    r2 = run_oracle(p2)
    p1 = dict(p2)
    p1["q_nope"] = p2["q_nope"][:, :1].copy()
    p1["q_pe"] = p2["q_pe"][:, :1].copy()
    p1["lens"] = p2["lens"] - 1
    p1["causal"] = False
    r1 = run_oracle(p1)
    for k in ("o_lat", "o", "lse"):
        np.testing.assert_allclose(r2[k][:, 0], r1[k][:, 0], rtol=0, atol=1e-13)


def split_merge():
    rng = np.random.default_rng(15)
    s = rng.standard_normal(37) * 3
    v = rng.standard_normal((37, 5))
    full = O.attend_range(s, v, 0, 37)
    for cuts in ([0, 37], [0, 10, 37], [0, 1, 2, 20, 36, 37], [0, 0, 5, 5, 37]):
        parts = [O.attend_range(s, v, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
        o, lse = O.merge_partials(parts)
        np.testing.assert_allclose(o, full[0], rtol=0, atol=1e-12)
        assert abs(lse - full[1]) < 1e-12
    # merge against a value computed without the oracle's softmax
    e = np.exp(s - s.max())
    np.testing.assert_allclose(full[0], (e / e.sum()) @ v, rtol=0, atol=1e-12)
    assert abs(full[1] - (s.max() + math.log(e.sum()))) < 1e-12
    o, lse = O.merge_partials([O.attend_range(s, v, 3, 3), O.attend_range(s, v, 4, 4)])
    assert np.isneginf(lse) and not o.any()


def streaming():
    rng = np.random.default_rng(16)
    for n in (1, 2, 50):
        s = rng.standard_normal(n) * 4
        v = rng.standard_normal((n, 3))
        acc, lse = O.online_softmax_stream(s, v)
        e = np.exp(s - s.max())
        np.testing.assert_allclose(acc, (e / e.sum()) @ v, rtol=0, atol=1e-12)
        assert abs(lse - (s.max() + math.log(e.sum()))) < 1e-12


def append_worked_example():
    """A hand-worked cache append (page "DeepSeek-V3 Multi-head Latent Attention (MLA) 深度工程",
    section 4.3: the new token's row goes into its page before attention; the lengths count the
    new tokens). Pages of 4 rows, rows 3 wide, s_q = 2:
      sequence 0, L = 5: new rows are tokens 3 and 4 -> page bt[0, 0] = 2 slot 3, page bt[0, 1] = 0 slot 0;
      sequence 1, L = 2: tokens 0 and 1 -> page bt[1, 0] = 1 slots 0 and 1;
      sequence 2, L = 1 < s_q: token -1 is skipped, token 0 -> page bt[2, 0] = 3 slot 0;
      sequence 3, L = 9: tokens 7 (page bt[3, 1] = -1: skipped) and 8 (past the 2-entry table: skipped)."""
    kv = np.full((4, 4, 3), -1.0)
    bt = np.array([[2, 0], [1, -1], [3, -1], [0, -1]])
    L = np.array([5, 2, 1, 9])
    new = np.arange(4 * 2 * 3, dtype=np.float64).reshape(4, 2, 3) + 100.0
    out = O.append_rows(kv, bt, L, new)
    want = np.full((4, 4, 3), -1.0)
    want[2, 3] = [100, 101, 102]   # seq 0, j 0
    want[0, 0] = [103, 104, 105]   # seq 0, j 1
    want[1, 0] = [106, 107, 108]   # seq 1, j 0
    want[1, 1] = [109, 110, 111]   # seq 1, j 1
    want[3, 0] = [115, 116, 117]   # seq 2, j 1 (j 0 has token -1)
    assert np.array_equal(out, want)
    assert np.array_equal(kv, np.full((4, 4, 3), -1.0))  # the input is not modified


def append_round_trip():
    """Reading the cache back through the pinned token gather: the last s_q tokens of every
    sequence are the new rows, every earlier token and every other cache row is unchanged."""
    rng = np.random.default_rng(21)
    page, P, s_q = 64, 40, 3
    kv = rng.standard_normal((P, page, 5))
    L = np.array([3, 64, 65, 130, 1000 % 640])
    bt = rng.permutation(P)[:5 * 8].reshape(5, 8)
    new = rng.standard_normal((5, s_q, 5))
    out = O.append_rows(kv, bt, L, new)
    touched = np.zeros((P, page), dtype=bool)
    for b in range(5):
        before, after = O.token_rows(kv, bt, b, int(L[b])), O.token_rows(out, bt, b, int(L[b]))
        assert np.array_equal(after[L[b] - s_q:], new[b])
        assert np.array_equal(after[:L[b] - s_q], before[:L[b] - s_q])
        for t in range(L[b] - s_q, L[b]):
            touched[bt[b, t // page], t % page] = True
    assert np.array_equal(out[~touched], kv[~touched])


ALL_PINS = [brute_force_tiny, brute_force_real_dims, sdpa_library, absorb_identity, up_v_identity,
            rows_sum_to_one, page_permutation, gather_indexing, zero_query, single_token,
            identical_rows, causal_reduction, split_merge, streaming, append_worked_example,
            append_round_trip]
