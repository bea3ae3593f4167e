"""Naive MLA decode over a paged latent cache, written for reading, not speed.

TEST INFRASTRUCTURE ONLY (see the package docstring): only tests, the smoke
check and the benchmark's CPU-baseline leg may use this module.

What it computes, and where the pages define it:

* Cached token rows. Each token of a sequence is one row of the paged cache;
  token t of sequence b lives in physical page block_table[b, t // page] at
  slot t % page (paged KV cache, SC11 note "Page Attention" paragraph; FlashMLA
  release news: bf16 paged cache, block size 64). The first d_c = 512 values
  of a row are the latent c^KV (page "DeepSeek-V3 Multi-head Latent Attention
  (MLA) 深度工程", section 2.2, compression stage), the remaining 64 are the
  decoupled positional key k^pos, already rotated (section 3.1).
* Naive expansion (section 2.2, decompression stage; section 4.3's module
  expands with W_uk and W_uv before attending): per head i,
  k_{t,i} = W_UK[i] c_t and v_{t,i} = W_UV[i]^T c_t, with W_UK stored
  [h, d_h, d_c] and W_UV stored [h, d_c, d_h].
* Scores (section 3.1, decoupled RoPE): the content and positional parts are
  concatenated, so score = scale * (q_nope . k_t + q_pe . k_pe_t), with
  scale = 1/sqrt(d_h + d_rope) = 1/sqrt(192) passed in.
* Exact softmax over the visible keys, o = sum_t p_t v_t (naive output) and the
  latent output o_lat = sum_t p_t c_t, whose up-projection o_lat @ W_UV[i]
  equals o. lse = max + ln(sum exp(s - max)), natural log.
* Causal decode with s_q query tokens (FlashMLA call takes causal=True): the
  cache length L already counts the s_q new tokens, query j sits at position
  L - s_q + j and sees keys 0 .. L - s_q + j, i.e. L - s_q + 1 + j of them.
  A row with no visible key returns o = 0, o_lat = 0, lse = -inf.

Readings of the pages taken here are listed in the repository's design notes.
All arithmetic is float64 unless a caller asks for float32.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# small helpers (module level so mutation tests can replace them)


def token_rows(kv_cache: np.ndarray, block_table: np.ndarray, b: int, n: int) -> np.ndarray:
    """Rows of tokens 0..n-1 of sequence b: kv[block_table[b, t // page], t % page]."""
    page = kv_cache.shape[1]
    t = np.arange(n)
    return kv_cache[block_table[b, t // page], t % page]


def append_rows(kv_cache: np.ndarray, block_table: np.ndarray, seqlens: np.ndarray,
                new_rows: np.ndarray) -> np.ndarray:
    """Cache after appending the step's new rows (a copy; the input is untouched).

    Each new token's row (latent c^KV and rotated positional key, page
    "DeepSeek-V3 Multi-head Latent Attention (MLA) 深度工程" sections 2.2 and
    3.2) is stored into the paged cache before attention (section 4.3). The
    lengths count the s_q new tokens, so new row j of sequence b is token
    L_b - s_q + j, which lives at page block_table[b, t // page], slot t % page.
    Rows whose token index is negative, past the block table, or on a page id
    outside the cache are skipped (the library flags them as errors).
    """
    out = kv_cache.copy()
    page = kv_cache.shape[1]
    b_count, s_q = new_rows.shape[0], new_rows.shape[1]
    for b in range(b_count):
        for j in range(s_q):
            t = int(seqlens[b]) - s_q + j
            if t < 0 or t // page >= block_table.shape[1]:
                continue
            pid = int(block_table[b, t // page])
            if 0 <= pid < kv_cache.shape[0]:
                out[pid, t % page] = new_rows[b, j]
    return out


def visible_keys(L: int, s_q: int, j: int, causal: bool) -> int:
    """Number of keys query j (0-based among s_q new tokens) may attend to."""
    if not causal:
        return max(int(L), 0)
    return max(int(L) - s_q + 1 + j, 0)


def expand_k(c: np.ndarray, w_uk_i: np.ndarray) -> np.ndarray:
    """k_t = W_UK[i] c_t for every row c_t of c; c [n, d_c], w_uk_i [d_h, d_c] -> [n, d_h]."""
    return c @ w_uk_i.T


def expand_v(c: np.ndarray, w_uv_i: np.ndarray) -> np.ndarray:
    """v_t = W_UV[i]^T c_t; c [n, d_c], w_uv_i [d_c, d_h] -> [n, d_h]."""
    return c @ w_uv_i


def scores_naive(k: np.ndarray, kpe: np.ndarray, qn: np.ndarray, qp: np.ndarray, scale: float) -> np.ndarray:
    """scale * (q_nope . k_t + q_pe . k_pe_t) for every key t."""
    return scale * (k @ qn + kpe @ qp)


def softmax_stats(s: np.ndarray):
    """Exact softmax of a score vector: (probabilities, lse). Empty -> ([], -inf)."""
    if s.size == 0:
        return s.copy(), -np.inf
    m = s.max()
    e = np.exp(s - m)
    l = e.sum()
    return e / l, m + np.log(l)


# ---------------------------------------------------------------------------
# projections


def absorb_q(q_nope: np.ndarray, w_uk: np.ndarray, dtype=np.float64) -> np.ndarray:
    """q_lat[b,s,i,:] = q_nope[b,s,i,:] @ W_UK[i]  (absorption trick, section 2.4).

    q_nope [b, s_q, h, d_h], w_uk [h, d_h, d_c] -> [b, s_q, h, d_c].
    """
    q = q_nope.astype(dtype)
    w = w_uk.astype(dtype)
    out = np.empty(q.shape[:3] + (w.shape[2],), dtype=dtype)
    for i in range(w.shape[0]):
        out[:, :, i, :] = q[:, :, i, :] @ w[i]
    return out


def up_v(o_lat: np.ndarray, w_uv: np.ndarray, dtype=np.float64) -> np.ndarray:
    """o[b,s,i,:] = o_lat[b,s,i,:] @ W_UV[i]; o_lat [b,s_q,h,d_c], w_uv [h,d_c,d_h]."""
    x = o_lat.astype(dtype)
    w = w_uv.astype(dtype)
    out = np.empty(x.shape[:3] + (w.shape[2],), dtype=dtype)
    for i in range(w.shape[0]):
        out[:, :, i, :] = x[:, :, i, :] @ w[i]
    return out


# ---------------------------------------------------------------------------
# the naive decode (the oracle proper)


def decode_naive(kv_cache, block_table, seqlens, q_nope, q_pe, w_uk, w_uv, scale, causal,
                 seqs=None, heads=None, dtype=np.float64):
    """Naive expand-then-attend decode.

    Arrays are float (already decoded from bf16). Shapes: kv_cache [P, page, d_c + d_r],
    block_table [b, max_blocks], seqlens [b], q_nope [b, s_q, h, d_h], q_pe [b, s_q, h, d_r],
    w_uk [h, d_h, d_c], w_uv [h, d_c, d_h].

    ``seqs`` / ``heads`` select a subset (default: all). Returns a dict with
    o_lat [ns, s_q, nh, d_c], o [ns, s_q, nh, d_h], lse [ns, s_q, nh] and the
    selected ``seqs`` and ``heads``.
    """
    B, s_q, H, d_h = q_nope.shape
    d_c = w_uk.shape[2]
    seqs = list(range(B)) if seqs is None else list(seqs)
    heads = list(range(H)) if heads is None else list(heads)
    o_lat = np.zeros((len(seqs), s_q, len(heads), d_c), dtype=dtype)
    o = np.zeros((len(seqs), s_q, len(heads), d_h), dtype=dtype)
    lse = np.full((len(seqs), s_q, len(heads)), -np.inf, dtype=dtype)
    for si, b in enumerate(seqs):
        L = int(seqlens[b])
        n_all = visible_keys(L, s_q, s_q - 1, causal)  # the last query sees the most keys
        rows = token_rows(kv_cache, block_table, b, n_all).astype(dtype)
        c = rows[:, :d_c]
        kpe = rows[:, d_c:]
        for hi, i in enumerate(heads):
            k = expand_k(c, w_uk[i].astype(dtype))
            v = expand_v(c, w_uv[i].astype(dtype))
            for j in range(s_q):
                n = visible_keys(L, s_q, j, causal)
                if n == 0:
                    continue
                s = scores_naive(k[:n], kpe[:n], q_nope[b, j, i].astype(dtype),
                                 q_pe[b, j, i].astype(dtype), scale)
                p, lse[si, j, hi] = softmax_stats(s)
                o[si, j, hi] = p @ v[:n]
                o_lat[si, j, hi] = p @ c[:n]
    return dict(o_lat=o_lat, o=o, lse=lse, seqs=seqs, heads=heads)


def decode_naive_inputs(inp, seqs=None, heads=None, dtype=np.float64):
    """decode_naive on an ``mla_inputs.MLAInputs`` (bf16 bits decoded exactly)."""
    from mla_inputs import f32
    return decode_naive(f32(inp.kv_cache), inp.block_table, inp.seqlens, f32(inp.q_nope),
                        f32(inp.q_pe), f32(inp.w_uk), f32(inp.w_uv), inp.scale, inp.causal,
                        seqs=seqs, heads=heads, dtype=dtype)


# ---------------------------------------------------------------------------
# the absorbed form: a second formulation, used only to pin the naive one


def decode_absorbed(kv_cache, block_table, seqlens, q_lat, q_pe, w_uv, scale, causal,
                    seqs=None, heads=None, dtype=np.float64):
    """Decode in the absorbed form: every head scores directly against the latent.

    score_t = scale * (q_lat . c_t + q_pe . k_pe_t), q_lat = W_UK[i]^T q_nope
    (section 2.4); o_lat = sum p_t c_t; o = o_lat @ W_UV[i].
    """
    B, s_q, H, d_c = q_lat.shape
    seqs = list(range(B)) if seqs is None else list(seqs)
    heads = list(range(H)) if heads is None else list(heads)
    o_lat = np.zeros((len(seqs), s_q, len(heads), d_c), dtype=dtype)
    lse = np.full((len(seqs), s_q, len(heads)), -np.inf, dtype=dtype)
    for si, b in enumerate(seqs):
        L = int(seqlens[b])
        rows = token_rows(kv_cache, block_table, b, visible_keys(L, s_q, s_q - 1, causal)).astype(dtype)
        c, kpe = rows[:, :d_c], rows[:, d_c:]
        for hi, i in enumerate(heads):
            for j in range(s_q):
                n = visible_keys(L, s_q, j, causal)
                if n == 0:
                    continue
                s = scale * (c[:n] @ q_lat[b, j, i].astype(dtype) + kpe[:n] @ q_pe[b, j, i].astype(dtype))
                p, lse[si, j, hi] = softmax_stats(s)
                o_lat[si, j, hi] = p @ c[:n]
    sel_w = w_uv[heads].astype(dtype)
    o = np.einsum("bshc,hcd->bshd", o_lat, sel_w)
    return dict(o_lat=o_lat, o=o, lse=lse, seqs=seqs, heads=heads)


# ---------------------------------------------------------------------------
# split-KV partials and their merge


def attend_range(s: np.ndarray, values: np.ndarray, lo: int, hi: int):
    """Exact attention restricted to keys [lo, hi): (output, lse); empty -> (0, -inf)."""
    if hi <= lo:
        return np.zeros(values.shape[1], dtype=values.dtype), -np.inf
    p, lse = softmax_stats(s[lo:hi])
    return p @ values[lo:hi], lse


def merge_partials(parts):
    """Merge per-range (o_k, lse_k) into the full result.

    lse = ln sum_k exp(lse_k); o = sum_k exp(lse_k - lse) o_k. Ranges with
    lse_k = -inf carry no weight; if all are -inf the result is (0, -inf).
    """
    lses = np.array([p[1] for p in parts], dtype=np.float64)
    if np.all(np.isneginf(lses)):
        return np.zeros_like(parts[0][0]), -np.inf
    m = lses.max()
    w = np.exp(lses - m)
    lse = m + np.log(w.sum())
    o = sum(np.exp(lk - lse) * ok for ok, lk in parts if not np.isneginf(lk))
    return o, lse


# ---------------------------------------------------------------------------
# the streaming recurrence printed on the pages (section 4.1 pseudocode)


def online_softmax_stream(s: np.ndarray, values: np.ndarray):
    """Key-by-key online softmax with a normalised accumulator.

    Follows the pages' recurrence (section 4.1): keep the running max m and
    running sum l; for each new score s_t, m' = max(m, s_t),
    l' = exp(m - m') l + exp(s_t - m'), and the accumulator becomes
    acc * (exp(m - m') l / l') + v_t * (exp(s_t - m') / l'). The start state
    m = -inf, l = 0 is handled so that exp(-inf - (-inf)) never appears.
    Returns (acc, lse).
    """
    m = -np.inf
    l = 0.0
    acc = np.zeros(values.shape[1], dtype=np.float64)
    for t in range(s.size):
        m_new = max(m, s[t])
        keep = 0.0 if m == -np.inf else np.exp(m - m_new) * l
        l_new = keep + np.exp(s[t] - m_new)
        acc = acc * (keep / l_new) + values[t] * (np.exp(s[t] - m_new) / l_new)
        m, l = m_new, l_new
    lse = m + np.log(l) if l > 0 else -np.inf
    return acc, lse
