"""Plant plausible mistakes in the CPU oracle and check that a pin catches each.

Every mutation here replaces one oracle helper for the duration of one test
(monkeypatch); the pins in oracle_pins.py must then fail (assertion or error).
"""
import math

import numpy as np
import pytest

import oracle_pins as pins
from mla_inputs import SOFTMAX_SCALE
from oracle import mla_oracle as O


def _rows_no_block_table(kv, bt, b, n):
    page = kv.shape[1]
    t = np.arange(n)
    return kv[t // page, t % page]


def _rows_slot_shift(kv, bt, b, n):
    page = kv.shape[1]
    t = np.arange(n)
    return kv[bt[b, t // page], (t + 1) % page]


def _rows_slot_reversed(kv, bt, b, n):
    page = kv.shape[1]
    t = np.arange(n)
    return kv[bt[b, t // page], page - 1 - t % page]


def _softmax_no_max(s):
    if s.size == 0:
        return s.copy(), -np.inf
    m = s.max()
    e = np.exp(s - m)
    return e / e.sum(), np.log(e.sum())


def _softmax_unnormalised(s):
    if s.size == 0:
        return s.copy(), -np.inf
    m = s.max()
    e = np.exp(s - m)
    return e, m + np.log(e.sum())


def _absorb_head0(q_nope, w_uk, dtype=np.float64):
    q, w = q_nope.astype(dtype), w_uk.astype(dtype)
    out = np.empty(q.shape[:3] + (w.shape[2],), dtype=dtype)
    for i in range(w.shape[0]):
        out[:, :, i, :] = q[:, :, i, :] @ w[0]
    return out


def _absorb_transposed(q_nope, w_uk, dtype=np.float64):
    q, w = q_nope.astype(dtype), w_uk.astype(dtype)
    out = np.empty(q.shape[:3] + (w.shape[2],), dtype=dtype)
    for i in range(w.shape[0]):
        out[:, :, i, :] = q[:, :, i, :] @ w[i].T
    return out


def _up_v_head0(o_lat, w_uv, dtype=np.float64):
    x, w = o_lat.astype(dtype), w_uv.astype(dtype)
    out = np.empty(x.shape[:3] + (w.shape[2],), dtype=dtype)
    for i in range(w.shape[0]):
        out[:, :, i, :] = x[:, :, i, :] @ w[0]
    return out


def _merge_no_rescale(parts):
    live = [p for p in parts if not np.isneginf(p[1])]
    if not live:
        return np.zeros_like(parts[0][0]), -np.inf
    lses = np.array([p[1] for p in live])
    return sum(p[0] for p in live) / len(live), lses.max() + np.log(np.exp(lses - lses.max()).sum())


def _merge_lse_max(parts):
    o, _ = O.__dict__["_orig_merge"](parts)
    lses = [p[1] for p in parts]
    return o, max(lses)


def _stream_no_keep(s, values):
    m, l = -np.inf, 0.0
    acc = np.zeros(values.shape[1])
    for t in range(s.size):
        m_new = max(m, s[t])
        keep = 0.0 if m == -np.inf else np.exp(m - m_new) * l
        l_new = keep + np.exp(s[t] - m_new)
        acc = acc + values[t] * (np.exp(s[t] - m_new) / l_new)
        m, l = m_new, l_new
    return acc, m + np.log(l)


def _append_with(token_of):
    def bad(kv, bt, L, new):
        out = kv.copy()
        page = kv.shape[1]
        for b in range(new.shape[0]):
            for j in range(new.shape[1]):
                t = token_of(int(L[b]), new.shape[1], j)
                if t < 0 or t // page >= bt.shape[1]:
                    continue
                pid = int(bt[b, t // page])
                if 0 <= pid < kv.shape[0]:
                    out[pid, t % page] = new[b, j]
        return out
    return bad


def _append_page_slot_swapped(kv, bt, L, new):
    out = kv.copy()
    page = kv.shape[1]
    for b in range(new.shape[0]):
        for j in range(new.shape[1]):
            t = int(L[b]) - new.shape[1] + j
            if t < 0 or t % page >= bt.shape[1] or t // page >= page:
                continue
            pid = int(bt[b, t % page])
            if 0 <= pid < kv.shape[0]:
                out[pid, t // page] = new[b, j]
    return out


MUTATIONS = {
    "append_off_by_one": ("append_rows", _append_with(lambda L, s_q, j: L - s_q + j + 1)),
    "append_reversed_rows": ("append_rows", _append_with(lambda L, s_q, j: L - 1 - j)),
    "append_at_start": ("append_rows", _append_with(lambda L, s_q, j: j)),
    "append_page_slot_swapped": ("append_rows", _append_page_slot_swapped),
    "rows_ignore_block_table": ("token_rows", _rows_no_block_table),
    "rows_slot_shift": ("token_rows", _rows_slot_shift),
    "rows_slot_reversed": ("token_rows", _rows_slot_reversed),
    "causal_off_by_one": ("visible_keys", lambda L, s_q, j, causal: max(L - s_q + j, 0) if causal else max(L, 0)),
    "causal_ignored": ("visible_keys", lambda L, s_q, j, causal: max(L, 0)),
    "k_weight_transposed": ("expand_k", lambda c, w: c @ w),
    "v_weight_transposed": ("expand_v", lambda c, w: c @ w.T),
    "rope_term_dropped": ("scores_naive", lambda k, kpe, qn, qp, scale: scale * (k @ qn)),
    "rope_term_sign": ("scores_naive", lambda k, kpe, qn, qp, scale: scale * (k @ qn - kpe @ qp)),
    "content_term_dropped": ("scores_naive", lambda k, kpe, qn, qp, scale: scale * (kpe @ qp)),
    "scale_dropped": ("scores_naive", lambda k, kpe, qn, qp, scale: k @ qn + kpe @ qp),
    "scale_squared": ("scores_naive", lambda k, kpe, qn, qp, scale: scale * scale * (k @ qn + kpe @ qp)),
    "lse_without_max": ("softmax_stats", _softmax_no_max),
    "softmax_unnormalised": ("softmax_stats", _softmax_unnormalised),
    "absorb_wrong_head": ("absorb_q", _absorb_head0),
    "absorb_transposed": ("absorb_q", _absorb_transposed),
    "up_v_wrong_head": ("up_v", _up_v_head0),
    "merge_without_rescale": ("merge_partials", _merge_no_rescale),
    "merge_lse_is_max": ("merge_partials", _merge_lse_max),
    "stream_drops_history": ("online_softmax_stream", _stream_no_keep),
}

# cheap pins first: the first failure ends a mutation's run
ORDER = [pins.append_worked_example, pins.append_round_trip,
         pins.split_merge, pins.streaming, pins.gather_indexing, pins.rows_sum_to_one, pins.zero_query,
         pins.single_token, pins.identical_rows, pins.causal_reduction, pins.up_v_identity,
         pins.absorb_identity, pins.page_permutation, pins.sdpa_library, pins.brute_force_tiny,
         pins.brute_force_real_dims]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, bad = MUTATIONS[name]
    monkeypatch.setitem(O.__dict__, "_orig_merge", O.merge_partials)
    monkeypatch.setattr(O, attr, bad)
    caught = []
    for pin in ORDER:
        try:
            pin()
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
            break
    assert caught, f"mutation {name} slipped past every pin"


def test_scale_reading():
    """The softmax scale is 1/sqrt(d_nope + d_rope) = 1/sqrt(192)."""
    assert SOFTMAX_SCALE == 1.0 / math.sqrt(192.0)
