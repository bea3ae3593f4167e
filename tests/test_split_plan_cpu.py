"""The split-KV plan model against a unit-by-unit brute force and its invariants."""
import numpy as np
import pytest

from oracle import split_plan as SP


def brute_plan(seqlens, n_slots, F, page=64):
    """Walk the cost line one unit at a time and cut it into n_slots chunks."""
    pages = [(-(-int(L) // page)) if L > 0 else 0 for L in seqlens]
    units = []  # (b, page or -1 for overhead)
    for b, n in enumerate(pages):
        if n == 0:
            continue
        units += [(b, -1)] * F + [(b, p) for p in range(n)]
    T = len(units)
    q = max(1, -(-T // n_slots)) if T else 1
    per_slot = []
    for s in range(n_slots):
        chunk = units[s * q:(s + 1) * q]
        pieces = {}
        for (b, p) in chunk:
            if p >= 0:
                lo, hi = pieces.get(b, (p, p))
                pieces[b] = (min(lo, p), max(hi, p + 1))
        per_slot.append(sorted(pieces.items()))
    return pages, per_slot


CASES = [
    ([37, 100], 4, 0), ([37, 100], 1, 2), ([512] * 128, 256, 2), ([0, 5, 0, 64, 65, 1], 3, 1),
    ([0, 0], 5, 2), ([1], 7, 0), ([65536, 1, 1, 8000], 256, 3),
]


def _random_cases():
    rng = np.random.default_rng(0)
    out = []
    for _ in range(40):
        b = int(rng.integers(1, 40))
        L = rng.integers(0, 3000, size=b)
        L[rng.random(b) < 0.1] = 0
        out.append((L.tolist(), int(rng.integers(1, 300)), int(rng.integers(0, 5))))
    return out


@pytest.mark.parametrize("seqlens,n_slots,F", CASES + _random_cases())
def test_plan_matches_brute_force(seqlens, n_slots, F):
    meta, ns, pieces = SP.plan(seqlens, n_slots, F)
    pages, per_slot = brute_plan(seqlens, n_slots, F)
    # pieces slot by slot
    got = {}
    for (s, b, lo, hi, k) in pieces:
        got.setdefault(s, []).append((b, (lo, hi)))
    for s in range(n_slots):
        assert got.get(s, []) == per_slot[s], s
    # every page covered exactly once
    cover = [np.zeros(n, dtype=int) for n in pages]
    for (s, b, lo, hi, k) in pieces:
        cover[b][lo:hi] += 1
    for c in cover:
        assert (c == 1).all()
    # split counts and indices
    for b, n in enumerate(pages):
        mine = [p for p in pieces if p[1] == b]
        assert ns[b + 1] - ns[b] == len(mine)
        assert [p[4] for p in mine] == list(range(ns[b], ns[b + 1]))
        assert [p[2] for p in mine] == sorted(p[2] for p in mine)
    assert ns[-1] <= SP.max_splits_bound(len(seqlens), n_slots)
    # tile_meta agrees with the pieces
    for s in range(n_slots):
        mine = [p for p in pieces if p[0] == s]
        if not mine:
            assert list(meta[s]) == [0, 0, -1, 0, 0, 0, 0, 0]
        else:
            assert meta[s][0] == mine[0][1] and meta[s][1] == mine[0][2]
            assert meta[s][2] == mine[-1][1] and meta[s][3] == mine[-1][3]
            assert meta[s][4] == mine[0][4]


def test_single_slot_never_splits():
    meta, ns, pieces = SP.plan([10, 200, 3000, 0, 64], 1, 2)
    assert list(np.diff(ns)) == [1, 1, 1, 0, 1]


def test_balance():
    rng = np.random.default_rng(1)
    L = rng.integers(256, 4097, size=128)
    F = 2
    meta, ns, pieces = SP.plan(L, 256, F)
    pages = SP.seq_pages(L)
    T = int(pages.sum()) + F * int((pages > 0).sum())
    q = -(-T // 256)
    per = np.zeros(256, dtype=int)
    for (s, b, lo, hi, k) in pieces:
        per[s] += hi - lo
    assert per.max() <= q
    assert per.sum() == pages.sum()
