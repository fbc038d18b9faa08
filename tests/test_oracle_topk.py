"""Pins of the oracle's TopK selection (CPU only).

Against: exhaustive search over every subset on tiny inputs (the unique subset whose every
member precedes every non-member in the order the reading defines, written here with plain
Python comparisons), the library's stable argsort, and the structural properties (count,
forced causal tail, threshold, ascending order, padding)."""
import itertools
import math

import numpy as np
import pytest

import oracle.topk as tk


def _precedes(a, b, s):
    """a before b: higher score, NaN after every number, equal scores by position."""
    sa, sb = s[a], s[b]
    na, nb = math.isnan(sa), math.isnan(sb)
    if na != nb:
        return nb
    if not na and sa != sb:
        return sa > sb
    return a < b


@pytest.mark.parametrize("seed", range(40))
def test_exhaustive_tiny(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 9))
    k = int(rng.integers(0, 9))
    tail = int(rng.integers(0, 4))
    # few distinct values, so ties are common; some NaN, infinities and signed zeros
    pool = np.array([1.0, -1.0, 0.0, -0.0, 2.5, np.inf, -np.inf, np.nan])
    s = pool[rng.integers(0, len(pool), size=n)]
    got = tk.select_row(s, n, k, tail)
    if n <= k:
        assert got.tolist() == list(range(n))
        return
    nt = min(tail, k, n)
    forced = set(range(n - nt, n))
    rest = [j for j in range(n) if j not in forced]
    valid = []
    for sub in itertools.combinations(rest, k - nt):
        inside = set(sub)
        if all(_precedes(a, b, s) for a in inside for b in rest if b not in inside):
            valid.append(sorted(inside | forced))
    assert len(valid) == 1
    assert got.tolist() == valid[0]


def test_matches_stable_argsort_without_nan():
    rng = np.random.default_rng(7)
    for _ in range(50):
        n = int(rng.integers(1, 3000))
        k = int(rng.integers(0, 600))
        s = np.round(rng.standard_normal(n) * 4) / 4          # many ties
        got = tk.select_row(s, n, k, 0)
        if n <= k:
            assert len(got) == n
            continue
        want = np.sort(np.argsort(-s, kind="stable")[:k])
        assert np.array_equal(got, want)


def test_threshold_tail_order_and_padding():
    rng = np.random.default_rng(9)
    T, H, L = 6, 3, 700
    scores = rng.standard_normal((T, H, L)).astype(np.float32)
    cu = np.array([0, 2, 6], dtype=np.int32)
    seqlens_k = np.array([400 - 1, 700 - 1], dtype=np.int32)   # kv_len 400 and 700
    sel, cnt = tk.topk_select(scores, cu, seqlens_k, k=128, tail=16, capacity=160)
    assert sel.shape == (T, H, 160) and cnt.shape == (T, H)
    for t in range(T):
        b = 0 if t < 2 else 1
        q_len = cu[b + 1] - cu[b]
        p = int(seqlens_k[b]) + 1 - q_len + (t - cu[b])
        n = min(p + 1, L)
        for c in range(H):
            m = int(cnt[t, c])
            assert m == min(128, n)
            idx = sel[t, c, :m]
            assert np.all(np.diff(idx) > 0) and idx[0] >= 0 and idx[-1] < n
            assert np.all(sel[t, c, m:] == -1)
            tail = set(range(n - 16, n))
            assert tail <= set(idx.tolist())
            chosen = [j for j in idx if j not in tail]
            others = [j for j in range(n - 16) if j not in set(idx.tolist())]
            assert min(scores[t, c, chosen]) >= max(scores[t, c, others])


def test_short_rows_and_empty_requests():
    scores = np.zeros((3, 1, 50), dtype=np.float32)
    cu = np.array([0, 0, 3], dtype=np.int32)            # request 0 has no rows
    seqlens_k = np.array([-1, 2], dtype=np.int32)        # request 1: 3 keys, 3 rows
    sel, cnt = tk.topk_select(scores, cu, seqlens_k, k=8, tail=2, capacity=8)
    assert cnt[:, 0].tolist() == [1, 2, 3]
    assert sel[2, 0].tolist() == [0, 1, 2, -1, -1, -1, -1, -1]
    # k = 0 selects nothing, whatever the tail
    sel, cnt = tk.topk_select(scores, cu, seqlens_k, k=0, tail=2, capacity=0)
    assert cnt.sum() == 0 and sel.shape == (3, 1, 0)
