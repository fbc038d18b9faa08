"""TopK selection of key positions from per-key scores, defined on the CPU (the producer of
``sel_idx`` / ``sel_count`` for the selected-token attention).  TEST INFRASTRUCTURE ONLY
(see the package docstring).

Pages: DynamicSparseAttention INT8 / fast QSA decode page (onnxruntime PR 33472), Key
Changes table (PackedSparseAttentionIndexer: hierarchical / compact TopK selection) and its
follow-up description (compact TopK over 2048-key chunks kept to 512 keys, preserving
stable keys, causal tails, capacity stride / padding and overflow handling).

The pages describe the selection only through those properties; the reading taken here:

* candidates of query row ``i`` of request ``b`` and KV head ``c``: the key positions the
  row may see causally, ``0 .. p`` with ``p = kv_len - q_len + i``, limited to the score
  row's length ``L`` (``n = clamp(p + 1, 0, L)``);
* causal tail: the last ``min(tail, k, n)`` candidates are always selected;
* the other ``k - n_tail`` selections are the highest-scoring remaining candidates; equal
  scores are ranked by position, lower first ("stable keys"); NaN ranks below every
  number (and NaNs by position); -0.0 equals +0.0;
* ``count = min(k, n)``; the selected positions are written in ascending order, then
  padded with -1 up to ``capacity`` (the row stride of ``sel_idx``);
* a row owned by no request selects nothing.

Pins (tests/test_oracle_topk.py): exhaustive search over every subset on tiny inputs, the
library's stable argsort, the threshold property (every selected non-tail score is at
least every unselected one), counts, the forced tail, ascending order and padding.
"""
from __future__ import annotations

import numpy as np


def _rank_key(scores):
    """Sort keys: descending score, NaN last, ties by position (float64 comparison, so
    -0.0 and +0.0 tie)."""
    s = np.asarray(scores, dtype=np.float64)
    nan = np.isnan(s)
    pos = np.arange(len(s))
    # lexsort sorts by the last key first: (nan flag, -score, position)
    return np.lexsort((pos, np.where(nan, 0.0, -s), nan.astype(np.int8)))


def select_row(scores_row, n: int, k: int, tail: int):
    """Selected positions (ascending) of one (row, KV head): candidates ``0 .. n-1``."""
    n = max(0, int(n))
    k = max(0, int(k))
    if n <= k:
        return np.arange(n, dtype=np.int64)
    nt = min(int(tail), k, n)
    forced = np.arange(n - nt, n)
    rest = np.asarray(scores_row[:n - nt])
    order = _rank_key(rest)
    taken = order[:k - nt]
    return np.sort(np.concatenate([taken, forced]).astype(np.int64))


def topk_select(scores, cu_seqlens_q, seqlens_k, *, k: int, tail: int, capacity: int):
    """``scores`` ``[T, H_kv, L]`` -> ``(sel_idx [T, H_kv, capacity] int32, sel_count
    [T, H_kv] int32)`` per the reading in the module docstring."""
    scores = np.asarray(scores)
    T, H_kv, L = scores.shape
    assert capacity >= k
    cu = [int(v) for v in np.asarray(cu_seqlens_q).reshape(-1)]
    sk = [int(v) for v in np.asarray(seqlens_k).reshape(-1)]
    sel = np.full((T, H_kv, capacity), -1, dtype=np.int32)
    cnt = np.zeros((T, H_kv), dtype=np.int32)
    for b in range(len(sk)):
        q_len = cu[b + 1] - cu[b]
        kv_len = sk[b] + 1
        for i in range(q_len):
            t = cu[b] + i
            p = kv_len - q_len + i
            n = min(max(p + 1, 0), L)
            for c in range(H_kv):
                idx = select_row(scores[t, c], n, k, tail)
                sel[t, c, :len(idx)] = idx
                cnt[t, c] = len(idx)
    return sel, cnt
