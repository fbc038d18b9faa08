"""Paged and selected-token sparse attention, defined on the CPU in float64.

The operators compute an ordinary softmax attention over a key set; paging and
selection only decide which cached rows form that set.  For packed row ``r`` of request
``b`` (``cu[b] <= r < cu[b+1]``, ``i = r - cu[b]``) and query head ``h``:

1. ``kv_len = seqlens_k[b] + 1`` and the row's key position is
   ``p = kv_len - q_len_b + i`` (query rows sit at the end of the key sequence: the
   window-start formula of review finding Q3 on the PagedAttention metadata page puts
   query ``i`` at past length + ``i``).
2. The KV head is ``c = h // (H_q / H_kv)`` (GQA head mapping, DynamicSparseAttention
   Description; H_q a multiple of H_kv as on the LinearAttention page).
3. The key set depends on the operator (``paged_attention`` / ``sparse_attention``).
4. INT8 / FP8 cache rows are dequantised per channel: ``k[d] = code[d] * key_scale[c][d]``
   (FP8 codes by their E4M3 value, ``decode_fp8_e4m3``) and
   ``v[d] = code[d] * value_scale[c][d]`` (PR 33472, Key Changes table).
5. ``s_j = scale * <q, k_j>`` with ``scale = 1/sqrt(D)`` when 0 is passed (the
   LinearAttention page's convention for a zero scale).
6. Softmax with a learned per-head sink logit (PagedAttention metadata page, Changes;
   DynamicSparseAttention Description): the sink joins the maximum and the normaliser
   only, it has no value row: ``m = max(max_j s_j, sink)``,
   ``o = sum_j e^(s_j - m) v_j / (sum_j e^(s_j - m) + e^(sink - m))``.  No sink = -inf.
7. An empty key set gives a zero row, with or without a sink (reading taken: the pages
   only show the empty-request sentinel; zero keeps every output finite).
"""
from __future__ import annotations

import math

import numpy as np

from .append import _check_cu, decode_fp8_e4m3
from .status import (STATUS_BAD_BLOCK, STATUS_BAD_COUNT, STATUS_BAD_INDEX, STATUS_CAPACITY,
                     STATUS_K_BOUND, STATUS_Q_BOUND, STATUS_SHORT_KV)


def attend(q, K, V, scale, sink=None):
    """Softmax attention of query vectors ``q`` ``[g, D]`` over keys ``K`` / values ``V``
    ``[n, D]`` with an optional per-query sink logit ``[g]``; float64 result ``[g, D]``.
    Step 6 and 7 of the module docstring."""
    q = np.asarray(q, dtype=np.float64)
    g, D = q.shape
    if K.shape[0] == 0:
        return np.zeros((g, D), dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    s = scale * (q @ K.T)                                   # [g, n]
    sig = np.full(g, -np.inf) if sink is None else np.asarray(sink, dtype=np.float64)
    m = np.maximum(s.max(axis=1), sig)                      # [g]
    w = np.exp(s - m[:, None])
    l = w.sum(axis=1) + np.exp(sig - m)
    return (w @ V) / l[:, None]


def _eff_scale(scale, D):
    return 1.0 / math.sqrt(D) if scale == 0 else float(scale)


class _Cache:
    """Addressing of a K/V cache: paged ``[nb, H_kv, bs, D]`` through a block table, or
    contiguous ``[B, H_kv, cap, D]``; rows come back dequantised in float64.  (The pages
    do not fix a layout; this library keeps each block's slots head by head.)"""

    def __init__(self, k, v, block_table, block_size, key_scale, value_scale):
        self.k, self.v, self.bt = k, v, block_table
        self.bs = int(block_size) if block_table is not None else int(k.shape[2])
        self.nb = int(k.shape[0])
        self.int8 = k.dtype == np.int8
        self.fp8 = k.dtype == np.uint8      # FP8 E4M3 codes (same per-channel scales)
        self.ks, self.vs = key_scale, value_scale

    def rows(self, b, c, js):
        """K and V rows of KV head ``c`` at positions ``js`` of request ``b``, the status
        bits raised, and a mask of positions whose slot exists (the others are excluded:
        beyond the capacity, or a block id outside [0, nb))."""
        js = np.asarray(js, dtype=np.int64)
        status = 0
        if self.bt is None:
            ok = (js < self.bs) & (b < self.nb)
            if not ok.all():
                status |= STATUS_CAPACITY
            blk = np.full(js.shape, b, dtype=np.int64)
            off = js
        else:
            lb = js // self.bs
            in_table = lb < self.bt.shape[1]
            if not in_table.all():
                status |= STATUS_CAPACITY
            blk = np.where(in_table, self.bt[b][np.minimum(lb, self.bt.shape[1] - 1)], -1)
            blk = blk.astype(np.int64)
            good_blk = (blk >= 0) & (blk < self.nb)
            if (in_table & ~good_blk).any():
                status |= STATUS_BAD_BLOCK
            ok = in_table & good_blk
            off = js % self.bs
        blk, off = blk[ok], off[ok]
        if self.fp8:
            K = decode_fp8_e4m3(self.k[blk, c, off])
            V = decode_fp8_e4m3(self.v[blk, c, off])
        else:
            K = self.k[blk, c, off].astype(np.float64)
            V = self.v[blk, c, off].astype(np.float64)
        if self.int8 or self.fp8:
            K = K * self.ks[c].astype(np.float64)
            V = V * self.vs[c].astype(np.float64)
        return K, V, status


def _rows_of(cu, B, rows):
    """(row, request, index within request) for the requested packed rows."""
    out = []
    want = None if rows is None else set(int(r) for r in rows)
    for b in range(B):
        for r in range(cu[b], cu[b + 1]):
            if want is None or r in want:
                out.append((r, b, r - cu[b]))
    return out


def paged_attention(q, k_cache, v_cache, cu_seqlens_q, seqlens_k, *, H_kv, block_table=None,
                    block_size=None, key_scale=None, value_scale=None, max_seqlen_q=None,
                    max_seqlen_k=None, scale=0.0, local_window=-1, sinks=None, rows=None):
    """Causal attention of packed queries ``q`` ``[T, H_q, D]`` over a paged (or
    contiguous) KV cache.  Key set of row ``r`` (position ``p``): cache positions
    ``lo <= j <= p`` with ``lo = max(0, p - W + 1)`` when ``local_window = W > 0`` (W keys
    including the row's own, per the window-start formula of review finding Q3 and the
    local-window change of the PagedAttention metadata page) and ``lo = 0`` otherwise.
    Positions whose slot does not exist are excluded (status bits, parity unpinned).

    Host bounds (parity unpinned, own contract): a request whose query length exceeds
    ``max_seqlen_q`` or whose key count exceeds ``max_seqlen_k`` gets zero rows and a
    status bit; a request with fewer keys than rows flags STATUS_SHORT_KV (its rows with
    ``p < 0`` see no key).

    ``rows`` restricts the computation to a subset of packed rows (then the returned
    array is ``[len(rows), H_q, D]`` in increasing row order and the status covers only
    those rows).  Returns ``(out float64, status)``.
    """
    q = np.asarray(q)
    T, H_q, D = q.shape
    cu = [int(x) for x in np.asarray(cu_seqlens_q).reshape(-1)]
    sk = [int(x) for x in np.asarray(seqlens_k).reshape(-1)]
    B = len(sk)
    _check_cu(cu, B, T)
    g = H_q // H_kv
    sc = _eff_scale(scale, D)
    cache = _Cache(k_cache, v_cache, block_table, block_size, key_scale, value_scale)
    todo = _rows_of(cu, B, rows)
    out = np.zeros((len(todo), H_q, D), dtype=np.float64)
    status = 0
    for n, (r, b, i) in enumerate(todo):
        q_len = cu[b + 1] - cu[b]
        kv_len = sk[b] + 1
        if max_seqlen_q is not None and q_len > max_seqlen_q:
            status |= STATUS_Q_BOUND
            continue
        if max_seqlen_k is not None and kv_len > max_seqlen_k:
            status |= STATUS_K_BOUND
            continue
        if kv_len < q_len:
            status |= STATUS_SHORT_KV
        p = kv_len - q_len + i
        lo = max(0, p - local_window + 1) if local_window > 0 else 0
        js = np.arange(lo, p + 1)
        for c in range(H_kv):
            K, V, st = cache.rows(b, c, js)
            status |= st
            hs = slice(c * g, (c + 1) * g)
            out[n, hs] = attend(q[r, hs], K, V, sc, None if sinks is None else sinks[hs])
    return out, status


def sparse_attention(q, mode, k_cache, v_cache, cu_seqlens_q, seqlens_k, sel_idx, sel_count,
                     max_selected, *, H_kv, block_table=None, block_size=None, key_scale=None,
                     value_scale=None, max_seqlen_q=None, local_window=-1, aux_k=None,
                     aux_v=None, aux_len=0, aux_batch_stride=0, scale=0.0, sinks=None,
                     rows=None):
    """Selected-token attention ("[WebGPU] Add DynamicSparseAttention", Description).

    For row ``r`` and KV head ``c`` the selection list is ``sel_idx[r][c][t]`` for
    ``t < n`` where ``n = sel_count[r][c]`` clamped to ``[0, max_selected]`` (every
    ``t`` when ``sel_count`` is None); the loop is bounded by the count, not by
    ``max_selected`` (review comment on the count-bounded loop).  Entry -1 is padding.

    * ``mode 0`` (selected main-cache rows): entry ``j`` names main-cache position ``j``
      of request ``b``; it is used when ``0 <= j < kv_len`` and ``j <= p`` (causal by
      position).  ``j = -1`` is skipped; any other ``j`` outside ``[0, kv_len)`` is
      excluded (guarded index) and flags STATUS_BAD_INDEX.
    * ``mode 1`` (local plus auxiliary): the main-cache positions ``lo <= j <= p`` of the
      row's local window (``lo`` as in ``paged_attention``) together with the auxiliary
      rows ``a = sel_idx[r][c][t]`` with ``0 <= a < aux_len`` (others excluded, -1 silent)
      read from ``aux_k`` / ``aux_v`` at element offset
      ``b * aux_batch_stride + (a * H_kv + c) * D``; auxiliary rows carry no position and
      are not masked.  One joint softmax over both sources and the sink (Description:
      joint FP32 stable softmax with optional sink).

    Duplicate entries count once per occurrence (a gather).  Returns ``(out, status)``.
    """
    q = np.asarray(q)
    T, H_q, D = q.shape
    cu = [int(x) for x in np.asarray(cu_seqlens_q).reshape(-1)]
    sk = [int(x) for x in np.asarray(seqlens_k).reshape(-1)]
    B = len(sk)
    _check_cu(cu, B, T)
    g = H_q // H_kv
    sc = _eff_scale(scale, D)
    cache = _Cache(k_cache, v_cache, block_table, block_size, key_scale, value_scale)
    if mode == 1:
        ak = np.asarray(aux_k).reshape(-1)
        av = np.asarray(aux_v).reshape(-1)
    todo = _rows_of(cu, B, rows)
    out = np.zeros((len(todo), H_q, D), dtype=np.float64)
    status = 0
    for n, (r, b, i) in enumerate(todo):
        q_len = cu[b + 1] - cu[b]
        kv_len = sk[b] + 1
        if max_seqlen_q is not None and q_len > max_seqlen_q:
            status |= STATUS_Q_BOUND
            continue
        if kv_len < q_len:
            status |= STATUS_SHORT_KV
        p = kv_len - q_len + i
        for c in range(H_kv):
            if sel_count is None:
                cnt = max_selected
            else:
                cnt = int(sel_count[r][c])
                if cnt < 0 or cnt > max_selected:
                    status |= STATUS_BAD_COUNT
                cnt = min(max(cnt, 0), max_selected)
            entries = [int(x) for x in sel_idx[r][c][:cnt]]
            if mode == 0:
                js = []
                for j in entries:
                    if j == -1:
                        continue
                    if j < 0 or j >= kv_len:
                        status |= STATUS_BAD_INDEX
                        continue
                    if j <= p:
                        js.append(j)
                K, V, st = cache.rows(b, c, js)
                status |= st
            else:
                lo = max(0, p - local_window + 1) if local_window > 0 else 0
                Kl, Vl, st = cache.rows(b, c, np.arange(lo, p + 1))
                status |= st
                ka, va = [], []
                for a in entries:
                    if a == -1:
                        continue
                    if a < 0 or a >= aux_len:
                        status |= STATUS_BAD_INDEX
                        continue
                    o = b * aux_batch_stride + (a * H_kv + c) * D
                    ka.append(ak[o:o + D].astype(np.float64))
                    va.append(av[o:o + D].astype(np.float64))
                Ka = np.array(ka, dtype=np.float64).reshape(-1, D)
                Va = np.array(va, dtype=np.float64).reshape(-1, D)
                K = np.concatenate([Kl, Ka], axis=0)
                V = np.concatenate([Vl, Va], axis=0)
            hs = slice(c * g, (c + 1) * g)
            out[n, hs] = attend(q[r, hs], K, V, sc, None if sinks is None else sinks[hs])
    return out, status
