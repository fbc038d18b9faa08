"""QKV prologue before the cache append: packed-QKV split, QK RMSNorm and rotary position
embedding, defined on the CPU.  TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages: "[WebGPU] Add DynamicSparseAttention", Description ("QKV and cache": packed and
unpacked QKV, GQA head mapping; "Position processing": QK RMSNorm, partial and interleaved
RoPE, rotary offsets and explicit position IDs) and its review comment that the RMS of a
head must be reduced once per (token, head) rather than once per channel; "[WebGPU] Add
SparsePagedAttention", pull-request overview (the PagedAttention prologue it reuses:
packed-QKV split, RoPE, block-table scatter).

The pages name these steps but print no formula for them, so the textbook definitions are
taken, each stated in the function that uses it:

* packed layout: row t of ``qkv`` is ``[H_q query heads | H_kv key heads | H_kv value
  heads]``, each head D contiguous elements;
* RMSNorm of one head: ``y_d = x_d / sqrt(mean_d(x^2) + eps) * w_d`` with a weight vector
  ``w`` of D entries shared by all heads (one for queries, one for keys);
* rotary embedding: each pair ``(a, b)`` of the first ``rotary_dim`` channels is rotated by
  the angle whose cosine and sine the tables hold at the token's position,
  ``(a, b) -> (a cos - b sin, b cos + a sin)``; pairs are ``(i, i + rotary_dim/2)``
  ("half" layout) or ``(2i, 2i+1)`` (interleaved), ``i < rotary_dim/2``; channels from
  ``rotary_dim`` on pass unchanged ("partial" RoPE);
* the position of row ``i`` of request ``b`` is ``position_ids[t]`` when given, else its
  key position ``kv_len - q_len + i``; ``rotary_offsets[b]`` (optional) is added.  A
  position outside ``[0, max_position)`` raises STATUS_POSITION; that row's query output
  is zero and its K/V row is not appended;
* order: split, then RMSNorm (queries and keys), then rotation (queries and keys); values
  pass through.  The results are rounded once to the activation dtype, and the rounded key
  row is what the cache append stores or quantises, so the fused step equals this
  prologue followed by ``kv_cache_append``.

Pins (tests/test_oracle_prologue.py): unit RMS after the norm, scale invariance, the
rotation equal to complex multiplication by ``exp(i*theta)`` (numpy complex arithmetic) in
both pair layouts, pair norms preserved, untouched channels past ``rotary_dim``, the
relative-position property of rotated dot products, packed equal to unpacked, explicit
positions equal to the default ones, offsets equal to shifted positions, and the
composition with the cache append.
"""
from __future__ import annotations

import numpy as np

from .append import kv_cache_append
from .status import STATUS_POSITION


def split_qkv(qkv, H_q: int, H_kv: int, D: int):
    """``[T, (H_q + 2 H_kv) * D]`` (or ``[T, H_q + 2 H_kv, D]``) -> q ``[T, H_q, D]``,
    k ``[T, H_kv, D]``, v ``[T, H_kv, D]``: query heads first, then key heads, then value
    heads."""
    a = np.asarray(qkv)
    T = a.shape[0]
    a = a.reshape(T, H_q + 2 * H_kv, D)
    return a[:, :H_q], a[:, H_q:H_q + H_kv], a[:, H_q + H_kv:]


def rms_norm(x, weight, eps: float):
    """RMSNorm over the last axis in float64: ``x / sqrt(mean(x^2) + eps) * weight``
    (``weight`` None = all ones)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    y = x / np.sqrt(ms + float(eps))
    if weight is not None:
        y = y * np.asarray(weight, dtype=np.float64)
    return y


def _pair_index(rotary_dim: int, interleaved: bool):
    half = rotary_dim // 2
    i = np.arange(half)
    if interleaved:
        return 2 * i, 2 * i + 1
    return i, i + half


def rotate(x, pos, cos_table, sin_table, rotary_dim: int, interleaved: bool):
    """Rotate each channel pair of ``x`` (``[..., D]``, float64) by the angle of row ``pos``
    (integer array of shape ``x.shape[:-1]``) of the tables (``[max_position,
    rotary_dim/2]``).  Returns ``(rotated, mag)``, where ``mag`` is the sum of the
    magnitudes of the terms that make each output element (``|a cos| + |b sin|`` on
    rotated channels, ``|x|`` elsewhere): the scale of the rounding error any evaluation
    of this sum in finite precision carries."""
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    mag = np.abs(x).copy()
    if rotary_dim <= 0:
        return out, mag
    ia, ib = _pair_index(rotary_dim, interleaved)
    c = np.asarray(cos_table, dtype=np.float64)[pos]
    s = np.asarray(sin_table, dtype=np.float64)[pos]
    a = x[..., ia]
    b = x[..., ib]
    out[..., ia] = a * c - b * s
    out[..., ib] = b * c + a * s
    mag[..., ia] = np.abs(a * c) + np.abs(b * s)
    mag[..., ib] = np.abs(b * c) + np.abs(a * s)
    return out, mag


def round_to(x, dtype: str):
    """Round float64 values once, to nearest with ties to even, to ``dtype`` ("f32",
    "f16", "bf16"; bf16 values are returned in a float32 array)."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        # bf16: 8 significant bits over float32's exponent range.  A value of magnitude in
        # [2^(e-1), 2^e) is rounded to a multiple of 2^(e-8); below 2^-126 the spacing stays
        # that of the smallest subnormal, 2^-133.  np.rint rounds ties to even.
        _, e = np.frexp(x)
        q = np.maximum(e - 8, -133)
        with np.errstate(over="ignore"):
            r = np.ldexp(np.rint(np.ldexp(x, -q)), q)
            return r.astype(np.float32)
    raise ValueError(dtype)


def positions(cu_seqlens_q, seqlens_k, T: int, position_ids=None, rotary_offsets=None):
    """Rotary position of every row: ``position_ids[t]`` or the key position
    ``kv_len - q_len + i``, plus ``rotary_offsets[b]``.  Rows owned by no request get -1
    (a well-formed ``cu`` owns every row)."""
    cu = [int(v) for v in np.asarray(cu_seqlens_q).reshape(-1)]
    sk = [int(v) for v in np.asarray(seqlens_k).reshape(-1)]
    pos = np.full(T, -1, dtype=np.int64)
    for b in range(len(sk)):
        q_len = cu[b + 1] - cu[b]
        kv_len = sk[b] + 1
        for i in range(q_len):
            t = cu[b] + i
            base = int(position_ids[t]) if position_ids is not None else kv_len - q_len + i
            off = int(rotary_offsets[b]) if rotary_offsets is not None else 0
            pos[t] = base + off
    return pos


def qkv_prologue(*, dtype: str, cu_seqlens_q, seqlens_k, H_q: int, H_kv: int, D: int,
                 k_cache, v_cache, qkv=None, q=None, k=None, v=None,
                 qk_norm: bool = False, q_norm_weight=None, k_norm_weight=None,
                 norm_eps: float = 1e-6, cos_table=None, sin_table=None, rotary_dim: int = 0,
                 interleaved: bool = False, position_ids=None, rotary_offsets=None,
                 block_table=None, block_size=None, key_scale=None, value_scale=None,
                 committed_length=None):
    """The prologue of one step, then the cache append of its key and value rows.

    Inputs are either ``qkv`` (packed) or ``q``, ``k``, ``v`` (``[T, H, D]``), holding
    values of the activation ``dtype``.  Returns a dict with ``q_out`` (``[T, H_q, D]``,
    rounded to ``dtype``), ``k_cache`` / ``v_cache`` (after the append), ``status``, and
    the unrounded float64 results with their term magnitudes (``q64``, ``q_mag``,
    ``k64``, ``k_mag``) for the comparison of a finite-precision evaluation.
    """
    if qkv is not None:
        q, k, v = split_qkv(qkv, H_q, H_kv, D)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    T = q.shape[0]
    if qk_norm:
        q = rms_norm(q, q_norm_weight, norm_eps)
        k = rms_norm(k, k_norm_weight, norm_eps)
    status = 0
    pos = positions(cu_seqlens_q, seqlens_k, T, position_ids, rotary_offsets)
    bad = np.zeros(T, dtype=bool)
    if rotary_dim > 0:
        max_position = np.asarray(cos_table).shape[0]
        bad = (pos < 0) | (pos >= max_position)
        if bad.any():
            status |= STATUS_POSITION
        pc = np.where(bad, 0, pos)
        q, q_mag = rotate(q, np.repeat(pc[:, None], H_q, axis=1), cos_table, sin_table,
                          rotary_dim, interleaved)
        k, k_mag = rotate(k, np.repeat(pc[:, None], H_kv, axis=1), cos_table, sin_table,
                          rotary_dim, interleaved)
    else:
        q_mag, k_mag = np.abs(q), np.abs(k)
    q[bad] = 0.0
    q_mag[bad] = 0.0
    q_out = round_to(q, dtype)
    k_new = round_to(k, dtype)
    v_new = np.asarray(v)
    kc, vc, st = kv_cache_append(k_new, v_new, cu_seqlens_q, seqlens_k, k_cache, v_cache,
                                 block_table, block_size, key_scale, value_scale,
                                 committed_length=committed_length, skip_rows=bad)
    return dict(q_out=q_out, k_cache=kc, v_cache=vc, status=status | st, q64=q, q_mag=q_mag,
                k64=k, k_mag=k_mag, k_new=k_new, skipped=bad)
