"""Seeded synthetic workloads for paged and selected-token attention.

Every array is drawn with ``numpy.random.default_rng(seed)`` in a fixed order
(lengths -> block table -> selected indices -> Q -> K -> V -> sinks -> scales -> new rows),
so the GPU path and the CPU oracle see the same bytes.  Nothing here evaluates the
operators: it only decides what the caller would pass in.

Conventions (these are input conventions, not arithmetic of the method):

* ``seqlens_k[b]`` is the key count of request ``b`` after this step's rows are appended,
  minus one (the PagedAttention metadata page prints ``seqlen_k = -1`` for an empty
  request and ``seqlen_k = 1`` for a request holding two keys).
* ``past_seqlens[b]`` is the key count already in the cache before this step.
* The paged cache is ``[num_blocks, H_kv, block_size, D]`` (each block holds its slots
  head by head); a contiguous cache is ``[B, H_kv, capacity, D]`` (``block_table`` is
  ``None``).  The auxiliary store is ``[B or 1, aux_len, H_kv, D]``.
* bf16 tensors are carried as float32 arrays whose values are exactly representable in
  bf16 (``round_bf16``), because numpy has no bf16 type.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

F32, F16, BF16, I8, FP8 = 0, 1, 2, 3, 4
DTYPE_NAMES = {F32: "f32", F16: "f16", BF16: "bf16", I8: "i8", FP8: "fp8"}
QUANTISED = (I8, FP8)           # cache dtypes with per-channel key / value scales


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    out = r.view(np.float32).copy()
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.nan
    return out


def _cast(x: np.ndarray, dtype: int) -> np.ndarray:
    """Round float32 draws to the storage dtype (round to nearest even)."""
    if dtype == F32:
        return x.astype(np.float32, copy=False)
    if dtype == F16:
        return x.astype(np.float16)
    if dtype == BF16:
        return round_bf16(x)
    raise ValueError(f"not a float dtype: {dtype}")


def _normal(rng: np.random.Generator, shape, dtype: int, chunk: int = 1 << 26) -> np.ndarray:
    """N(0, 1) draws in float32, rounded to ``dtype``; generated in chunks to bound memory."""
    n = int(np.prod(shape))
    np_dtype = {F32: np.float32, F16: np.float16, BF16: np.float32}[dtype]
    out = np.empty(n, dtype=np_dtype)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = _cast(rng.standard_normal(e - s, dtype=np.float32), dtype)
    return out.reshape(shape)


def _fp8_uniform(rng: np.random.Generator, shape, chunk: int = 1 << 26) -> np.ndarray:
    """FP8 E4M3 codes (uint8 arrays) shaped like scaled activations: random sign, uniform
    3-bit mantissa, exponent field round(N(7, 1.5)) clipped to [0, 15] (values of order 1
    with tails towards 2^-6 and 448), never the NaN code (exponent 15 with mantissa 7
    becomes mantissa 6)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint8)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        m = e - s
        exp = np.clip(np.rint(rng.normal(7.0, 1.5, size=m)), 0, 15).astype(np.uint8)
        man = rng.integers(0, 8, size=m, dtype=np.uint8)
        man = np.where((exp == 15) & (man == 7), np.uint8(6), man)
        sign = rng.integers(0, 2, size=m, dtype=np.uint8) << 7
        out[s:e] = sign | (exp << 3) | man
    return out.reshape(shape)


def _quantised_uniform(rng, shape, cache_dtype):
    return _int8_uniform(rng, shape) if cache_dtype == I8 else _fp8_uniform(rng, shape)


def _int8_uniform(rng: np.random.Generator, shape, chunk: int = 1 << 26) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.int8)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = rng.integers(-127, 128, size=e - s, dtype=np.int16).astype(np.int8)
    return out.reshape(shape)


@dataclass
class PagedCase:
    """Inputs of prepare_seqlens -> kv_cache_append -> paged_attention_fwd."""
    name: str
    B: int
    T: int
    H_q: int
    H_kv: int
    D: int
    dtype: int                 # Q / output / new-row dtype
    cache_dtype: int           # equals dtype, or I8 / FP8
    q: np.ndarray              # [T, H_q, D]
    cu_seqlens_q: np.ndarray   # int32 [B+1]
    past_seqlens: np.ndarray   # int32 [B]
    seqlens_k: np.ndarray      # int32 [B]  (total keys - 1)
    k_cache: np.ndarray        # [nb, H_kv, bs, D] or [B, H_kv, cap, D]
    v_cache: np.ndarray
    block_table: Optional[np.ndarray]   # int32 [B, max_blocks_per_seq] or None
    block_size: int            # block size, or capacity for a contiguous cache
    k_new: np.ndarray          # [T, H_kv, D] rows appended by this step (dtype)
    v_new: np.ndarray
    key_scale: Optional[np.ndarray] = None    # float32 [H_kv, D] (I8 / FP8 caches)
    value_scale: Optional[np.ndarray] = None
    sinks: Optional[np.ndarray] = None        # float32 [H_q]
    scale: float = 0.0
    local_window: int = -1
    max_seqlen_q: int = 0
    max_seqlen_k: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return 0 if self.block_table is None else int(self.block_table.shape[1])


@dataclass
class SparseCase:
    """Inputs of sparse_attention_fwd (mode 0: selected main-cache rows; mode 1: local
    window of the main cache plus selected rows of an auxiliary store)."""
    name: str
    mode: int
    B: int
    T: int
    H_q: int
    H_kv: int
    D: int
    dtype: int
    cache_dtype: int
    q: np.ndarray
    cu_seqlens_q: np.ndarray
    seqlens_k: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_table: Optional[np.ndarray]
    block_size: int
    sel_idx: np.ndarray            # int32 [T, H_kv, max_selected]
    sel_count: Optional[np.ndarray]  # int32 [T, H_kv] or None
    max_selected: int
    key_scale: Optional[np.ndarray] = None
    value_scale: Optional[np.ndarray] = None
    aux_k: Optional[np.ndarray] = None   # [B or 1, aux_len, H_kv, D]
    aux_v: Optional[np.ndarray] = None
    aux_dtype: int = F16
    aux_len: int = 0
    aux_batch_stride: int = 0            # elements; 0 = one store shared by all requests
    sinks: Optional[np.ndarray] = None
    scale: float = 0.0
    local_window: int = -1
    max_seqlen_q: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return 0 if self.block_table is None else int(self.block_table.shape[1])


def _draw_sinks(rng, H_q, sinks):
    if sinks is None or sinks is False:
        return None
    if isinstance(sinks, str) and sinks == "neg_inf":
        return np.full(H_q, -np.inf, dtype=np.float32)
    if isinstance(sinks, np.ndarray):
        return sinks.astype(np.float32)
    return rng.standard_normal(H_q, dtype=np.float32)


def _draw_scales(rng, H_kv, D, lo=0.005, hi=0.02):
    ks = rng.uniform(lo, hi, size=(H_kv, D)).astype(np.float32)
    vs = rng.uniform(lo, hi, size=(H_kv, D)).astype(np.float32)
    return ks, vs


def paged_case(seed: int, *, kv_lens, q_lens, H_q: int, H_kv: int, D: int,
               block_size: int = 16, dtype: int = F16, cache_dtype: Optional[int] = None,
               num_blocks: Optional[int] = None, max_blocks_per_seq: Optional[int] = None,
               contiguous: bool = False, capacity: Optional[int] = None,
               sinks=None, scale: float = 0.0, local_window: int = -1,
               poison: bool = False, max_seqlen_q: Optional[int] = None,
               max_seqlen_k: Optional[int] = None, rng: Optional[np.random.Generator] = None,
               name: str = "paged") -> PagedCase:
    """Build a paged (or contiguous) KV-cache case.

    ``kv_lens[b]`` is the key count after this step; ``q_lens[b]`` the rows appended now
    (``past = kv_len - q_len``).  Cache slots at positions ``past..kv_len-1`` are left for
    kv_cache_append to fill (NaN when ``poison``; otherwise random).  With ``poison`` every
    slot no request references holds NaN (float caches) so a stray read shows up.
    """
    rng = rng if rng is not None else np.random.default_rng(seed)
    cache_dtype = dtype if cache_dtype is None else cache_dtype
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    B = len(kv_lens)
    assert len(q_lens) == B and np.all(q_lens <= kv_lens) and np.all(q_lens >= 0)
    past = kv_lens - q_lens
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    T = int(cu[-1])

    # block table: consecutive slices of a random permutation of the physical pool
    if contiguous:
        cap = int(capacity if capacity is not None else max(1, int(kv_lens.max(initial=1))))
        assert np.all(kv_lens <= cap)
        block_table = None
        bs = cap
        shape = (B, H_kv, cap, D)
        nblk = B
    else:
        bs = block_size
        need = [(int(L) + bs - 1) // bs for L in kv_lens]
        mbps = max_blocks_per_seq if max_blocks_per_seq is not None else max(1, max(need))
        assert max(need, default=0) <= mbps
        nblk = num_blocks if num_blocks is not None else max(1, sum(need))
        assert sum(need) <= nblk
        perm = rng.permutation(nblk).astype(np.int32)
        block_table = np.full((B, mbps), -1, dtype=np.int32)
        o = 0
        for b in range(B):
            block_table[b, :need[b]] = perm[o:o + need[b]]
            o += need[b]
        shape = (nblk, H_kv, bs, D)

    q = _normal(rng, (T, H_q, D), dtype)
    if cache_dtype in QUANTISED:
        k_cache = _quantised_uniform(rng, shape, cache_dtype)
        v_cache = _quantised_uniform(rng, shape, cache_dtype)
    else:
        k_cache = _normal(rng, shape, cache_dtype)
        v_cache = _normal(rng, shape, cache_dtype)
    sink_arr = _draw_sinks(rng, H_q, sinks)
    key_scale = value_scale = None
    if cache_dtype in QUANTISED:
        key_scale, value_scale = _draw_scales(rng, H_kv, D)
    # rows appended by this step
    if cache_dtype in QUANTISED:
        # values around the representable range so quantisation hits rounding and clamping
        # (INT8: +-127; FP8 E4M3: +-448)
        spread = 45.0 if cache_dtype == I8 else 150.0
        k_new = _cast(rng.standard_normal((T, H_kv, D), dtype=np.float32), dtype)
        v_new = _cast(rng.standard_normal((T, H_kv, D), dtype=np.float32), dtype)
        k_new = _cast(k_new.astype(np.float32) * (spread * key_scale[None]), dtype)
        v_new = _cast(v_new.astype(np.float32) * (spread * value_scale[None]), dtype)
    else:
        k_new = _normal(rng, (T, H_kv, D), cache_dtype)
        v_new = _normal(rng, (T, H_kv, D), cache_dtype)

    def slot_of(b, j):
        if block_table is None:
            return b, j
        return int(block_table[b, j // bs]), j % bs

    if poison and cache_dtype != I8:
        live = np.zeros((shape[0], shape[2]), dtype=bool)
        for b in range(B):
            for j in range(int(past[b])):
                live[slot_of(b, j)] = True
        dead = ~live
        bad = np.uint8(0x7F) if cache_dtype == FP8 else np.nan   # the E4M3 NaN code
        k_cache.transpose(0, 2, 1, 3)[dead] = bad
        v_cache.transpose(0, 2, 1, 3)[dead] = bad

    if max_seqlen_q is None:
        max_seqlen_q = int(q_lens.max(initial=0))
    if max_seqlen_k is None:
        max_seqlen_k = int(kv_lens.max(initial=0))
    return PagedCase(
        name=name, B=B, T=T, H_q=H_q, H_kv=H_kv, D=D, dtype=dtype, cache_dtype=cache_dtype,
        q=q, cu_seqlens_q=cu, past_seqlens=past.astype(np.int32),
        seqlens_k=(kv_lens - 1).astype(np.int32), k_cache=k_cache, v_cache=v_cache,
        block_table=block_table, block_size=bs, k_new=k_new, v_new=v_new,
        key_scale=key_scale, value_scale=value_scale, sinks=sink_arr,
        scale=float(scale), local_window=int(local_window),
        max_seqlen_q=int(max_seqlen_q), max_seqlen_k=int(max_seqlen_k))


@dataclass
class PrologueCase:
    """Inputs of the QKV prologue (split, QK RMSNorm, rotary embedding, cache append)."""
    name: str
    B: int
    T: int
    H_q: int
    H_kv: int
    D: int
    dtype: int
    cache_dtype: int
    cu_seqlens_q: np.ndarray
    past_seqlens: np.ndarray
    seqlens_k: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_table: Optional[np.ndarray]
    block_size: int
    key_scale: Optional[np.ndarray]
    value_scale: Optional[np.ndarray]
    qkv: Optional[np.ndarray]          # [T, (H_q + 2 H_kv) * D] when packed, else None
    q: np.ndarray                      # [T, H_q, D] (views of qkv when packed)
    k: np.ndarray                      # [T, H_kv, D]
    v: np.ndarray
    qk_norm: bool
    q_norm_weight: Optional[np.ndarray]   # float32 [D]
    k_norm_weight: Optional[np.ndarray]
    norm_eps: float
    cos_table: Optional[np.ndarray]       # float32 [max_position, rotary_dim / 2]
    sin_table: Optional[np.ndarray]
    rotary_dim: int
    interleaved: bool
    position_ids: Optional[np.ndarray]    # int32 [T]
    rotary_offsets: Optional[np.ndarray]  # int32 [B]
    committed_length: Optional[np.ndarray] = None
    extra: dict = field(default_factory=dict)

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return 0 if self.block_table is None else int(self.block_table.shape[1])

    @property
    def max_position(self) -> int:
        return 0 if self.cos_table is None else int(self.cos_table.shape[0])


def rotary_tables(max_position: int, rotary_dim: int, base: float = 10000.0):
    """Rotary cos / sin tables as a model ships them (an input of the prologue, not part
    of it): angle(pos, i) = pos * base^(-2i / rotary_dim), evaluated in float64 and stored
    as float32 [max_position, rotary_dim / 2]."""
    half = rotary_dim // 2
    theta = base ** (-2.0 * np.arange(half, dtype=np.float64) / rotary_dim)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * theta[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def prologue_case(seed: int, *, kv_lens, q_lens, H_q: int, H_kv: int, D: int, dtype: int = F16,
                  cache_dtype: Optional[int] = None, packed: bool = False, rotary_dim: int = 0,
                  interleaved: bool = False, max_position: Optional[int] = None,
                  qk_norm: bool = False, norm_weights: bool = True, norm_eps: float = 1e-6,
                  explicit_positions: bool = False, offsets: bool = False,
                  block_size: int = 16, contiguous: bool = False, num_blocks: Optional[int] = None,
                  poison: bool = True, q_scale: float = 1.0, name: str = "prologue") -> PrologueCase:
    """A prologue case: the caches, block table and new rows of ``paged_case`` (same
    draws), the new rows as raw activations (packed into one ``[T, (H_q + 2 H_kv) D]``
    array when ``packed``), norm weights U[0.5, 2], rotary tables of base 10000, and
    optionally explicit positions (U[0, max_position)) and per-request offsets U{0..31}.
    ``q_scale`` multiplies the raw query and key activations (pre-norm activations of a
    real model are not unit-scale)."""
    rng = np.random.default_rng(seed)
    pc = paged_case(seed, kv_lens=kv_lens, q_lens=q_lens, H_q=H_q, H_kv=H_kv, D=D,
                    block_size=block_size, dtype=dtype, cache_dtype=cache_dtype,
                    num_blocks=num_blocks, contiguous=contiguous, poison=poison, rng=rng)
    T = pc.T
    q = _cast(pc.q.astype(np.float32) * np.float32(q_scale), dtype)
    k = _cast(pc.k_new.astype(np.float32) * np.float32(q_scale if qk_norm else 1.0), dtype)
    v = pc.v_new
    qkv = None
    if packed:
        qkv = np.concatenate([q.reshape(T, -1), k.reshape(T, -1), v.reshape(T, -1)], axis=1)
        qkv = np.ascontiguousarray(qkv)
        a = qkv.reshape(T, H_q + 2 * H_kv, D)
        q, k, v = a[:, :H_q], a[:, H_q:H_q + H_kv], a[:, H_q + H_kv:]
    qw = kw = None
    if qk_norm and norm_weights:
        qw = rng.uniform(0.5, 2.0, size=D).astype(np.float32)
        kw = rng.uniform(0.5, 2.0, size=D).astype(np.float32)
    cos = sin = None
    if max_position is None:
        max_position = int(np.max(kv_lens)) + 64
    if rotary_dim > 0:
        cos, sin = rotary_tables(max_position, rotary_dim)
    pos_ids = None
    if explicit_positions:
        pos_ids = rng.integers(0, max_position - 32, size=T).astype(np.int32)
    offs = None
    if offsets:
        offs = rng.integers(0, 32, size=pc.B).astype(np.int32)
    return PrologueCase(
        name=name, B=pc.B, T=T, H_q=H_q, H_kv=H_kv, D=D, dtype=dtype, cache_dtype=pc.cache_dtype,
        cu_seqlens_q=pc.cu_seqlens_q, past_seqlens=pc.past_seqlens, seqlens_k=pc.seqlens_k,
        k_cache=pc.k_cache, v_cache=pc.v_cache, block_table=pc.block_table,
        block_size=pc.block_size, key_scale=pc.key_scale, value_scale=pc.value_scale,
        qkv=qkv, q=q, k=k, v=v, qk_norm=qk_norm, q_norm_weight=qw, k_norm_weight=kw,
        norm_eps=float(norm_eps), cos_table=cos, sin_table=sin, rotary_dim=int(rotary_dim),
        interleaved=bool(interleaved), position_ids=pos_ids, rotary_offsets=offs)


@dataclass
class TopkCase:
    """Inputs of the TopK selection: per-key scores of each (row, KV head)."""
    name: str
    B: int
    T: int
    H_kv: int
    L: int
    scores: np.ndarray          # float32 [T, H_kv, L]
    cu_seqlens_q: np.ndarray
    seqlens_k: np.ndarray
    k: int
    tail: int
    capacity: int


def topk_case(seed: int, *, kv_lens, q_lens, H_kv: int, L: Optional[int] = None, k: int,
              tail: int = 0, capacity: Optional[int] = None, ties: float = 0.0,
              specials: float = 0.0, name: str = "topk") -> TopkCase:
    """Scores N(0, 1) in float32 (an indexer's output stands in as synthetic values); a
    fraction ``ties`` is rounded to multiples of 1/4 (many equal scores), a fraction
    ``specials`` replaced by NaN, +-inf or +-0.0."""
    rng = np.random.default_rng(seed)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    B = len(kv_lens)
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    T = int(cu[-1])
    L = int(L if L is not None else max(1, int(kv_lens.max(initial=1))))
    scores = rng.standard_normal((T, H_kv, L), dtype=np.float32)
    if ties > 0:
        m = rng.random(scores.shape) < ties
        scores[m] = np.round(scores[m] * 4) / 4
    if specials > 0:
        m = rng.random(scores.shape) < specials
        pool = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0], dtype=np.float32)
        scores[m] = pool[rng.integers(0, len(pool), size=int(m.sum()))]
    return TopkCase(name=name, B=B, T=T, H_kv=H_kv, L=L, scores=scores, cu_seqlens_q=cu,
                    seqlens_k=(kv_lens - 1).astype(np.int32), k=int(k), tail=int(tail),
                    capacity=int(capacity if capacity is not None else k))


def _selected_indices(rng, T, H_kv, max_selected, counts, hi_of_row, oor_frac=0.0):
    """Per (row, kv head): ``counts`` distinct indices from [0, hi), shuffled, padded with -1.
    A fraction ``oor_frac`` of in-count entries is replaced with out-of-range values, half
    at or above ``hi`` and half at or below -2."""
    sel = np.full((T, H_kv, max_selected), -1, dtype=np.int32)
    for r in range(T):
        hi = int(hi_of_row[r])
        for c in range(H_kv):
            n = int(min(counts[r, c], max_selected, max(hi, 0)))
            if n > 0:
                sel[r, c, :n] = rng.choice(hi, size=n, replace=False)
    if oor_frac > 0:
        for r in range(T):
            for c in range(H_kv):
                n = int(min(max(counts[r, c], 0), max_selected))
                if n == 0:
                    continue
                pick = rng.random(n) < oor_frac
                k = int(pick.sum())
                if k:
                    hi = int(hi_of_row[r])
                    up = rng.random(k) < 0.5
                    vals = np.where(up, hi + rng.integers(0, 1 << 20, size=k),
                                    -2 - rng.integers(0, 1 << 20, size=k))
                    sel[r, c, :n][pick] = vals.astype(np.int32)
    return sel


def sparse_selected_case(seed: int, *, B: int, S_q: int, H_q: int, H_kv: int, D: int,
                         capacity: int, kv_lens=None, max_selected: int = 2048,
                         counts=None, dtype: int = F16, cache_dtype: Optional[int] = None,
                         sinks=None, scale: float = 0.0, oor_frac: float = 0.0,
                         pass_count: bool = True, poison: bool = False,
                         block_size: Optional[int] = None,
                         name: str = "selected") -> SparseCase:
    """Mode 0: every row attends to its selected main-cache positions (count per
    (row, kv head), indices drawn without replacement from [0, kv_len), -1 padding).
    ``block_size`` switches the main cache to a paged layout with a random block table."""
    rng = np.random.default_rng(seed)
    cache_dtype = dtype if cache_dtype is None else cache_dtype
    kv_lens = np.full(B, capacity, dtype=np.int64) if kv_lens is None else np.asarray(kv_lens)
    T = B * S_q
    cu = (np.arange(B + 1) * S_q).astype(np.int32)
    row_req = np.repeat(np.arange(B), S_q)
    if counts is None:
        counts = rng.integers(0, max_selected + 1, size=(T, H_kv))
    counts = np.asarray(counts, dtype=np.int64).reshape(T, H_kv)
    bt = None
    if block_size is not None:
        need = [(int(L) + block_size - 1) // block_size for L in kv_lens]
        mbps = max(1, (capacity + block_size - 1) // block_size)
        nblk = max(1, sum(need))
        perm = rng.permutation(nblk).astype(np.int32)
        bt = np.full((B, mbps), -1, dtype=np.int32)
        o = 0
        for b in range(B):
            bt[b, :need[b]] = perm[o:o + need[b]]
            o += need[b]
        shape = (nblk, H_kv, block_size, D)
        bsz = block_size
    else:
        shape = (B, H_kv, capacity, D)
        bsz = capacity
    sel = _selected_indices(rng, T, H_kv, max_selected, counts, kv_lens[row_req], oor_frac)
    q = _normal(rng, (T, H_q, D), dtype)
    if cache_dtype in QUANTISED:
        k_cache = _quantised_uniform(rng, shape, cache_dtype)
        v_cache = _quantised_uniform(rng, shape, cache_dtype)
    else:
        k_cache = _normal(rng, shape, cache_dtype)
        v_cache = _normal(rng, shape, cache_dtype)
    sink_arr = _draw_sinks(rng, H_q, sinks)
    ks = vs = None
    if cache_dtype in QUANTISED:
        ks, vs = _draw_scales(rng, H_kv, D)
    if poison and cache_dtype != I8:
        # every main-cache row no (row, kv head) of its request selects becomes NaN
        keep = np.zeros(shape[:3], dtype=bool)
        for r in range(T):
            b = int(row_req[r])
            for c in range(H_kv):
                n = int(min(max(counts[r, c], 0), max_selected))
                js = sel[r, c, :n]
                js = js[(js >= 0) & (js < kv_lens[b])]
                if bt is None:
                    keep[b, c, js] = True
                else:
                    keep[bt[b, js // bsz], c, js % bsz] = True
        bad = np.uint8(0x7F) if cache_dtype == FP8 else np.nan   # the E4M3 NaN code
        k_cache[~keep] = bad
        v_cache[~keep] = bad
    return SparseCase(
        name=name, mode=0, B=B, T=T, H_q=H_q, H_kv=H_kv, D=D, dtype=dtype,
        cache_dtype=cache_dtype, q=q, cu_seqlens_q=cu,
        seqlens_k=(kv_lens - 1).astype(np.int32), k_cache=k_cache, v_cache=v_cache,
        block_table=bt, block_size=bsz, sel_idx=sel,
        sel_count=counts.astype(np.int32) if pass_count else None,
        max_selected=max_selected, key_scale=ks, value_scale=vs, sinks=sink_arr,
        scale=float(scale), max_seqlen_q=S_q)


def sparse_local_aux_case(seed: int, *, B: int, S_q: int, H_q: int, H_kv: int, D: int,
                          capacity: int, kv_lens=None, local_window: int = 128,
                          aux_len: int = 4096, n_selected: int = 1024,
                          max_selected: Optional[int] = None, counts=None,
                          dtype: int = F16, cache_dtype: int = I8, aux_dtype: Optional[int] = None,
                          sinks=True, scale: float = 0.0, shared_aux: bool = False,
                          oor_frac: float = 0.0, name: str = "local_aux") -> SparseCase:
    """Mode 1: each row attends to the last ``local_window`` main-cache positions up to its
    own, plus ``n_selected`` rows of an auxiliary K/V store (drawn without replacement)."""
    rng = np.random.default_rng(seed)
    aux_dtype = dtype if aux_dtype is None else aux_dtype
    max_selected = n_selected if max_selected is None else max_selected
    kv_lens = np.full(B, capacity, dtype=np.int64) if kv_lens is None else np.asarray(kv_lens)
    T = B * S_q
    cu = (np.arange(B + 1) * S_q).astype(np.int32)
    if counts is None:
        counts = np.full((T, H_kv), n_selected, dtype=np.int64)
    counts = np.asarray(counts, dtype=np.int64).reshape(T, H_kv)
    sel = _selected_indices(rng, T, H_kv, max_selected, counts, np.full(T, aux_len), oor_frac)
    q = _normal(rng, (T, H_q, D), dtype)
    shape = (B, H_kv, capacity, D)
    if cache_dtype in QUANTISED:
        k_cache = _quantised_uniform(rng, shape, cache_dtype)
        v_cache = _quantised_uniform(rng, shape, cache_dtype)
    else:
        k_cache = _normal(rng, shape, cache_dtype)
        v_cache = _normal(rng, shape, cache_dtype)
    nb_aux = 1 if shared_aux else B
    aux_k = _normal(rng, (nb_aux, aux_len, H_kv, D), aux_dtype)
    aux_v = _normal(rng, (nb_aux, aux_len, H_kv, D), aux_dtype)
    sink_arr = _draw_sinks(rng, H_q, sinks)
    ks = vs = None
    if cache_dtype in QUANTISED:
        ks, vs = _draw_scales(rng, H_kv, D)
    return SparseCase(
        name=name, mode=1, B=B, T=T, H_q=H_q, H_kv=H_kv, D=D, dtype=dtype,
        cache_dtype=cache_dtype, q=q, cu_seqlens_q=cu,
        seqlens_k=(kv_lens - 1).astype(np.int32), k_cache=k_cache, v_cache=v_cache,
        block_table=None, block_size=capacity, sel_idx=sel, sel_count=counts.astype(np.int32),
        max_selected=max_selected, key_scale=ks, value_scale=vs, aux_k=aux_k, aux_v=aux_v,
        aux_dtype=aux_dtype, aux_len=aux_len,
        aux_batch_stride=0 if shared_aux else aux_len * H_kv * D,
        sinks=sink_arr, scale=float(scale), local_window=local_window, max_seqlen_q=S_q)


# ----------------------------------------------------------------------------------------
# The five workloads (tiny paged decode, GQA paged decode, windowed paged prefill,
# selected-token grouped decode, local-plus-selected INT8).  Seed = 1000 + workload number.
# ----------------------------------------------------------------------------------------

def config_tiny_paged_decode(poison: bool = False) -> PagedCase:
    """fp32, B=2, one new row each, H 4/2, D 64, block 16, key counts 37 and 100, the
    block table a seeded permutation of 10 physical blocks, scale 1/8, no sink/window."""
    rng = np.random.default_rng(1001)
    return paged_case(1001, kv_lens=[37, 100], q_lens=[1, 1], H_q=4, H_kv=2, D=64,
                      block_size=16, dtype=F32, num_blocks=10, scale=0.125, sinks=None,
                      poison=poison, rng=rng, name="tiny_paged_decode_f32")


def config_gqa_paged_decode(poison: bool = False, B: int = 32, max_len: int = 8192,
                            seed: int = 1002, cache_dtype: int = F16) -> PagedCase:
    """fp16, B=32, one new row per non-empty request, H 64/8, D 64, block 16, key counts
    ~ U{0..8192} with one request forced to 0 (an empty request owns no rows: its
    seqlens_k is -1), a 20000-block pool, 512 table entries per request, sinks ~ N(0,1).
    ``cache_dtype`` I8 / FP8 stores the cache as codes with per-channel scales."""
    rng = np.random.default_rng(seed)
    L = rng.integers(0, max_len + 1, size=B)
    L[int(rng.integers(0, B))] = 0
    q_lens = (L > 0).astype(np.int64)
    return paged_case(seed, kv_lens=L, q_lens=q_lens, H_q=64, H_kv=8, D=64, block_size=16,
                      dtype=F16, cache_dtype=cache_dtype,
                      num_blocks=max(20000, int(((L + 15) // 16).sum())),
                      max_blocks_per_seq=(max_len + 15) // 16, sinks=True,
                      scale=1.0 / 8.0, poison=poison, max_seqlen_k=max_len, rng=rng,
                      name="gqa_paged_decode_f16")


def config_paged_prefill_window(window: int = 128, poison: bool = False,
                                lens=(1024, 512, 2048, 1536),
                                cache_dtype: Optional[int] = None) -> PagedCase:
    """fp16 fresh prompts (past = 0), B=4 with query lengths 1024, 512, 2048, 1536 in that
    order, H 64/8, D 64, block 16, a 1024-block pool, window 128, sinks ~ N(0,1)."""
    rng = np.random.default_rng(1003)
    return paged_case(1003, kv_lens=list(lens), q_lens=list(lens), H_q=64, H_kv=8, D=64,
                      block_size=16, dtype=F16, cache_dtype=cache_dtype,
                      num_blocks=max(1024, sum((x + 15) // 16 for x in lens)),
                      sinks=True, scale=1.0 / 8.0,
                      local_window=window, poison=poison, rng=rng,
                      name=(f"paged_prefill_w{window}_f16" if window > 0 else "paged_prefill_f16")
                      + {None: "", F16: "", I8: "_int8_cache", FP8: "_fp8_cache"}.get(cache_dtype, ""))


def config_selected_decode(sinks: bool = True, poison: bool = False, B: int = 16,
                           capacity: int = 65536) -> SparseCase:
    """fp16, B=16 with 8 rows each, H 48/4 (12 query heads per KV head), D 128, contiguous
    65536-token cache, up to 2048 selected positions per (row, KV head) with counts
    ~ U{0..2048}, -1 padding, 1% of in-count entries out of range, optional sink."""
    return sparse_selected_case(1004, B=B, S_q=8, H_q=48, H_kv=4, D=128, capacity=capacity,
                                max_selected=2048, dtype=F16, sinks=sinks, scale=1.0 / np.sqrt(128.0),
                                oor_frac=0.01, poison=poison,
                                name="selected_decode_f16" + ("_sink" if sinks else ""))


def config_local_plus_aux_int8(B: int = 8, capacity: int = 32768) -> SparseCase:
    """INT8 main cache (values U{-127..127}, per-channel scales U[0.005, 0.02]) of 32768
    tokens, window 128, plus 1024 selected rows of a 4096-token fp16 auxiliary store per
    request; B=8 with 8 rows each, H 48/4, D 128, sinks ~ N(0,1), one joint softmax."""
    return sparse_local_aux_case(1005, B=B, S_q=8, H_q=48, H_kv=4, D=128, capacity=capacity,
                                 local_window=128, aux_len=4096, n_selected=1024, dtype=F16,
                                 cache_dtype=I8, aux_dtype=F16, sinks=True,
                                 scale=1.0 / np.sqrt(128.0), name="local_plus_aux_int8")
