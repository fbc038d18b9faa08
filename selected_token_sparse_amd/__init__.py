"""Paged and selected-token sparse attention for MI355X (gfx950).

Thin Python binding over the C ABI of ``libspattn.so`` (declared in ``include/spattn.h``):
the functions below only turn torch tensors (device memory) into pointers and sizes and
pass the current HIP stream.  Every step runs in the library's HIP kernels; if the
library is missing the calls raise, there is no CPU path.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib

F32, F16, BF16, I8, FP8 = 0, 1, 2, 3, 4  # FP8: E4M3 (caches only)
KIND_PAGED, KIND_SELECTED, KIND_LOCAL_AUX = 0, 1, 2

STATUS_BAD_CU = 1 << 0
STATUS_Q_BOUND = 1 << 1
STATUS_K_BOUND = 1 << 2
STATUS_CAPACITY = 1 << 3
STATUS_BAD_BLOCK = 1 << 4
STATUS_BAD_INDEX = 1 << 5
STATUS_BAD_COUNT = 1 << 6
STATUS_SHORT_KV = 1 << 7
STATUS_CURSOR = 1 << 8
STATUS_POSITION = 1 << 9

_ERRORS = {-1: "null pointer", -2: "shape", -3: "dtype", -4: "unsupported", -5: "workspace too small",
           -6: "launch failed"}

_DTYPES = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16, torch.int8: I8,
           torch.float8_e4m3fn: FP8}


class SpattnError(RuntimeError):
    def __init__(self, fn: str, rc: int):
        super().__init__(f"{fn} returned {rc} ({_ERRORS.get(rc, 'error')})")
        self.rc = rc


def _dt(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def _ptr(t: Optional[torch.Tensor], what: str = "tensor") -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t.data_ptr()


def _i32(t: Optional[torch.Tensor], what: str) -> Optional[int]:
    if t is not None and t.dtype != torch.int32:
        raise TypeError(f"{what} must be int32")
    return _ptr(t, what)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _check(fn: str, rc: int) -> int:
    if rc != 0:
        raise SpattnError(fn, rc)
    return rc


def _cache_dims(k_cache: torch.Tensor, block_table: Optional[torch.Tensor]):
    """(num_blocks, block_size or capacity, max_blocks_per_seq) of a cache tensor laid out
    [num_blocks, H_kv, block_size, D] (paged) or [B, H_kv, capacity, D] (contiguous)."""
    nb, bs = int(k_cache.shape[0]), int(k_cache.shape[2])
    mbps = int(block_table.shape[1]) if block_table is not None else 0
    return nb, bs, mbps


def prepare_seqlens(cu_seqlens_q: torch.Tensor, past_seqlens: torch.Tensor, T: int,
                    seqlens_q: torch.Tensor, seqlens_k: torch.Tensor,
                    token_req: Optional[torch.Tensor] = None,
                    token_pos: Optional[torch.Tensor] = None,
                    status: Optional[torch.Tensor] = None) -> None:
    """Device metadata: seqlens_q, seqlens_k (total - 1) and per-token request/position."""
    B = int(past_seqlens.shape[0])
    lib = _lib.load()
    _check("prepare_seqlens", lib.prepare_seqlens(
        _i32(cu_seqlens_q, "cu_seqlens_q"), _i32(past_seqlens, "past_seqlens"), B, int(T),
        _i32(seqlens_q, "seqlens_q"), _i32(seqlens_k, "seqlens_k"), _i32(token_req, "token_req"),
        _i32(token_pos, "token_pos"), _i32(status, "status"), _stream(cu_seqlens_q)))


def kv_cache_append(k_new: torch.Tensor, v_new: torch.Tensor, cu_seqlens_q: torch.Tensor,
                    seqlens_k: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                    block_table: Optional[torch.Tensor] = None,
                    key_scale: Optional[torch.Tensor] = None,
                    value_scale: Optional[torch.Tensor] = None,
                    status: Optional[torch.Tensor] = None,
                    committed_length: Optional[torch.Tensor] = None) -> None:
    """Write this step's K/V rows ([T, H_kv, D]) into the cache in place.  With
    `committed_length` ([B] int32), a request whose cursor disagrees with its append
    position is flagged (STATUS_CURSOR) and left unwritten."""
    T, H_kv, D = (int(x) for x in k_new.shape)
    B = int(seqlens_k.shape[0])
    nb, bs, mbps = _cache_dims(k_cache, block_table)
    lib = _lib.load()
    _check("kv_cache_append", lib.kv_cache_append(
        _ptr(k_new, "k_new"), _ptr(v_new, "v_new"), _dt(k_new), _i32(cu_seqlens_q, "cu_seqlens_q"),
        _i32(seqlens_k, "seqlens_k"), B, T, _ptr(k_cache, "k_cache"), _ptr(v_cache, "v_cache"),
        _dt(k_cache), _i32(block_table, "block_table"), mbps, bs, nb,
        _ptr(key_scale, "key_scale"), _ptr(value_scale, "value_scale"), H_kv, D,
        _i32(committed_length, "committed_length"), _i32(status, "status"), _stream(k_new)))


def prepare_and_append(cu_seqlens_q: torch.Tensor, past_seqlens: torch.Tensor, T: int,
                       seqlens_q: torch.Tensor, seqlens_k: torch.Tensor, k_new: torch.Tensor,
                       v_new: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                       block_table: Optional[torch.Tensor] = None,
                       token_req: Optional[torch.Tensor] = None,
                       token_pos: Optional[torch.Tensor] = None,
                       key_scale: Optional[torch.Tensor] = None,
                       value_scale: Optional[torch.Tensor] = None,
                       committed_length: Optional[torch.Tensor] = None,
                       status: Optional[torch.Tensor] = None) -> None:
    """prepare_seqlens then kv_cache_append with the seqlens_k it produced, in one launch."""
    B = int(past_seqlens.shape[0])
    _, H_kv, D = (int(x) for x in k_new.shape)
    nb, bs, mbps = _cache_dims(k_cache, block_table)
    lib = _lib.load()
    _check("prepare_and_append", lib.prepare_and_append(
        _i32(cu_seqlens_q, "cu_seqlens_q"), _i32(past_seqlens, "past_seqlens"), B, int(T),
        _i32(seqlens_q, "seqlens_q"), _i32(seqlens_k, "seqlens_k"), _i32(token_req, "token_req"),
        _i32(token_pos, "token_pos"), _ptr(k_new, "k_new"), _ptr(v_new, "v_new"), _dt(k_new),
        _ptr(k_cache, "k_cache"), _ptr(v_cache, "v_cache"), _dt(k_cache),
        _i32(block_table, "block_table"), mbps, bs, nb, _ptr(key_scale, "key_scale"),
        _ptr(value_scale, "value_scale"), H_kv, D, _i32(committed_length, "committed_length"),
        _i32(status, "status"), _stream(cu_seqlens_q)))


def qkv_prologue(q_out: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                 cu_seqlens_q: torch.Tensor, seqlens_k: torch.Tensor, *, H_q: int, H_kv: int,
                 qkv: Optional[torch.Tensor] = None, q: Optional[torch.Tensor] = None,
                 k: Optional[torch.Tensor] = None, v: Optional[torch.Tensor] = None,
                 qk_norm: bool = False, q_norm_weight: Optional[torch.Tensor] = None,
                 k_norm_weight: Optional[torch.Tensor] = None, norm_eps: float = 1e-6,
                 rotary_dim: int = 0, interleaved: bool = False,
                 cos_table: Optional[torch.Tensor] = None, sin_table: Optional[torch.Tensor] = None,
                 position_ids: Optional[torch.Tensor] = None,
                 rotary_offsets: Optional[torch.Tensor] = None,
                 block_table: Optional[torch.Tensor] = None,
                 key_scale: Optional[torch.Tensor] = None,
                 value_scale: Optional[torch.Tensor] = None,
                 committed_length: Optional[torch.Tensor] = None,
                 status: Optional[torch.Tensor] = None) -> None:
    """Split (packed `qkv` [T, (H_q + 2 H_kv) * D], or `q`, `k`, `v`), QK RMSNorm, rotary
    embedding; the queries go to `q_out` [T, H_q, D], the key and value rows into the cache
    as kv_cache_append stores them."""
    T, _, D = (int(x) for x in q_out.shape)
    B = int(seqlens_k.shape[0])
    src = qkv if qkv is not None else q
    if src is None or src.dtype != q_out.dtype:
        raise TypeError("the input rows and q_out must share one dtype")
    for what, t in (("q_norm_weight", q_norm_weight), ("k_norm_weight", k_norm_weight),
                    ("cos_table", cos_table), ("sin_table", sin_table)):
        if t is not None and t.dtype != torch.float32:
            raise TypeError(f"{what} must be float32")
    max_position = int(cos_table.shape[0]) if cos_table is not None else 0
    nb, bs, mbps = _cache_dims(k_cache, block_table)
    lib = _lib.load()
    _check("qkv_prologue", lib.qkv_prologue(
        _ptr(qkv, "qkv"), _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _dt(q_out),
        _i32(cu_seqlens_q, "cu_seqlens_q"), _i32(seqlens_k, "seqlens_k"), B, T, int(H_q),
        int(H_kv), D, int(bool(qk_norm)), _ptr(q_norm_weight, "q_norm_weight"),
        _ptr(k_norm_weight, "k_norm_weight"), float(norm_eps), int(rotary_dim),
        int(bool(interleaved)), _ptr(cos_table, "cos_table"), _ptr(sin_table, "sin_table"),
        max_position, _i32(position_ids, "position_ids"), _i32(rotary_offsets, "rotary_offsets"),
        _ptr(q_out, "q_out"), _ptr(k_cache, "k_cache"), _ptr(v_cache, "v_cache"), _dt(k_cache),
        _i32(block_table, "block_table"), mbps, bs, nb, _ptr(key_scale, "key_scale"),
        _ptr(value_scale, "value_scale"), _i32(committed_length, "committed_length"),
        _i32(status, "status"), _stream(q_out)))


def topk_select(scores: torch.Tensor, cu_seqlens_q: torch.Tensor, seqlens_k: torch.Tensor,
                k: int, sel_idx: torch.Tensor, sel_count: torch.Tensor, tail: int = 0,
                status: Optional[torch.Tensor] = None) -> None:
    """The k highest-scoring causal key positions of every (row, KV head) of `scores`
    [T, H_kv, L] (float32), the last `tail` always kept, into `sel_idx` [T, H_kv, capacity]
    (ascending, -1 padded) and `sel_count` [T, H_kv]."""
    if scores.dtype != torch.float32:
        raise TypeError("scores must be float32")
    T, H_kv, L = (int(x) for x in scores.shape)
    capacity = int(sel_idx.shape[-1])
    B = int(seqlens_k.shape[0])
    lib = _lib.load()
    _check("topk_select", lib.topk_select(
        _ptr(scores, "scores"), L, _i32(cu_seqlens_q, "cu_seqlens_q"), _i32(seqlens_k, "seqlens_k"),
        B, T, H_kv, int(k), int(tail), _i32(sel_idx, "sel_idx"), capacity,
        _i32(sel_count, "sel_count"), _i32(status, "status"), _stream(scores)))


def attention_workspace_bytes(kind: int, dtype: int, B: int, T: int, max_seqlen_q: int,
                              max_seqlen_k: int, max_selected: int, local_window: int,
                              H_q: int, H_kv: int, D: int) -> int:
    n = _lib.load().attention_workspace_bytes(kind, dtype, B, T, max_seqlen_q, max_seqlen_k,
                                              max_selected, local_window, H_q, H_kv, D)
    if n == (1 << 64) - 1:
        raise SpattnError("attention_workspace_bytes", -2)
    return int(n)


def _ws_need(*args) -> int:
    """Workspace bytes for a call, or 0 when the arguments are invalid (the call itself
    then reports the precise error)."""
    n = _lib.load().attention_workspace_bytes(*args)
    return 0 if n == (1 << 64) - 1 else int(n)


def _workspace(ws: Optional[torch.Tensor], nbytes: int, like: torch.Tensor):
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=like.device)
    return ws, int(ws.numel() * ws.element_size())


def paged_attention_fwd(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                        cu_seqlens_q: torch.Tensor, seqlens_k: torch.Tensor, max_seqlen_q: int,
                        max_seqlen_k: int, out: torch.Tensor,
                        block_table: Optional[torch.Tensor] = None,
                        key_scale: Optional[torch.Tensor] = None,
                        value_scale: Optional[torch.Tensor] = None, scale: float = 0.0,
                        is_causal: int = 1, local_window: int = -1,
                        sinks: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None,
                        status: Optional[torch.Tensor] = None) -> None:
    """Causal attention of packed q [T, H_q, D] over a paged/contiguous cache into out."""
    T, H_q, D = (int(x) for x in q.shape)
    H_kv = int(k_cache.shape[1])
    B = int(seqlens_k.shape[0])
    nb, bs, mbps = _cache_dims(k_cache, block_table)
    lib = _lib.load()
    need = _ws_need(KIND_PAGED, _dt(q), B, T, int(max_seqlen_q), int(max_seqlen_k), 0,
                    int(local_window), H_q, H_kv, D)
    ws, ws_bytes = _workspace(workspace, need, q)
    _check("paged_attention_fwd", lib.paged_attention_fwd(
        _ptr(q, "q"), _dt(q), _ptr(k_cache, "k_cache"), _ptr(v_cache, "v_cache"), _dt(k_cache),
        _i32(block_table, "block_table"), mbps, bs, nb, _ptr(key_scale, "key_scale"),
        _ptr(value_scale, "value_scale"), _i32(cu_seqlens_q, "cu_seqlens_q"),
        _i32(seqlens_k, "seqlens_k"), B, T, int(max_seqlen_q), int(max_seqlen_k), H_q, H_kv, D,
        float(scale), int(is_causal), int(local_window), _ptr(sinks, "sinks"), _ptr(out, "out"),
        _ptr(ws, "workspace"), ws_bytes, _i32(status, "status"), _stream(q)))


def paged_decode_step(cu_seqlens_q: torch.Tensor, past_seqlens: torch.Tensor, T: int,
                      seqlens_q: torch.Tensor, seqlens_k: torch.Tensor, q: torch.Tensor,
                      k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
                      v_cache: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
                      out: torch.Tensor, block_table: Optional[torch.Tensor] = None,
                      key_scale: Optional[torch.Tensor] = None,
                      value_scale: Optional[torch.Tensor] = None, scale: float = 0.0,
                      local_window: int = -1, sinks: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None,
                      committed_length: Optional[torch.Tensor] = None,
                      status: Optional[torch.Tensor] = None) -> None:
    """prepare_seqlens + kv_cache_append + paged_attention_fwd of a decode step in one call.
    With `committed_length` ([B] int32), a request whose cursor disagrees with its past
    length is flagged (STATUS_CURSOR) and appends nothing."""
    B = int(past_seqlens.shape[0])
    _, H_q, D = (int(x) for x in q.shape)
    H_kv = int(k_cache.shape[1])
    nb, bs, mbps = _cache_dims(k_cache, block_table)
    lib = _lib.load()
    need = _ws_need(KIND_PAGED, _dt(q), B, int(T), int(max_seqlen_q), int(max_seqlen_k), 0,
                    int(local_window), H_q, H_kv, D)
    ws, ws_bytes = _workspace(workspace, need, q)
    _check("paged_decode_step", lib.paged_decode_step(
        _i32(cu_seqlens_q, "cu_seqlens_q"), _i32(past_seqlens, "past_seqlens"), B, int(T),
        _i32(seqlens_q, "seqlens_q"), _i32(seqlens_k, "seqlens_k"), _ptr(q, "q"),
        _ptr(k_new, "k_new"), _ptr(v_new, "v_new"), _dt(q), _ptr(k_cache, "k_cache"),
        _ptr(v_cache, "v_cache"), _dt(k_cache), _i32(block_table, "block_table"), mbps, bs, nb,
        _ptr(key_scale, "key_scale"), _ptr(value_scale, "value_scale"), int(max_seqlen_q),
        int(max_seqlen_k), H_q, H_kv, D, float(scale), int(local_window), _ptr(sinks, "sinks"),
        _ptr(out, "out"), _ptr(ws, "workspace"), ws_bytes,
        _i32(committed_length, "committed_length"), _i32(status, "status"), _stream(cu_seqlens_q)))


def paged_decode_step_noalloc(cu_seqlens_q: torch.Tensor, past_seqlens: torch.Tensor, T: int,
                              seqlens_q: torch.Tensor, seqlens_k: torch.Tensor, q: torch.Tensor,
                              k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
                              v_cache: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
                              out: torch.Tensor, block_table: Optional[torch.Tensor] = None,
                              key_scale: Optional[torch.Tensor] = None,
                              value_scale: Optional[torch.Tensor] = None, scale: float = 0.0,
                              local_window: int = -1, sinks: Optional[torch.Tensor] = None,
                              committed_length: Optional[torch.Tensor] = None,
                              status: Optional[torch.Tensor] = None) -> None:
    """paged_decode_step with its split-K partials in the library's static device array
    (no allocation by the call or by this binding)."""
    B = int(past_seqlens.shape[0])
    _, H_q, D = (int(x) for x in q.shape)
    H_kv = int(k_cache.shape[1])
    nb, bs, mbps = _cache_dims(k_cache, block_table)
    lib = _lib.load()
    _check("paged_decode_step_noalloc", lib.paged_decode_step_noalloc(
        _i32(cu_seqlens_q, "cu_seqlens_q"), _i32(past_seqlens, "past_seqlens"), B, int(T),
        _i32(seqlens_q, "seqlens_q"), _i32(seqlens_k, "seqlens_k"), _ptr(q, "q"),
        _ptr(k_new, "k_new"), _ptr(v_new, "v_new"), _dt(q), _ptr(k_cache, "k_cache"),
        _ptr(v_cache, "v_cache"), _dt(k_cache), _i32(block_table, "block_table"), mbps, bs, nb,
        _ptr(key_scale, "key_scale"), _ptr(value_scale, "value_scale"), int(max_seqlen_q),
        int(max_seqlen_k), H_q, H_kv, D, float(scale), int(local_window), _ptr(sinks, "sinks"),
        _ptr(out, "out"), _i32(committed_length, "committed_length"), _i32(status, "status"),
        _stream(cu_seqlens_q)))


def sparse_attention_fwd(q: torch.Tensor, mode: int, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         cu_seqlens_q: torch.Tensor, seqlens_k: torch.Tensor, max_seqlen_q: int,
                         sel_idx: torch.Tensor, out: torch.Tensor,
                         sel_count: Optional[torch.Tensor] = None,
                         block_table: Optional[torch.Tensor] = None,
                         key_scale: Optional[torch.Tensor] = None,
                         value_scale: Optional[torch.Tensor] = None, local_window: int = -1,
                         aux_k: Optional[torch.Tensor] = None,
                         aux_v: Optional[torch.Tensor] = None,
                         aux_batch_stride: Optional[int] = None, scale: float = 0.0,
                         sinks: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None,
                         status: Optional[torch.Tensor] = None) -> None:
    """Selected-token attention (mode 0) or local window plus auxiliary rows (mode 1)."""
    T, H_q, D = (int(x) for x in q.shape)
    H_kv = int(k_cache.shape[1])
    B = int(seqlens_k.shape[0])
    max_sel = int(sel_idx.shape[2])
    nb, bs, mbps = _cache_dims(k_cache, block_table)
    aux_len, aux_dt = 0, _dt(q)
    if aux_k is not None:
        aux_len = int(aux_k.shape[1])
        aux_dt = _dt(aux_k)
        if aux_batch_stride is None:
            aux_batch_stride = 0 if aux_k.shape[0] == 1 else aux_len * H_kv * D
    aux_batch_stride = int(aux_batch_stride or 0)
    kind = KIND_SELECTED if mode == 0 else KIND_LOCAL_AUX
    need = _ws_need(kind, _dt(q), B, T, int(max_seqlen_q), 0, max_sel, int(local_window),
                    H_q, H_kv, D)
    ws, ws_bytes = _workspace(workspace, need, q)
    lib = _lib.load()
    _check("sparse_attention_fwd", lib.sparse_attention_fwd(
        _ptr(q, "q"), _dt(q), int(mode), _ptr(k_cache, "k_cache"), _ptr(v_cache, "v_cache"),
        _dt(k_cache), _i32(block_table, "block_table"), mbps, bs, nb,
        _ptr(key_scale, "key_scale"), _ptr(value_scale, "value_scale"),
        _i32(cu_seqlens_q, "cu_seqlens_q"), _i32(seqlens_k, "seqlens_k"), B, T, int(max_seqlen_q),
        _i32(sel_idx, "sel_idx"), _i32(sel_count, "sel_count"), max_sel, int(local_window),
        _ptr(aux_k, "aux_k"), _ptr(aux_v, "aux_v"), aux_dt, aux_len, aux_batch_stride, H_q, H_kv,
        D, float(scale), _ptr(sinks, "sinks"), _ptr(out, "out"), _ptr(ws, "workspace"), ws_bytes,
        _i32(status, "status"), _stream(q)))
