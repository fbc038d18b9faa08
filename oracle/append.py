"""KV-cache append (scatter of this step's K/V rows into the cache), defined on the CPU.

"[WebGPU] Add SparsePagedAttention", file summaries: the current K/V rows are scattered
into the paged cache through a token-to-slot mapping derived from the block table.
"[WebGPU] Add DynamicSparseAttention", Description: contiguous per-request caches are
updated in place (alias-safe).  DynamicSparseAttention INT8 KV cache (onnxruntime PR
33472), Key Changes table: INT8 caches carry per-channel fp32 key_scale / value_scale and
the append quantises with them.  The same page adds an optional committed_length input,
and its review finding "Strict mode ignores cursor validation errors" shows a cursor that
disagrees with the sequence lengths (batch 1, one new row, capacity 2, seqlens_k = {0},
committed_length = {1}) still appending; here such a request is flagged before any of its
rows is written, and none is.
"""
from __future__ import annotations

import numpy as np

from .status import STATUS_CAPACITY, STATUS_BAD_BLOCK, STATUS_CURSOR, STATUS_SHORT_KV


def quantize_int8(x, s):
    """Symmetric per-channel INT8 code of ``x`` with scale ``s``.

    Reading taken (the pages give per-channel scales but no rounding rule): the value and
    the scale are float32, the quotient is one IEEE float32 division, rounded to the
    nearest integer with ties to even, then clamped to [-127, 127]; a NaN quotient gives 0.
    Pinned by hand-worked values in the tests (ties, clamping, NaN).
    """
    x = np.asarray(x, dtype=np.float32)
    s = np.asarray(s, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        r = np.divide(x, s, dtype=np.float32)
    r = np.rint(r)
    r = np.where(np.isnan(r), np.float32(0), r)
    r = np.clip(r, -127, 127)
    return r.astype(np.int8)


def decode_fp8_e4m3(codes):
    """Exact float64 values of FP8 E4M3 codes.

    Reading taken: the pages name an FP8 KV cache (DynamicSparseAttention INT8 page, build
    notes: FP8/INT4 KV cache enabled) without a format; it is taken as the OCP "E4M3FN"
    encoding (ONNX float8e4m3fn): sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
    subnormals ``m * 2**-9`` for exponent 0, no infinities, and the two codes 0x7F / 0xFF
    (exponent 15, mantissa 7) are NaN.  Largest finite magnitude 448.  Scaled per channel
    like INT8: ``value = decode(code) * scale[c][d]``.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def quantize_fp8_e4m3(x, s):
    """FP8 E4M3 code of ``x`` with scale ``s``: the float32 quotient ``x / s`` (one IEEE
    float32 division) rounded to the nearest E4M3 value, ties to the even mantissa;
    magnitudes above 448 saturate to 448 (as INT8 clamps to 127); a NaN quotient gives
    code 0 (as INT8).  Reading taken; pinned by hand-worked codes and against the library
    float8_e4m3fn conversion in its finite range."""
    x = np.asarray(x, dtype=np.float32)
    s = np.asarray(s, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        q = np.divide(x, s, dtype=np.float32).astype(np.float64)
    sign = np.where(np.signbit(q), 0x80, 0x00)
    a = np.abs(q)
    nan = np.isnan(a)
    big = a > 448.0
    a = np.where(nan | big, 0.0, a)          # the codes of these are fixed below
    # subnormal range (below 2**-6): multiples of 2**-9, code = the multiple (8 = 2**-6)
    sub = np.rint(a * 2.0 ** 9)
    # normal range: a = f * 2**e with f in [1, 2); 3 mantissa bits after rounding
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    # log2 of an exact power of two is exact; guard the rounding of log2 anyway
    e = np.where(np.exp2(e) > a, e - 1, e)
    e = np.where(np.exp2(e + 1) <= a, e + 1, e)
    r = np.rint(a / np.exp2(e) * 8.0)               # in [8, 16]
    e = np.where(r == 16, e + 1, e)
    r = np.where(r == 16, 8, r)
    normal = ((e + 7).astype(np.int64) << 3) | (r.astype(np.int64) - 8)
    mag = np.where(a < 2.0 ** -6, sub.astype(np.int64), normal)
    mag = np.where(big, 0x7E, mag)
    code = np.where(nan, 0, sign | mag)
    return code.astype(np.uint8)


def _check_cu(cu, B, T):
    if not (cu[0] == 0 and cu[B] == T and all(cu[b] <= cu[b + 1] for b in range(B))):
        raise ValueError("oracle: kv_cache_append / attention need a well-formed cu_seqlens_q")


def kv_cache_append(k_new, v_new, cu_seqlens_q, seqlens_k, k_cache, v_cache,
                    block_table=None, block_size=None, key_scale=None, value_scale=None,
                    committed_length=None, skip_rows=None):
    """Write row ``cu[b] + i`` of ``k_new`` / ``v_new`` (``[T, H_kv, D]``) at key position
    ``p = (seqlens_k[b] + 1) - q_len_b + i`` of request ``b``.

    Slot of position ``p``: paged cache ``[nb, H_kv, bs, D]`` (each block holds its
    slots head by head) -> block ``block_table[b][p // bs]``, slot ``p % bs``; contiguous
    cache ``[B, H_kv, cap, D]`` (``block_table is None``) -> block ``b``, slot ``p``.  The
    row of KV head ``c`` goes to ``cache[block, c, slot]``.  Float caches store the row as
    is (same dtype); INT8 caches store ``quantize_int8(row, scale[c][d])``.

    ``committed_length[b]`` (optional) is the key count the caller believes request ``b``
    already holds.  It must equal ``kv_len - q_len_b`` (the position of the first row this
    step writes); otherwise STATUS_CURSOR is raised and none of the request's rows is
    written (checked before any write of the request).

    Rows whose slot does not exist are skipped and flagged (parity unpinned): ``p < 0``
    (STATUS_SHORT_KV), ``p // bs >= max_blocks_per_seq`` or ``p >= cap``
    (STATUS_CAPACITY), a block id outside ``[0, nb)`` (STATUS_BAD_BLOCK).

    ``skip_rows`` (optional, boolean ``[T]``): rows that are not written at all (the
    prologue's rows whose rotary position is out of range); no other effect.

    Returns ``(k_cache_out, v_cache_out, status)``; the inputs are not modified.
    """
    cu = [int(x) for x in np.asarray(cu_seqlens_q).reshape(-1)]
    sk = [int(x) for x in np.asarray(seqlens_k).reshape(-1)]
    B = len(sk)
    T = int(np.asarray(k_new).shape[0])
    _check_cu(cu, B, T)
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    int8 = kc.dtype == np.int8
    fp8 = kc.dtype == np.uint8      # FP8 E4M3 codes
    nb = kc.shape[0]
    status = 0
    committed = None if committed_length is None else [int(x) for x in np.asarray(committed_length).reshape(-1)]
    for b in range(B):
        q_len = cu[b + 1] - cu[b]
        kv_len = sk[b] + 1
        if committed is not None and q_len > 0 and committed[b] != kv_len - q_len:
            status |= STATUS_CURSOR
            continue
        for i in range(q_len):
            r = cu[b] + i
            p = kv_len - q_len + i
            if skip_rows is not None and skip_rows[r]:
                continue
            if p < 0:
                status |= STATUS_SHORT_KV
                continue
            if block_table is None:
                if p >= kc.shape[2] or b >= nb:
                    status |= STATUS_CAPACITY
                    continue
                blk, off = b, p
            else:
                bs = int(block_size)
                lb = p // bs
                if lb >= block_table.shape[1]:
                    status |= STATUS_CAPACITY
                    continue
                blk = int(block_table[b][lb])
                if blk < 0 or blk >= nb:
                    status |= STATUS_BAD_BLOCK
                    continue
                off = p % bs
            if int8:
                kc[blk, :, off] = quantize_int8(np.asarray(k_new[r], np.float32), key_scale)
                vc[blk, :, off] = quantize_int8(np.asarray(v_new[r], np.float32), value_scale)
            elif fp8:
                kc[blk, :, off] = quantize_fp8_e4m3(np.asarray(k_new[r], np.float32), key_scale)
                vc[blk, :, off] = quantize_fp8_e4m3(np.asarray(v_new[r], np.float32), value_scale)
            else:
                kc[blk, :, off] = k_new[r]
                vc[blk, :, off] = v_new[r]
    return kc, vc, status
