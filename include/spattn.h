/*
 * spattn.h - C ABI of the MI355X (gfx950) paged / selected-token attention library.
 *
 * Four operations and one sizing helper:
 *
 *   prepare_seqlens            per-request query/key lengths and per-token (request,
 *                              position) derived on the device from cumulative offsets;
 *   kv_cache_append            scatter of this step's K/V rows into the cache (INT8
 *                              per-channel quantisation for INT8 caches);
 *   paged_attention_fwd        causal attention over a paged (block table) or contiguous
 *                              cache, GQA, local window, learned per-head sink;
 *   sparse_attention_fwd       attention over selected cache rows (int32 indices padded
 *                              with -1), or over a local window plus selected rows of an
 *                              auxiliary store, with one joint softmax and sink;
 *   attention_workspace_bytes  bytes of device workspace the attention calls need.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer argument is a device pointer unless stated otherwise; the caller owns
 *   every buffer and keeps it alive until the enqueued work has finished.
 * - `stream` is a hipStream_t (NULL = the default stream).  Each call only enqueues
 *   kernels on it: the library never allocates, frees, synchronises, copies between host
 *   and device, or logs.  All calls can therefore be recorded into a HIP graph.
 * - Return value: 0 = enqueued.  A negative value is a host-detectable argument error and
 *   then NOTHING was enqueued: SPATTN_ERR_NULL (a required pointer is NULL),
 *   SPATTN_ERR_SHAPE (a size is negative or inconsistent, or a data pointer is not 16-byte
 *   aligned: activations, outputs, caches and auxiliary stores are accessed 16 bytes at a
 *   time; allocations are aligned), SPATTN_ERR_DTYPE (dtype
 *   combination not supported), SPATTN_ERR_UNSUPPORTED (e.g. is_causal = 0, head_dim not
 *   64/128, H_q not a multiple of H_kv), SPATTN_ERR_WORKSPACE (workspace too small),
 *   SPATTN_ERR_LAUNCH (the HIP launch itself failed; work before the failing launch of
 *   the same call may have been enqueued).
 * - `status` (optional, may be NULL): one int32 in device memory into which the kernels
 *   OR the SPATTN_STATUS_* bits for malformed device-side data.  The caller clears it.
 *   Affected keys are excluded and affected rows written as zeros; nothing is read or
 *   written out of bounds.
 * - Packed layouts (row-major): Q and out [T, H_q, D]; new K/V [T, H_kv, D]; paged cache
 *   [num_blocks, H_kv, block_size, D] (each block holds its slots head by head, so the
 *   keys of one KV head in a block are one contiguous run) addressed through block_table
 *   [B, max_blocks_per_seq] (int32, entries past a request's blocks unused); contiguous
 *   cache [num_blocks >= B, H_kv, capacity, D] when block_table is NULL (then block_size is
 *   the capacity and max_blocks_per_seq is ignored).  Auxiliary stores (sparse mode 1) are
 *   token-major: [.., aux_len, H_kv, D].
 * - Row r of request b (cu_seqlens_q[b] <= r < cu_seqlens_q[b+1]) sits at key position
 *   p = (seqlens_k[b] + 1) - q_len_b + (r - cu_seqlens_q[b]); seqlens_k[b] is the total
 *   key count minus one (-1 = empty request).  cu_seqlens_q must be well formed
 *   (0 = cu[0] <= ... <= cu[B] = T) for kv_cache_append and the attention calls; for a
 *   malformed one their results are unspecified but every access stays in bounds.
 *
 * Citations are to web pages by title and section:
 *   [PA]  "[WebGPU] Add PagedAttention metadata and GPT-OSS support" (onnxruntime PR 32277)
 *   [SPA] "[WebGPU] Add SparsePagedAttention" (onnxruntime PR 32533)
 *   [DSA] "[WebGPU] Add DynamicSparseAttention" (onnxruntime PR 32529)
 *   [I8]  DynamicSparseAttention INT8 KV cache / grouped decode (onnxruntime PR 33472)
 *   [LA]  "ai.onnx.LinearAttention" kernel page
 */
#ifndef SPATTN_H
#define SPATTN_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define SPATTN_API __attribute__((visibility("default")))
#else
#define SPATTN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
#define SPATTN_F32 0
#define SPATTN_F16 1
#define SPATTN_BF16 2
#define SPATTN_I8 3 /* caches only */
#define SPATTN_FP8 4 /* caches only: FP8 E4M3 codes (OCP E4M3FN), per-channel scales as for I8 */

/* return codes */
#define SPATTN_OK 0
#define SPATTN_ERR_NULL (-1)
#define SPATTN_ERR_SHAPE (-2)
#define SPATTN_ERR_DTYPE (-3)
#define SPATTN_ERR_UNSUPPORTED (-4)
#define SPATTN_ERR_WORKSPACE (-5)
#define SPATTN_ERR_LAUNCH (-6)

/* device status bits (OR-ed into *status) */
#define SPATTN_STATUS_BAD_CU (1 << 0)     /* cu_seqlens_q malformed, or past < 0 */
#define SPATTN_STATUS_Q_BOUND (1 << 1)    /* q_len > max_seqlen_q: the request's rows are 0 */
#define SPATTN_STATUS_K_BOUND (1 << 2)    /* key count > max_seqlen_k: the request's rows are 0 */
#define SPATTN_STATUS_CAPACITY (1 << 3)   /* a needed position lies past the cache capacity */
#define SPATTN_STATUS_BAD_BLOCK (1 << 4)  /* a needed block id is outside [0, num_blocks) */
#define SPATTN_STATUS_BAD_INDEX (1 << 5)  /* a selected index (inside the count) is neither -1 nor in range */
#define SPATTN_STATUS_BAD_COUNT (1 << 6)  /* a selected count outside [0, max_selected]; clamped */
#define SPATTN_STATUS_SHORT_KV (1 << 7)   /* fewer keys than query rows: rows before key 0 see nothing */
#define SPATTN_STATUS_CURSOR (1 << 8)     /* committed_length disagrees with the append position */
#define SPATTN_STATUS_POSITION (1 << 9)   /* qkv_prologue: a rotary position outside [0, max_position) */

/* attention kinds for attention_workspace_bytes */
#define SPATTN_KIND_PAGED 0
#define SPATTN_KIND_SELECTED 1    /* sparse_attention_fwd mode 0 */
#define SPATTN_KIND_LOCAL_AUX 2   /* sparse_attention_fwd mode 1 */

/*
 * prepare_seqlens - device-side sequence metadata ([PA] Description and Changes: exact
 * per-request lengths are derived on the device from cumulative query offsets and past
 * lengths, with no host readback; [PA] review finding T1 for the worked examples;
 * [SPA] file summaries: per-token request/position metadata).
 *
 *   cu_seqlens_q [B+1] int32, past_seqlens [B] int32 (keys already cached), T = packed rows.
 *   Outputs: seqlens_q[b] = cu[b+1] - cu[b]; seqlens_k[b] = past[b] + seqlens_q[b] - 1;
 *   token_req[t] = request owning row t (or -1), token_pos[t] = its key position (or -1).
 *   token_req / token_pos / status may be NULL.  Malformed cu (cu[0] != 0, decreasing,
 *   cu[B] != T) or negative past: SPATTN_STATUS_BAD_CU, and each boundary is replaced by
 *   the running maximum of cu[0..b] clamped to [0, T] (negative past by 0).
 *   Limits: 0 <= B <= 8192, T >= 0.
 */
SPATTN_API int prepare_seqlens(const int32_t* cu_seqlens_q, const int32_t* past_seqlens, int B, int T,
                    int32_t* seqlens_q, int32_t* seqlens_k, int32_t* token_req,
                    int32_t* token_pos, int32_t* status, void* stream);

/*
 * kv_cache_append - write this step's K/V rows into the cache in place ([SPA] file
 * summaries: scatter of current K/V through the block table; [DSA] Description:
 * alias-safe in-place update of contiguous caches; [I8] Key Changes: INT8 caches with
 * per-channel key_scale / value_scale).
 *
 *   k_new, v_new [T, H_kv, D] of new_dtype; row r of request b goes to position
 *   p = (seqlens_k[b] + 1) - q_len_b + i (seqlens_k as AFTER the append).
 *   Float caches: cache_dtype == new_dtype, stored unchanged.  INT8 caches
 *   (cache_dtype = SPATTN_I8, new_dtype F32/F16/BF16): code = clamp(rint_even(x / s),
 *   -127, 127) with x, s float32 and an IEEE float32 division (NaN quotient -> 0);
 *   key_scale / value_scale [H_kv, D] float32 are then required.  FP8 caches
 *   (SPATTN_FP8; the pages name an FP8 KV cache, its format is taken as OCP E4M3FN): x / s
 *   rounded to the nearest E4M3 value (ties to even), magnitudes above 448 saturate to
 *   448, NaN -> code 0; the same scales are required.  Attention reads a code as
 *   E4M3 value * scale[c][d] (0x7F / 0xFF are NaN).
 *   Rows without a slot are skipped: p < 0 (SHORT_KV), past the capacity (CAPACITY), a
 *   block id outside [0, num_blocks) (BAD_BLOCK).
 *   committed_length [B] (optional, may be NULL): the key count the caller's cursor says
 *   request b held before this step ([I8] Key Changes: optional committed_length input;
 *   review finding "Strict mode ignores cursor validation errors").  A request with rows
 *   whose committed_length[b] differs from seqlens_k[b] + 1 - q_len_b raises
 *   SPATTN_STATUS_CURSOR and none of its rows is written; other requests append normally.
 *   The check is on the device: a caller that must not run attention after a failed check
 *   reads `status` (or skips the call) itself.
 */
SPATTN_API int kv_cache_append(const void* k_new, const void* v_new, int new_dtype,
                    const int32_t* cu_seqlens_q, const int32_t* seqlens_k, int B, int T,
                    void* k_cache, void* v_cache, int cache_dtype, const int32_t* block_table,
                    int max_blocks_per_seq, int block_size, int num_blocks,
                    const float* key_scale, const float* value_scale, int H_kv, int D,
                    const int32_t* committed_length, int32_t* status, void* stream);

/*
 * prepare_and_append - prepare_seqlens followed by kv_cache_append with the seqlens_k it
 * produced, as one launch when B <= 255 (two otherwise).  Its outputs and status are
 * those of the two calls made in order (same citations): seqlens_q, seqlens_k, token_req /
 * token_pos (may be NULL), the appended rows, and the status bits of both.  For a decode
 * step it removes one kernel launch; no device metadata is read back either way.
 *   paged_decode_step goes further for decode steps: it makes this call's work part of
 *   the attention launch.
 *   Arguments: those of prepare_seqlens, then those of kv_cache_append after its
 *   seqlens_k (which is this call's output).  Limits: 0 <= B <= 8192.
 */
SPATTN_API int prepare_and_append(const int32_t* cu_seqlens_q, const int32_t* past_seqlens, int B,
                    int T, int32_t* seqlens_q, int32_t* seqlens_k, int32_t* token_req,
                    int32_t* token_pos, const void* k_new, const void* v_new, int new_dtype,
                    void* k_cache, void* v_cache, int cache_dtype, const int32_t* block_table,
                    int max_blocks_per_seq, int block_size, int num_blocks,
                    const float* key_scale, const float* value_scale, int H_kv, int D,
                    const int32_t* committed_length, int32_t* status, void* stream);

/*
 * qkv_prologue - the step before attention, fused with the cache append ([DSA]
 * Description, "QKV and cache" and "Position processing": packed or unpacked QKV, QK
 * RMSNorm, partial and interleaved RoPE, rotary offsets, explicit position IDs; [DSA]
 * review: a head's RMS is reduced once per (token, head); [SPA] overview: the
 * PagedAttention prologue of packed-QKV split, RoPE and block-table scatter).  The pages
 * print no formula for these steps; the textbook definitions below are the readings taken.
 *
 *   Input rows: qkv [T, (H_q + 2 H_kv) * D] (each row: the H_q query heads, then the H_kv
 *   key heads, then the H_kv value heads, D elements each) or, when qkv is NULL, q
 *   [T, H_q, D], k [T, H_kv, D], v [T, H_kv, D]; all of `dtype` (F32 / F16 / BF16).
 *   qk_norm != 0: every query and key head x becomes x / sqrt(mean(x^2) + norm_eps) * w,
 *   w = q_norm_weight / k_norm_weight [D] float32 (NULL = ones).
 *   rotary_dim > 0 (even, <= D): the channel pairs (i, i + rotary_dim/2) -- or (2i, 2i+1)
 *   when rotary_interleaved != 0 -- of every query and key head, i < rotary_dim/2, become
 *   (a cos - b sin, b cos + a sin) with cos = cos_table[pos][i], sin = sin_table[pos][i]
 *   (float32 [max_position, rotary_dim/2], row-major); channels >= rotary_dim pass
 *   unchanged.  pos = (position_ids ? position_ids[t] : p) + (rotary_offsets ?
 *   rotary_offsets[b] : 0), p the row's key position.  A pos outside [0, max_position)
 *   sets SPATTN_STATUS_POSITION; that row's q_out is 0 and its K/V row is not appended.
 *   Value heads are neither normalised nor rotated.
 *   The arithmetic is float32 (norm, then rotation).  q_out [T, H_q, D] (dtype) receives
 *   the query heads rounded once to dtype; the key heads are rounded once to dtype too,
 *   and the key and value rows are then stored exactly as kv_cache_append stores
 *   k_new / v_new, with the same cache arguments, INT8 / FP8 quantisation, committed_length
 *   cursor check and status bits.  Rows of no request (malformed cu): q_out 0,
 *   SPATTN_STATUS_BAD_CU, nothing appended.
 *   Limits: 8 <= D <= 256, D % 8 == 0; norm_eps >= 0.  qkv / q / k / v must not overlap
 *   q_out or the caches.
 */
SPATTN_API int qkv_prologue(const void* qkv, const void* q, const void* k, const void* v, int dtype,
                    const int32_t* cu_seqlens_q, const int32_t* seqlens_k, int B, int T,
                    int H_q, int H_kv, int D, int qk_norm, const float* q_norm_weight,
                    const float* k_norm_weight, float norm_eps, int rotary_dim,
                    int rotary_interleaved, const float* cos_table, const float* sin_table,
                    int max_position, const int32_t* position_ids, const int32_t* rotary_offsets,
                    void* q_out, void* k_cache, void* v_cache, int cache_dtype,
                    const int32_t* block_table, int max_blocks_per_seq, int block_size,
                    int num_blocks, const float* key_scale, const float* value_scale,
                    const int32_t* committed_length, int32_t* status, void* stream);

/*
 * topk_select - the k highest-scoring key positions of every (row, KV head): the producer of
 * sel_idx / sel_count for sparse_attention_fwd mode 0 (DynamicSparseAttention INT8 / fast
 * QSA decode page, Key Changes table: hierarchical / compact TopK selection; follow-up
 * description: stable keys, causal tails, capacity stride and padding).  The pages name
 * those properties only; this is the reading taken.
 *
 *   scores [T, H_kv, L] float32 (row-major; the score of key position j is scores[t][c][j]).
 *   Row t of request b sees positions 0 .. p, p = (seqlens_k[b] + 1) - q_len_b + i, so it
 *   has n = clamp(p + 1, 0, L) candidates.  If n <= k all are selected.  Otherwise the last
 *   min(tail, k) candidates (the causal tail) are selected, and the other selections are
 *   the highest-scoring remaining candidates: equal scores by position, lower first; NaN
 *   below every number; -0.0 equal to +0.0.
 *   Outputs: sel_idx [T, H_kv, capacity] int32 -- the min(k, n) selected positions in
 *   ascending order, then -1 -- and sel_count [T, H_kv] int32 = min(k, n).  Rows owned by
 *   no request (malformed cu): count 0, SPATTN_STATUS_BAD_CU.
 *   Limits: 1 <= L <= 65536, 0 <= k <= capacity, tail >= 0.
 */
SPATTN_API int topk_select(const float* scores, int L, const int32_t* cu_seqlens_q,
                    const int32_t* seqlens_k, int B, int T, int H_kv, int k, int tail,
                    int32_t* sel_idx, int capacity, int32_t* sel_count, int32_t* status,
                    void* stream);

/*
 * attention_workspace_bytes - device workspace (bytes) an attention call with these
 * arguments needs for its split-K partial softmax states ([SPA] file summaries and
 * follow-up description: FP32 partial states merged by a finalize stage).  Pure host
 * function; 0 means the call may pass workspace = NULL.  Its contents need no
 * initialisation; calls that may run at the same time need separate workspaces.  `kind`
 * is SPATTN_KIND_*;
 * max_seqlen_k is used by SPATTN_KIND_PAGED, max_selected by the sparse kinds,
 * local_window by SPATTN_KIND_PAGED and SPATTN_KIND_LOCAL_AUX, dtype is the Q dtype.
 * Returns (size_t)-1 for arguments the attention calls would reject (including key
 * ranges longer than 256 splits of 4096 keys).
 */
SPATTN_API size_t attention_workspace_bytes(int kind, int dtype, int B, int T, int max_seqlen_q,
                                 int max_seqlen_k, int max_selected, int local_window,
                                 int H_q, int H_kv, int D);

/*
 * paged_attention_fwd - causal attention of packed queries over a paged or contiguous
 * KV cache ([PA] Description and Changes: paged attention with device-derived lengths,
 * local-window masking and a learned head sink; [PA] Q2/Q3: window kept on the direct
 * paged path, key loop started at the earliest window tile; [DSA] Description: GQA head
 * mapping, joint FP32 softmax; [I8] Key Changes: INT8 per-channel K/V).
 *
 *   q, out [T, H_q, D] of dtype (F32, F16, BF16).  Cache dtype equals dtype, or is I8
 *   (then key_scale / value_scale [H_kv, D] float32 are required).
 *   Key set of the row at position p: cache positions lo..p with lo = max(0, p - W + 1)
 *   when local_window = W > 0, else 0.  Query head h uses KV head h / (H_q / H_kv).
 *   s = scale * <q, k> with scale = 1/sqrt(D) when 0 ([LA] Attributes).  The per-head
 *   sink logit sinks[h] (float32 [H_q], may be NULL) joins the softmax maximum and
 *   denominator only.  A row with no visible key is written as zeros.
 *   max_seqlen_q / max_seqlen_k are host upper bounds of q_len / key count (a request
 *   exceeding them gets zero rows and Q_BOUND / K_BOUND); they size the launch.
 *   is_causal must be 1 ([PA] Changes: non-causal is rejected).  D in {64, 128}.
 *   workspace: >= attention_workspace_bytes(SPATTN_KIND_PAGED, ...) bytes, 256-byte aligned.
 */
SPATTN_API int paged_attention_fwd(const void* q, int dtype, const void* k_cache, const void* v_cache,
                        int cache_dtype, const int32_t* block_table, int max_blocks_per_seq,
                        int block_size, int num_blocks, const float* key_scale,
                        const float* value_scale, const int32_t* cu_seqlens_q,
                        const int32_t* seqlens_k, int B, int T, int max_seqlen_q,
                        int max_seqlen_k, int H_q, int H_kv, int D, float scale, int is_causal,
                        int local_window, const float* sinks, void* out, void* workspace,
                        size_t workspace_bytes, int32_t* status, void* stream);

/*
 * paged_decode_step - prepare_seqlens, kv_cache_append and paged_attention_fwd of one
 * decode step in one launch of the split-K kernel (plus its merge when the key range is
 * split); the same citations as those three calls ([PA] Description: lengths derived on
 * the device, no readback; [SPA] file summaries: scatter of the step's K/V through the
 * block table; [PA] Description and Changes: paged attention with window and sink).
 *
 *   Arguments: those of prepare_seqlens (no token_req / token_pos), then q, k_new, v_new
 *   (all of dtype) and the cache, bounds, head, scale, window, sink, output and workspace
 *   arguments of paged_attention_fwd (is_causal is 1; workspace sized by
 *   attention_workspace_bytes(SPATTN_KIND_PAGED, ...) with the same arguments).
 *   Well-formed metadata (cu[0] = 0, non-decreasing, cu[B] = T, past >= 0): seqlens_q,
 *   seqlens_k, the cache, out and the status bits equal those of
 *   prepare_and_append(..., token_req = token_pos = committed_length = NULL) followed by
 *   paged_attention_fwd(..., seqlens_k, is_causal = 1), bit for bit.  Each workgroup
 *   writes the new keys of its own key range before reading them, so a slot this step
 *   writes must not be read by another request as one of its past keys (shared prefix
 *   blocks hold past keys only).  Malformed metadata: SPATTN_STATUS_BAD_CU, seqlens_q /
 *   seqlens_k as prepare_seqlens writes them, nothing appended, every out row zero.
 *   committed_length [B] (optional, may be NULL): the caller's cursor, as for
 *   kv_cache_append ([I8] Key Changes: optional committed_length; review: a cursor
 *   mismatch must not be followed by a cache update).  A request with rows whose
 *   committed_length[b] differs from past_seqlens[b] raises SPATTN_STATUS_CURSOR and none
 *   of its keys is written; its rows are still attended over the unchanged cache.  With it
 *   the step equals prepare_and_append(..., committed_length) followed by
 *   paged_attention_fwd, bit for bit, so a graph replayed with stale lengths cannot
 *   overwrite live slots when the caller passes its cursor.
 *   Supported: dtype F16 / BF16 with a cache of the same dtype, INT8 or FP8; B <= 255;
 *   max_seqlen_q <= 8 (the split-K path; longer query blocks take the prefill kernel).
 *   Other arguments that the separate calls accept return SPATTN_ERR_UNSUPPORTED and
 *   enqueue nothing.  T = 0 writes the metadata only.
 */
SPATTN_API int paged_decode_step(const int32_t* cu_seqlens_q, const int32_t* past_seqlens, int B,
                      int T, int32_t* seqlens_q, int32_t* seqlens_k, const void* q,
                      const void* k_new, const void* v_new, int dtype, void* k_cache,
                      void* v_cache, int cache_dtype, const int32_t* block_table,
                      int max_blocks_per_seq, int block_size, int num_blocks,
                      const float* key_scale, const float* value_scale, int max_seqlen_q,
                      int max_seqlen_k, int H_q, int H_kv, int D, float scale, int local_window,
                      const float* sinks, void* out, void* workspace, size_t workspace_bytes,
                      const int32_t* committed_length, int32_t* status, void* stream);

/*
 * paged_decode_step_noalloc - paged_decode_step for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without workspace / workspace_bytes, the same results
 * bit for bit.  The split-K partials go to a static device array of the library, 16 MiB
 * per GPU (SPATTN_NOALLOC_SCRATCH_BYTES), held from the first call on a device until the
 * process ends; the call itself allocates nothing.  A call whose partials need more
 * (attention_workspace_bytes(SPATTN_KIND_PAGED, ...) > SPATTN_NOALLOC_SCRATCH_BYTES, e.g.
 * more than about 60 decode rows of 64 heads x 8192 keys) returns SPATTN_ERR_WORKSPACE and
 * enqueues nothing.  The array needs no clearing between calls (every partial a call reads
 * was written by the same call).  All calls on one GPU share that GPU's array, which keeps
 * the last call's contents: calls that may overlap on one GPU (different streams without
 * ordering between them) race and must not be made.  The current device must be the
 * device of `stream` (SPATTN_ERR_UNSUPPORTED otherwise); SPATTN_ERR_LAUNCH if the array's
 * device address cannot be found.  Argument errors are reported as by paged_decode_step,
 * before the array is looked up.
 */
#define SPATTN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
SPATTN_API int paged_decode_step_noalloc(const int32_t* cu_seqlens_q, const int32_t* past_seqlens,
                      int B, int T, int32_t* seqlens_q, int32_t* seqlens_k, const void* q,
                      const void* k_new, const void* v_new, int dtype, void* k_cache,
                      void* v_cache, int cache_dtype, const int32_t* block_table,
                      int max_blocks_per_seq, int block_size, int num_blocks,
                      const float* key_scale, const float* value_scale, int max_seqlen_q,
                      int max_seqlen_k, int H_q, int H_kv, int D, float scale, int local_window,
                      const float* sinks, void* out, const int32_t* committed_length,
                      int32_t* status, void* stream);

/*
 * sparse_attention_fwd - attention over selected cache rows ([DSA] Description: selected
 * main-cache mode and local-plus-auxiliary mode, guarded int32 indices, joint FP32 stable
 * softmax with optional sink, shared auxiliary K/V storage; [DSA] review: the selection
 * loop is bounded by the device count, not by max_selected; [SPA] overview: selected
 * reads and local-plus-compressed attention over paged caches).
 *
 *   sel_idx [T, H_kv, max_selected] int32; sel_count [T, H_kv] int32 or NULL (NULL = all
 *   max_selected entries); counts outside [0, max_selected] are clamped (BAD_COUNT).
 *   Entry -1 is padding; any other entry outside its range is excluded (BAD_INDEX).
 *   mode 0 (selected main): entry j is main-cache position j of the row's request, used
 *     when 0 <= j < key count and j <= p (causal by position).  local_window must be <= 0.
 *   mode 1 (local + auxiliary): main positions max(0, p - W + 1)..p (local_window = W > 0
 *     required) plus auxiliary rows a (0 <= a < aux_len) of aux_k / aux_v, which are
 *     [.., aux_len, H_kv, D] of aux_dtype (== dtype) with request b's rows starting at
 *     element b * aux_batch_stride (0 = one store shared by every request); aux_k and
 *     aux_v may alias.  Auxiliary rows carry no position and are not masked.
 *   One softmax over every source and the sink; empty key set -> zero row.
 *   Main-cache arguments as in paged_attention_fwd (paged or contiguous, F32/F16/BF16
 *   equal to dtype, or I8 with scales).  D in {64, 128}.
 *   workspace: >= attention_workspace_bytes(SPATTN_KIND_SELECTED or _LOCAL_AUX, ...).
 */
SPATTN_API int sparse_attention_fwd(const void* q, int dtype, int mode, const void* k_cache,
                         const void* v_cache, int cache_dtype, const int32_t* block_table,
                         int max_blocks_per_seq, int block_size, int num_blocks,
                         const float* key_scale, const float* value_scale,
                         const int32_t* cu_seqlens_q, const int32_t* seqlens_k, int B, int T,
                         int max_seqlen_q, const int32_t* sel_idx, const int32_t* sel_count,
                         int max_selected, int local_window, const void* aux_k,
                         const void* aux_v, int aux_dtype, int aux_len,
                         int64_t aux_batch_stride, int H_q, int H_kv, int D, float scale,
                         const float* sinks, void* out, void* workspace,
                         size_t workspace_bytes, int32_t* status, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPATTN_H */
