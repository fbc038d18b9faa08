// C ABI entry points: argument validation on the host (nothing is enqueued when it fails),
// then the launchers.  The declarations and their contracts are in include/spattn.h.
#include <math.h>

#include <mutex>

#include "common.h"
#include "launch.h"
#include "append.h"
#include "prologue.h"
#include "topk.h"

using namespace spattn;

namespace {

bool float_dtype(int t) { return t == SPATTN_F32 || t == SPATTN_F16 || t == SPATTN_BF16; }
bool quantised_cache(int t) { return t == SPATTN_I8 || t == SPATTN_FP8; }

// The kernels read and write activations and cache rows with 16-byte vector accesses (a
// row of D elements is a multiple of 16 bytes), so every data pointer must be 16-byte
// aligned; null pointers are checked separately.
bool misaligned(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) != 0; }

// Shared checks of a KV cache description; returns SPATTN_OK or an error code.
int check_cache(const void* k_cache, const void* v_cache, int dtype, int cache_dtype,
                const int32_t* block_table, int max_blocks, int block_size, int num_blocks,
                const float* key_scale, const float* value_scale, int B, int H_kv, int D) {
  if (k_cache == nullptr || v_cache == nullptr) return SPATTN_ERR_NULL;
  if (misaligned(k_cache) || misaligned(v_cache)) return SPATTN_ERR_SHAPE;
  if (quantised_cache(cache_dtype)) {
    if (key_scale == nullptr || value_scale == nullptr) return SPATTN_ERR_NULL;
  } else if (cache_dtype != dtype) {
    return SPATTN_ERR_DTYPE;
  }
  if (block_size < 1 || num_blocks < 1) return SPATTN_ERR_SHAPE;
  if (block_table != nullptr) {
    if (max_blocks < 1) return SPATTN_ERR_SHAPE;
  } else if (num_blocks < B) {
    return SPATTN_ERR_SHAPE;
  }
  // cache rows (of D elements) are indexed with 32-bit integers
  if ((int64_t)num_blocks * block_size * H_kv >= (int64_t)1 << 31) return SPATTN_ERR_SHAPE;
  (void)D;
  return SPATTN_OK;
}

int check_heads(int H_q, int H_kv, int D) {
  if (H_q < 1 || H_kv < 1) return SPATTN_ERR_SHAPE;
  if (H_q % H_kv != 0) return SPATTN_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return SPATTN_ERR_UNSUPPORTED;
  return SPATTN_OK;
}

float resolve_scale(float scale, int D) { return scale == 0.0f ? 1.0f / sqrtf((float)D) : scale; }


// ---------------------------------------------------------------------------------------
// Scratch of paged_decode_step_noalloc: the split-K partials in a static device array
// (one copy per GPU, held until the process ends), for callers that cannot allocate.
// Host code never passes `scratch` itself (its host-side name is not a device address):
// the device address is looked up once per device with hipGetSymbolAddress and kept.
// ---------------------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = SPATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on its first use).  The
// stream must belong to the current device: each device has its own copy of the array.
int noalloc_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SPATTN_ERR_LAUNCH;
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess || sdev != dev) return SPATTN_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return SPATTN_ERR_LAUNCH;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SPATTN_OK;
}

}  // namespace

static int decode_step_impl(const int32_t* cu_seqlens_q, const int32_t* past_seqlens, int B, int T,
                      int32_t* seqlens_q, int32_t* seqlens_k, const void* q, const void* k_new,
                      const void* v_new, int dtype, void* k_cache, void* v_cache, int cache_dtype,
                      const int32_t* block_table, int max_blocks_per_seq, int block_size,
                      int num_blocks, const float* key_scale, const float* value_scale,
                      int max_seqlen_q, int max_seqlen_k, int H_q, int H_kv, int D, float scale,
                      int local_window, const float* sinks, void* out, void* workspace,
                      size_t workspace_bytes, const int32_t* committed_length, int32_t* status,
                      void* stream, bool static_scratch) {
  if (dtype != SPATTN_F16 && dtype != SPATTN_BF16) return float_dtype(dtype) ? SPATTN_ERR_UNSUPPORTED : SPATTN_ERR_DTYPE;
  int rc = check_heads(H_q, H_kv, D);
  if (rc != SPATTN_OK) return rc;
  if (B < 0 || T < 0 || max_seqlen_q < 0 || max_seqlen_k < 0) return SPATTN_ERR_SHAPE;
  if (B > kStepMaxB) return SPATTN_ERR_UNSUPPORTED;
  if (use_prefill_path(SPATTN_KIND_PAGED, dtype, max_seqlen_q)) return SPATTN_ERR_UNSUPPORTED;
  if (cu_seqlens_q == nullptr || past_seqlens == nullptr || seqlens_q == nullptr || seqlens_k == nullptr)
    return SPATTN_ERR_NULL;
  hipStream_t st = (hipStream_t)stream;
  // no rows: the metadata is all there is to do
  if (T == 0) return launch_prepare_seqlens(cu_seqlens_q, past_seqlens, B, T, seqlens_q, seqlens_k,
                                            nullptr, nullptr, status, st);
  if (B == 0) return SPATTN_ERR_SHAPE;
  if (q == nullptr || k_new == nullptr || v_new == nullptr || out == nullptr) return SPATTN_ERR_NULL;
  if (misaligned(q) || misaligned(k_new) || misaligned(v_new) || misaligned(out)) return SPATTN_ERR_SHAPE;
  rc = check_cache(k_cache, v_cache, dtype, cache_dtype, block_table, max_blocks_per_seq,
                   block_size, num_blocks, key_scale, value_scale, B, H_kv, D);
  if (rc != SPATTN_OK) return rc;

  AttnArgs a{};
  a.kind = SPATTN_KIND_PAGED;
  a.q = q; a.dtype = dtype; a.k_cache = k_cache; a.v_cache = v_cache; a.cache_dtype = cache_dtype;
  a.block_table = block_table; a.max_blocks = max_blocks_per_seq; a.block_size = block_size;
  a.num_blocks = num_blocks; a.key_scale = key_scale; a.value_scale = value_scale;
  a.cu = cu_seqlens_q; a.seqlens_k = nullptr; a.B = B; a.T = T;
  a.max_q = max_seqlen_q; a.max_k = max_seqlen_k;
  a.window = local_window > 0 ? local_window : 0;
  a.H_q = H_q; a.H_kv = H_kv; a.D = D;
  a.scale = resolve_scale(scale, D);
  a.sinks = sinks; a.out = out; a.workspace = workspace; a.status = status;
  a.past = past_seqlens; a.k_new = k_new; a.v_new = v_new;
  a.seqlens_q_out = seqlens_q; a.seqlens_k_out = seqlens_k;
  a.committed = committed_length;
  const SplitPlan plan = make_split_plan(a.kind, dtype, cache_dtype, B, T, max_seqlen_q,
                                         max_seqlen_k, 0, a.window, H_q, H_kv, D);
  if (plan.n_splits < 0) return SPATTN_ERR_SHAPE;
  if (static_scratch && plan.ws_bytes > 0) {
    // the partials go to the static array: checked against its size, then its address
    if (plan.ws_bytes > kNoAllocScratchBytes) return SPATTN_ERR_WORKSPACE;
    const int rc2 = noalloc_scratch(st, &a.workspace);
    if (rc2 != SPATTN_OK) return rc2;
  } else if (plan.ws_bytes > 0 && (workspace == nullptr || workspace_bytes < plan.ws_bytes)) {
    return SPATTN_ERR_WORKSPACE;
  }
  return launch_split_attention(a, plan, st);
}

extern "C" {

int prepare_seqlens(const int32_t* cu_seqlens_q, const int32_t* past_seqlens, int B, int T,
                    int32_t* seqlens_q, int32_t* seqlens_k, int32_t* token_req,
                    int32_t* token_pos, int32_t* status, void* stream) {
  if (cu_seqlens_q == nullptr) return SPATTN_ERR_NULL;
  if (B > 0 && (past_seqlens == nullptr || seqlens_q == nullptr || seqlens_k == nullptr))
    return SPATTN_ERR_NULL;
  if (B < 0 || T < 0) return SPATTN_ERR_SHAPE;
  return launch_prepare_seqlens(cu_seqlens_q, past_seqlens, B, T, seqlens_q, seqlens_k, token_req,
                                token_pos, status, (hipStream_t)stream);
}

int kv_cache_append(const void* k_new, const void* v_new, int new_dtype,
                    const int32_t* cu_seqlens_q, const int32_t* seqlens_k, int B, int T,
                    void* k_cache, void* v_cache, int cache_dtype, const int32_t* block_table,
                    int max_blocks_per_seq, int block_size, int num_blocks,
                    const float* key_scale, const float* value_scale, int H_kv, int D,
                    const int32_t* committed_length, int32_t* status, void* stream) {
  if (B < 0 || T < 0 || H_kv < 1 || D < 8 || D % 8 != 0) return SPATTN_ERR_SHAPE;
  if (!float_dtype(new_dtype)) return SPATTN_ERR_DTYPE;
  if (!quantised_cache(cache_dtype) && !float_dtype(cache_dtype)) return SPATTN_ERR_DTYPE;
  if (T == 0) return SPATTN_OK;
  if (B == 0) return SPATTN_ERR_SHAPE;
  if (k_new == nullptr || v_new == nullptr || cu_seqlens_q == nullptr || seqlens_k == nullptr)
    return SPATTN_ERR_NULL;
  if (misaligned(k_new) || misaligned(v_new)) return SPATTN_ERR_SHAPE;
  int rc = check_cache(k_cache, v_cache, new_dtype, cache_dtype, block_table, max_blocks_per_seq,
                       block_size, num_blocks, key_scale, value_scale, B, H_kv, D);
  if (rc != SPATTN_OK) return rc;
  return launch_kv_cache_append(k_new, v_new, new_dtype, cu_seqlens_q, seqlens_k, B, T, k_cache,
                                v_cache, cache_dtype, block_table, max_blocks_per_seq, block_size,
                                num_blocks, key_scale, value_scale, H_kv, D, committed_length,
                                status, (hipStream_t)stream);
}

int prepare_and_append(const int32_t* cu_seqlens_q, const int32_t* past_seqlens, int B, int T,
                       int32_t* seqlens_q, int32_t* seqlens_k, int32_t* token_req,
                       int32_t* token_pos, const void* k_new, const void* v_new, int new_dtype,
                       void* k_cache, void* v_cache, int cache_dtype, const int32_t* block_table,
                       int max_blocks_per_seq, int block_size, int num_blocks,
                       const float* key_scale, const float* value_scale, int H_kv, int D,
                       const int32_t* committed_length, int32_t* status, void* stream) {
  // the checks of both calls, before anything is enqueued
  if (B < 0 || B > 8192 || T < 0) return SPATTN_ERR_SHAPE;
  if (cu_seqlens_q == nullptr || past_seqlens == nullptr || seqlens_q == nullptr || seqlens_k == nullptr)
    return SPATTN_ERR_NULL;
  if (H_kv < 1 || D < 8 || D % 8 != 0) return SPATTN_ERR_SHAPE;
  if (!float_dtype(new_dtype)) return SPATTN_ERR_DTYPE;
  if (!quantised_cache(cache_dtype) && !float_dtype(cache_dtype)) return SPATTN_ERR_DTYPE;
  if (T > 0) {
    if (B == 0) return SPATTN_ERR_SHAPE;
    if (k_new == nullptr || v_new == nullptr) return SPATTN_ERR_NULL;
    if (misaligned(k_new) || misaligned(v_new)) return SPATTN_ERR_SHAPE;
    const int rc = check_cache(k_cache, v_cache, new_dtype, cache_dtype, block_table,
                               max_blocks_per_seq, block_size, num_blocks, key_scale, value_scale,
                               B, H_kv, D);
    if (rc != SPATTN_OK) return rc;
  }
  return spattn::launch_prepare_and_append(cu_seqlens_q, past_seqlens, B, T, seqlens_q, seqlens_k,
                                           token_req, token_pos, k_new, v_new, new_dtype, k_cache,
                                           v_cache, cache_dtype, block_table, max_blocks_per_seq,
                                           block_size, num_blocks, key_scale, value_scale, H_kv, D,
                                           committed_length, status, (hipStream_t)stream);
}

int qkv_prologue(const void* qkv, const void* q, const void* k, const void* v, int dtype,
                 const int32_t* cu_seqlens_q, const int32_t* seqlens_k, int B, int T, int H_q,
                 int H_kv, int D, int qk_norm, const float* q_norm_weight,
                 const float* k_norm_weight, float norm_eps, int rotary_dim,
                 int rotary_interleaved, const float* cos_table, const float* sin_table,
                 int max_position, const int32_t* position_ids, const int32_t* rotary_offsets,
                 void* q_out, void* k_cache, void* v_cache, int cache_dtype,
                 const int32_t* block_table, int max_blocks_per_seq, int block_size,
                 int num_blocks, const float* key_scale, const float* value_scale,
                 const int32_t* committed_length, int32_t* status, void* stream) {
  if (B < 0 || T < 0 || H_q < 1 || H_kv < 1 || D < 8 || D > 256 || D % 8 != 0)
    return SPATTN_ERR_SHAPE;
  if (!float_dtype(dtype)) return SPATTN_ERR_DTYPE;
  if (!quantised_cache(cache_dtype) && !float_dtype(cache_dtype)) return SPATTN_ERR_DTYPE;
  if (rotary_dim < 0 || rotary_dim > D || rotary_dim % 2 != 0) return SPATTN_ERR_SHAPE;
  if (rotary_dim > 0 && (cos_table == nullptr || sin_table == nullptr)) return SPATTN_ERR_NULL;
  if (rotary_dim > 0 && max_position < 1) return SPATTN_ERR_SHAPE;
  if (qk_norm && !(norm_eps >= 0.f && norm_eps < __builtin_huge_valf())) return SPATTN_ERR_SHAPE;
  if (T == 0) return SPATTN_OK;
  if (B == 0) return SPATTN_ERR_SHAPE;
  if (qkv == nullptr && (q == nullptr || k == nullptr || v == nullptr)) return SPATTN_ERR_NULL;
  if (q_out == nullptr || cu_seqlens_q == nullptr || seqlens_k == nullptr) return SPATTN_ERR_NULL;
  if (misaligned(qkv) || misaligned(q) || misaligned(k) || misaligned(v) || misaligned(q_out))
    return SPATTN_ERR_SHAPE;
  int rc = check_cache(k_cache, v_cache, dtype, cache_dtype, block_table, max_blocks_per_seq,
                       block_size, num_blocks, key_scale, value_scale, B, H_kv, D);
  if (rc != SPATTN_OK) return rc;
  spattn::PrologueArgs a{};
  a.qkv = qkv; a.q = q; a.k = k; a.v = v; a.dtype = dtype;
  a.cu = cu_seqlens_q; a.seqlens_k = seqlens_k;
  a.B = B; a.T = T; a.H_q = H_q; a.H_kv = H_kv; a.D = D;
  a.qk_norm = qk_norm != 0; a.q_norm_weight = q_norm_weight; a.k_norm_weight = k_norm_weight;
  a.norm_eps = norm_eps;
  a.rotary_dim = rotary_dim; a.interleaved = rotary_interleaved != 0;
  a.cos_table = cos_table; a.sin_table = sin_table; a.max_position = max_position;
  a.position_ids = position_ids; a.rotary_offsets = rotary_offsets;
  a.q_out = q_out; a.k_cache = k_cache; a.v_cache = v_cache; a.cache_dtype = cache_dtype;
  a.block_table = block_table; a.max_blocks = max_blocks_per_seq; a.block_size = block_size;
  a.num_blocks = num_blocks; a.key_scale = key_scale; a.value_scale = value_scale;
  a.committed = committed_length; a.status = status;
  return spattn::launch_qkv_prologue(a, (hipStream_t)stream);
}

int topk_select(const float* scores, int L, const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                int B, int T, int H_kv, int k, int tail, int32_t* sel_idx, int capacity,
                int32_t* sel_count, int32_t* status, void* stream) {
  if (B < 0 || T < 0 || H_kv < 1 || L < 1 || L > 65536) return L > 65536 ? SPATTN_ERR_UNSUPPORTED : SPATTN_ERR_SHAPE;
  if (k < 0 || tail < 0 || capacity < k) return SPATTN_ERR_SHAPE;
  if (T == 0) return SPATTN_OK;
  if (B == 0) return SPATTN_ERR_SHAPE;
  if (scores == nullptr || cu_seqlens_q == nullptr || seqlens_k == nullptr || sel_count == nullptr ||
      (capacity > 0 && sel_idx == nullptr))
    return SPATTN_ERR_NULL;
  spattn::TopkArgs a{};
  a.scores = scores; a.L = L; a.cu = cu_seqlens_q; a.seqlens_k = seqlens_k;
  a.B = B; a.T = T; a.H_kv = H_kv; a.k = k; a.tail = tail; a.capacity = capacity;
  a.sel_idx = sel_idx; a.sel_count = sel_count; a.status = status;
  return spattn::launch_topk_select(a, (hipStream_t)stream);
}

size_t attention_workspace_bytes(int kind, int dtype, int B, int T, int max_seqlen_q,
                                 int max_seqlen_k, int max_selected, int local_window,
                                 int H_q, int H_kv, int D) {
  const size_t bad = (size_t)-1;
  if (kind < SPATTN_KIND_PAGED || kind > SPATTN_KIND_LOCAL_AUX) return bad;
  if (!float_dtype(dtype)) return bad;
  if (B < 0 || T < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || max_selected < 0) return bad;
  if (check_heads(H_q, H_kv, D) != SPATTN_OK) return bad;
  if (kind == SPATTN_KIND_LOCAL_AUX && local_window <= 0) return bad;
  if (kind == SPATTN_KIND_PAGED && use_prefill_path(kind, dtype, max_seqlen_q)) return 0;
  // the plan of a 16-bit cache: over an 8-bit cache a call never needs more
  const SplitPlan plan = make_split_plan(kind, dtype, dtype, B, T, max_seqlen_q, max_seqlen_k,
                                         max_selected, local_window, H_q, H_kv, D);
  return plan.n_splits < 0 ? bad : plan.ws_bytes;
}

int paged_attention_fwd(const void* q, int dtype, const void* k_cache, const void* v_cache,
                        int cache_dtype, const int32_t* block_table, int max_blocks_per_seq,
                        int block_size, int num_blocks, const float* key_scale,
                        const float* value_scale, const int32_t* cu_seqlens_q,
                        const int32_t* seqlens_k, int B, int T, int max_seqlen_q,
                        int max_seqlen_k, int H_q, int H_kv, int D, float scale, int is_causal,
                        int local_window, const float* sinks, void* out, void* workspace,
                        size_t workspace_bytes, int32_t* status, void* stream) {
  if (!float_dtype(dtype)) return SPATTN_ERR_DTYPE;
  if (is_causal != 1) return SPATTN_ERR_UNSUPPORTED;
  int rc = check_heads(H_q, H_kv, D);
  if (rc != SPATTN_OK) return rc;
  if (B < 0 || T < 0 || max_seqlen_q < 0 || max_seqlen_k < 0) return SPATTN_ERR_SHAPE;
  if (T == 0) return SPATTN_OK;
  if (B == 0) return SPATTN_ERR_SHAPE;
  if (q == nullptr || out == nullptr || cu_seqlens_q == nullptr || seqlens_k == nullptr)
    return SPATTN_ERR_NULL;
  if (misaligned(q) || misaligned(out)) return SPATTN_ERR_SHAPE;
  rc = check_cache(k_cache, v_cache, dtype, cache_dtype, block_table, max_blocks_per_seq,
                   block_size, num_blocks, key_scale, value_scale, B, H_kv, D);
  if (rc != SPATTN_OK) return rc;

  AttnArgs a{};
  a.kind = SPATTN_KIND_PAGED;
  a.q = q; a.dtype = dtype; a.k_cache = k_cache; a.v_cache = v_cache; a.cache_dtype = cache_dtype;
  a.block_table = block_table; a.max_blocks = max_blocks_per_seq; a.block_size = block_size;
  a.num_blocks = num_blocks; a.key_scale = key_scale; a.value_scale = value_scale;
  a.cu = cu_seqlens_q; a.seqlens_k = seqlens_k; a.B = B; a.T = T;
  a.max_q = max_seqlen_q; a.max_k = max_seqlen_k;
  a.window = local_window > 0 ? local_window : 0;
  a.H_q = H_q; a.H_kv = H_kv; a.D = D;
  a.scale = resolve_scale(scale, D);
  a.sinks = sinks; a.out = out; a.workspace = workspace; a.status = status;
  hipStream_t st = (hipStream_t)stream;
  if (use_prefill_path(a.kind, dtype, max_seqlen_q)) return launch_prefill_attention(a, st);
  const SplitPlan plan = make_split_plan(a.kind, dtype, cache_dtype, B, T, max_seqlen_q,
                                         max_seqlen_k, 0, a.window, H_q, H_kv, D);
  if (plan.n_splits < 0) return SPATTN_ERR_SHAPE;
  if (plan.ws_bytes > 0 && (workspace == nullptr || workspace_bytes < plan.ws_bytes))
    return SPATTN_ERR_WORKSPACE;
  return launch_split_attention(a, plan, st);
}

int paged_decode_step(const int32_t* cu_seqlens_q, const int32_t* past_seqlens, int B, int T,
                      int32_t* seqlens_q, int32_t* seqlens_k, const void* q, const void* k_new,
                      const void* v_new, int dtype, void* k_cache, void* v_cache, int cache_dtype,
                      const int32_t* block_table, int max_blocks_per_seq, int block_size,
                      int num_blocks, const float* key_scale, const float* value_scale,
                      int max_seqlen_q, int max_seqlen_k, int H_q, int H_kv, int D, float scale,
                      int local_window, const float* sinks, void* out, void* workspace,
                      size_t workspace_bytes, const int32_t* committed_length, int32_t* status,
                      void* stream) {
  return decode_step_impl(cu_seqlens_q, past_seqlens, B, T, seqlens_q, seqlens_k, q, k_new, v_new,
                          dtype, k_cache, v_cache, cache_dtype, block_table, max_blocks_per_seq,
                          block_size, num_blocks, key_scale, value_scale, max_seqlen_q,
                          max_seqlen_k, H_q, H_kv, D, scale, local_window, sinks, out, workspace,
                          workspace_bytes, committed_length, status, stream, false);
}

int paged_decode_step_noalloc(const int32_t* cu_seqlens_q, const int32_t* past_seqlens, int B,
                              int T, int32_t* seqlens_q, int32_t* seqlens_k, const void* q,
                              const void* k_new, const void* v_new, int dtype, void* k_cache,
                              void* v_cache, int cache_dtype, const int32_t* block_table,
                              int max_blocks_per_seq, int block_size, int num_blocks,
                              const float* key_scale, const float* value_scale, int max_seqlen_q,
                              int max_seqlen_k, int H_q, int H_kv, int D, float scale,
                              int local_window, const float* sinks, void* out,
                              const int32_t* committed_length, int32_t* status, void* stream) {
  return decode_step_impl(cu_seqlens_q, past_seqlens, B, T, seqlens_q, seqlens_k, q, k_new, v_new,
                          dtype, k_cache, v_cache, cache_dtype, block_table, max_blocks_per_seq,
                          block_size, num_blocks, key_scale, value_scale, max_seqlen_q,
                          max_seqlen_k, H_q, H_kv, D, scale, local_window, sinks, out, nullptr, 0,
                          committed_length, status, stream, true);
}

int sparse_attention_fwd(const void* q, int dtype, int mode, const void* k_cache,
                         const void* v_cache, int cache_dtype, const int32_t* block_table,
                         int max_blocks_per_seq, int block_size, int num_blocks,
                         const float* key_scale, const float* value_scale,
                         const int32_t* cu_seqlens_q, const int32_t* seqlens_k, int B, int T,
                         int max_seqlen_q, const int32_t* sel_idx, const int32_t* sel_count,
                         int max_selected, int local_window, const void* aux_k,
                         const void* aux_v, int aux_dtype, int aux_len,
                         int64_t aux_batch_stride, int H_q, int H_kv, int D, float scale,
                         const float* sinks, void* out, void* workspace,
                         size_t workspace_bytes, int32_t* status, void* stream) {
  if (!float_dtype(dtype)) return SPATTN_ERR_DTYPE;
  if (mode != 0 && mode != 1) return SPATTN_ERR_UNSUPPORTED;
  if (mode == 0 && local_window > 0) return SPATTN_ERR_UNSUPPORTED;
  if (mode == 1 && local_window <= 0) return SPATTN_ERR_UNSUPPORTED;
  int rc = check_heads(H_q, H_kv, D);
  if (rc != SPATTN_OK) return rc;
  if (B < 0 || T < 0 || max_seqlen_q < 0 || max_selected < 0) return SPATTN_ERR_SHAPE;
  if (T == 0) return SPATTN_OK;
  if (B == 0) return SPATTN_ERR_SHAPE;
  if (q == nullptr || out == nullptr || cu_seqlens_q == nullptr || seqlens_k == nullptr)
    return SPATTN_ERR_NULL;
  if (max_selected > 0 && sel_idx == nullptr) return SPATTN_ERR_NULL;
  if (misaligned(q) || misaligned(out) || misaligned(aux_k) || misaligned(aux_v))
    return SPATTN_ERR_SHAPE;
  rc = check_cache(k_cache, v_cache, dtype, cache_dtype, block_table, max_blocks_per_seq,
                   block_size, num_blocks, key_scale, value_scale, B, H_kv, D);
  if (rc != SPATTN_OK) return rc;
  if (mode == 1) {
    if (aux_k == nullptr || aux_v == nullptr) return SPATTN_ERR_NULL;
    if (aux_dtype != dtype) return SPATTN_ERR_DTYPE;
    if (aux_len < 0 || aux_batch_stride < 0 || aux_batch_stride % D != 0) return SPATTN_ERR_SHAPE;
    const int64_t rows = (int64_t)(B - 1) * (aux_batch_stride / D) + (int64_t)aux_len * H_kv;
    if (rows >= (int64_t)1 << 31) return SPATTN_ERR_SHAPE;
  }
  AttnArgs a{};
  a.kind = mode == 0 ? SPATTN_KIND_SELECTED : SPATTN_KIND_LOCAL_AUX;
  a.q = q; a.dtype = dtype; a.k_cache = k_cache; a.v_cache = v_cache; a.cache_dtype = cache_dtype;
  a.block_table = block_table; a.max_blocks = max_blocks_per_seq; a.block_size = block_size;
  a.num_blocks = num_blocks; a.key_scale = key_scale; a.value_scale = value_scale;
  a.cu = cu_seqlens_q; a.seqlens_k = seqlens_k; a.B = B; a.T = T;
  a.max_q = max_seqlen_q; a.max_k = -1;
  a.sel_idx = sel_idx; a.sel_count = sel_count; a.max_selected = max_selected;
  a.window = mode == 1 ? local_window : 0;
  a.aux_k = aux_k; a.aux_v = aux_v; a.aux_len = aux_len; a.aux_stride = aux_batch_stride;
  a.H_q = H_q; a.H_kv = H_kv; a.D = D;
  a.scale = resolve_scale(scale, D);
  a.sinks = sinks; a.out = out; a.workspace = workspace; a.status = status;
  const SplitPlan plan = make_split_plan(a.kind, dtype, a.cache_dtype, B, T, max_seqlen_q, 0,
                                         max_selected, a.window, H_q, H_kv, D);
  if (plan.n_splits < 0) return SPATTN_ERR_SHAPE;
  if (plan.ws_bytes > 0 && (workspace == nullptr || workspace_bytes < plan.ws_bytes))
    return SPATTN_ERR_WORKSPACE;
  return launch_split_attention(a, plan, (hipStream_t)stream);
}

}  // extern "C"
