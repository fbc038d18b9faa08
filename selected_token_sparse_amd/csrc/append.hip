// kv_cache_append (and prepare_and_append): scatter this step's K/V rows into the cache in place ("[WebGPU] Add
// SparsePagedAttention", file summaries: scatter through the token-to-slot mapping;
// "[WebGPU] Add DynamicSparseAttention", Description: alias-safe in-place update of
// contiguous caches; INT8 per-channel quantisation per the Key Changes table of the
// DynamicSparseAttention INT8 KV cache page).
//
// The packed input row holds all KV heads of one position; in the cache each head's row
// of D elements sits in its own head-major run of the block ([nb, H_kv, bs, D]), so lanes
// copy 16-byte pieces to slot `off` of every head (an INT8 append turns eight input
// elements into eight codes per lane).
#include "common.h"
#include "launch.h"
#include "append.h"

namespace spattn {

constexpr int kAppendThreads = 256;
constexpr int kFusedMaxB = kAppendThreads - 1;   // boundaries staged one per thread

// Row r of k_new / v_new into the cache row `dst` (element offset of KV head 0's slot).
// kQuant: 0 = float cache (rows stored as they are), 1 = INT8 codes, 2 = FP8 E4M3 codes.
template <typename NewT, int kQuant>
__device__ __forceinline__ void append_row(const NewT* __restrict__ k_new, const NewT* __restrict__ v_new,
                                           int r, int64_t dst, void* __restrict__ k_cache,
                                           void* __restrict__ v_cache, const CacheDesc& cd,
                                           const float* __restrict__ key_scale,
                                           const float* __restrict__ value_scale) {
  const int row_elems = cd.H_kv * cd.D;
  const int64_t src = (int64_t)r * row_elems;
  const int64_t head_stride = (int64_t)cd.block_size * cd.D;  // between heads in a block
  if constexpr (kQuant != 0) {
    int8_t* kc = reinterpret_cast<int8_t*>(k_cache) + dst;
    int8_t* vc = reinterpret_cast<int8_t*>(v_cache) + dst;
    for (int e = threadIdx.x * 8; e < row_elems; e += kAppendThreads * 8) {
      const int c = e / cd.D, d = e - c * cd.D;
      quantize8<kQuant == 2>(k_new + src + e, key_scale + e, kc + c * head_stride + d);
      quantize8<kQuant == 2>(v_new + src + e, value_scale + e, vc + c * head_stride + d);
    }
  } else {
    constexpr int kPer = 16 / sizeof(NewT);
    NewT* kc = reinterpret_cast<NewT*>(k_cache) + dst;
    NewT* vc = reinterpret_cast<NewT*>(v_cache) + dst;
    for (int e = threadIdx.x * kPer; e < row_elems; e += kAppendThreads * kPer) {
      const int c = e / cd.D, d = e - c * cd.D;
      store16(kc + c * head_stride + d, load16(k_new + src + e));
      store16(vc + c * head_stride + d, load16(v_new + src + e));
    }
  }
}

// The checks of row r of request b before it is written; returns the cache row or -1.
__device__ __forceinline__ int64_t append_slot(const int32_t* __restrict__ cu, int b, int r, int kv_len,
                                               const CacheDesc& cd, const int32_t* __restrict__ committed,
                                               int& flags) {
  const int q_len = cu[b + 1] - cu[b];
  const int p = kv_len - q_len + (r - cu[b]);
  // the caller's cursor must agree with the first position this step writes; every row
  // of the request makes the same check, so a disagreeing request writes nothing
  if (committed != nullptr && committed[b] != kv_len - q_len) { flags |= SPATTN_STATUS_CURSOR; return -1; }
  if (p < 0) { flags |= SPATTN_STATUS_SHORT_KV; return -1; }
  return cache_row(cd, b, p, 0, flags);
}

template <typename NewT, int kQuant>
__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(
    const NewT* __restrict__ k_new, const NewT* __restrict__ v_new, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ seqlens_k, int B, void* __restrict__ k_cache,
    void* __restrict__ v_cache, CacheDesc cd, const float* __restrict__ key_scale,
    const float* __restrict__ value_scale, const int32_t* __restrict__ committed,
    int32_t* status) {
  const int r = blockIdx.x;
  int flags = 0;
  const int b = find_request(cu, B, r);
  int64_t dst = -1;
  if (b < 0) flags |= SPATTN_STATUS_BAD_CU;
  else dst = append_slot(cu, b, r, seqlens_k[b] + 1, cd, committed, flags);
  if (threadIdx.x == 0) raise_status(status, flags);
  if (dst < 0) return;
  append_row<NewT, kQuant>(k_new, v_new, r, dst, k_cache, v_cache, cd, key_scale, value_scale);
}

// prepare_seqlens followed by kv_cache_append in one launch (B <= kFusedMaxB).  Every
// workgroup rebuilds the sanitised request boundaries (running maximum of cu, clamped to
// [0, T]) in LDS with the metadata kernel's arithmetic; workgroup 0 writes the per-request
// lengths and the malformed-input flag, workgroup r the metadata of token r, and then
// appends row r exactly as kv_append_kernel does with the seqlens_k just computed.
template <typename NewT, int kQuant>
__global__ __launch_bounds__(kAppendThreads) void prepare_append_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ past, int B, int T,
    int32_t* __restrict__ seqlens_q, int32_t* __restrict__ seqlens_k,
    int32_t* __restrict__ token_req, int32_t* __restrict__ token_pos,
    const NewT* __restrict__ k_new, const NewT* __restrict__ v_new, void* __restrict__ k_cache,
    void* __restrict__ v_cache, CacheDesc cd, const float* __restrict__ key_scale,
    const float* __restrict__ value_scale, const int32_t* __restrict__ committed,
    int32_t* status) {
  __shared__ int bound[kFusedMaxB + 1];
  __shared__ int wave_max[kAppendThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = B + 1;                       // <= kAppendThreads
  // running maximum of cu over the boundaries (one per thread), clamped to [0, T]
  int v = tid < n ? cu[tid] : INT32_MIN;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(v, o, 64);
    if (lane >= o) v = max(v, y);
  }
  if (lane == 63) wave_max[wave] = v;
  __syncthreads();
  for (int w = 0; w < wave; ++w) v = max(v, wave_max[w]);
  if (tid < n) bound[tid] = min(max(v, 0), T);
  __syncthreads();

  if (blockIdx.x == 0) {
    int bad = 0;
    for (int b = tid; b < B; b += kAppendThreads) {
      const int c0 = cu[b], c1 = cu[b + 1];
      int pb = past[b];
      if (c1 < c0 || pb < 0) bad = 1;
      pb = max(pb, 0);
      const int q_len = bound[b + 1] - bound[b];
      seqlens_q[b] = q_len;
      seqlens_k[b] = pb + q_len - 1;
    }
    if (tid == 0 && (cu[0] != 0 || cu[B] != T)) bad = 1;
    if (__ballot(bad) != 0 && lane == 0) raise_status(status, SPATTN_STATUS_BAD_CU);
  }
  const int r = blockIdx.x;
  if (r >= T) return;
  // token r: its request and key position over the sanitised boundaries
  int req = -1;
  if (B > 0 && bound[0] <= r) {
    int lo = 0, hi = B - 1;                  // largest b with bound[b] <= r
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (bound[mid] <= r) lo = mid; else hi = mid - 1;
    }
    if (r < bound[lo + 1]) req = lo;
  }
  if (tid == 0) {
    if (token_req != nullptr) token_req[r] = req;
    if (token_pos != nullptr) token_pos[r] = req >= 0 ? max(past[req], 0) + (r - bound[req]) : -1;
  }
  // the append of row r, as kv_append_kernel makes it (request found on the raw cu)
  int flags = 0;
  const int b = find_request(cu, B, r);
  int64_t dst = -1;
  if (b < 0) {
    flags |= SPATTN_STATUS_BAD_CU;
  } else {
    const int kv_len = max(past[b], 0) + (bound[b + 1] - bound[b]);   // seqlens_k[b] + 1
    dst = append_slot(cu, b, r, kv_len, cd, committed, flags);
  }
  if (tid == 0) raise_status(status, flags);
  if (dst < 0) return;
  append_row<NewT, kQuant>(k_new, v_new, r, dst, k_cache, v_cache, cd, key_scale, value_scale);
}

int launch_kv_cache_append(const void* k_new, const void* v_new, int new_dtype,
                           const int32_t* cu, const int32_t* seqlens_k, int B, int T,
                           void* k_cache, void* v_cache, int cache_dtype,
                           const int32_t* block_table, int max_blocks, int block_size,
                           int num_blocks, const float* key_scale, const float* value_scale,
                           int H_kv, int D, const int32_t* committed, int32_t* status,
                           hipStream_t stream) {
  if (T == 0) return SPATTN_OK;
  CacheDesc cd;
  cd.block_table = block_table;
  cd.max_blocks = max_blocks;
  cd.block_size = block_size;
  cd.bs_shift = (block_size & (block_size - 1)) == 0 ? __builtin_ctz(block_size) : -1;
  cd.num_blocks = num_blocks;
  cd.H_kv = H_kv;
  cd.D = D;
  dim3 grid(T), block(kAppendThreads);
  const int quant = cache_dtype == SPATTN_I8 ? 1 : (cache_dtype == SPATTN_FP8 ? 2 : 0);
#define SPATTN_APPEND(NT, Q)                                                               \
  hipLaunchKernelGGL((kv_append_kernel<NT, Q>), grid, block, 0, stream,                    \
                     reinterpret_cast<const NT*>(k_new), reinterpret_cast<const NT*>(v_new), \
                     cu, seqlens_k, B, k_cache, v_cache, cd, key_scale, value_scale, committed, \
                     status)
#define SPATTN_APPEND_Q(NT)                         \
  if (quant == 1) SPATTN_APPEND(NT, 1);             \
  else if (quant == 2) SPATTN_APPEND(NT, 2);        \
  else SPATTN_APPEND(NT, 0)
  switch (new_dtype) {
    case SPATTN_F32: SPATTN_APPEND_Q(float); break;
    case SPATTN_F16: SPATTN_APPEND_Q(f16); break;
    case SPATTN_BF16: SPATTN_APPEND_Q(bf16); break;
    default: return SPATTN_ERR_DTYPE;
  }
#undef SPATTN_APPEND_Q
#undef SPATTN_APPEND
  return hipGetLastError() == hipSuccess ? SPATTN_OK : SPATTN_ERR_LAUNCH;
}

int launch_prepare_and_append(const int32_t* cu, const int32_t* past, int B, int T,
                              int32_t* seqlens_q, int32_t* seqlens_k, int32_t* token_req,
                              int32_t* token_pos, const void* k_new, const void* v_new,
                              int new_dtype, void* k_cache, void* v_cache, int cache_dtype,
                              const int32_t* block_table, int max_blocks, int block_size,
                              int num_blocks, const float* key_scale, const float* value_scale,
                              int H_kv, int D, const int32_t* committed, int32_t* status,
                              hipStream_t stream) {
  if (B > kFusedMaxB) {
    // too many requests to stage per workgroup: the two kernels, in order
    int rc = launch_prepare_seqlens(cu, past, B, T, seqlens_q, seqlens_k, token_req, token_pos,
                                    status, stream);
    if (rc != SPATTN_OK) return rc;
    return launch_kv_cache_append(k_new, v_new, new_dtype, cu, seqlens_k, B, T, k_cache, v_cache,
                                  cache_dtype, block_table, max_blocks, block_size, num_blocks,
                                  key_scale, value_scale, H_kv, D, committed, status, stream);
  }
  CacheDesc cd;
  cd.block_table = block_table;
  cd.max_blocks = max_blocks;
  cd.block_size = block_size;
  cd.bs_shift = (block_size & (block_size - 1)) == 0 ? __builtin_ctz(block_size) : -1;
  cd.num_blocks = num_blocks;
  cd.H_kv = H_kv;
  cd.D = D;
  dim3 grid(T > 0 ? T : 1), block(kAppendThreads);
  const int quant = cache_dtype == SPATTN_I8 ? 1 : (cache_dtype == SPATTN_FP8 ? 2 : 0);
#define SPATTN_FUSED(NT, Q)                                                                   \
  hipLaunchKernelGGL((prepare_append_kernel<NT, Q>), grid, block, 0, stream, cu, past, B, T,  \
                     seqlens_q, seqlens_k, token_req, token_pos,                              \
                     reinterpret_cast<const NT*>(k_new), reinterpret_cast<const NT*>(v_new),  \
                     k_cache, v_cache, cd, key_scale, value_scale, committed, status)
#define SPATTN_FUSED_Q(NT)                         \
  if (quant == 1) SPATTN_FUSED(NT, 1);             \
  else if (quant == 2) SPATTN_FUSED(NT, 2);        \
  else SPATTN_FUSED(NT, 0)
  switch (new_dtype) {
    case SPATTN_F32: SPATTN_FUSED_Q(float); break;
    case SPATTN_F16: SPATTN_FUSED_Q(f16); break;
    case SPATTN_BF16: SPATTN_FUSED_Q(bf16); break;
    default: return SPATTN_ERR_DTYPE;
  }
#undef SPATTN_FUSED_Q
#undef SPATTN_FUSED
  return hipGetLastError() == hipSuccess ? SPATTN_OK : SPATTN_ERR_LAUNCH;
}

}  // namespace spattn
