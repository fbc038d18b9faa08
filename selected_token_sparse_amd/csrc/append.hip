// kv_cache_append: scatter this step's K/V rows into the cache in place ("[WebGPU] Add
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

namespace spattn {

constexpr int kAppendThreads = 256;

__device__ __forceinline__ int8_t quantize_one(float x, float s) {
  float r = __builtin_rintf(x / s);  // IEEE float32 division, ties to even
  if (r != r) return 0;              // NaN quotient
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int8_t)(int)r;
}

// Eight consecutive elements of one KV head (D is a multiple of 8) into eight codes:
// INT8 (kFp8 = false) or FP8 E4M3 (kFp8 = true).
template <bool kFp8, typename NewT>
__device__ __forceinline__ void quantize8(const NewT* __restrict__ src, const float* __restrict__ scale,
                                          int8_t* __restrict__ dst) {
  union { int8_t c[8]; int2 v; } u;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if constexpr (kFp8) u.c[e] = (int8_t)quantize_fp8(to_f32(src[e]), scale[e]);
    else u.c[e] = quantize_one(to_f32(src[e]), scale[e]);
  }
  *reinterpret_cast<int2*>(dst) = u.v;
}

// kQuant: 0 = float cache (rows stored as they are), 1 = INT8 codes, 2 = FP8 E4M3 codes
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
  if (b < 0) {
    flags |= SPATTN_STATUS_BAD_CU;
  } else {
    const int q_len = cu[b + 1] - cu[b];
    const int kv_len = seqlens_k[b] + 1;
    const int p = kv_len - q_len + (r - cu[b]);
    // the caller's cursor must agree with the first position this step writes; every row
    // of the request makes the same check, so a disagreeing request writes nothing
    if (committed != nullptr && committed[b] != kv_len - q_len) flags |= SPATTN_STATUS_CURSOR;
    else if (p < 0) flags |= SPATTN_STATUS_SHORT_KV;
    else dst = cache_row(cd, b, p, 0, flags);
  }
  if (threadIdx.x == 0) raise_status(status, flags);
  if (dst < 0) return;
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

}  // namespace spattn
