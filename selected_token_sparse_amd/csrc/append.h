// INT8 / FP8 code writers shared by the cache append and the fused decode step, and the
// launcher of prepare_and_append (api.hip validates the arguments, then calls it).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace spattn {

// One value x / s as an INT8 code (IEEE float32 division, round half to even, clamped to
// [-127, 127], NaN quotient -> 0), and eight of them: the cache append and the fused decode
// step write codes with these two functions only.
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

int launch_prepare_and_append(const int32_t* cu, const int32_t* past, int B, int T,
                              int32_t* seqlens_q, int32_t* seqlens_k, int32_t* token_req,
                              int32_t* token_pos, const void* k_new, const void* v_new,
                              int new_dtype, void* k_cache, void* v_cache, int cache_dtype,
                              const int32_t* block_table, int max_blocks, int block_size,
                              int num_blocks, const float* key_scale, const float* value_scale,
                              int H_kv, int D, const int32_t* committed, int32_t* status,
                              hipStream_t stream);

}  // namespace spattn
