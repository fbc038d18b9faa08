// Launcher of prepare_and_append (api.hip validates the arguments, then calls it).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spattn {

int launch_prepare_and_append(const int32_t* cu, const int32_t* past, int B, int T,
                              int32_t* seqlens_q, int32_t* seqlens_k, int32_t* token_req,
                              int32_t* token_pos, const void* k_new, const void* v_new,
                              int new_dtype, void* k_cache, void* v_cache, int cache_dtype,
                              const int32_t* block_table, int max_blocks, int block_size,
                              int num_blocks, const float* key_scale, const float* value_scale,
                              int H_kv, int D, const int32_t* committed, int32_t* status,
                              hipStream_t stream);

}  // namespace spattn
