// Launcher of the QKV prologue (api.hip validates the arguments, then calls it).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace spattn {

// Everything the QKV prologue needs; filled and validated by api.hip.
struct PrologueArgs {
  const void* qkv;        // packed [T, (H_q + 2 H_kv) * D], or nullptr (then q, k, v)
  const void* q;
  const void* k;
  const void* v;
  int dtype;
  const int32_t* cu;
  const int32_t* seqlens_k;
  int B, T, H_q, H_kv, D;
  int qk_norm;
  const float* q_norm_weight;
  const float* k_norm_weight;
  float norm_eps;
  int rotary_dim;         // 0: no rotation
  int interleaved;
  const float* cos_table;
  const float* sin_table;
  int max_position;
  const int32_t* position_ids;
  const int32_t* rotary_offsets;
  void* q_out;
  void* k_cache;
  void* v_cache;
  int cache_dtype;
  const int32_t* block_table;
  int max_blocks;
  int block_size;
  int num_blocks;
  const float* key_scale;
  const float* value_scale;
  const int32_t* committed;
  int32_t* status;
};

int launch_qkv_prologue(const PrologueArgs& a, hipStream_t stream);

}  // namespace spattn
