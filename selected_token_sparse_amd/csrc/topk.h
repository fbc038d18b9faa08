// Launcher of the TopK selection (api.hip validates the arguments, then calls it).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace spattn {

struct TopkArgs {
  const float* scores;      // [T, H_kv, L]
  int L;
  const int32_t* cu;
  const int32_t* seqlens_k;
  int B, T, H_kv;
  int k, tail, capacity;
  int32_t* sel_idx;         // [T, H_kv, capacity]
  int32_t* sel_count;       // [T, H_kv]
  int32_t* status;
};

int launch_topk_select(const TopkArgs& a, hipStream_t stream);

}  // namespace spattn
