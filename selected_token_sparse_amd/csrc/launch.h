// Internal launchers behind the C ABI (api.hip validates arguments, then calls these).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace spattn {

int launch_prepare_seqlens(const int32_t* cu, const int32_t* past, int B, int T,
                           int32_t* seqlens_q, int32_t* seqlens_k, int32_t* token_req,
                           int32_t* token_pos, int32_t* status, hipStream_t stream);

int launch_kv_cache_append(const void* k_new, const void* v_new, int new_dtype,
                           const int32_t* cu, const int32_t* seqlens_k, int B, int T,
                           void* k_cache, void* v_cache, int cache_dtype,
                           const int32_t* block_table, int max_blocks, int block_size,
                           int num_blocks, const float* key_scale, const float* value_scale,
                           int H_kv, int D, const int32_t* committed_length, int32_t* status,
                           hipStream_t stream);

// Everything an attention launch needs; filled and validated by api.hip.
struct AttnArgs {
  int kind;               // SPATTN_KIND_*
  const void* q;
  int dtype;              // Q / out dtype
  const void* k_cache;
  const void* v_cache;
  int cache_dtype;
  const int32_t* block_table;
  int max_blocks;
  int block_size;
  int num_blocks;
  const float* key_scale;
  const float* value_scale;
  const int32_t* cu;
  const int32_t* seqlens_k;
  int B, T, max_q, max_k;  // max_k < 0: no key-count bound (sparse kinds)
  const int32_t* sel_idx;
  const int32_t* sel_count;
  int max_selected;
  int window;             // <= 0: off
  const void* aux_k;
  const void* aux_v;
  int aux_len;
  int64_t aux_stride;
  int H_q, H_kv, D;
  float scale;            // already resolved (0 -> 1/sqrt(D))
  const float* sinks;
  void* out;
  void* workspace;
  int32_t* status;
  // fused decode step only (paged kind, 16-bit q, split path, B < 256); nullptr otherwise
  const int32_t* past;
  const void* k_new;
  const void* v_new;
  int32_t* seqlens_q_out;
  int32_t* seqlens_k_out;
  const int32_t* committed;   // fused decode step only: the caller's cursor [B] or nullptr
};

// Largest B of the fused decode step (its boundaries are staged one per thread).
constexpr int kStepMaxB = 255;

// Work plan of the split-K (per-row) path: how the key range of one (row, KV head) is cut.
struct SplitPlan {
  int chunk;        // keys per split (multiple of the 128-key workgroup step)
  int n_main;       // splits over the main source (range or selection)
  int n_aux;        // splits over the auxiliary selection (LOCAL_AUX only)
  int n_splits;     // n_main + n_aux
  int head_tiles;   // ceil(group / 16)
  size_t ws_bytes;  // partial-state workspace (0 when one split writes the output directly)
};

// Prefill (MFMA tile) path is used when true; otherwise the split-K path.
bool use_prefill_path(int kind, int dtype, int max_q);
SplitPlan make_split_plan(int kind, int dtype, int cache_dtype, int B, int T, int max_q,
                          int max_k, int max_sel, int window, int H_q, int H_kv, int D);

int launch_split_attention(const AttnArgs& a, const SplitPlan& plan, hipStream_t stream);
int launch_prefill_attention(const AttnArgs& a, hipStream_t stream);

}  // namespace spattn
