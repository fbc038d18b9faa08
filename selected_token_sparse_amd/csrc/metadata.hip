// prepare_seqlens: per-request lengths and per-token (request, position), computed on the
// device from cumulative query offsets and past lengths so the host never reads device
// metadata back ("[WebGPU] Add PagedAttention metadata and GPT-OSS support", Description
// and Changes; per-token metadata as in the token-metadata stage of "[WebGPU] Add
// SparsePagedAttention", with a binary search instead of a per-token linear scan).
#include "common.h"
#include "launch.h"

namespace spattn {

constexpr int kMetaThreads = 1024;
constexpr int kMetaMaxB = 8192;

// Every workgroup rebuilds the sanitised boundaries (running maximum of cu clamped to
// [0, T]) in LDS; workgroup 0 writes the per-request outputs and the status, and every
// workgroup resolves its share of tokens by binary search over the boundaries.
__global__ __launch_bounds__(kMetaThreads) void prepare_seqlens_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ past, int B, int T,
    int32_t* __restrict__ seqlens_q, int32_t* __restrict__ seqlens_k,
    int32_t* __restrict__ token_req, int32_t* __restrict__ token_pos, int32_t* status) {
  __shared__ int bound[kMetaMaxB + 1];
  __shared__ int chunk_max[kMetaThreads];
  __shared__ int bad;
  const int tid = threadIdx.x;
  const int n = B + 1;
  if (tid == 0) bad = 0;
  // each thread owns a contiguous chunk of boundaries
  const int per = (n + kMetaThreads - 1) / kMetaThreads;
  const int s0 = tid * per, s1 = min(n, s0 + per);
  int run = INT32_MIN;
  for (int i = s0; i < s1; ++i) {
    run = max(run, cu[i]);
    bound[i] = run;
  }
  chunk_max[tid] = run;
  __syncthreads();
  // inclusive scan (max) over chunk maxima
  for (int off = 1; off < kMetaThreads; off <<= 1) {
    int v = (tid >= off) ? chunk_max[tid - off] : INT32_MIN;
    __syncthreads();
    chunk_max[tid] = max(chunk_max[tid], v);
    __syncthreads();
  }
  const int prefix = (tid > 0) ? chunk_max[tid - 1] : INT32_MIN;
  int local_bad = 0;
  for (int i = s0; i < s1; ++i) {
    int v = max(bound[i], prefix);
    bound[i] = min(max(v, 0), T);
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int b = tid; b < B; b += kMetaThreads) {
      const int c0 = cu[b], c1 = cu[b + 1];
      int pb = past[b];
      if (c1 < c0 || pb < 0) local_bad = 1;
      pb = max(pb, 0);
      const int q_len = bound[b + 1] - bound[b];
      seqlens_q[b] = q_len;
      seqlens_k[b] = pb + q_len - 1;
    }
    if (tid == 0 && (cu[0] != 0 || cu[B] != T)) local_bad = 1;
    if (local_bad) bad = 1;
  }
  // tokens
  if (token_req != nullptr || token_pos != nullptr) {
    for (int t = blockIdx.x * kMetaThreads + tid; t < T; t += gridDim.x * kMetaThreads) {
      int req = -1, pos = -1;
      if (B > 0 && bound[0] <= t) {
        int lo = 0, hi = B - 1;  // largest b with bound[b] <= t
        while (lo < hi) {
          int mid = (lo + hi + 1) >> 1;
          if (bound[mid] <= t) lo = mid; else hi = mid - 1;
        }
        if (t < bound[lo + 1]) {
          req = lo;
          pos = max(past[lo], 0) + (t - bound[lo]);
        }
      }
      if (token_req != nullptr) token_req[t] = req;
      if (token_pos != nullptr) token_pos[t] = pos;
    }
  }
  __syncthreads();
  if (blockIdx.x == 0 && tid == 0 && bad) raise_status(status, SPATTN_STATUS_BAD_CU);
}

int launch_prepare_seqlens(const int32_t* cu, const int32_t* past, int B, int T,
                           int32_t* seqlens_q, int32_t* seqlens_k, int32_t* token_req,
                           int32_t* token_pos, int32_t* status, hipStream_t stream) {
  if (B > kMetaMaxB) return SPATTN_ERR_SHAPE;
  int grid = (T + kMetaThreads - 1) / kMetaThreads;
  grid = max(1, min(grid, 64));
  hipLaunchKernelGGL(prepare_seqlens_kernel, dim3(grid), dim3(kMetaThreads), 0, stream, cu, past,
                     B, T, seqlens_q, seqlens_k, token_req, token_pos, status);
  return hipGetLastError() == hipSuccess ? SPATTN_OK : SPATTN_ERR_LAUNCH;
}

}  // namespace spattn
