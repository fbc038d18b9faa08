// topk_select: the k highest-scoring key positions of each (row, KV head), the producer of
// the selected-token index lists.  (DynamicSparseAttention INT8 / fast QSA decode page,
// Key Changes table: hierarchical / compact TopK selection; its follow-up description: the
// selection keeps stable keys, causal tails and the capacity stride with padding.)
//
// One workgroup of 1024 threads per (row, KV head).  The scores are loaded coalesced into
// LDS and each thread takes up to 64 candidates (in words of 32 consecutive positions) as
// order-preserving 32-bit keys, which it transposes into 32 bit planes (one mask bit per
// key).  A bitwise search over the key space (32 steps of a few mask operations, a
// popcount and one block sum; no atomics) finds the exact key of the last selection and
// how many keys equal to it are taken; one emit pass with block-wide scans writes the
// selected positions in ascending order.  The chunked sort-and-merge of the pages' CUDA
// design is replaced by this select: no sort is needed, because the output order is the
// position order.  (Measured at 65536 candidates a row: a radix select with LDS histograms
// took 147 us for 512 rows, because scores cluster in few exponent bins and a wave's
// histogram atomics serialise on one address; a compare-per-key search 168 us; this 84 us.)
#include "common.h"
#include "launch.h"
#include "topk.h"

namespace spattn {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / 64;

struct TopkParams {
  const float* scores;
  int L;
  const int32_t* cu;
  const int32_t* seqlens_k;
  int B, T, H_kv, k, tail, capacity;
  int32_t* sel_idx;
  int32_t* sel_count;
  int32_t* status;
};

// Order-preserving key of a score: larger score, larger key; NaN (1) below every number
// (-inf is 0x007FFFFF); -0 = +0.  Key 0 marks a position that is not ranked: the target of
// the select is always a ranked key (>= 1), so zero keys are never selected and never move
// it, and no per-position test is needed in the passes.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t b = __builtin_bit_cast(uint32_t, f);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 1u;   // NaN
  if (b == 0x80000000u) b = 0u;                     // -0 -> +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Sum of one value per thread over the workgroup.  `slot` (kTkWaves ints) must not be the
// slot of the previous call: alternating two slots needs a single barrier per call.
__device__ __forceinline__ int block_sum(int v, int* slot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // sums of 16-lane rows by DPP (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
  // row_mirror), then the four row sums by readlane
  v += __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);
  v += __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);
  v += __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true);
  v += __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, true);
  v = __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
      __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
  if (lane == 0) slot[wave] = v;
  __syncthreads();
  int all = 0;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) all += slot[w];
  return all;
}

// Exclusive prefix sum of one value per thread over the workgroup; *total gets the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_sums, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wave_sums[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) {
    const int s = wave_sums[w];
    before += w < wave ? s : 0;
    all += s;
  }
  __syncthreads();   // wave_sums is reused by the next scan
  *total = all;
  return before + x - v;
}

// 32 x 32 bit transpose in place (recursive block swap; B is part of a register array and
// every index is a compile-time constant).  On return B[b] holds, in bit c, bit b of the
// word that was B[c] on entry: the bit planes of 32 keys.
__device__ __forceinline__ void transpose32(uint32_t* B) {
  // the block swap below is written for the reversed view A[i] = B[31 - i]
  uint32_t m = 0x0000FFFFu;
#pragma unroll
  for (int j = 16; j != 0; j >>= 1, m ^= (m << j)) {
#pragma unroll
    for (int k = 0; k < 32; k = (k + j + 1) & ~j) {
      uint32_t& a = B[31 - k];
      uint32_t& c = B[31 - (k + j)];
      const uint32_t t = (a ^ (c >> j)) & m;
      a ^= t;
      c ^= t << j;
      // (an empty statement that keeps the swaps in order: left free, the compiler computes
      // a whole stage's temporaries first and runs out of registers at 64 keys a thread)
      asm volatile("" : "+v"(a), "+v"(c));
    }
  }
}

// Keys staged through LDS per round: 32768 floats plus 16 bytes of padding per 256 (a
// thread's 64 consecutive keys are read with b128 loads 272 bytes apart: no bank conflicts).
constexpr int kTkRound = 32768;
__host__ __device__ constexpr int tk_pad(int i) { return i + ((i >> 6) << 2); }

// KPT keys per thread, in NW words of KW keys: word w of thread t holds the positions
// w * R + t * KW .. + KW - 1 (R = KW * 1024), so round w of the LDS staging fills word w of
// every thread and each register is written exactly once.
template <int KPT>
__global__ __launch_bounds__(kTkThreads) void topk_select_kernel(TopkParams P) {
  constexpr int KW = KPT < 32 ? KPT : 32;   // keys per word
  constexpr int NW = KPT / KW;              // words per thread
  constexpr int R = KW * kTkThreads;        // positions per word (one staging round)
  static_assert(R <= kTkRound, "a round must fit the stage");
  __shared__ float stage[tk_pad(kTkRound)];
  __shared__ int sums[2][kTkWaves];
  __shared__ int wave_sums[kTkWaves];
  __shared__ int bcast[1];
  const int tid = threadIdx.x;
  const int seg = blockIdx.x;
  const int t = seg / P.H_kv;

  // the row's candidates: positions 0 .. n-1 (causal), the last nt always selected
  if (tid == 0) {
    const int b = find_request(P.cu, P.B, t);
    int n = 0;
    if (b < 0) {
      raise_status(P.status, SPATTN_STATUS_BAD_CU);
    } else {
      const int q_len = P.cu[b + 1] - P.cu[b];
      const int p = P.seqlens_k[b] + 1 - q_len + (t - P.cu[b]);
      n = min(max(p + 1, 0), P.L);
    }
    bcast[0] = n;
  }
  __syncthreads();
  const int n = bcast[0];
  int32_t* out = P.sel_idx + (int64_t)seg * P.capacity;
  const int count = min(P.k, n);
  if (n <= P.k) {
    for (int j = tid; j < P.capacity; j += kTkThreads) out[j] = j < n ? j : -1;
    if (tid == 0) P.sel_count[seg] = count;
    return;
  }
  const int nt = min(min(P.tail, P.k), n);
  const int m = n - nt;            // ranked candidates: positions 0 .. m-1
  const int need = P.k - nt;       // how many of them are selected (< m)

  // keys (0 = not ranked), loaded coalesced through LDS, one word per round: all loads of
  // a round are issued together, and the next round's loads are in flight while this
  // round's keys are read back and transposed into bit planes (afterwards key[32 w + b]
  // bit e = bit b of the word's key e)
  const float* row = P.scores + (int64_t)seg * P.L;
  constexpr int NV = R / (4 * kTkThreads);   // float4 loads per thread and round
  // float4 loads when every row starts on a 16-byte boundary
  const bool vec = (P.L & 3) == 0 && (reinterpret_cast<uintptr_t>(P.scores) & 15u) == 0;
  f32x4 buf[NV];
  auto load_round = [&](int w) {
    const int r0 = w * R;
    const int len = max(0, min(R, m - r0));
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int i = 4 * (tid + q * kTkThreads);
      if (vec && i + 4 <= len) {
        buf[q] = *reinterpret_cast<const f32x4*>(row + r0 + i);
      } else {
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) if (i + c < len) v[c] = row[r0 + i + c];
        buf[q] = v;
      }
    }
  };
  uint32_t key[NW * 32];
  load_round(0);
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int len = max(0, min(R, m - w * R));
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int i = 4 * (tid + q * kTkThreads);
      if (i < len) *reinterpret_cast<f32x4*>(stage + tk_pad(i)) = buf[q];
    }
    __syncthreads();
    if (w + 1 < NW) load_round(w + 1);
    const int base = tid * KW;
#pragma unroll
    for (int e = 0; e < 32; e += 4) {
      if (e < KW && base + e + 4 <= len) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(stage + tk_pad(base + e));
#pragma unroll
        for (int q = 0; q < 4; ++q) key[32 * w + e + q] = score_key(v[q]);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          key[32 * w + e + q] = (e + q < KW && base + e + q < len) ? score_key(stage[tk_pad(base + e + q)]) : 0u;
      }
    }
    transpose32(key + 32 * w);
    __syncthreads();   // the stage is refilled by the next round
  }
#define PLANE(b, w) key[32 * (w) + (b)]

  // select: the need-th largest key among positions < m, bit by bit from the top.  gt:
  // keys above the prefix so far, eq: keys equal to it so far (bit masks over the thread's
  // keys); a step counts gt | (eq & plane) and keeps the bit if that count reaches need.
  // At the end gt = the keys above the selected key, eq = the keys equal to it.
  uint32_t gt[NW], eq[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) { gt[w] = 0u; eq[w] = need > 0 ? 0xFFFFFFFFu : 0u; }
  int remaining = need;
  if (need > 0) {
    int gt_total = 0;
#pragma unroll
    for (int b = 31; b >= 0; --b) {
      int c = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) c += __builtin_popcount(gt[w] | (eq[w] & PLANE(b, w)));
      const int total = block_sum(c, sums[b & 1]);
      if (total >= need) {
#pragma unroll
        for (int w = 0; w < NW; ++w) eq[w] &= PLANE(b, w);
      } else {
#pragma unroll
        for (int w = 0; w < NW; ++w) { gt[w] |= eq[w] & PLANE(b, w); eq[w] &= ~PLANE(b, w); }
        gt_total = total;
      }
    }
    remaining = need - gt_total;
  }
#undef PLANE

  // emit in position order (word 0 of every thread, then word 1): the keys above the
  // selected one, the first `remaining` keys equal to it, the tail
  int eq_base = 0, out_base = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int pw = w * R + tid * KW;          // position of bit 0 of this word
    const uint32_t e_mask = eq[w];
    const int eqn = __builtin_popcount(e_mask);
    int total;
    const int eq_before = eq_base + block_exclusive_scan(eqn, wave_sums, &total);
    eq_base += total;
    int eq_take = min(max(remaining - eq_before, 0), eqn);
    uint32_t first = 0u, x = e_mask;
    for (; eq_take > 0; --eq_take) { const uint32_t low = x & (0u - x); first |= low; x ^= low; }
    const int lo = min(max(m - pw, 0), KW), hi = min(max(n - pw, 0), KW);
    const uint32_t below_hi = hi >= 32 ? 0xFFFFFFFFu : ((1u << hi) - 1u);
    const uint32_t below_lo = lo >= 32 ? 0xFFFFFFFFu : ((1u << lo) - 1u);
    uint32_t take = gt[w] | first | (below_hi & ~below_lo);
    int off = out_base + block_exclusive_scan(__builtin_popcount(take), wave_sums, &total);
    out_base += total;
    while (take != 0u) {
      const int e = __builtin_ctz(take);
      take &= take - 1u;
      if (off < P.capacity) out[off] = pw + e;
      ++off;
    }
  }
  for (int j = count + tid; j < P.capacity; j += kTkThreads) out[j] = -1;
  if (tid == 0) P.sel_count[seg] = count;
}

int launch_topk_select(const TopkArgs& a, hipStream_t stream) {
  if (a.T == 0 || a.H_kv == 0) return SPATTN_OK;
  TopkParams P{};
  P.scores = a.scores; P.L = a.L; P.cu = a.cu; P.seqlens_k = a.seqlens_k;
  P.B = a.B; P.T = a.T; P.H_kv = a.H_kv; P.k = a.k; P.tail = a.tail; P.capacity = a.capacity;
  P.sel_idx = a.sel_idx; P.sel_count = a.sel_count; P.status = a.status;
  const int64_t blocks = (int64_t)a.T * a.H_kv;
  if (blocks > 0x7FFFFFFF) return SPATTN_ERR_SHAPE;
  dim3 grid((unsigned)blocks), block(kTkThreads);
  const int per = (a.L + kTkThreads - 1) / kTkThreads;
  if (per <= 4) hipLaunchKernelGGL((topk_select_kernel<4>), grid, block, 0, stream, P);
  else if (per <= 8) hipLaunchKernelGGL((topk_select_kernel<8>), grid, block, 0, stream, P);
  else if (per <= 16) hipLaunchKernelGGL((topk_select_kernel<16>), grid, block, 0, stream, P);
  else if (per <= 32) hipLaunchKernelGGL((topk_select_kernel<32>), grid, block, 0, stream, P);
  else if (per <= 64) hipLaunchKernelGGL((topk_select_kernel<64>), grid, block, 0, stream, P);
  else return SPATTN_ERR_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? SPATTN_OK : SPATTN_ERR_LAUNCH;
}

}  // namespace spattn
