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
__device__ __forceinline__ uint32_t score_key_bits(uint32_t b) {
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 1u;   // NaN
  if (b == 0x80000000u) b = 0u;                     // -0 -> +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ uint32_t score_key(float f) {
  return score_key_bits(__builtin_bit_cast(uint32_t, f));
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

// ---------------------------------------------------------------------------------------
// Long rows (16384 < L <= 65536, float4-aligned): one persistent workgroup per CU walks
// its segments (seg = blockIdx.x + i * gridDim.x).  A thread holds 32 keys per word of
// 32768 positions (one or two words): word w of thread t is positions w * 32768 + 32 t ..
// + 31.  Each word reaches a 128 KB LDS stage by LDS DMA (coalesced 1 KB per wave
// instruction, no registers held) and is read back with a per-thread rotation of its eight
// 16-byte units (thread t starts at unit (t + t / 8) mod 8: conflict-free b128 reads).  The
// next segment's first word is copied during the current segment's search, one
// instruction a wave per step (a wave that issues a long burst of memory instructions
// stalls until the memory system takes them).  The search takes two bit planes per step
// (three counts, one barrier) and stops once the keys at or above the prefix are exactly
// the ones needed; the emit runs one scan per word for the selected and the tied counts.
// ---------------------------------------------------------------------------------------
constexpr int kTsWord = 32768;   // positions per word and per stage

typedef const int32_t __attribute__((address_space(4))) ts_const_i32;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Candidates of segment seg (key positions 0 .. n-1), from uniform scalar loads: no vector
// memory counter is involved, so the lookup never waits for the stage copies in flight.
__device__ __forceinline__ int ts_candidates(const TopkParams& P, int seg) {
  ts_const_i32* cu = (ts_const_i32*)P.cu;
  ts_const_i32* sk = (ts_const_i32*)P.seqlens_k;
  const int t = __builtin_amdgcn_readfirstlane(seg) / P.H_kv;   // uniform: scalar loads
  if (P.B <= 0 || cu[0] > t) return -1;
  int lo = 0, hi = P.B - 1;   // largest b with cu[b] <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int c0 = cu[lo], c1 = cu[lo + 1];
  if (t >= c1) return -1;
  const int p = sk[lo] + 1 - (c1 - c0) + (t - c0);
  return min(max(p + 1, 0), P.L);
}

// One stage of the 32 x 32 bit transpose: rows k and k + J (k without bit J) exchange the
// upper J-bit halves of row k's 2J-bit groups with the lower halves of row k + J's.  The
// stages J = 16, 8, 4, 2, 1 in turn leave W[b] bit c = bit b of the word that was W[c].
template <int J>
__device__ __forceinline__ void ts_transpose_stage(uint32_t* W) {
  constexpr uint32_t m = J == 16 ? 0x0000FFFFu : J == 8 ? 0x00FF00FFu : J == 4 ? 0x0F0F0F0Fu
                       : J == 2 ? 0x33333333u : 0x55555555u;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    if (k & J) continue;
    uint32_t a = W[k], c = W[k + J];
    uint32_t a2, c2;
    if (J >= 8) {
      // whole bytes move: one byte permute per row (selector bytes 0-3 pick a's bytes,
      // 4-7 c's)
      a2 = __builtin_amdgcn_perm(c, a, J == 16 ? 0x05040100u : 0x06020400u);
      c2 = __builtin_amdgcn_perm(c, a, J == 16 ? 0x07060302u : 0x07030501u);
    } else {
      a2 = (a & m) | ((c << J) & ~m);
      c2 = (c & ~m) | ((a >> J) & m);
    }
    a = a2; c = c2;
    asm volatile("" : "+v"(a), "+v"(c));   // keeps the exchanges in order (register pressure)
    W[k] = a; W[k + J] = c;
  }
}


// Sum over the wave (every lane gets it, as a scalar).
__device__ __forceinline__ uint32_t ts_wave_sum(uint32_t v) {
  v += __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);
  v += __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);
  v += __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true);
  v += __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, true);
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
         __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

// Inclusive sum over lanes 0 .. lane of the wave (row_shr steps within rows of 16, then the
// row_bcast:15 / row_bcast:31 steps across rows).
__device__ __forceinline__ uint32_t ts_wave_scan(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false);
  return x;
}

// LDS DMA of 16 bytes a lane (lane l writes LDS byte lds + 16 l), written out so that the
// compiler does not see an LDS write in flight: it would otherwise wait for every
// outstanding vector-memory operation before each LDS access of the search and the emit,
// serialising them with the next word's copy.  The kernel orders the stage itself
// (vmcnt(0) and a barrier before the stage is read, a barrier before it is refilled).
__device__ __forceinline__ void ts_dma16(const void* g, uint32_t lds) {
  // (one wait state between the M0 write and the LDS DMA that reads it)
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}

// LDS add without a return value (the caller waits with lgkmcnt before the barrier).
__device__ __forceinline__ void ts_lds_add(uint32_t lds, uint32_t v) {
  asm volatile("ds_add_u32 %0, %1" :: "v"(lds), "v"(v) : "memory");
}

template <int NW>
__global__ __launch_bounds__(kTkThreads) void topk_stream_kernel(TopkParams P) {
  __shared__ __align__(16) uint32_t stage[kTsWord];
  __shared__ __align__(16) uint32_t cnt[3][4];         // search counts, a ring of three
  __shared__ __align__(16) uint32_t wtot[kTkWaves][NW];  // emit: per-wave totals
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = P.T * P.H_kv;
  const int rot = 4 * ((tid + (tid >> 3)) & 7);   // slot c holds position offset (c + rot) & 31
  const uint32_t stage_lds = (uint32_t)reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) uint32_t*)stage);
  const uint32_t cnt_lds = (uint32_t)reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) uint32_t*)&cnt[0][0]);
  if (tid < 12) (&cnt[0][0])[tid] = 0u;

  // The first segment at or after s (this workgroup's stride) that needs a ranked
  // selection (more than k candidates and a tail shorter than k); the ones passed on the way
  // are written here: every candidate, or the last k (the tail covers k).
  auto advance = [&](int s, int& n_out) -> int {
    for (; s < S; s += gridDim.x) {
      int n = ts_candidates(P, s);
      if (n < 0) {
        if (tid == 0) raise_status(P.status, SPATTN_STATUS_BAD_CU);
        n = 0;
      }
      if (n > P.k && P.tail < P.k) { n_out = n; return s; }
      const int count = min(n, P.k), first = n - count;
      int32_t* out = P.sel_idx + (int64_t)s * P.capacity;
      for (int j = tid; j < P.capacity; j += kTkThreads) out[j] = j < count ? first + j : -1;
      if (tid == 0) P.sel_count[s] = count;
    }
    n_out = 0;
    return S;
  };
  // Stage copy of one word (its positions below m): wave instruction q moves 1 KB (16
  // bytes a lane) to stage byte 1024 q; wave v issues q = v + 16 i as slice i (i < 8).
  // Lanes past m re-read the word's first unit.
  const float* dma_row = nullptr;
  int dma_len = 0, dma_slice = 8;
  auto dma_begin = [&](int s, int w, int m) {
    dma_row = P.scores + (int64_t)s * P.L + w * kTsWord;
    dma_len = min(kTsWord, m - w * kTsWord);
    dma_slice = 0;
  };
  auto dma_step = [&]() {
    if (dma_slice < 8) {
      const int q = wave + kTkWaves * dma_slice;
      if (256 * q < dma_len) {
        int u = 64 * q + lane;
        asm volatile("" : "+v"(u));   // (computed here, not hoisted and held for every slice)
        ts_dma16(4 * u < dma_len ? dma_row + 4 * u : dma_row, stage_lds + 1024 * q);
      }
      ++dma_slice;
    }
  };
  // Word w of this thread from the stage (its eight 16-byte units, rotated), then order-
  // preserving keys transposed into planes; positions past m get key 0.
  auto load_word = [&](uint32_t* kw, int w, int m) {
    const unsigned char* base = reinterpret_cast<const unsigned char*>(stage) + tid * 128;
    int r4 = rot * 4;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      asm volatile("" : "+v"(r4));   // offsets computed here, not held across the loop
      const u32x4 v = *reinterpret_cast<const u32x4*>(base + ((16 * j + r4) & 127));
      kw[4 * j] = v[0]; kw[4 * j + 1] = v[1]; kw[4 * j + 2] = v[2]; kw[4 * j + 3] = v[3];
    }
  };
  // (copy_steps: one DMA slice of the copy in flight between each pair of phases, eight
  // in all, so that no wave stalls on a burst of them)
  auto make_planes = [&](uint32_t* kw, int w, int m, bool copy_steps) {
    if (copy_steps) dma_step();
    // order-preserving keys: adding +0 turns -0 into +0 and leaves every other number
    // (subnormals included: the kernels keep float32 denormals) unchanged, the sign flip
    // orders the numbers, and a NaN gets key 1
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      const float f = __builtin_bit_cast(float, kw[c]);
      const uint32_t b = __builtin_bit_cast(uint32_t, f + 0.0f);
      const uint32_t k = b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
      kw[c] = __builtin_isnan(f) ? 1u : k;
      if (copy_steps && c == 15) dma_step();
    }
    if (copy_steps) dma_step();
    ts_transpose_stage<16>(kw);
    if (copy_steps) dma_step();
    ts_transpose_stage<8>(kw);
    if (copy_steps) dma_step();
    ts_transpose_stage<4>(kw);
    if (copy_steps) dma_step();
    ts_transpose_stage<2>(kw);
    if (copy_steps) dma_step();
    ts_transpose_stage<1>(kw);
    if (copy_steps) dma_step();
    const int valid = min(max(m - w * kTsWord - 32 * tid, 0), 32);
    if (valid < 32) {
      const uint32_t slots = __builtin_rotateright32(valid ? (0xFFFFFFFFu >> (32 - valid)) : 0u, rot);
#pragma unroll
      for (int b = 0; b < 32; ++b) kw[b] &= slots;
    }
  };

  int n = 0;
  int seg = advance(blockIdx.x, n);
  if (seg < S) {
    dma_begin(seg, 0, n - min(min(P.tail, P.k), n));
    for (int i = 0; i < 8; ++i) dma_step();
  }
  uint32_t key[NW * 32];
  int slot = 0;   // the search counts' ring position, carried from segment to segment
  while (seg < S) {
    n = __builtin_amdgcn_readfirstlane(n);
    const int nt = min(min(P.tail, P.k), n);
    const int m = n - nt;          // ranked candidates: positions 0 .. m-1
    const int need = P.k - nt;     // selected among them (1 .. m-1)
    const int words = (m + kTsWord - 1) / kTsWord;   // 1 .. NW
    int n_next = 0;
    const int next = __builtin_amdgcn_readfirstlane(advance(seg + gridDim.x, n_next));
    const int wb = 2048 * wave;   // the wave's first position offset in a word
    // (every key register defined afresh each segment: nothing of the previous segment's
    // planes is carried around the loop; waves whose positions all lie past m keep these
    // zeros, the planes of unranked positions)
#pragma unroll
    for (int c = 0; c < NW * 32; ++c) key[c] = 0u;

    // word 0 from the stage
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();   // word 0 of this segment is in the stage
    if (wb < m) load_word(key, 0, m);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();   // the stage is free
    if (NW == 1) {
      if (next < S) dma_begin(next, 0, n_next - min(min(P.tail, P.k), n_next));
      if (wb < m) make_planes(key, 0, m, true);
    } else {
      // word 1 through the stage, its copy spread through word 0's conversion (a wave that
      // issues a burst of memory instructions stalls until the memory system takes them;
      // copies issued by only a few waves ran slower)
      if (words > 1) dma_begin(seg, 1, m);
      if (wb < m) make_planes(key, 0, m, words > 1);
      while (dma_slice < 8) dma_step();
      if (words > 1) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();   // word 1 is in the stage
      if (kTsWord + wb < m) load_word(key + 32, 1, m);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __syncthreads();   // the stage is free
      if (kTsWord + wb < m) make_planes(key + 32, 1, m, false);
      if (next < S) dma_begin(next, 0, n_next - min(min(P.tail, P.k), n_next));
    }

    // select the need-th largest key, two bits a step: gt = keys above the prefix so far,
    // eq = keys equal to it.  A step counts the keys of eq whose next two bits are 11, 1x and
    // non-zero, takes the largest digit d whose keys at or above it reach need, and stops
    // once the keys at or above the prefix are exactly need.
    uint32_t gt[NW], eq[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) { gt[w] = 0u; eq[w] = 0xFFFFFFFFu; }
    int gt_total = 0, ge_total = -1;   // counts of keys above / at or above the prefix
#pragma unroll
    for (int b = 31; b >= 1; b -= 2) {
      if (ge_total != need) {
        dma_step();
        uint32_t c3 = 0, c2 = 0, c1 = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const uint32_t H = key[32 * w + b], L = key[32 * w + b - 1];
          c3 += __builtin_popcount(eq[w] & H & L);
          c2 += __builtin_popcount(eq[w] & H);
          c1 += __builtin_popcount(eq[w] & (H | L));
        }
        const uint32_t s32 = ts_wave_sum(c3 | (c2 << 16));   // per-wave counts <= 4096
        const uint32_t s1 = ts_wave_sum(c1);
        if (lane == 0) {
          const uint32_t a = cnt_lds + 16 * slot;
          ts_lds_add(a, s32 & 0xFFFFu);
          ts_lds_add(a + 4, s32 >> 16);
          ts_lds_add(a + 8, s1);
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
        if (tid < 3) cnt[slot == 2 ? 0 : slot + 1][tid] = 0u;
        __syncthreads();
        const u32x4 tv = *reinterpret_cast<const u32x4*>(cnt[slot]);
        const int t3 = gt_total + __builtin_amdgcn_readfirstlane((int)tv[0]);
        const int t2 = gt_total + __builtin_amdgcn_readfirstlane((int)tv[1]);
        const int t1 = gt_total + __builtin_amdgcn_readfirstlane((int)tv[2]);
        slot = slot == 2 ? 0 : slot + 1;
        if (t3 >= need) {
#pragma unroll
          for (int w = 0; w < NW; ++w) eq[w] &= key[32 * w + b] & key[32 * w + b - 1];
          ge_total = t3;
        } else if (t2 >= need) {
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            const uint32_t H = key[32 * w + b], L = key[32 * w + b - 1];
            gt[w] |= eq[w] & H & L;
            eq[w] &= H & ~L;
          }
          gt_total = t3; ge_total = t2;
        } else if (t1 >= need) {
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            const uint32_t H = key[32 * w + b], L = key[32 * w + b - 1];
            gt[w] |= eq[w] & H;
            eq[w] &= ~H & L;
          }
          gt_total = t2; ge_total = t1;
        } else {
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            const uint32_t H = key[32 * w + b], L = key[32 * w + b - 1];
            gt[w] |= eq[w] & (H | L);
            eq[w] &= ~(H | L);
          }
          gt_total = t1;
        }
      }
    }
    const int remaining = need - gt_total;   // taken from eq, lowest positions first

    // emit in position order: word 0 of every thread, then word 1; one scan per word counts
    // the selected keys above the selected one and the tied ones together.  The tail
    // (positions m .. n-1, after every ranked one) fills the last nt entries.
    int pe = 32 * tid;
    asm volatile("" : "+v"(pe));   // (none of this computed early)
    uint32_t Gp[NW], Ep[NW], sc[NW], incl[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      Gp[w] = __builtin_rotateleft32(gt[w], rot);
      Ep[w] = __builtin_rotateleft32(eq[w], rot);
      sc[w] = (uint32_t)__builtin_popcount(Gp[w]) | ((uint32_t)__builtin_popcount(Ep[w]) << 16);
      incl[w] = ts_wave_scan(sc[w]);   // per-word block totals <= 32768 in each half
      if (lane == 63) wtot[wave][w] = incl[w];
    }
    __syncthreads();
    int32_t* out = P.sel_idx + (int64_t)seg * P.capacity;
    int base_a = 0, base_e = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      uint32_t before = 0u, total = 0u;
#pragma unroll
      for (int v = 0; v < kTkWaves; ++v) {
        const uint32_t x = wtot[v][w];
        before += v < wave ? x : 0u;
        total += x;
      }
      const uint32_t x = before + incl[w] - sc[w];
      const int a_before = base_a + (int)(x & 0xFFFFu);
      const int e_before = base_e + (int)(x >> 16);
      const int eqn = (int)(sc[w] >> 16);
      const int eq_take = min(max(remaining - e_before, 0), eqn);
      uint32_t take = Gp[w];
      if (eq_take == eqn) {
        take |= Ep[w];
      } else {
        uint32_t y = Ep[w];
        for (int i = 0; i < eq_take; ++i) { const uint32_t low = y & (0u - y); take |= low; y ^= low; }
      }
      int off = a_before + min(e_before, remaining);
      const int pw = w * kTsWord + pe;
      while (take != 0u) {
        const int e = __builtin_ctz(take);
        take &= take - 1u;
        if (off < P.capacity) out[off] = pw + e;
        ++off;
      }
      base_a += (int)(total & 0xFFFFu);
      base_e += (int)(total >> 16);
    }
    for (int j = tid; j < nt; j += kTkThreads) out[need + j] = m + j;
    for (int j = P.k + tid; j < P.capacity; j += kTkThreads) out[j] = -1;
    if (tid == 0) P.sel_count[seg] = P.k;
    // the rest of the next segment's copy after the stores (queued behind the copy, the
    // stores would wait for it)
    while (dma_slice < 8) dma_step();
    seg = next;
    n = n_next;
  }
}

// CUs of the current device (queried once a device).
static int ts_cu_count() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = __atomic_load_n(&cached[dev], __ATOMIC_RELAXED);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    __atomic_store_n(&cached[dev], v, __ATOMIC_RELAXED);
  }
  return v;
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
  const bool vec = (a.L & 3) == 0 && (reinterpret_cast<uintptr_t>(a.scores) & 15u) == 0;
  if (vec && per > 16 && per <= 64) {
    const int64_t cus = ts_cu_count();
    dim3 pgrid((unsigned)(blocks < cus ? blocks : cus));
    if (per <= 32) hipLaunchKernelGGL((topk_stream_kernel<1>), pgrid, block, 0, stream, P);
    else hipLaunchKernelGGL((topk_stream_kernel<2>), pgrid, block, 0, stream, P);
    return hipGetLastError() == hipSuccess ? SPATTN_OK : SPATTN_ERR_LAUNCH;
  }
  if (per <= 4) hipLaunchKernelGGL((topk_select_kernel<4>), grid, block, 0, stream, P);
  else if (per <= 8) hipLaunchKernelGGL((topk_select_kernel<8>), grid, block, 0, stream, P);
  else if (per <= 16) hipLaunchKernelGGL((topk_select_kernel<16>), grid, block, 0, stream, P);
  else if (per <= 32) hipLaunchKernelGGL((topk_select_kernel<32>), grid, block, 0, stream, P);
  else if (per <= 64) hipLaunchKernelGGL((topk_select_kernel<64>), grid, block, 0, stream, P);
  else return SPATTN_ERR_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? SPATTN_OK : SPATTN_ERR_LAUNCH;
}

}  // namespace spattn
