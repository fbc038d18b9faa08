// Split-K attention for short queries (decode) and for selected-token attention.
//
// One workgroup (4 waves) handles one (packed row, KV head, tile of <= 16 query heads of
// that KV head's group, split of the row's key list).  The key list is, per source:
//   range      cache positions lo..p (lo = window start or 0), paged or contiguous;
//   selected   main-cache positions named by an int32 index list (count-bounded, -1 padded);
//   auxiliary  rows of an auxiliary store named by an index list (local-plus-aux mode).
// ("[WebGPU] Add PagedAttention metadata and GPT-OSS support": direct paged split-reduce
// decode with sinks, review Q2 asks for the window on that path; "[WebGPU] Add
// SparsePagedAttention": main and auxiliary partial FP32 softmax states merged by a
// finalize stage; "[WebGPU] Add DynamicSparseAttention": guarded indices, count-bounded
// loop, joint softmax with sink; DynamicSparseAttention INT8 page: per-channel INT8 K/V.)
//
// Per workgroup:
//  1. cu_seqlens_q / seqlens_k are staged in LDS in one parallel round and the row's
//     request and key position are found by binary search there;
//  2. the split's keys are turned into cache-row indices in LDS (one pass, guarded);
//  3. each wave takes 32-key tiles: K rows are loaded straight into the A operand of
//     S^T = K Q^T (v_mfma_f32_16x16x32, 16-byte loads) while V rows go into the wave's LDS
//     buffer by DMA (global_load_lds_dwordx4, no registers held while in flight); an online
//     softmax in the log2 domain (the accumulator is rescaled only when a running maximum
//     moved), then O^T += V^T P^T with V^T read through ds_read_b64_tr_b16;
//  4. the four wave states are merged in LDS.  With one split the workgroup writes the
//     normalised output; otherwise it writes its partial (m, l, acc) and a merge kernel
//     combines the splits of every (row, query head) and applies the sink.  (Merging in the
//     last-arriving workgroup instead needs an agent-scope release per workgroup, which on
//     this chip writes back the L2 and measured several times slower.)
//
// INT8 and FP8 E4M3 caches: key_scale is folded into the query operand (f16), value_scale
// is applied to the accumulator before it leaves the workgroup.
//
// Fused decode step (paged_decode_step, the kStep instantiation): step 1 derives seqlens_k
// from cu and past in the same load round, and before the barrier that ends step 2 the
// workgroup writes the step's new K/V rows that fall in its own key split (quantised as
// the cache append quantises them); workgroup 0 writes seqlens_q / seqlens_k last.
#include <type_traits>

#include "append.h"
#include "common.h"
#include "launch.h"

namespace spattn {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kTile = 32;          // keys per wave iteration
constexpr int kWgStep = kWaves * kTile;
constexpr int kMaxChunk = 2048;    // sparse kinds: keys per split while there are enough workgroups
constexpr int kChunkCap = 4096;    // keys per split, hard limit (LDS row table)
constexpr int kMaxSplits = 256;    // splits per item (LDS merge coefficients)
// Workgroups the split plan aims for.  Paged ranges: one round of resident workgroups, i.e.
// 256 CUs x the workgroups a CU holds at D = 64 (4; 3 over FP8 caches, whose kernel needs
// more registers), split evenly.  Measured on the GQA decode (248 row-head items, up to
// 8192 keys): 992 workgroups of 2048 keys match 3968 of 512 over a 16-bit cache and are
// 10-20% faster over 8-bit caches, whose shorter byte streams leave more of the time to
// per-workgroup set-up and partial states.  Selected and local-plus-aux rows run fastest at
// one workgroup per item and key range (the split length doubles until the plan has at
// most this many): 512 workgroups of 2048 selected keys need no merge at all.
constexpr int kTargetWorkgroupsPaged = 1024;
constexpr int kTargetWorkgroupsPagedFp8 = 768;
constexpr int kTargetWorkgroupsSparse = 512;
constexpr int kMetaLdsMax = 512;   // cu entries staged in LDS (more: binary search in memory)
static_assert(kStepMaxB + 1 <= kThreads, "a fused step stages one boundary per thread");

enum Src { SRC_RANGE = 0, SRC_SELECT = 1, SRC_AUX = 2 };

template <typename T> struct OpVec;
template <> struct OpVec<f16> { typedef f16x8 v8; typedef f16x4 v4; };
template <> struct OpVec<bf16> { typedef bf16x8 v8; typedef bf16x4 v4; };

__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Eight 16-bit cache elements as an MFMA operand.
template <typename OpT, typename KT>
__device__ __forceinline__ typename OpVec<OpT>::v8 load_op8(const KT* p) {
  static_assert(sizeof(KT) == 2, "8-bit caches load raw codes (see issue_tile)");
  return __builtin_bit_cast(typename OpVec<OpT>::v8, load16(p));
}

// Parameters of the split kernels (by value).
struct SplitParams {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const void* aux_k;
  const void* aux_v;
  const float* key_scale;
  const float* value_scale;
  const int32_t* cu;
  const int32_t* seqlens_k;
  const int32_t* sel_idx;
  const int32_t* sel_count;
  const float* sinks;
  void* out;
  float* ws_acc;    // [n_splits][T][H_q][D]
  float2* ws_ml;    // [n_splits][T][H_q]
  int32_t* status;
  CacheDesc cd;
  int B, T, H_q, H_kv, D, group, head_tiles;
  int max_q, max_k, max_sel, window, aux_len;
  int64_t aux_row_stride;   // rows (of D elements) between requests in the aux store
  int chunk, n_main, n_splits;
  int row_slots;            // LDS entries of the split's row table (see split_row_slots)
  int cu_slots;             // > 0: paged splits dealt to CUs by size (see deal_split); the
                            // CUs one KV head's workgroups spread over
  int meta_lds;             // 1: cu / seqlens_k staged in LDS
  float scale_log2;         // scale * log2(e)
  // Fused decode step (past != nullptr, paged kind, B + 1 <= kThreads): seqlens_k is
  // derived here from cu and past as prepare_seqlens derives it, and every workgroup first
  // writes the step's new K/V rows that fall in its own key range (see step_write_keys).
  const int32_t* past;
  const void* k_new;        // [T, H_kv, D] of the query dtype
  const void* v_new;
  int32_t* seqlens_q_out;   // [B], written by workgroup 0
  int32_t* seqlens_k_out;
  // [B] or nullptr: the caller's cursor; a request whose past length differs appends nothing
  const int32_t* committed;
};

// OR of the per-lane status flags across the wave (uniform result; every SPATTN_STATUS_*
// bit, 0 .. 9).
__device__ __forceinline__ int wave_or_flags(int flags) {
  int wave_flags = 0;
#pragma unroll
  for (int bit = 0; bit < 10; ++bit)
    if (__ballot(flags & (1 << bit))) wave_flags |= 1 << bit;
  return wave_flags;
}
// Flags reach the status word through raise_status: one atomic OR whose result is unused,
// so nothing waits for it (a read-then-OR would put a contended load on the critical path).

// LDS layout (bytes): per-wave V tiles (reused as the combine / merge area after the key
// loop), then the split's row table, then the staged metadata.  The row table holds one
// cache-row index per key for selected and auxiliary rows, and one base row per cache block
// for paged ranges (a key's row is its block's base plus its offset in the block), so a
// 2048-key paged split needs 129 entries at block size 16 instead of 2048.
template <int D>
struct SplitLds {
  // two tiles in flight per wave: a wave's two V tile buffers
  static constexpr int kVTileBytes = 2 * kTile * D * 2;
  static constexpr int kCombineRow = D + 4;   // floats per (wave, head) row of the combine area
  static constexpr int kCombineBytes = (kWaves * 16 * kCombineRow + 4 * kWaves * 16) * 4;
  static constexpr int kAreaBytes = (kWaves * kVTileBytes > kCombineBytes) ? kWaves * kVTileBytes : kCombineBytes;
};

template <int D>
static size_t split_lds_bytes(int row_slots, int meta_ints) {
  return SplitLds<D>::kAreaBytes + (size_t)row_slots * 4 + (size_t)meta_ints * 4;
}

// Row-table entries of a split of `chunk` keys: with a block table, one per block a paged
// range can touch (a split may start inside a block); otherwise one per key.
static int split_row_slots(int kind, int chunk, bool paged, int block_size) {
  if (kind != SPATTN_KIND_PAGED || !paged) return chunk;
  return (chunk + block_size - 2) / block_size + 1;
}

// LDS-DMA of 16 bytes per lane: lane l's bytes land at lds + 16 * l (the LDS address is
// wave-uniform; lanes that skip the call leave their 16 bytes untouched).
__device__ __forceinline__ void dma16(const void* gptr, void* lds) {
  __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void*)(lds), 16, 0, 0);
}
// The compiler does not track LDS-DMA completion: wait for every vector memory operation
// of this wave, and for every LDS operation before an LDS buffer is overwritten by DMA.
__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// vmcnt wait with a compile-time count (gfx9 encoding: low 4 bits at [3:0], high 2 at [15:14]).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Issue the loads of one 32-key tile.  K rows 16*st + lam, dims 32*kc + 8*grp .. +7 come
// straight into the A operand of S^T = K Q^T; 16-bit V rows go into the wave's LDS buffer
// by DMA in the same lane layout (block (st, kc) of 1 KB, lane l at 16*l); INT8 V is loaded
// into registers and converted.  Every lane issues every load (a masked key reads the
// in-bounds rows `dk` / `dv`: its score is replaced by -inf and its V row, which must be
// finite, gets weight 0), so each tile costs exactly 4*D/32 vector memory instructions and
// can be waited for with a fixed vmcnt.
template <typename OpT, typename KT, int D, bool kQuant = sizeof(KT) == 1>
struct TileRegs {
  typename OpVec<OpT>::v8 k[2][D / 32];   // 16-bit caches: the K operands as loaded
};
template <typename OpT, typename KT, int D>
struct TileRegs<OpT, KT, D, true> {
  i32x4 kq[2][D / 64], vq[2][D / 64];     // 8-bit caches: raw codes, 16 per lane and load
};

// Dimensions of the K operand of QK step kc held by lane group grp: 8 at 32 kc + 8 grp for
// 16-bit caches (16-byte loads); for 8-bit caches one 16-byte load brings 16 codes, dims
// 64 j + 16 grp .. + 15, which feed steps 2j and 2j + 1.  The query operand uses the same
// dimensions (the contraction does not depend on their order).
template <typename KT>
__device__ __forceinline__ int qk_col(int kc, int grp) {
  return sizeof(KT) == 2 ? 32 * kc + 8 * grp : 64 * (kc >> 1) + 16 * grp + 8 * (kc & 1);
}

template <typename OpT, typename KT, int D>
__device__ __forceinline__ void issue_tile(TileRegs<OpT, KT, D>& t, const KT* __restrict__ kbase,
                                           const KT* __restrict__ vbase, const KT* dk,
                                           const KT* dv, int row0, int row1, unsigned char* vbuf,
                                           int grp) {
  constexpr int KC = D / 32;
  const int rows[2] = {row0, row1};
  if constexpr (sizeof(KT) == 2) {
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int col = kc * 32 + grp * 8;
        const KT* kp = rows[st] >= 0 ? kbase + (int64_t)rows[st] * D + col : dk + col;
        const KT* vp = rows[st] >= 0 ? vbase + (int64_t)rows[st] * D + col : dv + col;
        dma16(vp, vbuf + (st * KC + kc) * 1024);
        t.k[st][kc] = load_op8<OpT>(kp);
      }
  } else {
    // raw codes stay in flight; they are converted when the tile is consumed
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int j = 0; j < D / 64; ++j) {
        const int col = 64 * j + 16 * grp;
        const KT* kp = rows[st] >= 0 ? kbase + (int64_t)rows[st] * D + col : dk + col;
        const KT* vp = rows[st] >= 0 ? vbase + (int64_t)rows[st] * D + col : dv + col;
        t.vq[st][j] = load16(vp);
        t.kq[st][j] = load16(kp);
      }
  }
}

// The f16 operands of 16 codes (an E4M3 code as value / 256, the factor riding on the
// scales; an INT8 code exactly).
template <typename KT>
__device__ __forceinline__ void codes_to_f16(i32x4 r, f16x8& a, f16x8& b) {
  if constexpr (std::is_same<KT, uint8_t>::value) {
    a = fp8x8_to_f16(r[0], r[1]);
    b = fp8x8_to_f16(r[2], r[3]);
  } else {
    a = int8x8_to_f16(r[0], r[1]);
    b = int8x8_to_f16(r[2], r[3]);
  }
}

// Softmax update and both products for a tile whose loads have completed.
template <typename OpT, typename KT, int D>
__device__ __forceinline__ void consume_tile(TileRegs<OpT, KT, D>& t, uint32_t valid,
                                             const typename OpVec<OpT>::v8 (&qop)[2][D / 32],
                                             float scale_log2, unsigned char* vbuf, float& m_run,
                                             float& l_run, f32x4 (&acc)[D / 16], int lam, int grp) {
  typedef typename OpVec<OpT>::v8 V8;
  constexpr int KC = D / 32;
  constexpr int MT = D / 16;
  constexpr bool kQuant = sizeof(KT) == 1;
  V8 kop[2][kQuant ? KC : 1];   // 8-bit caches: the converted K operands
  if constexpr (kQuant) {
    // V codes to f16, into the LDS buffer in the DMA lane layout (block (st, dim / 32),
    // slot key % 16 + 16 * ((dim % 32) / 8)), masked keys as zeros; then the K codes
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const bool ok = (valid >> (16 * st + lam)) & 1u;
#pragma unroll
      for (int j = 0; j < D / 64; ++j) {
        V8 v0, v1;
        codes_to_f16<KT>(t.vq[st][j], v0, v1);
        unsigned char* blk = vbuf + (st * KC + 2 * j + (grp >> 1)) * 1024 + 16 * (lam + 32 * (grp & 1));
        *reinterpret_cast<V8*>(blk) = ok ? v0 : V8{};
        *reinterpret_cast<V8*>(blk + 256) = ok ? v1 : V8{};
      }
    }
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int j = 0; j < D / 64; ++j) codes_to_f16<KT>(t.kq[st][j], kop[st][2 * j], kop[st][2 * j + 1]);
  }
  // S^T[key][head] for keys 16*st + 4*grp + i, head lam
  f32x4 s[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      if constexpr (kQuant) {
        c = mfma16(kop[st][kc], qop[0][kc], c);
        // the low half of the folded query (see the query set-up)
        c = mfma16(kop[st][kc], qop[1][kc], c);
      } else {
        c = mfma16(t.k[st][kc], qop[0][kc], c);
      }
    }
    s[st] = c;
  }
  float mt = kNegInf;
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = 16 * st + 4 * grp + i;
      const float v = ((valid >> key) & 1u) ? s[st][i] * scale_log2 : kNegInf;
      s[st][i] = v;
      mt = fmaxf(mt, v);
    }
  mt = xor_max(mt, 16);
  mt = xor_max(mt, 32);
  const float m_new = fmaxf(m_run, mt);
  // the reference maximum m_run moves only when some head's maximum outgrows it by more
  // than kLazyRescaleLog2 (a head's first visible key always moves it: x - -inf = inf);
  // -inf - -inf is NaN and compares false, so a head with no visible key keeps m = -inf
  if (__ballot(m_new - m_run > kLazyRescaleLog2)) {
    const float alpha = m_new == m_run ? 1.f : exp2_safe(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] *= alpha;
    m_run = m_new;
  }
  // a head with no visible key so far keeps l = 0, acc = 0 (its scores are all -inf)
  const float m_use = m_run == kNegInf ? 0.f : m_run;
  // bf16 operands keep 8 significant bits: the weights are carried as hi + lo (hi = p
  // rounded, lo = its rounding error rounded) and PV takes one product with each, so the
  // weights keep about 16 bits, as f16 operands keep 11
  constexpr bool kSplitP = std::is_same<OpT, bf16>::value;
  float psum = 0.f;
  V8 pop, plo;
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = exp2_safe(s[st][i] - m_use);
      psum += p;
      pop[st * 4 + i] = (OpT)p;
      if constexpr (kSplitP) plo[st * 4 + i] = (OpT)(p - (float)pop[st * 4 + i]);
    }
  psum = xor_sum(psum, 16);
  psum = xor_sum(psum, 32);
  l_run += psum;
  if constexpr (sizeof(KT) == 1) wait_lgkm0();
  const int s4 = lam >> 2, u = lam & 3;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    // V[key][dim] sits in block (key / 16, dim / 32) at lane slot (key % 16) + 16 * ((dim % 32) / 8)
    // and byte 2 * (dim % 8); lane (grp, 4*s4 + u) fetches key 4*grp + s4 (+16), dims 16m + 4u ..
    const int slot = 4 * grp + s4 + 16 * (2 * (m & 1) + (u >> 1));
    const unsigned char* a0 = vbuf + (m >> 1) * 1024 + slot * 16 + (u & 1) * 8;
    const unsigned char* a1 = a0 + KC * 1024;
    s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a0));
    s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a1));
    typename OpVec<OpT>::v4 h0 = __builtin_bit_cast(typename OpVec<OpT>::v4, r0);
    typename OpVec<OpT>::v4 h1 = __builtin_bit_cast(typename OpVec<OpT>::v4, r1);
    V8 aop = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
    acc[m] = mfma16(aop, pop, acc[m]);
    if constexpr (kSplitP) acc[m] = mfma16(aop, plo, acc[m]);
  }
}

__device__ __forceinline__ uint32_t tile_valid(int row0, int row1) {
  const uint64_t b0 = __ballot(row0 >= 0);
  const uint64_t b1 = __ballot(row1 >= 0);
  return (uint32_t)(b0 & 0xFFFFu) | ((uint32_t)(b1 & 0xFFFFu) << 16);
}

// The key loop of one wave over one source, two tiles deep: the next tile's loads are in
// flight while the current tile is computed (V tiles alternate between two LDS buffers).
// `row_at(k)` gives the cache-row index (row of D elements counted from kbase / vbase) of
// key k < n_keys of the split, or -1; `dk` is any in-bounds row and `dv` an in-bounds row
// of finite values, read for masked keys.
template <typename OpT, typename KT, int D, typename RowAt>
__device__ __forceinline__ void wave_keys(const KT* __restrict__ kbase, const KT* __restrict__ vbase,
                                          const KT* dk, const KT* dv, RowAt row_at, int n_keys,
                                          const typename OpVec<OpT>::v8 (&qop)[2][D / 32],
                                          float scale_log2, unsigned char* vbuf2, float& m_run,
                                          float& l_run, f32x4 (&acc)[D / 16]) {
  constexpr int kTileBytes = (D / 32) * 2 * 1024;
  // vector memory instructions per tile (K and V, both key halves)
  constexpr int kOps = sizeof(KT) == 2 ? 4 * (D / 32) : 4 * (D / 64);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lam = lane & 15;
  const int grp = lane >> 4;
  const int n_tiles = (n_keys + kTile - 1) / kTile;
  auto row_of = [&](int tile, int k) {
    const int key = tile * kTile + k;
    return key < n_keys ? row_at(key) : -1;
  };
  TileRegs<OpT, KT, D> ta, tb;
  int tile = wave;
  if (tile >= n_tiles) return;
  int a0 = row_of(tile, lam), a1 = row_of(tile, 16 + lam);
  uint32_t va = tile_valid(a0, a1);
  issue_tile<OpT, KT, D>(ta, kbase, vbase, dk, dv, a0, a1, vbuf2, grp);
  int buf = 0;
  for (;;) {
    const int next = tile + kWaves;
    if (next < n_tiles) {
      const int b0 = row_of(next, lam), b1 = row_of(next, 16 + lam);
      const uint32_t vb = tile_valid(b0, b1);
      wait_lgkm0();  // the LDS buffer about to be refilled has been read
      issue_tile<OpT, KT, D>(tb, kbase, vbase, dk, dv, b0, b1, vbuf2 + (buf ^ 1) * kTileBytes, grp);
      wait_vm<kOps>();  // everything but the next tile has landed
      consume_tile<OpT, KT, D>(ta, va, qop, scale_log2, vbuf2 + buf * kTileBytes, m_run, l_run, acc, lam, grp);
      ta = tb;
      va = vb;
      buf ^= 1;
      tile = next;
    } else {
      wait_vm<0>();
      consume_tile<OpT, KT, D>(ta, va, qop, scale_log2, vbuf2 + buf * kTileBytes, m_run, l_run, acc, lam, grp);
      break;
    }
  }
}

// The split's source and key range for a resolved row.
struct SplitRange {
  int src, v0, n_keys, lo;
  const int32_t* sel;
};

template <int KIND>
__device__ __forceinline__ SplitRange split_range(const SplitParams& P, const RowInfo& ri, int r,
                                                  int c, int split, int& flags) {
  SplitRange sr{SRC_RANGE, 0, 0, 0, nullptr};
  if (ri.b < 0) return sr;
  int s = split, cnt;
  if (KIND == SPATTN_KIND_LOCAL_AUX && split >= P.n_main) { sr.src = SRC_AUX; s = split - P.n_main; }
  else if (KIND == SPATTN_KIND_SELECTED) sr.src = SRC_SELECT;
  if (sr.src == SRC_RANGE) {
    sr.lo = P.window > 0 ? max(0, ri.p - P.window + 1) : 0;
    cnt = ri.p - sr.lo + 1;
  } else {
    sr.sel = P.sel_idx + ((int64_t)r * P.H_kv + c) * P.max_sel;
    if (P.sel_count != nullptr) {
      cnt = P.sel_count[(int64_t)r * P.H_kv + c];
      if (cnt < 0 || cnt > P.max_sel) flags |= SPATTN_STATUS_BAD_COUNT;
      cnt = min(max(cnt, 0), P.max_sel);
    } else {
      cnt = P.max_sel;
    }
  }
  sr.v0 = s * P.chunk;
  sr.n_keys = max(0, min(sr.v0 + P.chunk, cnt) - sr.v0);
  return sr;
}

// Cache-row index of key v of the split, or -1 (guards raise status bits).
__device__ __forceinline__ int split_key_row(const SplitParams& P, const SplitRange& sr,
                                             const RowInfo& ri, int c, int v, int& flags) {
  if (sr.src == SRC_RANGE) return cache_row_index(P.cd, ri.b, sr.lo + sr.v0 + v, c, flags);
  const int j = sr.sel[sr.v0 + v];
  if (sr.src == SRC_SELECT) {
    if (j != -1 && (j < 0 || j >= ri.kv_len)) { flags |= SPATTN_STATUS_BAD_INDEX; return -1; }
    if (j >= 0 && j <= ri.p) return cache_row_index(P.cd, ri.b, j, c, flags);
    return -1;
  }
  if (j != -1 && (j < 0 || j >= P.aux_len)) { flags |= SPATTN_STATUS_BAD_INDEX; return -1; }
  if (j >= 0) return (int)(ri.b * P.aux_row_stride + (int64_t)j * P.H_kv + c);
  return -1;
}

// Splits dealt to CUs by size (paged ranges and selected rows).  The workgroups of a launch
// that fits the GPU are
// all resident at once, and workgroup i runs on XCD i % 8 and, within it, on CU
// (i / 8) % 32; a CU streams its workgroups' keys at a rate of its own, so the call lasts
// as long as the CU with the most keys.  With fixed splits the key counts of the splits
// sharing a CU follow from the rows' lengths (four long rows' splits can meet on one CU
// while another gets empty splits; selected rows' counts vary the same way).  Instead
// every workgroup computes all U = n_splits * T split sizes of its KV head (paged: from
// the metadata; selected: from the per-row counts), ranks them (largest first, ties by
// index) and takes the split of the rank that a serpentine deal gives its position:
// position j = (its index among the head's workgroups) sits on CU slot j % cus, round
// j / cus; even rounds deal ranks in slot order, odd rounds in reverse, so each CU gets one
// split of each size class.  The partial-state layout does not change.  Needs U <=
// kThreads and scratch for kThreads + 1 ints.
template <int KIND>
__device__ __forceinline__ void deal_split(const SplitParams& P, const int32_t* cu,
                                           const int32_t* skl, bool step_bad, int c, int* sm,
                                           int& split, int& r) {
  const int tid = threadIdx.x;
  const int U = P.n_splits * P.T;
  int* s_size = sm;                  // [kThreads]
  int* s_pick = sm + kThreads;       // [1]
  int sz = 0;
  if (tid < U) {
    const int rr = tid % P.T, ss = tid / P.T;
    int L = 0;
    if constexpr (KIND == SPATTN_KIND_SELECTED) {
      // the row's count as split_range reads it (a dead row's splits are empty, but are
      // ranked by their count: only the deal's balance depends on it)
      L = P.sel_count != nullptr ? min(max(P.sel_count[(int64_t)rr * P.H_kv + c], 0), P.max_sel)
                                 : P.max_sel;
    } else if (!step_bad) {
      int f = 0;   // each row's own workgroups raise its flags
      const RowInfo x = resolve_row(cu, skl, P.B, rr, P.max_q, P.max_k, f);
      if (x.b >= 0) {
        const int lo = P.window > 0 ? max(0, x.p - P.window + 1) : 0;
        L = max(0, x.p - lo + 1);
      }
    }
    sz = min(max(L - ss * P.chunk, 0), P.chunk);
  }
  // one sort key per split: the size, ties by index (sizes <= kChunkCap, U <= 512)
  const int key = sz * 512 + (511 - tid);
  if (tid < ((U + 3) & ~3)) s_size[tid] = tid < U ? key : -1;   // padding ranks last
  __syncthreads();
  const int j = blockIdx.x / P.H_kv;
  const int cus = P.cu_slots;
  const int R = j / cus, pos = j - R * cus;
  const int nR = min(cus, U - R * cus);
  const int k = R * cus + ((R & 1) ? nR - 1 - pos : pos);
  if (tid < U) {
    int rank = 0;                    // splits with a larger key
    for (int u = 0; u < U; u += 4) {
      const i32x4 o = *reinterpret_cast<const i32x4*>(s_size + u);
#pragma unroll
      for (int e = 0; e < 4; ++e) rank += o[e] > key ? 1 : 0;
    }
    if (rank == k) *s_pick = tid;
  }
  __syncthreads();
  const int unit = __builtin_amdgcn_readfirstlane(*s_pick);   // (uniform: one writer)
  split = unit / P.T;
  r = unit - split * P.T;
  __syncthreads();                   // the scratch is free again
}

// Per-request metadata of a workgroup, staged in LDS (`meta`, 2 B + 1 ints) when `to_lds`.
// Fused decode step (kStep), one load round and one barrier: meta[0..B] = cu,
// meta[B+1+b] = past[b] + q_len_b - 1 (seqlens_k, as prepare_seqlens derives it for
// well-formed metadata), and with a cursor, meta[2B+1+b] = 1 when committed[b] differs
// from past[b] (3 B + 1 ints); returns whether the metadata is malformed (B + 1 <=
// kThreads).  Otherwise cu / seqlens_k are copied, or read from global memory when !to_lds.
template <bool kStep>
__device__ __forceinline__ bool stage_metadata(const SplitParams& P, int32_t* meta, bool to_lds,
                                               const int32_t*& cu, const int32_t*& skl) {
  const int tid = threadIdx.x;
  cu = P.cu;
  skl = P.seqlens_k;
  if constexpr (kStep) {
    const int n = P.B + 1;
    const int cv = tid < n ? P.cu[tid] : 0;
    const int cn = tid < P.B ? P.cu[tid + 1] : 0;
    const int pb = tid < P.B ? P.past[tid] : 0;
    const int cm = tid < P.B && P.committed != nullptr ? P.committed[tid] : pb;
    const bool bad = (tid < P.B && (cn < cv || pb < 0)) ||
                     (tid == 0 && (cv != 0 || P.cu[P.B] != P.T));
    if (tid < n) meta[tid] = cv;
    if (tid < P.B) {
      meta[n + tid] = pb + (cn - cv) - 1;
      if (P.committed != nullptr) meta[n + P.B + tid] = cm != pb ? 1 : 0;
    }
    const bool step_bad = __syncthreads_or(bad) != 0;
    cu = meta;
    skl = meta + n;
    return step_bad;
  } else {
    if (to_lds) {
      for (int i = tid; i <= P.B; i += kThreads) {
        meta[i] = P.cu[i];
        if (i < P.B) meta[P.B + 1 + i] = P.seqlens_k[i];
      }
      __syncthreads();
      cu = meta;
      skl = meta + P.B + 1;
    }
    return false;
  }
}

// Fused decode step, workgroup 0: seqlens_q / seqlens_k exactly as prepare_seqlens writes
// them.  Malformed metadata takes its sanitised boundaries: the running maximum of cu
// clamped to [0, T] (one per thread, B + 1 <= kThreads) and negative past read as 0.
__device__ __forceinline__ void step_lengths(const SplitParams& P, bool bad, int* wave_max) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (!bad) {
    if (tid < P.B) {
      const int q = P.cu[tid + 1] - P.cu[tid];
      P.seqlens_q_out[tid] = q;
      P.seqlens_k_out[tid] = P.past[tid] + q - 1;
    }
    return;
  }
  const int n = P.B + 1;
  int v = tid < n ? P.cu[tid] : INT32_MIN;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(v, o, 64);
    if (lane >= o) v = max(v, y);
  }
  if (lane == 63) wave_max[wave] = v;
  __syncthreads();
  for (int w = 0; w < wave; ++w) v = max(v, wave_max[w]);
  const int bound = min(max(v, 0), P.T);
  // bound of the next boundary: from the next lane, or from the next wave's first lane
  const int up = __shfl_down(bound, 1, 64);
  __shared__ int first_bound[kWaves];
  if (lane == 0) first_bound[wave] = bound;
  __syncthreads();
  const int next = lane < 63 ? up : (wave + 1 < kWaves ? first_bound[wave + 1] : 0);
  if (tid < P.B) {
    const int q = next - bound;
    P.seqlens_q_out[tid] = q;
    P.seqlens_k_out[tid] = max(P.past[tid], 0) + q - 1;
  }
  __syncthreads();                                     // wave_max is reused by the caller
}

// Fused decode step: new keys j0 .. j1 - 1 (positions >= first_new) of request b, KV head c.
// Key j is row c0 + (j - first_new) of k_new / v_new and goes to its cache slot exactly as
// kv_cache_append stores it (16-bit rows copied, 8-bit rows quantised by the same code
// writers).  Each workgroup writes the new keys its own split reads before it reads them;
// workgroups that share a key write identical bytes.  Threads take 16-byte pieces.
template <typename QT, typename KT, int D>
__device__ __forceinline__ void step_write_keys(const SplitParams& P, int b, int c, int j0, int j1,
                                                int first_new, int c0, int& flags) {
  constexpr int kPieces = D / 8;                 // 8-element pieces per row
  const int n = max(0, j1 - j0) * 2 * kPieces;   // K and V
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const int key = i / (2 * kPieces), rest = i - key * 2 * kPieces;
    const bool is_v = rest >= kPieces;
    const int d = (is_v ? rest - kPieces : rest) * 8;
    const int j = j0 + key;
    const QT* src = reinterpret_cast<const QT*>(is_v ? P.v_new : P.k_new) +
                    ((int64_t)(c0 + j - first_new) * P.H_kv + c) * D + d;
    // the new row's piece loads before the block-id lookup, so the two loads overlap
    const i32x4 raw = load16(src);
    const int row = cache_row_index(P.cd, b, j, c, flags);
    if (row < 0) continue;
    // the cache arguments are read-only everywhere else in this kernel
    void* cache = const_cast<void*>(is_v ? P.v_cache : P.k_cache);
    if constexpr (sizeof(KT) == 1) {
      const typename OpVec<QT>::v8 x = __builtin_bit_cast(typename OpVec<QT>::v8, raw);
      QT piece[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) piece[e] = x[e];
      quantize8<std::is_same<KT, uint8_t>::value>(
          piece, (is_v ? P.value_scale : P.key_scale) + c * D + d,
          reinterpret_cast<int8_t*>(cache) + (int64_t)row * D + d);
    } else {
      store16(reinterpret_cast<KT*>(cache) + (int64_t)row * D + d, raw);
    }
  }
}

// One wave's key loop over main-cache rows.  Quantised caches fold the per-channel key
// scale into the query.  The folded value x = q * s is carried as hi + lo, two 16-bit
// operands (hi = x rounded, lo = the rounding error rounded), and S takes one product with
// each, so the scores keep about 22 bits of x instead of 11: a single 16-bit operand would
// put a relative error of 2^-11 on every term q_d k_d, i.e. score errors up to
// 2^-11 sum_d |q_d k_d|.  `qraw` holds this lane's query dims as loaded (16-bit caches);
// lanes with hv false loaded the tile's first head and carry a zero query.
template <typename QT, typename KT, int D, typename RowAt>
__device__ __forceinline__ void main_cache_keys(const SplitParams& P, const QT* qrow,
                                                const QT* q0row, bool hv,
                                                const i32x4 (&qraw)[D / 32], int c, RowAt row_at,
                                                int n_keys, unsigned char* vbuf2, float& m_run,
                                                float& l_run, f32x4 (&acc)[D / 16]) {
  typedef typename std::conditional<sizeof(KT) == 1, f16, KT>::type OpM;
  constexpr float kUnit = std::is_same<KT, uint8_t>::value ? kFp8Unit : 1.0f;
  const int grp = (threadIdx.x & 63) >> 4;
  typename OpVec<OpM>::v8 qop[2][D / 32];
#pragma unroll
  for (int kc = 0; kc < D / 32; ++kc) {
    const int col = qk_col<KT>(kc, grp);
    if constexpr (sizeof(KT) == 1) {
      // the query dims of this step's K operand (not those of qraw's layout)
      const typename OpVec<QT>::v8 qv = __builtin_bit_cast(
          typename OpVec<QT>::v8, hv ? load16(qrow + col) : i32x4{0, 0, 0, 0});
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = hv ? to_f32((QT)qv[e]) * (P.key_scale[c * D + col + e] * kUnit) : 0.f;
        const OpM hi = (OpM)x;
        qop[0][kc][e] = hi;
        qop[1][kc][e] = (OpM)(x - (float)hi);
      }
    } else {
      qop[0][kc] = __builtin_bit_cast(typename OpVec<OpM>::v8, hv ? qraw[kc] : i32x4{0, 0, 0, 0});
      qop[1][kc] = typename OpVec<OpM>::v8{};
    }
  }
  // masked keys read row 0 of the cache for K and, with 16-bit caches, the query row of
  // the tile's first head for V (in bounds for every lane, and finite); 8-bit V of masked
  // keys is replaced by zeros
  const KT* dv = sizeof(KT) == 2 ? reinterpret_cast<const KT*>(q0row)
                                 : reinterpret_cast<const KT*>(P.k_cache);
  wave_keys<OpM, KT, D>(reinterpret_cast<const KT*>(P.k_cache),
                        reinterpret_cast<const KT*>(P.v_cache),
                        reinterpret_cast<const KT*>(P.k_cache), dv, row_at, n_keys, qop,
                        P.scale_log2, vbuf2, m_run, l_run, acc);
}

// End of a workgroup's part of one (row, KV head, head tile): the four wave states (head
// lam, dims 16m + 4grp + i) are merged in LDS and stored.  Rows of the accumulator area are
// padded by 4 floats so the 16-byte stores of the 16 heads of a lane group fall in
// different banks; the merge factors of each (wave, head) are computed once, by 16
// threads.  `direct`: the workgroup saw every key of the row, so it writes the normalised
// output (the sink folded into the normaliser); otherwise the partial (m, l, acc) of head
// h goes to acc_dst[h * D ..] and ml_dst[h] for the merge kernel.  8-bit caches apply
// value_scale here.  The caller has synchronised after the key loop; `area` is free
// again when this returns.
template <typename QT, int D>
__device__ __forceinline__ void combine_and_store(const SplitParams& P, unsigned char* area,
                                                  float m_run, float l_run,
                                                  const f32x4 (&acc)[D / 16], int nh, int r,
                                                  int c, int h0, bool use_scale, float unit,
                                                  bool direct, float* acc_dst, float2* ml_dst) {
  constexpr int CR = SplitLds<D>::kCombineRow;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lam = lane & 15, grp = lane >> 4;
  float* cm = reinterpret_cast<float*>(area);              // [wave][16] m
  float* cl = cm + kWaves * 16;                           // [wave][16] l
  float* cf = cl + kWaves * 16;                           // [wave][16] merge factor
  float* cML = cf + kWaves * 16;                          // [16] (M, L)
  float* ca = cML + kWaves * 16;                          // [wave][16][CR] acc
  if (grp == 0) { cm[wave * 16 + lam] = m_run; cl[wave * 16 + lam] = l_run; }
#pragma unroll
  for (int m = 0; m < D / 16; ++m)
    *reinterpret_cast<f32x4*>(ca + (wave * 16 + lam) * CR + 16 * m + 4 * grp) = acc[m];
  __syncthreads();
  if (tid < 16) {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, cm[w * 16 + tid]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = M != kNegInf ? exp2_safe(cm[w * 16 + tid] - M) : 0.f;
      cf[w * 16 + tid] = f;
      L += cl[w * 16 + tid] * f;
    }
    cML[2 * tid] = M;
    cML[2 * tid + 1] = L;
  }
  __syncthreads();
  for (int e = tid; e < 16 * D; e += kThreads) {
    const int h = e / D, d = e - h * D;
    if (h >= nh) continue;
    const float M = cML[2 * h], L = cML[2 * h + 1];
    float A = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) A += ca[(w * 16 + h) * CR + d] * cf[w * 16 + h];
      if (use_scale) A *= P.value_scale[c * D + d] * unit;
    }
    const int head = h0 + h;
    if (direct) {
      float res = 0.f;
      if (M != kNegInf) {
        const float sg = P.sinks != nullptr ? P.sinks[head] * kLog2e : kNegInf;
        const float M2 = fmaxf(M, sg);
        const float f = exp2_safe(M - M2);
        res = A * f / (L * f + exp2_safe(sg - M2));
      }
      reinterpret_cast<QT*>(P.out)[((int64_t)r * P.H_q + head) * D + d] = from_f32<QT>(res);
    } else {
      acc_dst[h * D + d] = A;
      if (d == 0) ml_dst[h] = make_float2(M, L);
    }
  }
  __syncthreads();
}

// Occupancy hint for D = 64, where each wave keeps two tiles in flight: 4 waves per SIMD
// for 16-bit and INT8 caches (the double-buffered V tiles take 32 KB of LDS per
// workgroup, so a CU holds at most 4 workgroups of 4 waves whatever the registers allow;
// INT8 tiles hold the raw K and V codes and the query has a second, low operand); one
// fewer when the kernel also carries the second (window) source over an 8-bit cache; 3
// for FP8 caches, whose conversion needs a few more registers (at 4 it spills inside the
// key loop: 63.6 us against 56.6 at 3 for the FP8 decode).
template <int KIND, typename KT, int D>
constexpr int split_waves_per_eu() {
  if (D != 64) return 1;
  if (KIND == SPATTN_KIND_LOCAL_AUX) return sizeof(KT) == 1 ? 3 : 4;
  return std::is_same<KT, uint8_t>::value ? 3 : 4;
}

template <int KIND, typename QT, typename KT, typename AT, int D, bool kStep>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(split_waves_per_eu<KIND, KT, D>(), 8)))
void split_attn_kernel(SplitParams P) {
  typedef typename std::conditional<sizeof(KT) == 1, f16, KT>::type OpM;  // main operand
  // FP8 operands hold code values / kFp8Unit; the factor rides on the scales
  constexpr float kUnit = std::is_same<KT, uint8_t>::value ? kFp8Unit : 1.0f;
  typedef QT OpA;                                                          // aux operand
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* area = smem;
  int32_t* rows = reinterpret_cast<int32_t*>(smem + SplitLds<D>::kAreaBytes);
  int32_t* meta = rows + P.row_slots;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lam = lane & 15;
  const int grp = lane >> 4;

  const int hkt = P.H_kv * P.head_tiles;
  const int per_split = P.T * hkt;
  int split = blockIdx.x / per_split;
  const int rem = blockIdx.x - split * per_split;
  int r = rem / hkt;
  const int kvt = rem - r * hkt;
  const int c = kvt / P.head_tiles;
  const int ht = kvt - c * P.head_tiles;
  const int h0 = c * P.group + ht * 16;                 // first query head of the tile
  const int nh = min(16, P.group - ht * 16);            // heads in the tile
  const bool dealt = KIND != SPATTN_KIND_LOCAL_AUX && P.cu_slots > 0;

  // the query rows: without the deal they depend on the grid position only and load
  // under the metadata round
  const bool hv = lam < nh;
  i32x4 qraw[D / 32];
  auto load_query = [&]() {
    const QT* qrow = reinterpret_cast<const QT*>(P.q) + ((int64_t)r * P.H_q + h0 + (hv ? lam : 0)) * D;
#pragma unroll
    for (int kc = 0; kc < D / 32; ++kc)
      qraw[kc] = load16(qrow + kc * 32 + grp * 8);
  };
  if (!dealt) load_query();

  // ---- 1. the row's request and position ----
  const int32_t* cu = P.cu;
  const int32_t* skl = P.seqlens_k;
  __shared__ int wave_flags[kWaves];
  // fused step: malformed metadata
  const bool step_bad = stage_metadata<kStep>(P, meta, P.meta_lds != 0, cu, skl);
  if (dealt) {
    deal_split<KIND>(P, cu, skl, step_bad, c, reinterpret_cast<int*>(area), split, r);
    load_query();
  }
  const QT* qrow = reinterpret_cast<const QT*>(P.q) + ((int64_t)r * P.H_q + h0 + (hv ? lam : 0)) * D;
  const QT* q0row = reinterpret_cast<const QT*>(P.q) + ((int64_t)r * P.H_q + h0) * D;
  int flags = 0;
  RowInfo ri;
  if (step_bad) {
    // malformed metadata in a fused step: every row is zero and nothing is appended
    ri.b = -1; ri.q_len = 0; ri.kv_len = 0; ri.p = -1;
    if (blockIdx.x == 0) flags |= SPATTN_STATUS_BAD_CU;
  } else {
    ri = resolve_row(cu, skl, P.B, r, P.max_q, P.max_k, flags);
  }
  // fused step with a cursor: requests whose cursor disagrees append nothing (their rows
  // are still attended over the unchanged cache); workgroup 0 flags them
  auto cursor_bad = [&](int b) { return kStep && P.committed != nullptr && meta[2 * P.B + 1 + b] != 0; };
  if (kStep && !step_bad && P.committed != nullptr && blockIdx.x == 0) {
    // (a uniform branch: every thread of workgroup 0 holds the flag)
    if (__syncthreads_or(tid < P.B && cu[tid + 1] > cu[tid] && cursor_bad(tid)))
      flags |= SPATTN_STATUS_CURSOR;
  }
  if (kStep && !step_bad && ri.b < 0 && ri.q_len > 0 &&
      split == 0 && ht == 0 && !cursor_bad(find_request(cu, P.B, r))) {
    // a fused step's row beyond the host bounds reads nothing, but its key is still appended
    const int b = find_request(cu, P.B, r);
    const int first_new = ri.kv_len - ri.q_len, j = first_new + (r - cu[b]);
    if (j < 0) flags |= SPATTN_STATUS_SHORT_KV;
    else step_write_keys<QT, KT, D>(P, b, c, j, j + 1, first_new, cu[b], flags);
  }

  // ---- 2. the split's keys -> cache-row indices ----
  const SplitRange sr = split_range<KIND>(P, ri, r, c, split, flags);
  if (sr.n_keys == 0 && P.n_splits > 1) {
    // nothing in this split: (m, l) = (-inf, 0) tells the merge to skip it; no accumulator
    // (the flags raised so far are the same in every wave)
    if (kStep && blockIdx.x == 0) step_lengths(P, step_bad, wave_flags);
    if (tid == 0) raise_status(P.status, flags);
    if (tid < nh)
      P.ws_ml[(int64_t)split * P.T * P.H_q + (int64_t)r * P.H_q + h0 + tid] = make_float2(kNegInf, 0.f);
    return;
  }
  // paged range through a block table: keys j0 .. j0 + n_keys - 1, the base row of block
  // lb at rows[lb - lb0] (-1: missing); other sources: key k's row at rows[k]
  const bool blocks = KIND == SPATTN_KIND_PAGED && P.cd.block_table != nullptr;
  const int j0 = sr.lo + sr.v0;
  const int bs = P.cd.block_size, bsh = P.cd.bs_shift;
  auto block_of = [&](int j) { return bsh >= 0 ? j >> bsh : j / bs; };
  const int lb0 = block_of(j0);
  if (blocks) {
    const int n_ent = sr.n_keys > 0 ? block_of(j0 + sr.n_keys - 1) - lb0 + 1 : 0;
    for (int v = tid; v < n_ent; v += kThreads) {
      const int lb = lb0 + v;
      int e = -1;
      if (lb >= P.cd.max_blocks) {
        flags |= SPATTN_STATUS_CAPACITY;
      } else {
        const int blk = P.cd.block_table[(int64_t)ri.b * P.cd.max_blocks + lb];
        if (blk < 0 || blk >= P.cd.num_blocks) flags |= SPATTN_STATUS_BAD_BLOCK;
        else e = (blk * P.cd.H_kv + c) * bs;
      }
      rows[v] = e;
    }
  } else {
    for (int v = tid; v < sr.n_keys; v += kThreads) rows[v] = split_key_row(P, sr, ri, c, v, flags);
  }
  if (kStep && ri.b >= 0 && !cursor_bad(ri.b)) {
    // fused step: the new keys of this split's range, written before the barrier below
    const int first_new = ri.kv_len - ri.q_len, k0 = sr.lo + sr.v0;
    step_write_keys<QT, KT, D>(P, ri.b, c, max(k0, first_new), k0 + sr.n_keys, first_new,
                               cu[ri.b], flags);
  }
  {
    const int wf = wave_or_flags(flags);
    if (lane == 0) wave_flags[wave] = wf;
  }
  __syncthreads();
  if (tid == 0) raise_status(P.status, wave_flags[0] | wave_flags[1] | wave_flags[2] | wave_flags[3]);

  // ---- 3. per-wave key loop ----
  float m_run = kNegInf, l_run = 0.f;
  f32x4 acc[D / 16];
#pragma unroll
  for (int m = 0; m < D / 16; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bool use_scale = sizeof(KT) == 1 && sr.src != SRC_AUX;
  auto row_at = [&](int k) -> int {
    if (!blocks) return rows[k];
    const int j = j0 + k;
    const int lb = block_of(j);
    const int e = rows[lb - lb0];
    return e < 0 ? -1 : e + (j - lb * bs);
  };
  if (sr.n_keys > 0) {
    if (KIND != SPATTN_KIND_LOCAL_AUX || sr.src != SRC_AUX) {
      main_cache_keys<QT, KT, D>(P, qrow, q0row, hv, qraw, c, row_at, sr.n_keys,
                                 area + wave * SplitLds<D>::kVTileBytes, m_run, l_run, acc);
    } else if constexpr (sizeof(AT) == 2) {
      typename OpVec<OpA>::v8 qop[2][D / 32];
#pragma unroll
      for (int kc = 0; kc < D / 32; ++kc) {
        qop[0][kc] = __builtin_bit_cast(typename OpVec<OpA>::v8, hv ? qraw[kc] : i32x4{0, 0, 0, 0});
        qop[1][kc] = typename OpVec<OpA>::v8{};
      }
      wave_keys<OpA, AT, D>(reinterpret_cast<const AT*>(P.aux_k),
                            reinterpret_cast<const AT*>(P.aux_v),
                            reinterpret_cast<const AT*>(q0row), reinterpret_cast<const AT*>(q0row),
                            row_at, sr.n_keys, qop,
                            P.scale_log2, area + wave * SplitLds<D>::kVTileBytes, m_run, l_run, acc);
    }
  }
  __syncthreads();

  // ---- 4. merge the four wave states and store ----
  const bool single = P.n_splits == 1;
  const int64_t so = (int64_t)split * P.T * P.H_q + (int64_t)r * P.H_q + h0;
  combine_and_store<QT, D>(P, area, m_run, l_run, acc, nh, r, c, h0, use_scale, kUnit, single,
                           single ? nullptr : P.ws_acc + so * D, single ? nullptr : P.ws_ml + so);
  // fused step: the lengths, written last so that nothing of it is live in the key loop
  if (kStep && blockIdx.x == 0) step_lengths(P, step_bad, wave_flags);
}

// ---------------------------------------------------------------------------------------
// Merge of split partial states plus the sink for the float32 path ("[WebGPU] Add
// SparsePagedAttention", finalize stage; one wave per (row, query head), merge
// coefficients shared across the head's output channels).
// ---------------------------------------------------------------------------------------
template <typename QT, int D, int kBatch>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ ws_acc,
                                                    const float2* __restrict__ ws_ml,
                                                    const float* __restrict__ sinks,
                                                    void* __restrict__ out, int T, int H_q,
                                                    int n_splits) {
  // Splits without a visible key wrote m = -inf and no accumulator (their accumulator
  // memory is stale and is not read).  Per batch of kBatch splits (n_splits rounded up to
  // a power of two, at most 16): the (m, l) pairs in one round, then the accumulators of
  // the live splits, every load issued before any is used.
  constexpr int PER = D / 64;
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (pair >= T * H_q) return;
  const int head = pair % H_q;
  const int64_t stride = (int64_t)T * H_q;
  // the sink, loaded before the partial states: loads complete in order, so the waits for
  // the states cover it (loaded after them, it cost a round trip of its own at the end).
  // Every lane loads (a workspace word when there are no sinks, unused), so no register is
  // cleared while the load is in flight.
  const float sink_raw = *(sinks != nullptr ? sinks + head : reinterpret_cast<const float*>(ws_ml));
  float M = kNegInf, L = 0.f;   // running reference maximum and normaliser
  float A[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) A[e] = 0.f;
  // one batch (the first is peeled from the loop: a call with at most kBatch splits then has
  // no loop, whose back edge would make the compiler wait for the sink before the first
  // batch's loads)
  auto batch = [&](int s0) {
    float2 ml[kBatch];
    float a[kBatch][PER];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int sp = min(s0 + k, n_splits - 1);   // (in range; repeats are dropped below)
      ml[k] = ws_ml[sp * stride + pair];
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int sp = min(s0 + k, n_splits - 1);
#pragma unroll
      for (int e = 0; e < PER; ++e) a[k][e] = 0.f;
      if (s0 + k < n_splits && ml[k].x != kNegInf) {   // (uniform across the wave)
#pragma unroll
        for (int e = 0; e < PER; ++e) a[k][e] = ws_acc[(sp * stride + pair) * D + lane + 64 * e];
      }
    }
    float Mb = M;
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      if (s0 + k < n_splits) Mb = fmaxf(Mb, ml[k].x);
    if (Mb == kNegInf) return;                    // nothing visible yet
    const float r = M == kNegInf ? 0.f : exp2_safe(M - Mb);
    L *= r;
#pragma unroll
    for (int e = 0; e < PER; ++e) A[e] *= r;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const bool live = s0 + k < n_splits && ml[k].x != kNegInf;
      const float f = live ? exp2_safe(ml[k].x - Mb) : 0.f;
      L += live ? ml[k].y * f : 0.f;
#pragma unroll
      for (int e = 0; e < PER; ++e) A[e] += live ? a[k][e] * f : 0.f;
    }
    M = Mb;
  };
  if (n_splits > 0) batch(0);
  for (int s0 = kBatch; s0 < n_splits; s0 += kBatch) batch(s0);
  // the sink joins the maximum and the normaliser only; no visible key (A = 0): zeros
  const float sg = sinks != nullptr ? sink_raw * kLog2e : kNegInf;
  const float Mf = fmaxf(M, sg);
  float Lt = 0.f;
  if (Mf != kNegInf) {
    const float r = M == kNegInf ? 0.f : exp2_safe(M - Mf);
    Lt = L * r + (sg == kNegInf ? 0.f : exp2_safe(sg - Mf));
#pragma unroll
    for (int e = 0; e < PER; ++e) A[e] *= r;
  }
  float res[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) res[e] = Lt > 0.f ? A[e] / Lt : 0.f;
  QT* o = reinterpret_cast<QT*>(out) + (int64_t)pair * D;
#pragma unroll
  for (int e = 0; e < PER; ++e) o[lane + 64 * e] = from_f32<QT>(res[e]);
}

// ---------------------------------------------------------------------------------------
// float32 path (float32 queries, float32 or INT8 caches): plain VALU arithmetic, one wave
// per (split, row, query head); same key lists and partial format, merged by merge_kernel.
// ---------------------------------------------------------------------------------------
template <int KIND, typename KT, typename AT, int D, bool DIRECT>
__global__ __launch_bounds__(64) void split_attn_f32_kernel(SplitParams P) {
  __shared__ int32_t rows[64];
  __shared__ float pw[64];
  const int lane = threadIdx.x;
  const int per_split = P.T * P.H_q;
  const int split = blockIdx.x / per_split;
  const int rem = blockIdx.x - split * per_split;
  const int r = rem / P.H_q;
  const int head = rem - r * P.H_q;
  const int c = head / P.group;
  int flags = 0;
  const RowInfo ri = resolve_row(P.cu, P.seqlens_k, P.B, r, P.max_q, P.max_k, flags);
  const SplitRange sr = split_range<KIND>(P, ri, r, c, split, flags);
  const bool is_i8 = sizeof(KT) == 1 && sr.src != SRC_AUX;
  constexpr int PER = D / 64;
  float qv[D];
  const float* q32 = reinterpret_cast<const float*>(P.q) + ((int64_t)r * P.H_q + head) * D;
  for (int d = 0; d < D; ++d) qv[d] = is_i8 ? q32[d] * P.key_scale[c * D + d] : q32[d];
  float m_run = kNegInf, l_run = 0.f, acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
  for (int base = 0; base < sr.n_keys; base += 64) {
    const int v = base + lane;
    const int row = v < sr.n_keys ? split_key_row(P, sr, ri, c, v, flags) : -1;
    float s = kNegInf;
    if (row >= 0) {
      float dot = 0.f;
      if (sr.src == SRC_AUX) {
        const AT* kr = reinterpret_cast<const AT*>(P.aux_k) + (int64_t)row * D;
        for (int d = 0; d < D; ++d) dot += qv[d] * to_f32(kr[d]);
      } else {
        const KT* kr = reinterpret_cast<const KT*>(P.k_cache) + (int64_t)row * D;
        for (int d = 0; d < D; ++d) dot += qv[d] * to_f32(kr[d]);
      }
      s = dot * P.scale_log2;
    }
    float mt = s;
    for (int o = 32; o >= 1; o >>= 1) mt = fmaxf(mt, __shfl_xor(mt, o, 64));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    rows[lane] = row;
    const float p = exp2_safe(s - m_use);
    pw[lane] = p;
    __syncthreads();
    float ps = p;
    for (int o = 32; o >= 1; o >>= 1) ps += __shfl_xor(ps, o, 64);
    const float alpha = exp2_safe(m_run - m_use);
    l_run = l_run * alpha + ps;
    m_run = m_new;
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] *= alpha;
    for (int kk = 0; kk < 64; ++kk) {
      const int rw = rows[kk];
      if (rw < 0) continue;
      const float w = pw[kk];
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int d = lane + 64 * k;
        float x;
        if (sr.src == SRC_AUX) x = to_f32(reinterpret_cast<const AT*>(P.aux_v)[(int64_t)rw * D + d]);
        else x = to_f32(reinterpret_cast<const KT*>(P.v_cache)[(int64_t)rw * D + d]);
        acc[k] += w * x;
      }
    }
    __syncthreads();
  }
  {
    const int wf = wave_or_flags(flags);
    if (lane == 0) raise_status(P.status, wf);
  }
  const int64_t o = ((int64_t)r * P.H_q + head) * D;
  if constexpr (DIRECT) {
    float* out = reinterpret_cast<float*>(P.out) + o;
    const float sg = P.sinks != nullptr ? P.sinks[head] * kLog2e : kNegInf;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int d = lane + 64 * k;
      float res = 0.f;
      if (m_run != kNegInf) {
        const float M2 = fmaxf(m_run, sg);
        const float f = exp2_safe(m_run - M2);
        float a = acc[k];
        if (is_i8) a *= P.value_scale[c * D + d];
        res = a * f / (l_run * f + exp2_safe(sg - M2));
      }
      out[d] = res;
    }
  } else {
    const int64_t so = (int64_t)split * P.T * P.H_q;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int d = lane + 64 * k;
      float a = acc[k];
      if (is_i8 && m_run != kNegInf) a *= P.value_scale[c * D + d];
      P.ws_acc[so * D + o + d] = a;
    }
    if (lane == 0) P.ws_ml[so + (int64_t)r * P.H_q + head] = make_float2(m_run, l_run);
  }
}

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------
bool use_prefill_path(int kind, int dtype, int max_q) {
  return kind == SPATTN_KIND_PAGED && dtype != SPATTN_F32 && max_q > 8;
}

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

SplitPlan make_split_plan(int kind, int dtype, int cache_dtype, int B, int T, int max_q,
                          int max_k, int max_sel, int window, int H_q, int H_kv, int D) {
  (void)B; (void)max_q;
  SplitPlan pl{};
  const int group = H_q / H_kv;
  const bool f32 = dtype == SPATTN_F32;
  pl.head_tiles = f32 ? 1 : (group + 15) / 16;
  long n_main = 0, n_aux = 0;
  if (kind == SPATTN_KIND_PAGED) n_main = window > 0 ? std::min(window, max_k) : max_k;
  else if (kind == SPATTN_KIND_SELECTED) n_main = max_sel;
  else { n_main = window; n_aux = max_sel; }
  n_main = std::max(0L, n_main);
  n_aux = std::max(0L, n_aux);
  const long items = (long)T * (f32 ? H_q : (long)H_kv * pl.head_tiles);
  const long total = n_main + n_aux;
  int chunk = kWgStep;
  auto splits_for = [&](int ch) {
    long s = (n_main + ch - 1) / ch + (n_aux + ch - 1) / ch;
    return std::max(1L, s);
  };
  if (kind == SPATTN_KIND_PAGED && !f32) {
    // as many equal splits per item as fill the target, each of kWgStep .. kChunkCap keys
    // (a multiple of kWgStep)
    const long target = cache_dtype == SPATTN_FP8 ? kTargetWorkgroupsPagedFp8 : kTargetWorkgroupsPaged;
    long s = std::max(1L, target / std::max(1L, items));
    s = std::min(s, std::max(1L, (n_main + kWgStep - 1) / kWgStep));
    s = std::max(s, (n_main + kChunkCap - 1) / kChunkCap);
    if (s > kMaxSplits) {  // key range too long for one call
      pl.n_splits = -1;
      return pl;
    }
    const long per = (n_main + s - 1) / s;
    chunk = (int)std::max((long)kWgStep, (per + kWgStep - 1) / kWgStep * kWgStep);
  } else {
    const long target = kind == SPATTN_KIND_PAGED ? kTargetWorkgroupsPaged : kTargetWorkgroupsSparse;
    while (chunk < kMaxChunk && chunk < total && items * splits_for(chunk) > target) chunk *= 2;
    while (splits_for(chunk) > kMaxSplits && chunk < kChunkCap) chunk *= 2;
    if (splits_for(chunk) > kMaxSplits) {  // key range too long for one call
      pl.n_splits = -1;
      return pl;
    }
  }
  pl.chunk = chunk;
  pl.n_main = (int)std::max(1L, (n_main + chunk - 1) / chunk);
  pl.n_aux = (int)((n_aux + chunk - 1) / chunk);
  if (kind != SPATTN_KIND_LOCAL_AUX) pl.n_aux = 0;
  pl.n_splits = pl.n_main + pl.n_aux;
  pl.ws_bytes = 0;
  if (pl.n_splits > 1) {
    const size_t acc = (size_t)pl.n_splits * T * H_q * D * sizeof(float);
    const size_t ml = (size_t)pl.n_splits * T * H_q * sizeof(float2);
    pl.ws_bytes = align256(acc) + align256(ml);
  }
  return pl;
}

template <int KIND, typename QT, typename KT, typename AT, int D>
static void launch_split_typed(const SplitParams& P, hipStream_t stream) {
  const int blocks = P.n_splits * P.T * P.H_kv * P.head_tiles;
  const size_t lds = split_lds_bytes<D>(P.row_slots, P.meta_lds || P.past != nullptr ? 3 * P.B + 1 : 0);
  // the fused decode step is its own instantiation, so the other kernels carry none of it
  if constexpr (KIND == SPATTN_KIND_PAGED) {
    if (P.past != nullptr) {
      hipLaunchKernelGGL((split_attn_kernel<KIND, QT, KT, AT, D, true>), dim3(blocks), dim3(kThreads), lds, stream, P);
      return;
    }
  }
  hipLaunchKernelGGL((split_attn_kernel<KIND, QT, KT, AT, D, false>), dim3(blocks), dim3(kThreads), lds, stream, P);
}

template <int KIND, typename KT, typename AT, int D>
static void launch_split_f32(const SplitParams& P, bool direct, hipStream_t stream) {
  const int blocks = P.n_splits * P.T * P.H_q;
  if (direct)
    hipLaunchKernelGGL((split_attn_f32_kernel<KIND, KT, AT, D, true>), dim3(blocks), dim3(64), 0, stream, P);
  else
    hipLaunchKernelGGL((split_attn_f32_kernel<KIND, KT, AT, D, false>), dim3(blocks), dim3(64), 0, stream, P);
}

template <int KIND, typename QT, int D>
static void dispatch_cache(const AttnArgs& a, const SplitParams& P, bool direct, hipStream_t stream) {
  // INT8 caches are int8_t, FP8 E4M3 caches uint8_t
  const bool i8 = a.cache_dtype == SPATTN_I8;
  const bool fp8 = a.cache_dtype == SPATTN_FP8;
  if constexpr (std::is_same<QT, float>::value) {
    if (i8) launch_split_f32<KIND, int8_t, float, D>(P, direct, stream);
    else if (fp8) launch_split_f32<KIND, uint8_t, float, D>(P, direct, stream);
    else launch_split_f32<KIND, float, float, D>(P, direct, stream);
  } else {
    if (i8) launch_split_typed<KIND, QT, int8_t, QT, D>(P, stream);
    else if (fp8) launch_split_typed<KIND, QT, uint8_t, QT, D>(P, stream);
    else launch_split_typed<KIND, QT, QT, QT, D>(P, stream);
  }
}

template <int KIND>
static void dispatch_q(const AttnArgs& a, const SplitParams& P, bool direct, hipStream_t stream) {
  if (a.D == 64) {
    if (a.dtype == SPATTN_F32) dispatch_cache<KIND, float, 64>(a, P, direct, stream);
    else if (a.dtype == SPATTN_F16) dispatch_cache<KIND, f16, 64>(a, P, direct, stream);
    else dispatch_cache<KIND, bf16, 64>(a, P, direct, stream);
  } else {
    if (a.dtype == SPATTN_F32) dispatch_cache<KIND, float, 128>(a, P, direct, stream);
    else if (a.dtype == SPATTN_F16) dispatch_cache<KIND, f16, 128>(a, P, direct, stream);
    else dispatch_cache<KIND, bf16, 128>(a, P, direct, stream);
  }
}

int launch_split_attention(const AttnArgs& a, const SplitPlan& plan, hipStream_t stream) {
  if (a.T == 0) return SPATTN_OK;
  SplitParams P;
  P.q = a.q; P.k_cache = a.k_cache; P.v_cache = a.v_cache; P.aux_k = a.aux_k; P.aux_v = a.aux_v;
  P.key_scale = a.key_scale; P.value_scale = a.value_scale; P.cu = a.cu; P.seqlens_k = a.seqlens_k;
  P.sel_idx = a.sel_idx; P.sel_count = a.sel_count; P.sinks = a.sinks; P.out = a.out;
  P.status = a.status;
  P.cd.block_table = a.block_table;
  P.cd.max_blocks = a.max_blocks;
  P.cd.block_size = a.block_size;
  P.cd.bs_shift = (a.block_size & (a.block_size - 1)) == 0 ? __builtin_ctz(a.block_size) : -1;
  P.cd.num_blocks = a.num_blocks;
  P.cd.H_kv = a.H_kv;
  P.cd.D = a.D;
  P.B = a.B; P.T = a.T; P.H_q = a.H_q; P.H_kv = a.H_kv; P.D = a.D;
  P.group = a.H_q / a.H_kv;
  P.head_tiles = plan.head_tiles;
  P.max_q = a.max_q; P.max_k = a.max_k; P.max_sel = a.max_selected; P.window = a.window;
  P.aux_len = a.aux_len;
  P.aux_row_stride = a.aux_stride / a.D;
  P.chunk = plan.chunk; P.n_main = plan.n_main; P.n_splits = plan.n_splits;
  P.row_slots = split_row_slots(a.kind, plan.chunk, a.block_table != nullptr, a.block_size);
  // the deal of splits to CUs (paged ranges and selected rows): one head tile, 8 XCDs of
  // 32 CUs shared evenly by the KV heads, every split of a head ranked by one thread.
  // Measured on the decode workload: f16 call 71.2 -> 62.7 us, INT8 cache 42.4 -> 40.1,
  // FP8 unchanged; selected grouped decode 80.2 -> 63.9 us.
  P.cu_slots = 0;
  if ((a.kind == SPATTN_KIND_PAGED || a.kind == SPATTN_KIND_SELECTED) && a.dtype != SPATTN_F32 &&
      plan.head_tiles == 1 && 8 % a.H_kv == 0 && (long)plan.n_splits * a.T <= kThreads)
    P.cu_slots = 32 * (8 / a.H_kv);
  P.meta_lds = a.B + 1 <= kMetaLdsMax ? 1 : 0;
  P.scale_log2 = a.scale * kLog2e;
  P.past = a.past; P.k_new = a.k_new; P.v_new = a.v_new; P.committed = a.committed;
  P.seqlens_q_out = a.seqlens_q_out; P.seqlens_k_out = a.seqlens_k_out;
  const bool direct = plan.n_splits == 1;
  P.ws_acc = nullptr; P.ws_ml = nullptr;
  if (!direct) {
    const size_t acc = align256((size_t)plan.n_splits * a.T * a.H_q * a.D * sizeof(float));
    const size_t ml = align256((size_t)plan.n_splits * a.T * a.H_q * sizeof(float2));
    char* ws = reinterpret_cast<char*>(a.workspace);
    P.ws_acc = reinterpret_cast<float*>(ws);
    P.ws_ml = reinterpret_cast<float2*>(ws + acc);
  }
  switch (a.kind) {
    case SPATTN_KIND_PAGED: dispatch_q<SPATTN_KIND_PAGED>(a, P, direct, stream); break;
    case SPATTN_KIND_SELECTED: dispatch_q<SPATTN_KIND_SELECTED>(a, P, direct, stream); break;
    default: dispatch_q<SPATTN_KIND_LOCAL_AUX>(a, P, direct, stream); break;
  }
  if (hipGetLastError() != hipSuccess) return SPATTN_ERR_LAUNCH;
  if (!direct) {
    const int pairs = a.T * a.H_q;
    dim3 grid((pairs + 3) / 4);
#define SPATTN_MERGE_B(QT, DD, NB)                                                           \
  hipLaunchKernelGGL((merge_kernel<QT, DD, NB>), grid, dim3(256), 0, stream, P.ws_acc,       \
                     P.ws_ml, a.sinks, a.out, a.T, a.H_q, plan.n_splits)
#define SPATTN_MERGE(QT, DD)                                                                 \
  do {                                                                                       \
    if (plan.n_splits <= 2) SPATTN_MERGE_B(QT, DD, 2);                                       \
    else if (plan.n_splits <= 4) SPATTN_MERGE_B(QT, DD, 4);                                  \
    else if (plan.n_splits <= 8) SPATTN_MERGE_B(QT, DD, 8);                                  \
    else SPATTN_MERGE_B(QT, DD, 16);                                                         \
  } while (0)
    if (a.D == 64) {
      if (a.dtype == SPATTN_F32) SPATTN_MERGE(float, 64);
      else if (a.dtype == SPATTN_F16) SPATTN_MERGE(f16, 64);
      else SPATTN_MERGE(bf16, 64);
    } else {
      if (a.dtype == SPATTN_F32) SPATTN_MERGE(float, 128);
      else if (a.dtype == SPATTN_F16) SPATTN_MERGE(f16, 128);
      else SPATTN_MERGE(bf16, 128);
    }
#undef SPATTN_MERGE
#undef SPATTN_MERGE_B
    if (hipGetLastError() != hipSuccess) return SPATTN_ERR_LAUNCH;
  }
  return SPATTN_OK;
}

}  // namespace spattn
