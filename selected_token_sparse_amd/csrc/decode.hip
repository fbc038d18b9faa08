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
//  1. the row's request and key position are resolved from cu_seqlens_q / seqlens_k;
//  2. the split's keys are turned into cache-row indices in LDS (one pass, guarded);
//  3. each wave takes 32-key tiles: S^T = K Q^T with v_mfma_f32_16x16x32 (K rows loaded
//     straight into the A operand with 16-byte loads), an online softmax in the log2
//     domain, then O^T += V^T P^T where V^T comes from LDS through ds_read_b64_tr_b16;
//  4. the four wave states are merged in LDS and written either as a partial (m, l, acc)
//     for the merge kernel or, with a single split, as the final normalised output.
//
// INT8 caches: key_scale is folded into the query operand (f16), value_scale is applied
// to the accumulator before it leaves the workgroup.
#include "common.h"
#include "launch.h"

namespace spattn {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kTile = 32;          // keys per wave iteration
constexpr int kWgStep = kWaves * kTile;
constexpr int kMaxChunk = 2048;    // keys per split (LDS row-index buffer)
constexpr int kTargetWorkgroups = 4096;

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

// 8 cache elements at `p` as an MFMA operand of type OpT (int8 codes convert exactly).
template <typename OpT, typename KT>
__device__ __forceinline__ typename OpVec<OpT>::v8 load_op8(const KT* p) {
  typedef typename OpVec<OpT>::v8 V8;
  if constexpr (sizeof(KT) == 2) {
    i32x4 raw = load16(p);
    return __builtin_bit_cast(V8, raw);
  } else {
    int2 raw = *reinterpret_cast<const int2*>(p);
    const int8_t* c = reinterpret_cast<const int8_t*>(&raw);
    V8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (OpT)(float)c[e];
    return v;
  }
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
  float scale_log2;         // scale * log2(e)
};

__device__ __forceinline__ void flush_flags(int flags, int32_t* status) {
  // OR the per-lane flags across the wave, then one atomic per wave and only when the
  // bits are not set yet.
  int wave_flags = 0;
#pragma unroll
  for (int bit = 0; bit < 8; ++bit)
    if (__ballot(flags & (1 << bit))) wave_flags |= 1 << bit;
  if (wave_flags && (threadIdx.x & 63) == 0 && status != nullptr) {
    int cur = __atomic_load_n(status, __ATOMIC_RELAXED);
    if ((cur & wave_flags) != wave_flags) atomicOr(status, wave_flags);
  }
}

// LDS layout (bytes): row indices of the split's keys, then per-wave V tiles (reused as
// the combine area after the key loop).
template <int D>
struct SplitLds {
  static constexpr int kVld = D + 16;                       // padded V tile row (elements)
  static constexpr int kVTileBytes = kTile * kVld * 2;
  static constexpr int kCombineBytes = kWaves * 16 * (D + 2) * 4;
  static constexpr int kAreaBytes = (kWaves * kVTileBytes > kCombineBytes) ? kWaves * kVTileBytes : kCombineBytes;
  static constexpr int kRowsBytes = kMaxChunk * 4;
  static constexpr int kTotal = kRowsBytes + kAreaBytes;
};

// The key loop of one wave over one source.  `rows` holds the cache-row index (row of D
// elements counted from kbase / vbase) of each key of the split, or -1.
template <typename OpT, typename KT, int D>
__device__ __forceinline__ void wave_keys(const KT* __restrict__ kbase, const KT* __restrict__ vbase,
                                          const int32_t* rows, int n_keys,
                                          const typename OpVec<OpT>::v8 (&qop)[D / 32],
                                          float scale_log2, OpT* vtile, float& m_run,
                                          float& l_run, f32x4 (&acc)[D / 16]) {
  typedef typename OpVec<OpT>::v8 V8;
  constexpr int KC = D / 32;
  constexpr int MT = D / 16;
  constexpr int VLD = SplitLds<D>::kVld;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lam = lane & 15;
  const int grp = lane >> 4;
  const int n_tiles = (n_keys + kTile - 1) / kTile;
  for (int tile = wave; tile < n_tiles; tile += kWaves) {
    const int base = tile * kTile;
    int row0 = (base + lam < n_keys) ? rows[base + lam] : -1;
    int row1 = (base + 16 + lam < n_keys) ? rows[base + 16 + lam] : -1;
    V8 kop[2][KC];
    V8 vop[2][KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int col = kc * 32 + grp * 8;
      V8 z = {};
      kop[0][kc] = row0 >= 0 ? load_op8<OpT>(kbase + (int64_t)row0 * D + col) : z;
      kop[1][kc] = row1 >= 0 ? load_op8<OpT>(kbase + (int64_t)row1 * D + col) : z;
      vop[0][kc] = row0 >= 0 ? load_op8<OpT>(vbase + (int64_t)row0 * D + col) : z;
      vop[1][kc] = row1 >= 0 ? load_op8<OpT>(vbase + (int64_t)row1 * D + col) : z;
    }
    const uint64_t b0 = __ballot(row0 >= 0);
    const uint64_t b1 = __ballot(row1 >= 0);
    const uint32_t valid = (uint32_t)(b0 & 0xFFFFu) | ((uint32_t)(b1 & 0xFFFFu) << 16);

    // S^T[key][head] for keys 16*st + 4*grp + i, head lam
    f32x4 s[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) c = mfma16(kop[st][kc], qop[kc], c);
      s[st] = c;
    }
    float mt = kNegInf;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * st + 4 * grp + i;
        float v = ((valid >> key) & 1u) ? s[st][i] * scale_log2 : kNegInf;
        s[st][i] = v;
        mt = fmaxf(mt, v);
      }
    mt = xor_max(mt, 16);
    mt = xor_max(mt, 32);
    const float m_new = fmaxf(m_run, mt);

    // V tile -> LDS (row-major, padded), read back transposed below
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        *reinterpret_cast<V8*>(vtile + (16 * st + lam) * VLD + kc * 32 + grp * 8) = vop[st][kc];

    // Every lane runs the update and the MFMAs (they read operands of all 64 lanes); a
    // head with no visible key so far keeps m = -inf, l = 0, acc = 0.
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    {
      const float alpha = exp2_safe(m_run - m_use);
      float psum = 0.f;
      V8 pop;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = exp2_safe(s[st][i] - m_use);
          psum += p;
          pop[st * 4 + i] = (OpT)p;
        }
      psum = xor_sum(psum, 16);
      psum = xor_sum(psum, 32);
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m] *= alpha;
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the V tile writes have landed
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        // lane (grp, lam) provides rows 4*grp + lam/4 (+16), columns 16*m + 4*(lam%4)
        const OpT* a0 = vtile + (4 * grp + (lam >> 2)) * VLD + 16 * m + 4 * (lam & 3);
        const OpT* a1 = a0 + 16 * VLD;
        s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(a0));
        s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(a1));
        typename OpVec<OpT>::v4 h0 = __builtin_bit_cast(typename OpVec<OpT>::v4, r0);
        typename OpVec<OpT>::v4 h1 = __builtin_bit_cast(typename OpVec<OpT>::v4, r1);
        V8 aop = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
        acc[m] = mfma16(aop, pop, acc[m]);
      }
    }
  }
}

// Cache-row index of key v of the split (or -1), for each source.
__device__ __forceinline__ int key_row_range(const SplitParams& P, int b, int c, int lo, int v,
                                             int& flags) {
  const int64_t off = cache_row(P.cd, b, lo + v, c, flags);
  return off < 0 ? -1 : (int)(off / P.D);
}

template <int KIND, typename QT, typename KT, typename AT, int D, bool DIRECT>
__global__ __launch_bounds__(kThreads) void split_attn_kernel(SplitParams P) {
  typedef typename std::conditional<sizeof(KT) == 1, f16, KT>::type OpM;  // main operand
  typedef QT OpA;                                                          // aux operand
  extern __shared__ __align__(16) unsigned char smem[];
  int32_t* rows = reinterpret_cast<int32_t*>(smem);
  unsigned char* area = smem + SplitLds<D>::kRowsBytes;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lam = lane & 15;
  const int grp = lane >> 4;

  const int hkt = P.H_kv * P.head_tiles;
  const int per_split = P.T * hkt;
  const int split = blockIdx.x / per_split;
  const int rem = blockIdx.x - split * per_split;
  const int r = rem / hkt;
  const int kvt = rem - r * hkt;
  const int c = kvt / P.head_tiles;
  const int ht = kvt - c * P.head_tiles;
  const int h0 = c * P.group + ht * 16;                 // first query head of the tile
  const int nh = min(16, P.group - ht * 16);            // heads in the tile

  int flags = 0;
  RowInfo ri = resolve_row(P.cu, P.seqlens_k, P.B, r, P.max_q, P.max_k, flags);

  // ---- the split's source and key range ----
  int src = SRC_RANGE, v0 = 0, v1 = 0, lo = 0, cnt = 0;
  const int32_t* sel = nullptr;
  if (ri.b >= 0) {
    int s = split;
    if (KIND == SPATTN_KIND_LOCAL_AUX && split >= P.n_main) { src = SRC_AUX; s = split - P.n_main; }
    else if (KIND == SPATTN_KIND_SELECTED) src = SRC_SELECT;
    if (src == SRC_RANGE) {
      lo = P.window > 0 ? max(0, ri.p - P.window + 1) : 0;
      cnt = ri.p - lo + 1;
    } else {
      sel = P.sel_idx + ((int64_t)r * P.H_kv + c) * P.max_sel;
      if (P.sel_count != nullptr) {
        cnt = P.sel_count[(int64_t)r * P.H_kv + c];
        if (cnt < 0 || cnt > P.max_sel) flags |= SPATTN_STATUS_BAD_COUNT;
        cnt = min(max(cnt, 0), P.max_sel);
      } else {
        cnt = P.max_sel;
      }
    }
    v0 = s * P.chunk;
    v1 = min(v0 + P.chunk, cnt);
  }
  const int n_keys = max(0, v1 - v0);

  // ---- key -> cache-row indices (guarded) ----
  for (int v = tid; v < n_keys; v += kThreads) {
    int row = -1;
    if (src == SRC_RANGE) {
      row = key_row_range(P, ri.b, c, lo, v0 + v, flags);
    } else {
      const int j = sel[v0 + v];
      if (src == SRC_SELECT) {
        if (j != -1 && (j < 0 || j >= ri.kv_len)) flags |= SPATTN_STATUS_BAD_INDEX;
        else if (j >= 0 && j <= ri.p) {
          const int64_t off = cache_row(P.cd, ri.b, j, c, flags);
          row = off < 0 ? -1 : (int)(off / P.D);
        }
      } else {
        if (j != -1 && (j < 0 || j >= P.aux_len)) flags |= SPATTN_STATUS_BAD_INDEX;
        else if (j >= 0) row = (int)(ri.b * P.aux_row_stride + (int64_t)j * P.H_kv + c);
      }
    }
    rows[v] = row;
  }
  flush_flags(flags, P.status);
  __syncthreads();

  // ---- per-wave key loop ----
  float m_run = kNegInf, l_run = 0.f;
  f32x4 acc[D / 16];
#pragma unroll
  for (int m = 0; m < D / 16; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bool use_scale = sizeof(KT) == 1 && src != SRC_AUX;
  if (n_keys > 0) {
    const int head = h0 + lam;
    const bool hv = lam < nh;
    if (src != SRC_AUX) {
      typename OpVec<OpM>::v8 qop[D / 32];
      const QT* qrow = reinterpret_cast<const QT*>(P.q) + ((int64_t)r * P.H_q + head) * D;
#pragma unroll
      for (int kc = 0; kc < D / 32; ++kc) {
        const int col = kc * 32 + grp * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float x = hv ? to_f32(qrow[col + e]) : 0.f;
          if (use_scale) x *= P.key_scale[c * D + col + e];
          qop[kc][e] = (OpM)x;
        }
      }
      const KT* kb = reinterpret_cast<const KT*>(P.k_cache);
      const KT* vb = reinterpret_cast<const KT*>(P.v_cache);
      wave_keys<OpM, KT, D>(kb, vb, rows, n_keys, qop, P.scale_log2,
                            reinterpret_cast<OpM*>(area + wave * SplitLds<D>::kVTileBytes),
                            m_run, l_run, acc);
    } else {
      typename OpVec<OpA>::v8 qop[D / 32];
      const QT* qrow = reinterpret_cast<const QT*>(P.q) + ((int64_t)r * P.H_q + head) * D;
#pragma unroll
      for (int kc = 0; kc < D / 32; ++kc) {
        const int col = kc * 32 + grp * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) qop[kc][e] = hv ? qrow[col + e] : (QT)0.f;
      }
      const AT* kb = reinterpret_cast<const AT*>(P.aux_k);
      const AT* vb = reinterpret_cast<const AT*>(P.aux_v);
      if constexpr (sizeof(AT) == 2)
        wave_keys<OpA, AT, D>(kb, vb, rows, n_keys, qop, P.scale_log2,
                              reinterpret_cast<OpA*>(area + wave * SplitLds<D>::kVTileBytes),
                              m_run, l_run, acc);
    }
  }
  __syncthreads();

  // ---- merge the four wave states (head lam, dims 16m + 4grp + i) ----
  float* cm = reinterpret_cast<float*>(area);              // [wave][16] m
  float* cl = cm + kWaves * 16;                           // [wave][16] l
  float* ca = cl + kWaves * 16;                           // [wave][16][D] acc
  if (grp == 0) { cm[wave * 16 + lam] = m_run; cl[wave * 16 + lam] = l_run; }
#pragma unroll
  for (int m = 0; m < D / 16; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) ca[(wave * 16 + lam) * D + 16 * m + 4 * grp + i] = acc[m][i];
  __syncthreads();

  for (int e = tid; e < 16 * D; e += kThreads) {
    const int h = e / D, d = e - h * D;
    if (h >= nh) continue;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, cm[w * 16 + h]);
    float L = 0.f, A = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = exp2_safe(cm[w * 16 + h] - M);
        L += cl[w * 16 + h] * f;
        A += ca[(w * 16 + h) * D + d] * f;
      }
      if (use_scale) A *= P.value_scale[c * D + d];
    }
    const int head = h0 + h;
    const int64_t o = ((int64_t)r * P.H_q + head) * D + d;
    if constexpr (DIRECT) {
      float res = 0.f;
      if (M != kNegInf) {
        const float sg = P.sinks != nullptr ? P.sinks[head] * kLog2e : kNegInf;
        const float M2 = fmaxf(M, sg);
        const float f = exp2_safe(M - M2);
        res = A * f / (L * f + exp2_safe(sg - M2));
      }
      reinterpret_cast<QT*>(P.out)[o] = from_f32<QT>(res);
    } else {
      const int64_t so = (int64_t)split * P.T * P.H_q;
      P.ws_acc[so * D + o] = A;
      if (d == 0) P.ws_ml[so + (int64_t)r * P.H_q + head] = make_float2(M, L);
    }
  }
}

// ---------------------------------------------------------------------------------------
// Merge of split partial states plus the sink ("[WebGPU] Add SparsePagedAttention",
// finalize stage; one wave per (row, query head), merge coefficients shared across the
// head's output channels).
// ---------------------------------------------------------------------------------------
template <typename QT, int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ ws_acc,
                                                    const float2* __restrict__ ws_ml,
                                                    const float* __restrict__ sinks,
                                                    void* __restrict__ out, int T, int H_q,
                                                    int n_splits) {
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (pair >= T * H_q) return;
  const int head = pair % H_q;
  const int64_t stride = (int64_t)T * H_q;
  float M = kNegInf;
  for (int s = 0; s < n_splits; ++s) M = fmaxf(M, ws_ml[s * stride + pair].x);
  constexpr int PER = D / 64;
  float res[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) res[k] = 0.f;
  if (M != kNegInf) {
    const float sg = sinks != nullptr ? sinks[head] * kLog2e : kNegInf;
    const float M2 = fmaxf(M, sg);
    float L = exp2_safe(sg - M2);
    float A[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) A[k] = 0.f;
    for (int s = 0; s < n_splits; ++s) {
      const float2 ml = ws_ml[s * stride + pair];
      if (ml.x == kNegInf) continue;
      const float f = exp2_safe(ml.x - M2);
      L += ml.y * f;
      const float* a = ws_acc + (s * stride + pair) * D;
#pragma unroll
      for (int k = 0; k < PER; ++k) A[k] += a[lane + 64 * k] * f;
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) res[k] = A[k] / L;
  }
  QT* o = reinterpret_cast<QT*>(out) + (int64_t)pair * D;
#pragma unroll
  for (int k = 0; k < PER; ++k) o[lane + 64 * k] = from_f32<QT>(res[k]);
}

// ---------------------------------------------------------------------------------------
// float32 path (and any dtype with float32 queries): plain VALU arithmetic, one wave per
// (split, row, query head); same key lists, same partial format and merge.
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
  RowInfo ri = resolve_row(P.cu, P.seqlens_k, P.B, r, P.max_q, P.max_k, flags);
  int src = SRC_RANGE, v0 = 0, v1 = 0, lo = 0, cnt = 0;
  const int32_t* sel = nullptr;
  if (ri.b >= 0) {
    int s = split;
    if (KIND == SPATTN_KIND_LOCAL_AUX && split >= P.n_main) { src = SRC_AUX; s = split - P.n_main; }
    else if (KIND == SPATTN_KIND_SELECTED) src = SRC_SELECT;
    if (src == SRC_RANGE) {
      lo = P.window > 0 ? max(0, ri.p - P.window + 1) : 0;
      cnt = ri.p - lo + 1;
    } else {
      sel = P.sel_idx + ((int64_t)r * P.H_kv + c) * P.max_sel;
      if (P.sel_count != nullptr) {
        cnt = P.sel_count[(int64_t)r * P.H_kv + c];
        if (cnt < 0 || cnt > P.max_sel) flags |= SPATTN_STATUS_BAD_COUNT;
        cnt = min(max(cnt, 0), P.max_sel);
      } else {
        cnt = P.max_sel;
      }
    }
    v0 = s * P.chunk;
    v1 = min(v0 + P.chunk, cnt);
  }
  const int n_keys = max(0, v1 - v0);
  const bool is_i8 = sizeof(KT) == 1 && src != SRC_AUX;
  // the query (key_scale folded in for INT8 caches)
  constexpr int PER = D / 64;
  float qv[D];
  const float* q32 = reinterpret_cast<const float*>(P.q) + ((int64_t)r * P.H_q + head) * D;
  for (int d = 0; d < D; ++d) qv[d] = is_i8 ? q32[d] * P.key_scale[c * D + d] : q32[d];
  float m_run = kNegInf, l_run = 0.f, acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
  for (int base = 0; base < n_keys; base += 64) {
    const int v = base + lane;
    int row = -1;
    if (v < n_keys) {
      if (src == SRC_RANGE) {
        row = key_row_range(P, ri.b, c, lo, v0 + v, flags);
      } else {
        const int j = sel[v0 + v];
        if (src == SRC_SELECT) {
          if (j != -1 && (j < 0 || j >= ri.kv_len)) flags |= SPATTN_STATUS_BAD_INDEX;
          else if (j >= 0 && j <= ri.p) {
            const int64_t off = cache_row(P.cd, ri.b, j, c, flags);
            row = off < 0 ? -1 : (int)(off / P.D);
          }
        } else {
          if (j != -1 && (j < 0 || j >= P.aux_len)) flags |= SPATTN_STATUS_BAD_INDEX;
          else if (j >= 0) row = (int)(ri.b * P.aux_row_stride + (int64_t)j * P.H_kv + c);
        }
      }
    }
    float s = kNegInf;
    if (row >= 0) {
      float dot = 0.f;
      if (src == SRC_AUX) {
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
    rows[lane] = row;
    float p = 0.f;
    if (m_new != kNegInf) p = exp2_safe(s - m_new);
    pw[lane] = p;
    __syncthreads();
    if (m_new != kNegInf) {
      float ps = p;
      for (int o = 32; o >= 1; o >>= 1) ps += __shfl_xor(ps, o, 64);
      const float alpha = exp2_safe(m_run - m_new);
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
          if (src == SRC_AUX) x = to_f32(reinterpret_cast<const AT*>(P.aux_v)[(int64_t)rw * D + d]);
          else x = to_f32(reinterpret_cast<const KT*>(P.v_cache)[(int64_t)rw * D + d]);
          acc[k] += w * x;
        }
      }
    }
    __syncthreads();
  }
  flush_flags(flags, P.status);
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

SplitPlan make_split_plan(int kind, int dtype, int B, int T, int max_q, int max_k, int max_sel,
                          int window, int H_q, int H_kv, int D) {
  (void)B; (void)max_q;
  SplitPlan pl{};
  const int group = H_q / H_kv;
  pl.head_tiles = dtype == SPATTN_F32 ? 1 : (group + 15) / 16;
  long n_main = 0, n_aux = 0;
  if (kind == SPATTN_KIND_PAGED) n_main = window > 0 ? std::min(window, max_k) : max_k;
  else if (kind == SPATTN_KIND_SELECTED) n_main = max_sel;
  else { n_main = window; n_aux = max_sel; }
  n_main = std::max(0L, n_main);
  n_aux = std::max(0L, n_aux);
  const long items = (long)T * (dtype == SPATTN_F32 ? H_q : (long)H_kv * pl.head_tiles);
  const long total = n_main + n_aux;
  int chunk = kWgStep;
  auto splits_for = [&](int ch) {
    long s = (n_main + ch - 1) / ch + (n_aux + ch - 1) / ch;
    return std::max(1L, s);
  };
  while (chunk < kMaxChunk && chunk < total && items * splits_for(chunk) > kTargetWorkgroups) chunk *= 2;
  pl.chunk = chunk;
  pl.n_main = (int)std::max(1L, (n_main + chunk - 1) / chunk);
  pl.n_aux = (int)((n_aux + chunk - 1) / chunk);
  if (kind != SPATTN_KIND_LOCAL_AUX) pl.n_aux = 0;
  pl.n_splits = pl.n_main + pl.n_aux;
  pl.ws_bytes = 0;
  if (pl.n_splits > 1) {
    const size_t acc = (size_t)pl.n_splits * T * H_q * D * sizeof(float);
    const size_t ml = (size_t)pl.n_splits * T * H_q * sizeof(float2);
    pl.ws_bytes = ((acc + 255) / 256) * 256 + ((ml + 255) / 256) * 256;
  }
  return pl;
}

template <int KIND, typename QT, typename KT, typename AT, int D>
static void launch_split_typed(const SplitParams& P, bool direct, hipStream_t stream) {
  const int blocks = P.n_splits * P.T * P.H_kv * P.head_tiles;
  const size_t lds = SplitLds<D>::kTotal;
  if (direct)
    hipLaunchKernelGGL((split_attn_kernel<KIND, QT, KT, AT, D, true>), dim3(blocks), dim3(kThreads), lds, stream, P);
  else
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
static int dispatch_cache(const AttnArgs& a, const SplitParams& P, bool direct, hipStream_t stream) {
  const bool i8 = a.cache_dtype == SPATTN_I8;
  if constexpr (std::is_same<QT, float>::value) {
    if (i8) launch_split_f32<KIND, int8_t, float, D>(P, direct, stream);
    else launch_split_f32<KIND, float, float, D>(P, direct, stream);
  } else {
    if (i8) launch_split_typed<KIND, QT, int8_t, QT, D>(P, direct, stream);
    else launch_split_typed<KIND, QT, QT, QT, D>(P, direct, stream);
  }
  return SPATTN_OK;
}

template <int KIND>
static int dispatch_q(const AttnArgs& a, const SplitParams& P, bool direct, hipStream_t stream) {
  if (a.D == 64) {
    if (a.dtype == SPATTN_F32) return dispatch_cache<KIND, float, 64>(a, P, direct, stream);
    if (a.dtype == SPATTN_F16) return dispatch_cache<KIND, f16, 64>(a, P, direct, stream);
    return dispatch_cache<KIND, bf16, 64>(a, P, direct, stream);
  }
  if (a.dtype == SPATTN_F32) return dispatch_cache<KIND, float, 128>(a, P, direct, stream);
  if (a.dtype == SPATTN_F16) return dispatch_cache<KIND, f16, 128>(a, P, direct, stream);
  return dispatch_cache<KIND, bf16, 128>(a, P, direct, stream);
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
  P.scale_log2 = a.scale * kLog2e;
  const bool direct = plan.n_splits == 1;
  P.ws_acc = nullptr; P.ws_ml = nullptr;
  if (!direct) {
    const size_t acc = (size_t)plan.n_splits * a.T * a.H_q * a.D * sizeof(float);
    P.ws_acc = reinterpret_cast<float*>(a.workspace);
    P.ws_ml = reinterpret_cast<float2*>(reinterpret_cast<char*>(a.workspace) + ((acc + 255) / 256) * 256);
  }
  int rc;
  switch (a.kind) {
    case SPATTN_KIND_PAGED: rc = dispatch_q<SPATTN_KIND_PAGED>(a, P, direct, stream); break;
    case SPATTN_KIND_SELECTED: rc = dispatch_q<SPATTN_KIND_SELECTED>(a, P, direct, stream); break;
    default: rc = dispatch_q<SPATTN_KIND_LOCAL_AUX>(a, P, direct, stream); break;
  }
  if (rc != SPATTN_OK) return rc;
  if (hipGetLastError() != hipSuccess) return SPATTN_ERR_LAUNCH;
  if (!direct) {
    const int pairs = a.T * a.H_q;
    dim3 grid((pairs + 3) / 4);
#define SPATTN_MERGE(QT, DD)                                                              \
  hipLaunchKernelGGL((merge_kernel<QT, DD>), grid, dim3(256), 0, stream, P.ws_acc, P.ws_ml, \
                     a.sinks, a.out, a.T, a.H_q, plan.n_splits)
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
    if (hipGetLastError() != hipSuccess) return SPATTN_ERR_LAUNCH;
  }
  return SPATTN_OK;
}

}  // namespace spattn
