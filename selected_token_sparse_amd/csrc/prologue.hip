// qkv_prologue: the step before attention, fused with the cache append.
// ("[WebGPU] Add DynamicSparseAttention", Description: packed and unpacked QKV, QK RMSNorm,
// partial and interleaved RoPE, rotary offsets and explicit position IDs, with a review
// comment that a head's RMS is to be reduced once per (token, head), not once per channel;
// "[WebGPU] Add SparsePagedAttention", overview: the PagedAttention prologue of packed-QKV
// split, RoPE and block-table scatter.)
//
// The work is the flat list of (token, head) rows of the packed layout: per token the
// query heads, then the key heads, then the value heads.  A group of G = D/8 lanes owns one
// row, each lane 8 consecutive channels (one 16-byte load and store for 16-bit types), so
// a wave covers 64/G rows (8 at D = 64) and consecutive rows of a token share a wave.  The
// head's sum of squares is reduced within the group (an xor butterfly when G is a power of
// two, else a sum over the group's partials in LDS); the rotation reads each channel's
// partner from the wave's LDS copy of its rows.  Query rows go to q_out; key rows (rounded
// to the activation type) and value rows go to their cache slot with the same store or
// quantisation, cursor check and status bits as kv_cache_append.
#include "common.h"
#include "launch.h"
#include "prologue.h"

namespace spattn {

constexpr int kProWaves = 4;
constexpr int kProThreads = kProWaves * 64;
constexpr int kProDeepMinBlocks = 1024;   // workgroups a 2-batch launch must still have

struct PrologueParams {
  const void* qkv;          // packed rows, or nullptr
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cu;
  const int32_t* seqlens_k;
  int B, T, H_q, H_kv, D;
  int qk_norm;
  const float* q_norm_weight;
  const float* k_norm_weight;
  float norm_eps;
  int rotary_dim;
  int interleaved;
  const float* cos_table;
  const float* sin_table;
  int max_position;
  const int32_t* position_ids;
  const int32_t* rotary_offsets;
  void* q_out;
  void* k_cache;
  void* v_cache;
  CacheDesc cd;
  const float* key_scale;
  const float* value_scale;
  const int32_t* committed;
  int32_t* status;
  int G;                    // lanes per row (D / 8)
  int rows_per_wave;        // 64 / G
  int64_t n_rows;           // T * (H_q + 2 H_kv)
};

__device__ __forceinline__ int8_t pro_quantize_i8(float x, float s) {
  float r = __builtin_rintf(x / s);  // IEEE float32 division, ties to even
  if (r != r) return 0;
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int8_t)(int)r;
}

// eight consecutive elements <-> float
template <typename T> __device__ __forceinline__ void load8(const T* p, float (&x)[8]) {
  const i32x4 r = load16(p);
  const T* e = reinterpret_cast<const T*>(&r);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = to_f32(e[i]);
}
template <> __device__ __forceinline__ void load8<float>(const float* p, float (&x)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
}
// the same, split into the load and the conversion, so that the loads can stay in flight
// across the metadata lookups (a conversion right after a load waits for it)
struct Raw8 { i32x4 a, b; };
template <typename T> __device__ __forceinline__ Raw8 load_raw8(const T* p) {
  Raw8 r;
  r.a = load16(p);
  r.b = sizeof(T) == 4 ? load16(p + 16 / sizeof(T)) : i32x4{0, 0, 0, 0};
  return r;
}
template <typename T> __device__ __forceinline__ void convert8(const Raw8& r, float (&x)[8]) {
  if constexpr (sizeof(T) == 4) {
    const f32x4 a = __builtin_bit_cast(f32x4, r.a), b = __builtin_bit_cast(f32x4, r.b);
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
  } else {
    const T* e = reinterpret_cast<const T*>(&r.a);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = to_f32(e[i]);
  }
}
template <typename T> __device__ __forceinline__ void store8(T* p, const float (&x)[8]) {
  i32x4 r;
  T* e = reinterpret_cast<T*>(&r);
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = from_f32<T>(x[i]);
  store16(p, r);
}
template <> __device__ __forceinline__ void store8<float>(float* p, const float (&x)[8]) {
  *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}

// Per-row state between the phases of the kernel.
struct ProRow {
  int t, task, kind, head, pos;
  bool active, compute, append_ok;
  int64_t dst;
};

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// kQuant: 0 = float cache (stores T), 1 = INT8 codes, 2 = FP8 E4M3 codes.  ITER: row
// batches per wave (all their loads are issued before the metadata).  A wave's rows are
// consecutive, so they span few tokens (at most 64, which the host guarantees): lane j
// resolves the request, positions, cursor and cache slot of the wave's j-th token once,
// and each row reads its token's entry by a lane shuffle.
template <typename T, int kQuant, int ITER>
__global__ __launch_bounds__(kProThreads) void qkv_prologue_kernel(PrologueParams P) {
  __shared__ float rowbuf[kProWaves][64 * 8];   // each lane's 8 channels, row after row
  __shared__ float partial[kProWaves][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // (uniform: scalar)
  const int G = P.G;
  const int gi = lane / G;                      // row slot of this lane in a batch
  const int li = lane - gi * G;                 // lane within the row's group
  const int d0 = 8 * li;                        // first channel of this lane
  const int D = P.D;
  const int NH = P.H_q + 2 * P.H_kv;
  const bool slot_ok = gi < P.rows_per_wave;
  const int64_t r0 = ((int64_t)blockIdx.x * kProWaves + wave) * ITER * P.rows_per_wave;
  if (r0 >= P.n_rows) return;                   // the whole wave is past the end
  const int t_first = (int)(r0 / NH);
  const int base = (int)(r0 - (int64_t)t_first * NH);   // r0's head index in its token

  // phase 1: which rows, and their source loads (independent of any metadata)
  // (every lane loads: an inactive lane reads the wave's first row, so no register is
  // cleared while a load is in flight; the loaded bits are converted after the metadata)
  ProRow R[ITER];
  Raw8 raw[ITER];
  float x[ITER][8];
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    ProRow& r = R[it];
    const int k = it * P.rows_per_wave + gi;    // row of the wave
    const int tok = (base + k) / NH;            // token of the wave (0, 1, ...)
    r.t = t_first + tok;
    r.task = base + k - tok * NH;
    r.active = slot_ok && r0 + k < P.n_rows;
    r.kind = r.task < P.H_q ? 0 : (r.task < P.H_q + P.H_kv ? 1 : 2);   // Q, K, V
    r.head = r.kind == 0 ? r.task : (r.kind == 1 ? r.task - P.H_q : r.task - P.H_q - P.H_kv);
    const T* src;
    if (!r.active) src = reinterpret_cast<const T*>(P.qkv != nullptr ? P.qkv : P.q) + (P.qkv != nullptr ? r0 * D : 0);
    else if (P.qkv != nullptr) src = reinterpret_cast<const T*>(P.qkv) + (r0 + k) * D;
    else if (r.kind == 0) src = reinterpret_cast<const T*>(P.q) + ((int64_t)r.t * P.H_q + r.head) * D;
    else src = reinterpret_cast<const T*>(r.kind == 1 ? P.k : P.v) + ((int64_t)r.t * P.H_kv + r.head) * D;
    raw[it] = load_raw8<T>(src + d0);
  }
  // the norm weight of each row's kind depends on no metadata: it loads with the rows
  const float* w_any = P.q_norm_weight != nullptr ? P.q_norm_weight : P.k_norm_weight;
  const bool pre_w = P.qk_norm && w_any != nullptr;
  Raw8 wraw[ITER];
  if (pre_w) {
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const float* w = R[it].kind == 0 ? P.q_norm_weight : P.k_norm_weight;
      wraw[it] = load_raw8<float>((w != nullptr ? w : w_any) + d0);
    }
  }

  // phase 2: token metadata, lane j for the wave's token j
  int m_state = 0, m_pos = 0;                   // state: 1 = queries computed, 2 = K/V appended
  int64_t m_dst = -1;
  {
    const int last = (int)((min(r0 + (int64_t)ITER * P.rows_per_wave, P.n_rows) - 1) / NH);
    const int tj = t_first + lane;
    // The request of the wave's first and of its last token, by a binary search with
    // scalar loads (the metadata is read-only here, and waiting for a scalar load never
    // waits for the row loads in flight).  When both give request b, every token between
    // them does too: the search for each of them takes the same comparisons (whatever the
    // order of cu), so the request's lengths, offset and cursor are read once, by scalar
    // loads, instead of by a chain of vector loads per lane.
    typedef const __attribute__((address_space(4))) int32_t* CI;
    const CI ccu = (CI)P.cu;
    auto find_uniform = [&](int r) {
      int lo = 0, hi = P.B - 1;
      if (P.B <= 0 || ccu[0] > r) return -1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (ccu[mid] <= r) lo = mid; else hi = mid - 1;
      }
      return r < ccu[lo + 1] ? lo : -1;
    };
    const int b_first = find_uniform(t_first);
    const bool one_request = b_first >= 0 && find_uniform(last) == b_first;
    int ub_c0 = 0, ub_qlen = 0, ub_kvlen = 0, ub_off = 0;
    bool ub_cursor_bad = false;
    if (one_request) {
      ub_c0 = ccu[b_first];
      ub_qlen = ccu[b_first + 1] - ub_c0;
      ub_kvlen = ((CI)P.seqlens_k)[b_first] + 1;
      ub_off = P.rotary_offsets != nullptr ? ((CI)P.rotary_offsets)[b_first] : 0;
      ub_cursor_bad = P.committed != nullptr && ((CI)P.committed)[b_first] != ub_kvlen - ub_qlen;
    }
    if (tj <= last && one_request) {
      int flags = 0;
      const int b = b_first;
      const int q_len = ub_qlen;
      const int kv_len = ub_kvlen;
      const int p = kv_len - q_len + (tj - ub_c0);
      bool pos_ok = true;
      if (P.rotary_dim > 0) {
        m_pos = (P.position_ids != nullptr ? P.position_ids[tj] : p) + ub_off;
        if (m_pos < 0 || m_pos >= P.max_position) { pos_ok = false; flags |= SPATTN_STATUS_POSITION; }
      }
      if (pos_ok) m_state |= 1;
      if (ub_cursor_bad) flags |= SPATTN_STATUS_CURSOR;
      else if (!pos_ok) {}
      else if (p < 0) flags |= SPATTN_STATUS_SHORT_KV;
      else m_dst = cache_row(P.cd, b, p, 0, flags);
      if (m_dst >= 0) m_state |= 2;
      raise_status(P.status, flags);           // a token split over two waves reports twice
    } else if (tj <= last) {
      int flags = 0;
      const int b = find_request(P.cu, P.B, tj);
      if (b < 0) {
        flags |= SPATTN_STATUS_BAD_CU;
      } else {
        const int q_len = P.cu[b + 1] - P.cu[b];
        const int kv_len = P.seqlens_k[b] + 1;
        const int p = kv_len - q_len + (tj - P.cu[b]);
        bool pos_ok = true;
        if (P.rotary_dim > 0) {
          m_pos = (P.position_ids != nullptr ? P.position_ids[tj] : p) +
                  (P.rotary_offsets != nullptr ? P.rotary_offsets[b] : 0);
          if (m_pos < 0 || m_pos >= P.max_position) { pos_ok = false; flags |= SPATTN_STATUS_POSITION; }
        }
        if (pos_ok) m_state |= 1;
        // the cursor check is per request, whatever the row's position; a row without a
        // rotary position is then skipped with no further check
        if (P.committed != nullptr && P.committed[b] != kv_len - q_len) flags |= SPATTN_STATUS_CURSOR;
        else if (!pos_ok) {}
        else if (p < 0) flags |= SPATTN_STATUS_SHORT_KV;
        else m_dst = cache_row(P.cd, b, p, 0, flags);
        if (m_dst >= 0) m_state |= 2;
      }
      raise_status(P.status, flags);           // a token split over two waves reports twice
    }
  }
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    ProRow& r = R[it];
    const int src_lane = r.t - t_first;
    const int st = __shfl(m_state, src_lane, 64);
    r.pos = __shfl(m_pos, src_lane, 64);
    const int lo = __shfl((int)(uint32_t)(m_dst & 0xFFFFFFFF), src_lane, 64);
    const int hi = __shfl((int)(m_dst >> 32), src_lane, 64);
    r.dst = (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
    r.append_ok = r.active && r.kind != 0 && (st & 2) != 0;
    r.compute = r.active && (r.kind == 0 ? (st & 1) != 0 : r.append_ok);
    convert8<T>(raw[it], x[it]);
    if (!r.compute) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[it][e] = 0.f;   // rows of no request or position: zero queries
    }
  }

  // phase 3: norm, rotation, stores.  Every lane of the wave runs the reductions and the
  // LDS exchanges; rows that do not compute carry zeros and write nothing but zero queries.
  const int rd = P.rotary_dim;
  const int half = rd >> 1;
  const bool vec_tables = (half & 7) == 0;      // 8 (half layout) or 4 (interleaved) angles per lane
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const ProRow& r = R[it];
    float (&xv)[8] = x[it];
    if (P.qk_norm) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += xv[e] * xv[e];
      if ((G & (G - 1)) == 0) {
        for (int m = 1; m < G; m <<= 1) ss += __shfl_xor(ss, m, 64);
      } else {
        partial[wave][lane] = ss;
        wave_lds_sync();
        ss = 0.f;
        if (slot_ok)
          for (int j = 0; j < G; ++j) ss += partial[wave][gi * G + j];
        wave_lds_sync();   // partial[] is rewritten by the next batch
      }
      if (r.kind != 2 && r.compute) {
        const float inv = 1.0f / sqrtf(ss / (float)D + P.norm_eps);
        const float* w = r.kind == 0 ? P.q_norm_weight : P.k_norm_weight;
        if (w != nullptr) {
          float wv[8];
          convert8<float>(wraw[it], wv);
#pragma unroll
          for (int e = 0; e < 8; ++e) xv[e] = xv[e] * inv * wv[e];
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) xv[e] = xv[e] * inv;
        }
      }
    }
    if (rd > 0) {
      const bool rot = r.kind != 2 && r.compute && d0 < rd;
      const float* ct = P.cos_table + (int64_t)r.pos * half;
      const float* st = P.sin_table + (int64_t)r.pos * half;
      float y[8];
      if (P.interleaved && vec_tables) {
        // pairs (2i, 2i+1) sit inside the lane: angles d0/2 .. d0/2 + 3
        if (rot) {
          const f32x4 c4 = *reinterpret_cast<const f32x4*>(ct + (d0 >> 1));
          const f32x4 s4 = *reinterpret_cast<const f32x4*>(st + (d0 >> 1));
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float a = xv[2 * i], b = xv[2 * i + 1];
            xv[2 * i] = a * c4[i] - b * s4[i];
            xv[2 * i + 1] = b * c4[i] + a * s4[i];
          }
        }
      } else {
        float* rb = rowbuf[wave];
#pragma unroll
        for (int e = 0; e < 8; ++e) rb[8 * lane + e] = xv[e];
        wave_lds_sync();
        if (rot) {
          const float* myrow = rb + gi * D;     // this row's channels in LDS
          if (!P.interleaved && vec_tables) {
            // half layout, 8 consecutive angles and partners per lane
            const bool first = d0 < half;
            const int i0 = first ? d0 : d0 - half;
            const int p0 = first ? d0 + half : d0 - half;
            float c[8], sn[8], o[8];
            load8<float>(ct + i0, c);
            load8<float>(st + i0, sn);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = myrow[p0 + e];
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = first ? xv[e] * c[e] - o[e] * sn[e] : xv[e] * c[e] + o[e] * sn[e];
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int d = d0 + e;
              y[e] = xv[e];
              if (d < rd) {
                int i, partner;
                bool first;
                if (P.interleaved) { i = d >> 1; partner = d ^ 1; first = (d & 1) == 0; }
                else { first = d < half; i = first ? d : d - half; partner = first ? d + half : d - half; }
                const float cc = ct[i], ss2 = st[i];
                const float o = myrow[partner];
                y[e] = first ? xv[e] * cc - o * ss2 : xv[e] * cc + o * ss2;
              }
            }
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) xv[e] = y[e];
        }
        wave_lds_sync();   // rowbuf is rewritten by the next batch
      }
    }
    if (!r.active) continue;
    if (r.kind == 0) {
      T* dq = reinterpret_cast<T*>(P.q_out) + ((int64_t)r.t * P.H_q + r.head) * D + d0;
      store8<T>(dq, xv);
      continue;
    }
    if (!r.append_ok) continue;
    // key or value row into its slot (the key rounded to the activation type first)
    const int64_t off = r.dst + (int64_t)r.head * P.cd.block_size * D + d0;
    if constexpr (kQuant == 0) {
      store8<T>(reinterpret_cast<T*>(r.kind == 1 ? P.k_cache : P.v_cache) + off, xv);
    } else {
      const float* sc = (r.kind == 1 ? P.key_scale : P.value_scale) + r.head * D + d0;
      float sv[8];
      load8<float>(sc, sv);
      union { int8_t c[8]; int2 v; } u;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float q = to_f32(from_f32<T>(xv[e]));
        if constexpr (kQuant == 1) u.c[e] = pro_quantize_i8(q, sv[e]);
        else u.c[e] = (int8_t)quantize_fp8(q, sv[e]);
      }
      *reinterpret_cast<int2*>(reinterpret_cast<int8_t*>(r.kind == 1 ? P.k_cache : P.v_cache) + off) = u.v;
    }
  }
}

int launch_qkv_prologue(const PrologueArgs& a, hipStream_t stream) {
  if (a.T == 0) return SPATTN_OK;
  PrologueParams P{};
  P.qkv = a.qkv; P.q = a.q; P.k = a.k; P.v = a.v;
  P.cu = a.cu; P.seqlens_k = a.seqlens_k;
  P.B = a.B; P.T = a.T; P.H_q = a.H_q; P.H_kv = a.H_kv; P.D = a.D;
  P.qk_norm = a.qk_norm; P.q_norm_weight = a.q_norm_weight; P.k_norm_weight = a.k_norm_weight;
  P.norm_eps = a.norm_eps;
  P.rotary_dim = a.rotary_dim; P.interleaved = a.interleaved;
  P.cos_table = a.cos_table; P.sin_table = a.sin_table; P.max_position = a.max_position;
  P.position_ids = a.position_ids; P.rotary_offsets = a.rotary_offsets;
  P.q_out = a.q_out; P.k_cache = a.k_cache; P.v_cache = a.v_cache;
  P.cd.block_table = a.block_table;
  P.cd.max_blocks = a.max_blocks;
  P.cd.block_size = a.block_size;
  P.cd.bs_shift = (a.block_size & (a.block_size - 1)) == 0 ? __builtin_ctz(a.block_size) : -1;
  P.cd.num_blocks = a.num_blocks;
  P.cd.H_kv = a.H_kv;
  P.cd.D = a.D;
  P.key_scale = a.key_scale; P.value_scale = a.value_scale;
  P.committed = a.committed; P.status = a.status;
  P.G = a.D / 8;
  P.rows_per_wave = 64 / P.G;
  P.n_rows = (int64_t)a.T * (a.H_q + 2 * a.H_kv);
  // two row batches per wave once there are enough rows to fill the chip that way (more
  // bytes in flight per wave; measured at 5120 rows: 1 batch 49.6 us, 2 batches 42.8,
  // 4 batches 51.8, 8 batches 61.7, as registers cut occupancy); one batch otherwise
  const int64_t rows_one = (int64_t)kProWaves * P.rows_per_wave;
  // (the tokens a wave spans must fit its 64 lanes: 2 * rows_per_wave rows span at most
  // (2 * rows_per_wave - 1) / NH + 2 tokens)
  const int NH = a.H_q + 2 * a.H_kv;
  const bool deep = P.n_rows >= (int64_t)kProDeepMinBlocks * 2 * rows_one &&
                    (2 * P.rows_per_wave - 1) / NH + 2 <= 64;
  const int64_t rows_per_block = rows_one * (deep ? 2 : 1);
  const int64_t blocks = (P.n_rows + rows_per_block - 1) / rows_per_block;
  if (blocks > 0x7FFFFFFF) return SPATTN_ERR_SHAPE;
  dim3 grid((unsigned)blocks), block(kProThreads);
  const int quant = a.cache_dtype == SPATTN_I8 ? 1 : (a.cache_dtype == SPATTN_FP8 ? 2 : 0);
#define SPATTN_PROLOGUE(TT, Q)                                                                \
  if (deep) hipLaunchKernelGGL((qkv_prologue_kernel<TT, Q, 2>), grid, block, 0, stream, P);  \
  else hipLaunchKernelGGL((qkv_prologue_kernel<TT, Q, 1>), grid, block, 0, stream, P)
#define SPATTN_PROLOGUE_Q(TT)                   \
  if (quant == 1) { SPATTN_PROLOGUE(TT, 1); }   \
  else if (quant == 2) { SPATTN_PROLOGUE(TT, 2); } \
  else { SPATTN_PROLOGUE(TT, 0); }
  switch (a.dtype) {
    case SPATTN_F32: SPATTN_PROLOGUE_Q(float); break;
    case SPATTN_F16: SPATTN_PROLOGUE_Q(f16); break;
    case SPATTN_BF16: SPATTN_PROLOGUE_Q(bf16); break;
    default: return SPATTN_ERR_DTYPE;
  }
#undef SPATTN_PROLOGUE_Q
#undef SPATTN_PROLOGUE
  return hipGetLastError() == hipSuccess ? SPATTN_OK : SPATTN_ERR_LAUNCH;
}

}  // namespace spattn
