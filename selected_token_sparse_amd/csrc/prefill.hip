// MFMA prefill: causal paged attention for long query blocks, fp16/bf16 operands, fp32
// softmax and accumulation ("[WebGPU] Add PagedAttention metadata and GPT-OSS support":
// paged attention with local window and learned sink; review finding Q3: start the key
// loop at the tile holding the earliest window key of the workgroup's first row, so the
// traversal is about one window plus one query tile instead of the whole history).
//
// Workgroup = 4 waves = 32*RW query rows x HW query heads of one KV head (RW * HW = 4);
// every wave owns 32 rows of one head.  All waves share each 32-key K/V tile, staged
// through LDS (two stages, one barrier per tile).  Per wave and tile:
//   S^T[32 keys x 32 rows] = K Q^T      (v_mfma_f32_32x32x16, D/16 steps)
//   online softmax per row (a lane holds 16 keys of its row; one cross-lane exchange)
//   O^T[D x 32 rows] += V^T P^T         (V^T from LDS via ds_read_b64_tr_b16)
// Masks: key j is visible to the row at position p when lo(p) <= j <= p and its cache
// slot exists.  The sink joins the normaliser once at the end of the row.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace spattn {

constexpr int kPfThreads = 256;
constexpr int kPfTile = 32;

template <typename T> struct Op32;

// a + b + c in fp32 for two 16-bit values (v_dot2c_f32_{f16,bf16} against (1, 1))
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_ones(f16 a, f16 b, float c) {
  return __builtin_amdgcn_fdot2(f16x2{a, b}, f16x2{(f16)1.f, (f16)1.f}, c, false);
}
__device__ __forceinline__ float dot2_ones(bf16 a, bf16 b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(bf16x2{a, b}, bf16x2{(bf16)1.f, (bf16)1.f}, c, false);
}
template <> struct Op32<f16> { typedef f16x8 v8; typedef f16x4 v4; };
template <> struct Op32<bf16> { typedef bf16x8 v8; typedef bf16x4 v4; };

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

struct PrefillParams {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const float* key_scale;
  const float* value_scale;
  const int32_t* cu;
  const int32_t* seqlens_k;
  const float* sinks;
  void* out;
  int32_t* status;
  CacheDesc cd;
  int B, T, H_q, H_kv, D, group;
  int max_q, max_k, window;
  int n_rt;        // row tiles per request (host bound)
  int n_hg;        // head groups per KV head
  int total;       // workgroups
  int xcd_pairs;   // 1: (request, KV head) pairs split evenly over the 8 XCDs
  float scale_log2;
};

// LDS stage of a 32-key K/V tile.  16-bit caches arrive by LDS DMA, which writes each
// lane's 16 bytes at a fixed place, so their rows are unpadded and the 16-byte chunks of key
// k are XOR-swizzled by k (pf_swizzle) to spread the operand reads over the banks; INT8
// caches are converted in registers and stored with padded rows.
template <int D, bool kDma>
struct PfLds {
  static constexpr int kKld = kDma ? D : D + 8;    // K tile row (elements)
  static constexpr int kVld = kDma ? D : D + 16;   // V tile row (elements)
  static constexpr int kKBytes = kPfTile * kKld * 2;
  static constexpr int kVBytes = kPfTile * kVld * 2;
  static constexpr int kStage = kKBytes + kVBytes + kPfTile * 4 + 16;  // + key validity words
                                                                       // + 4 per-wave flags
  static constexpr int kStages = kDma ? 3 : 2;     // DMA: compute, landed, in flight
  static constexpr int kBtCap = 512;     // window of block ids staged in LDS
  static constexpr int kBtOffset = kStages * kStage;
  static constexpr int kTotal = kBtOffset + kBtCap * 4;
  static_assert(kStage % 16 == 0, "DMA destinations are 16-byte aligned");
};

// Slot XOR of key kk's 16-byte chunks in a DMA-staged tile row (chunk c sits in slot
// c ^ pf_swizzle(kk)).  At D = 64 the XOR is a bit rotation of kk mod 8, so the four keys
// one transposed V read of 16 lanes covers (kk = 4i .. 4i + 3) land in four different
// 32-byte slot pairs, while any 8 consecutive keys still get 8 different XORs for the K
// operand reads; measured, it halves the LDS bank-conflict cycles of the kernel.
template <int D>
__device__ __forceinline__ int pf_swizzle(int kk) {
  if constexpr (D == 64) return ((kk & 3) << 1) | ((kk >> 2) & 1);
  else return kk & (D / 8 - 1);
}

// LDS-DMA of 16 bytes per lane (lane l's bytes land at lds + 16 * l) and the waits the
// compiler does not insert for it.
__device__ __forceinline__ void pf_dma16(const void* gptr, void* lds) {
  __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void*)(lds), 16, 0, 0);
}
template <int N>
__device__ __forceinline__ void pf_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void pf_wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// One wave's step over one 32-key tile staged in LDS, for its 32 query rows (lane l32 =
// row, lane half h):
//   S^T[32 keys x 32 rows] = K Q^T  (v_mfma_f32_32x32x16, D/16 steps; with kQlo a second
//                                    product with the low half of a folded query)
//   masks(s): the caller's masks on the lane's 16 scores (keys 8*(i/4) + 4*h + i%4)
//   online softmax per row in the log2 domain with a lazy rescale (c_scale = |scale| log2 e
//   applied in the exponent; the running maximum is on raw scores)
//   O^T[D x 32 rows] += V^T P^T     (V^T from LDS via ds_read_b64_tr_b16)
// kchunk(kk, c) / vchunk(kk, c): byte offset of 16-byte chunk c of key kk in the K / V tile.
//
// kPair: two tiles in one softmax pass, for a full 32-row block of a window W that is a
// multiple of 32: the first tile of its key span (keys j_lo + k, visible to row r when
// k >= r) and the last (keys j_lo + W + k, visible when k < r) cover complementary
// triangles, so each row sees exactly 32 of their 64 keys.  Both QK products are taken;
// element i holds the key of the first tile when that key is at or after the row, else the
// one of the second; the softmax runs once over the merged 16 elements, and the weights go
// to the PV product of their own tile (0 in the other).  kl1 / vl1: the second tile.
template <typename OpT, int D, bool kQlo, bool kPair = false, typename KChunk, typename VChunk,
          typename Masks>
__device__ __forceinline__ void pf_tile_math(const unsigned char* kl, const unsigned char* vl,
                                             KChunk k_chunk, VChunk v_chunk,
                                             const typename Op32<OpT>::v8 (&qop)[D / 16],
                                             const typename Op32<OpT>::v8 (&qlo)[kQlo ? D / 16 : 1],
                                             Masks masks, float c_scale, float lazy_raw, float& m_run,
                                             float& l_run, f32x16 (&acc)[D / 32],
                                             const unsigned char* kl1 = nullptr,
                                             const unsigned char* vl1 = nullptr) {
  typedef typename Op32<OpT>::v8 V8;
  typedef typename Op32<OpT>::v4 V4;
  constexpr int KC = D / 16;
  constexpr int MT = D / 32;
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  // p = exp2(c * (s - m)) <= 2^8 with nm = -c m; a row with no visible key yet keeps p = 0.
  // nm is formed here, off the tile's dependent chain, and again only when m moves.
  float nm = m_run == kNegInf ? 0.f : -m_run * c_scale;
  // S^T: A = K[key l32][16kc + 8h ..], B = qop
  f32x16 s = f32x16{};
  f32x16 s1 = f32x16{};
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    V8 a = *reinterpret_cast<const V8*>(kl + k_chunk(l32, 2 * kc + h));
    s = mfma32(a, qop[kc], s);
    if constexpr (kQlo) s = mfma32(a, qlo[kc], s);
    if constexpr (kPair) {
      V8 a1 = *reinterpret_cast<const V8*>(kl1 + k_chunk(l32, 2 * kc + h));
      s1 = mfma32(a1, qop[kc], s1);
    }
  }
  // (pair) first[i]: element i's key, 8 (i / 4) + 4 h + i % 4 of the tile, is at or after
  // the lane's row, so it comes from the first tile
  bool first[16];
  if constexpr (kPair) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      first[i] = 8 * (i >> 2) + 4 * h + (i & 3) >= l32;
      s[i] = first[i] ? s[i] : s1[i];
    }
  } else {
    masks(s);
  }
  // the lane's maximum by a tree of three-input maxima (depth 3 instead of a chain of 8)
  float m5[5];
#pragma unroll
  for (int k = 0; k < 5; ++k) m5[k] = fmaxf(fmaxf(s[3 * k], s[3 * k + 1]), s[3 * k + 2]);
  float mt = fmaxf(fmaxf(fmaxf(m5[0], m5[1]), m5[2]), fmaxf(fmaxf(m5[3], m5[4]), s[15]));
  mt = half_swap_max(mt);                    // the row's other lane half
  const float m_new = fmaxf(m_run, mt);      // raw-score maximum of the row
  // the reference maximum moves only when some row's maximum outgrows it by more than
  // kLazyRescaleLog2 in the exponent, i.e. by lazy_raw = kLazyRescaleLog2 / c_scale in raw
  // scores; a row's first visible key always moves it (-inf + lazy_raw = -inf)
  if (__ballot(m_new > m_run + lazy_raw)) {
    // rows whose max did not move keep alpha = 1 (including rows that have seen no key
    // yet: -inf - -inf must not reach the exponent); a row seeing its first key gets
    // alpha = 0 on acc = 0, l = 0
    const float alpha = m_new == m_run ? 1.f : exp2_safe((m_run - m_new) * c_scale);
    l_run *= alpha;
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] *= alpha;
    m_run = m_new;
    nm = m_run == kNegInf ? 0.f : -m_run * c_scale;
  }
  // bf16 operands keep 8 significant bits: the weights are carried as hi + lo (hi = p
  // rounded, lo = its rounding error rounded) and PV takes one product with each, so
  // the weights keep about 16 bits, as f16 operands keep 11
  constexpr bool kSplitP = std::is_same<OpT, bf16>::value;
  V8 pop[2];
  V8 plo[kSplitP ? 2 : 1];
  V8 pop1[kPair ? 2 : 1];
  V8 plo1[kPair && kSplitP ? 2 : 1];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float p = exp2_safe(__builtin_fmaf(s[i], c_scale, nm));
    if constexpr (kPair) {
      const float p0 = first[i] ? p : 0.f, p1 = first[i] ? 0.f : p;
      pop[i >> 3][i & 7] = (OpT)p0;
      pop1[i >> 3][i & 7] = (OpT)p1;
      if constexpr (kSplitP) {
        plo[i >> 3][i & 7] = (OpT)(p0 - (float)pop[i >> 3][i & 7]);
        plo1[i >> 3][i & 7] = (OpT)(p1 - (float)pop1[i >> 3][i & 7]);
      }
    } else {
      pop[i >> 3][i & 7] = (OpT)p;
      if constexpr (kSplitP) plo[i >> 3][i & 7] = (OpT)(p - (float)pop[i >> 3][i & 7]);
    }
  }
  // this lane's part of the row sum, over the rounded weights the PV product uses, two
  // per instruction (products with 1 are exact; the sum is fp32)
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    l_run = dot2_ones(pop[i >> 3][i & 7], pop[i >> 3][(i & 7) + 1], l_run);
    if constexpr (kSplitP) l_run = dot2_ones(plo[i >> 3][i & 7], plo[i >> 3][(i & 7) + 1], l_run);
    if constexpr (kPair) {
      l_run = dot2_ones(pop1[i >> 3][i & 7], pop1[i >> 3][(i & 7) + 1], l_run);
      if constexpr (kSplitP) l_run = dot2_ones(plo1[i >> 3][i & 7], plo1[i >> 3][(i & 7) + 1], l_run);
    }
  }
  {
    const int grp = lane >> 4, lam = lane & 15;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        // key vk, dims d .. d + 3 (8 bytes inside chunk d / 8), and key vk + 8
        const int vk = 16 * ks + 4 * h + (lam >> 2);
        const int d = 32 * m + 16 * (grp & 1) + 4 * (lam & 3);
        const OpT* a0 = reinterpret_cast<const OpT*>(vl + v_chunk(vk, d >> 3) + (d & 7) * 2);
        const OpT* a1 = reinterpret_cast<const OpT*>(vl + v_chunk(vk + 8, d >> 3) + (d & 7) * 2);
        s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(a0));
        s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(a1));
        V4 x0 = __builtin_bit_cast(V4, r0);
        V4 x1 = __builtin_bit_cast(V4, r1);
        V8 av = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        acc[m] = mfma32(av, pop[ks], acc[m]);
        if constexpr (kSplitP) acc[m] = mfma32(av, plo[ks], acc[m]);
      }
  }
  if constexpr (kPair) {   // the same product over the pair's second V tile
    const int grp = lane >> 4, lam = lane & 15;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int vk = 16 * ks + 4 * h + (lam >> 2);
        const int d = 32 * m + 16 * (grp & 1) + 4 * (lam & 3);
        const OpT* a0 = reinterpret_cast<const OpT*>(vl1 + v_chunk(vk, d >> 3) + (d & 7) * 2);
        const OpT* a1 = reinterpret_cast<const OpT*>(vl1 + v_chunk(vk + 8, d >> 3) + (d & 7) * 2);
        s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(a0));
        s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(a1));
        V4 x0 = __builtin_bit_cast(V4, r0);
        V4 x1 = __builtin_bit_cast(V4, r1);
        V8 av = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        acc[m] = mfma32(av, pop1[ks], acc[m]);
        if constexpr (kSplitP) acc[m] = mfma32(av, plo1[ks], acc[m]);
      }
  }
}

// 4 waves per SIMD at D = 64 (128 registers: both tile buffers, the accumulators and the
// query operand fit), 3 at D = 64 with a quantised cache (the query's low operand needs
// 16 more registers), 2 at D = 128.
template <typename KT, int D>
constexpr int prefill_waves_per_eu() { return D != 64 ? 2 : sizeof(KT) == 1 ? 3 : 4; }

template <typename QT, typename KT, int D, int RW>
__global__ __launch_bounds__(kPfThreads)
__attribute__((amdgpu_waves_per_eu(prefill_waves_per_eu<KT, D>(), 8)))
void prefill_kernel(PrefillParams P) {
  constexpr int HW = 4 / RW;
  constexpr int KC = D / 16;          // QK k-steps
  constexpr int MT = D / 32;          // PV m-tiles
  constexpr int CH = D / 8;           // 8-element chunks per row
  constexpr int NCH = kPfTile * CH / kPfThreads;
  constexpr bool kI8 = sizeof(KT) == 1;                       // INT8 or FP8 E4M3 codes
  constexpr bool kFp8 = std::is_same<KT, uint8_t>::value;
  // FP8 operands hold code values / kFp8Unit; the factor rides on the scales
  constexpr float kUnit = kFp8 ? kFp8Unit : 1.0f;
  constexpr bool kDma = !kI8;
  typedef PfLds<D, kDma> L;
  constexpr int CHK = D / 8;          // 16-byte chunks per K/V row
  typedef typename std::conditional<kI8, f16, QT>::type OpT;
  typedef typename Op32<OpT>::v8 V8;
  typedef typename Op32<OpT>::v4 V4;
  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rw = wave / HW;
  const int hw = wave - rw * HW;
  const int h = lane >> 5;            // lane half
  const int l32 = lane & 31;

  // Work order: heaviest row tiles (the last ones of a request, which see the most keys)
  // first.  Workgroup i runs on XCD i % 8; when the (request, KV head) pairs split evenly
  // over the 8 XCDs, pair p is kept on XCD p % 8, so every XCD gets the same mix of row
  // tiles and the K/V of a pair is read through one L2.
  int rt, b, c, hg;
  {
    const int i = blockIdx.x;
    const int pairs = P.B * P.H_kv;
    int pair, rt_idx;
    if (P.xcd_pairs) {
      const int x = i & 7, k = i >> 3;
      const int per_rt = (pairs >> 3) * P.n_hg;       // items of one row-tile index per XCD
      rt_idx = k / per_rt;
      const int rem = k - rt_idx * per_rt;
      hg = rem % P.n_hg;
      pair = (rem / P.n_hg) * 8 + x;
    } else {
      hg = i % P.n_hg;
      const int t = i / P.n_hg;
      pair = t % pairs;
      rt_idx = t / pairs;
    }
    c = pair % P.H_kv;
    b = pair / P.H_kv;
    rt = P.n_rt - 1 - rt_idx;
  }

  int flags = 0;
  const int c0 = P.cu[b];
  int q_len = P.cu[b + 1] - c0;
  const int kv_len = P.seqlens_k[b] + 1;
  bool dead = false;
  if (q_len < 0 || c0 < 0 || c0 + q_len > P.T) { flags |= SPATTN_STATUS_BAD_CU; q_len = 0; }
  else if (q_len > P.max_q) { flags |= SPATTN_STATUS_Q_BOUND; dead = true; }
  else if (kv_len > P.max_k) { flags |= SPATTN_STATUS_K_BOUND; dead = true; }
  else if (kv_len < q_len) flags |= SPATTN_STATUS_SHORT_KV;

  const int head_local = hg * HW + hw;
  const bool head_ok = head_local < P.group;
  const int head = c * P.group + head_local;

  if (dead) {
    // the request's rows are zero; rows past the host bound are covered by striding
    if (head_ok) {
      for (int i = rt * 32 * RW + rw * 32 + (lane & 31); i < q_len; i += P.n_rt * 32 * RW) {
        QT* o = reinterpret_cast<QT*>(P.out) + ((int64_t)(c0 + i) * P.H_q + head) * D;
        for (int d = h; d < D; d += 2) o[d] = from_f32<QT>(0.f);
      }
    }
    if (tid == 0) raise_status(P.status, flags);
    return;
  }
  const int row_base = rt * 32 * RW;                 // first row (within the request) of the WG
  if (row_base >= q_len) { if (tid == 0) raise_status(P.status, flags); return; }
  const int wg_rows = min(32 * RW, q_len - row_base);
  const int pos0 = kv_len - q_len;                   // position of row 0
  const int p_first = pos0 + row_base;
  const int p_last = pos0 + row_base + wg_rows - 1;
  const int j_lo = P.window > 0 ? max(0, p_first - P.window + 1) : 0;
  const int j_hi = min(p_last, kv_len - 1);
  // this wave's rows
  const int wrow0 = row_base + rw * 32;
  const int my_row = wrow0 + l32;                    // row (within the request) of this lane
  const bool row_ok = my_row < q_len && head_ok;
  const int my_p = pos0 + my_row;
  const int my_lo = P.window > 0 ? my_p - P.window + 1 : INT32_MIN;
  const int wave_rows = max(0, min(32, q_len - wrow0));
  const int w_p_first = pos0 + wrow0;
  const int w_p_last = pos0 + wrow0 + wave_rows - 1;
  const int w_lo = P.window > 0 ? max(0, w_p_first - P.window + 1) : 0;
  const bool wave_active = head_ok && wave_rows > 0;

  // query operand (B of S^T = K Q^T): row my_row, dims 16*kc + 8*h .. +7.  The running max
  // is kept on raw scores q.k and the positive factor c = |scale| * log2(e) is applied inside
  // the exponent, so a negative scale is folded into the query's sign.
  const float c_scale = fabsf(P.scale_log2);
  const float lazy_raw = kLazyRescaleLog2 / c_scale;   // the rescale threshold in raw scores
  const bool q_neg = P.scale_log2 < 0.f;
  // Quantised caches fold the per-channel key scale into the query and carry the folded
  // value x = q * s as hi + lo (hi = x rounded to the operand type, lo = its rounding error
  // rounded); S takes one product with each, so the scores keep about 22 bits of x.  With
  // hi alone every term q_d k_d would carry a relative error up to 2^-11.
  V8 qop[KC];
  V8 qlo[kI8 ? KC : 1];
  {
    const QT* qr = reinterpret_cast<const QT*>(P.q) + ((int64_t)(c0 + my_row) * P.H_q + head) * D;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int col = kc * 16 + h * 8;
      if (row_ok) {
        if constexpr (kI8) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = to_f32(qr[col + e]) * (P.key_scale[c * D + col + e] * kUnit);
            const OpT hi = (OpT)x;
            qop[kc][e] = hi;
            qlo[kc][e] = (OpT)(x - (float)hi);
          }
        } else {
          qop[kc] = __builtin_bit_cast(V8, load16(qr + col));
        }
      } else {
        qop[kc] = V8{};
        if constexpr (kI8) qlo[kc] = V8{};
      }
      if (q_neg) {
        qop[kc] = -qop[kc];
        if constexpr (kI8) qlo[kc] = -qlo[kc];
      }
    }
  }

  f32x16 acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;

  const int kt_begin = (j_lo / kPfTile) * kPfTile;
  const int n_tiles = j_hi >= j_lo ? (j_hi - kt_begin) / kPfTile + 1 : 0;

  const KT* kcache = reinterpret_cast<const KT*>(P.k_cache);
  const KT* vcache = reinterpret_cast<const KT*>(P.v_cache);

  // ---- block ids of the key range, staged in LDS (paged caches) ----
  // The window holds the ids of logical blocks win_lb .. win_lb + kBtCap - 1; a workgroup
  // whose key range needs more refills it between barriers (block size 16: every 8192 keys).
  int32_t* bt_lds = reinterpret_cast<int32_t*>(smem + L::kBtOffset);
  const bool paged = P.cd.block_table != nullptr;
  const int bs = P.cd.block_size;
  const bool pow2 = P.cd.bs_shift >= 0;
  auto lblock = [&](int j) { return pow2 ? j >> P.cd.bs_shift : j / bs; };
  const int lb_last = n_tiles > 0 ? lblock(j_hi) : 0;
  int win_lb = n_tiles > 0 ? lblock(j_lo) : 0;
  auto fill_window = [&]() {
    const int32_t* row = P.cd.block_table + (int64_t)b * P.cd.max_blocks;
    for (int i = tid; i < L::kBtCap; i += kPfThreads) {
      const int lb = win_lb + i;
      // never read past the table width or the blocks of the key range
      bt_lds[i] = lb < P.cd.max_blocks && lb <= lb_last ? row[lb] : 0;
    }
  };
  if (paged && n_tiles > 0) {
    fill_window();
    __syncthreads();
  }
  // before loading tile `it`: move the window when the tile's last key lies beyond it
  auto ensure_window = [&](int it) {
    if (!paged) return;
    const int kt = kt_begin + it * kPfTile;
    if (lblock(min(kt + kPfTile - 1, j_hi)) < win_lb + L::kBtCap) return;
    __syncthreads();                       // every thread is done with the old window
    win_lb = lblock(max(kt, j_lo));
    fill_window();
    __syncthreads();
  };

  // ---- tile loader: global -> registers -> LDS stage; two tiles in registers at a time ----
  // A thread always loads the same 16-byte piece (key lkey, columns lcol..+7) of each tile,
  // so the address is   block * blk_stride + slot * D + head_col   (paged) or
  //                     req_base + j * D                         (contiguous).
  typedef typename std::conditional<kI8, int2, i32x4>::type Raw;
  struct TileRegs { Raw k[NCH], v[NCH]; bool ok[NCH]; };
  // a finite row of D elements for the loads of missing keys: the workgroup's first query
  // row for 16-bit caches (same element size), the cache's first row for INT8 caches
  const KT* safe_k = kI8 ? kcache : reinterpret_cast<const KT*>(
      reinterpret_cast<const QT*>(P.q) + ((int64_t)(c0 + row_base) * P.H_q + c * P.group) * D);
  const KT* safe_v = kI8 ? vcache : safe_k;
  const int64_t blk_stride = (int64_t)P.cd.H_kv * bs * D;
  const int64_t head_off = (int64_t)c * bs * D;
  const int64_t req_base = ((int64_t)b * P.cd.H_kv + c) * bs * D;   // contiguous caches
  // element offset of key j's cache row (KV head c), or ok = false (missing key: flagged,
  // never read)
  auto key_row = [&](int j, bool& ok) -> int64_t {
    ok = j >= j_lo && j <= j_hi;
    if (paged) {
      const int lb = lblock(j);
      const int o = j - lb * bs;
      const bool in_tab = lb < P.cd.max_blocks;
      // in-range keys index the window; others read any entry and are dropped
      const int blk = bt_lds[min(max(lb - win_lb, 0), L::kBtCap - 1)];
      const bool blk_ok = blk >= 0 && blk < P.cd.num_blocks;
      if (ok && !(in_tab && blk_ok))
        flags |= in_tab ? SPATTN_STATUS_BAD_BLOCK : SPATTN_STATUS_CAPACITY;
      ok = ok && in_tab && blk_ok;
      return (int64_t)blk * blk_stride + head_off + o * D;
    }
    const bool in_cap = j < bs && b < P.cd.num_blocks;
    if (ok && !in_cap) flags |= SPATTN_STATUS_CAPACITY;
    ok = ok && in_cap;
    return req_base + (int64_t)j * D;
  };
  auto load_tile = [&](TileRegs& tr, int kt) {
#pragma unroll
    for (int n = 0; n < NCH; ++n) {
      const int qi = tid + n * kPfThreads;
      const int key = qi / CH, col = (qi % CH) * 8;
      bool ok;
      const int64_t off = key_row(kt + key, ok) + col;
      tr.ok[n] = ok;
      // every lane loads (no register is cleared, so nothing waits for loads in flight): a
      // missing key reads a safe finite row instead; its score is masked to -inf and its
      // weight is exactly 0
      const KT* kp = ok ? kcache + off : safe_k + col;
      const KT* vp = ok ? vcache + off : safe_v + col;
      tr.k[n] = *reinterpret_cast<const Raw*>(kp);
      tr.v[n] = *reinterpret_cast<const Raw*>(vp);
    }
  };
  // 16-bit caches: DMA of a tile straight into an LDS stage.  Instruction q of the tile
  // (wave w issues q = w * kDmaPerWave + n) fills 16-byte positions 64q .. 64q + 63, i.e.
  // key p / CHK, slot p % CHK, which holds the key's chunk slot ^ pf_swizzle(key).
  constexpr int kDmaPerWave = kPfTile * CHK / (64 * (kPfThreads / 64));
  // Paged cache with a power-of-two block size and blocks under 4 GiB apart: the byte
  // address of key j is  base + blk * blk_bytes + (j mod bs) * row_bytes + column bytes,
  // formed with one 32 x 32 -> 64-bit multiply-add per tile instead of the general
  // element-offset arithmetic of key_row.
  const uint64_t blk_bytes64 = (uint64_t)blk_stride * sizeof(KT);
  const bool dma_fast = paged && pow2 && blk_bytes64 < (1ull << 32);
  const uint32_t blk_bytes = (uint32_t)P.cd.H_kv * (uint32_t)bs * (uint32_t)(D * sizeof(KT));
  const char* kbytes = reinterpret_cast<const char*>(kcache + head_off);
  const char* vbytes = reinterpret_cast<const char*>(vcache + head_off);
  // One DMA instruction covers kKeysPerInst consecutive keys.  With a power-of-two block
  // size of at least that many keys, they lie in one block; when they are all in the key
  // range and the block's id (read by a scalar load: the table is read-only here) is valid,
  // the instruction's address is  block base (uniform) + a per-lane offset that is the same
  // for every tile, so the tile's DMAs need no per-lane block lookup, bounds checks or
  // address arithmetic.  Other instructions (range edges, missing blocks) go per lane.
  constexpr int kKeysPerInst = 64 / CHK;
  const bool uniform_dma = dma_fast && (1 << P.cd.bs_shift) >= kKeysPerInst;
  const __attribute__((address_space(4))) int32_t* ctable =
      (const __attribute__((address_space(4))) int32_t*)(paged ? P.cd.block_table + (int64_t)b * P.cd.max_blocks
                                                               : nullptr);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  uint32_t lane_off[kDmaPerWave];      // bytes from the instruction's first key row
#pragma unroll
  for (int n = 0; n < kDmaPerWave; ++n) {
    const int p = (wave * kDmaPerWave + n) * 64 + lane;
    const int key = p / CHK, slot = p % CHK;
    lane_off[n] = (uint32_t)(((key % kKeysPerInst) * D + (slot ^ pf_swizzle<D>(key)) * 8) * sizeof(KT));
  }
  auto issue_dma = [&](int kt, int stage) {
    unsigned char* base = smem + stage * L::kStage;
    int32_t* vb = reinterpret_cast<int32_t*>(base + L::kKBytes + L::kVBytes);
    bool all_ok = true;
#pragma unroll
    for (int n = 0; n < kDmaPerWave; ++n) {
      const int q = wave * kDmaPerWave + n;
      const int p = q * 64 + lane;
      const int key = p / CHK, slot = p % CHK;
      const int col = (slot ^ pf_swizzle<D>(key)) * 8;
      bool ok;
      const KT* kp;
      const KT* vp;
      // the uniform case: first key of the instruction, its block and that block's id
      const int ja = kt + (wave_u * kDmaPerWave + n) * kKeysPerInst;
      int blk_u = -1;
      if (uniform_dma && ja >= j_lo && ja + kKeysPerInst - 1 <= j_hi) {
        const int lb = ja >> P.cd.bs_shift;
        if (lb < P.cd.max_blocks) blk_u = ctable[lb];
      }
      if ((unsigned)blk_u < (unsigned)P.cd.num_blocks) {
        ok = true;
        const uint64_t boff = (uint64_t)(uint32_t)blk_u * blk_bytes +
                              (uint32_t)(ja & (bs - 1)) * (uint32_t)(D * sizeof(KT));   // (uniform)
        kp = reinterpret_cast<const KT*>(kbytes + boff + lane_off[n]);
        vp = reinterpret_cast<const KT*>(vbytes + boff + lane_off[n]);
      } else if (dma_fast) {
        const int j = kt + key;
        const int lb = j >> P.cd.bs_shift;
        const int blk = bt_lds[min(max(lb - win_lb, 0), L::kBtCap - 1)];
        const bool in_range = j >= j_lo && j <= j_hi;
        const bool in_tab = lb < P.cd.max_blocks;
        const bool blk_ok = (unsigned)blk < (unsigned)P.cd.num_blocks;
        if (in_range && !(in_tab && blk_ok))
          flags |= in_tab ? SPATTN_STATUS_BAD_BLOCK : SPATTN_STATUS_CAPACITY;
        ok = in_range && in_tab && blk_ok;
        const uint32_t in_blk = (uint32_t)((j & (bs - 1)) * D + col) * (uint32_t)sizeof(KT);
        const uint64_t boff = (uint64_t)(uint32_t)blk * blk_bytes + in_blk;
        kp = ok ? reinterpret_cast<const KT*>(kbytes + boff) : safe_k + col;
        vp = ok ? reinterpret_cast<const KT*>(vbytes + boff) : safe_v + col;
      } else {
        const int64_t off = key_row(kt + key, ok) + col;
        kp = ok ? kcache + off : safe_k + col;
        vp = ok ? vcache + off : safe_v + col;
      }
      // (the LDS destination is uniform: wave_u keeps it in scalar registers)
      const int q_u = wave_u * kDmaPerWave + n;
      pf_dma16(kp, base + q_u * 1024);
      pf_dma16(vp, base + L::kKBytes + q_u * 1024);
      if (slot == 0) vb[key] = ok ? 1 : 0;
      all_ok = all_ok && ok;
    }
    const bool wave_ok = __ballot(!all_ok) == 0;
    if (lane == 0) vb[kPfTile + wave] = wave_ok ? 1 : 0;
  };
  auto store_tile = [&](const TileRegs& tr, int stage) {
    unsigned char* base = smem + stage * L::kStage;
    OpT* kl = reinterpret_cast<OpT*>(base);
    OpT* vl = reinterpret_cast<OpT*>(base + L::kKBytes);
    int32_t* vb = reinterpret_cast<int32_t*>(base + L::kKBytes + L::kVBytes);
#pragma unroll
    for (int n = 0; n < NCH; ++n) {
      const int qi = tid + n * kPfThreads;
      const int key = qi / CH, col = (qi % CH) * 8;
      V8 kv, vv;
      if constexpr (kFp8) {
        kv = fp8x8_to_f16(tr.k[n].x, tr.k[n].y);
        vv = fp8x8_to_f16(tr.v[n].x, tr.v[n].y);
      } else if constexpr (kI8) {
        kv = int8x8_to_f16(tr.k[n].x, tr.k[n].y);
        vv = int8x8_to_f16(tr.v[n].x, tr.v[n].y);
      } else {
        kv = __builtin_bit_cast(V8, tr.k[n]);
        vv = __builtin_bit_cast(V8, tr.v[n]);
      }
      if constexpr (kI8) {
        // a missing key read the cache's first row, whose FP8 codes may be NaN: its weight
        // is 0, so its row must be finite
        if (!tr.ok[n]) { kv = V8{}; vv = V8{}; }
      }
      *reinterpret_cast<V8*>(kl + key * L::kKld + col) = kv;
      *reinterpret_cast<V8*>(vl + key * L::kVld + col) = vv;
      if (col == 0) vb[key] = tr.ok[n] ? 1 : 0;
    }
    // one flag per loading wave: every key it loaded exists
    bool all_ok = true;
#pragma unroll
    for (int n = 0; n < NCH; ++n) all_ok = all_ok && tr.ok[n];
    const bool wave_ok = __ballot(!all_ok) == 0;
    if (lane == 0) vb[kPfTile + wave] = wave_ok ? 1 : 0;
  };

  // byte offset of logical 16-byte chunk c of key kk within a K / V tile
  auto k_chunk = [&](int kk, int c) -> int {
    if constexpr (kDma) return kk * D * 2 + ((c ^ pf_swizzle<D>(kk)) << 4);
    else return (kk * L::kKld + c * 8) * 2;
  };
  auto v_chunk = [&](int kk, int c) -> int {
    if constexpr (kDma) return kk * D * 2 + ((c ^ pf_swizzle<D>(kk)) << 4);
    else return (kk * L::kVld + c * 8) * 2;
  };
  auto compute_tile = [&](int it, int stage) {
    const int kt = kt_begin + it * kPfTile;
    // skip tiles outside this wave's key range (fully masked for every row it owns)
    if (wave_active && kt + kPfTile - 1 >= w_lo && kt <= w_p_last) {
      const unsigned char* base = smem + stage * L::kStage;
      const OpT* kl = reinterpret_cast<const OpT*>(base);
      const OpT* vl = reinterpret_cast<const OpT*>(base + L::kKBytes);
      const int32_t* vb = reinterpret_cast<const int32_t*>(base + L::kKBytes + L::kVBytes);
      // lane holds keys 8*(i/4) + 4*h + i%4 of row l32.  Masks only on tiles some row of the
      // wave does not fully see (the diagonal, the window edge, missing keys).
      // (the loaders' flags are read here, after the K operand reads are issued, so the two
      // LDS round trips overlap)
      const bool full_rows = kt + kPfTile - 1 <= w_p_first &&
                             (P.window <= 0 || kt >= w_p_last - P.window + 1);
      auto masks = [&](f32x16& s) {
        const i32x4 wflags = *reinterpret_cast<const i32x4*>(vb + kPfTile);
        const bool tile_ok = (wflags[0] & wflags[1] & wflags[2] & wflags[3]) != 0;
        if (!(tile_ok && full_rows)) {
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int k0 = 8 * g4 + 4 * h;
            const i32x4 ok = *reinterpret_cast<const i32x4*>(vb + k0);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int j = kt + k0 + e;
              if (!(ok[e] && j <= my_p && j >= my_lo)) s[4 * g4 + e] = kNegInf;
            }
          }
        }
      };
      pf_tile_math<OpT, D, kI8>(reinterpret_cast<const unsigned char*>(kl),
                                reinterpret_cast<const unsigned char*>(vl), k_chunk, v_chunk, qop,
                                qlo, masks, c_scale, lazy_raw, m_run, l_run, acc);
    }
  };

  if constexpr (kDma) {
    // Iteration it computes tile it from stage it % 3 while tile it + 2 streams into stage
    // (it + 2) % 3 (last read in iteration it - 1, before its barrier); before the barrier
    // each wave waits for its DMAs of tile it + 1.  One barrier per tile.
    if (n_tiles > 0) issue_dma(kt_begin, 0);
    if (n_tiles > 1) {
      ensure_window(1);
      issue_dma(kt_begin + kPfTile, 1);
    }
    if (n_tiles > 1) pf_wait_vm<2 * kDmaPerWave>(); else pf_wait_vm<0>();
    pf_wait_lgkm0();
    __syncthreads();
    int stage = 0;
    for (int it = 0; it < n_tiles; ++it) {
      const bool more = it + 2 < n_tiles;
      if (more) {
        ensure_window(it + 2);
        issue_dma(kt_begin + (it + 2) * kPfTile, stage == 0 ? 2 : stage - 1);
      }
      compute_tile(it, stage);
      if (more) pf_wait_vm<2 * kDmaPerWave>(); else pf_wait_vm<0>();   // tile it + 1 landed
      pf_wait_lgkm0();
      __syncthreads();
      stage = stage == 2 ? 0 : stage + 1;
    }
  } else {
    // Iteration it computes tile it from LDS stage it & 1 while tile it + 2 loads into the
    // register buffer tile it freed; tile it + 1 (loaded one iteration earlier) then goes to
    // the other stage.  One barrier per tile.
    auto step = [&](int it, TileRegs& next, TileRegs& later) {
      if (it + 2 < n_tiles) {
        ensure_window(it + 2);
        load_tile(later, kt_begin + (it + 2) * kPfTile);
      }
      compute_tile(it, it & 1);
      if (it + 1 < n_tiles) store_tile(next, (it + 1) & 1);
      __syncthreads();
    };
    TileRegs ra, rb;
    if (n_tiles > 0) load_tile(ra, kt_begin);
    if (n_tiles > 1) {
      ensure_window(1);
      load_tile(rb, kt_begin + kPfTile);
    }
    if (n_tiles > 0) store_tile(ra, 0);
    __syncthreads();
    // two steps per trip with fixed buffer roles, so no register copies (which would wait
    // for the loads in flight) are needed; an odd last tile runs after the loop
    int it = 0;
    for (; it + 1 < n_tiles; it += 2) {
      step(it, rb, ra);
      step(it + 1, ra, rb);
    }
    if (it < n_tiles) step(it, rb, ra);
  }

  // ---- finalise: sink, normalise, store (lane: row l32, dims 32m + 8(i/4) + 4h + i%4) ----
  l_run = half_swap_sum(l_run);                      // both lane halves of the row
  float f = 0.f, inv = 0.f;
  if (row_ok && m_run != kNegInf) {
    const float ms = m_run * c_scale;                // log2-domain maximum
    const float sg = P.sinks != nullptr ? P.sinks[head] * kLog2e : kNegInf;
    const float M2 = fmaxf(ms, sg);
    f = exp2_safe(ms - M2);
    inv = f / (l_run * f + exp2_safe(sg - M2));
  }
  // The wave's 32 rows go through LDS (the tile stages: every wave has passed the key
  // loop's last barrier, so none reads them again) and out with 16 bytes a lane and D / 8
  // lanes a row; in the accumulator layout each row would be stored as D / 4 separate
  // 8-byte pieces.  Rows are padded by 16 bytes to spread the 8-byte writes over the banks.
  constexpr int kORow = D * 2 + 16;
  static_assert(L::kStages * L::kStage >= 4 * 32 * kORow, "output staging fits the tile stages");
  unsigned char* ost = smem + wave * (32 * kORow);
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = 32 * m + 8 * g4 + 4 * h;
      typename Op32<QT>::v4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = acc[m][4 * g4 + e] * inv;
        if constexpr (kI8) x *= P.value_scale[c * D + d0 + e] * kUnit;
        w[e] = from_f32<QT>(x);
      }
      *reinterpret_cast<typename Op32<QT>::v4*>(ost + l32 * kORow + d0 * 2) = w;
    }
  constexpr int kRowsPerStore = 64 / CH;
#pragma unroll
  for (int i = 0; i < 32 / kRowsPerStore; ++i) {
    const int r = i * kRowsPerStore + lane / CH, ch = lane % CH;
    const i32x4 v = *reinterpret_cast<const i32x4*>(ost + r * kORow + ch * 16);
    if (head_ok && wrow0 + r < q_len)
      store16(reinterpret_cast<QT*>(P.out) + ((int64_t)(c0 + wrow0 + r) * P.H_q + head) * D + ch * 8, v);
  }
  // flags from the loaders (keys visible to some row of the workgroup) and the row checks
  int wave_flags = 0;
#pragma unroll
  for (int bit = 0; bit < 8; ++bit)
    if (__ballot(flags & (1 << bit))) wave_flags |= 1 << bit;
  if (wave_flags && lane == 0) raise_status(P.status, wave_flags);
}

// ---------------------------------------------------------------------------------------
// Windowed prefill over 16-bit caches ("[WebGPU] Add PagedAttention metadata and GPT-OSS
// support": local window; review finding Q3: the keys a query block needs are one window
// plus the block).  Workgroup = one 32-row block of one request and one KV head, with every
// query head of its group: the block's whole key span, max(0, p_first - W + 1) .. p_last
// (at most 31 + W keys), goes into LDS by DMA once, behind one barrier.  Then each wave
// takes the group's heads h = wave, wave + NW, ... and runs every tile of the span for the
// 32 rows, with no further barrier.  K and V are read once per group of heads, and the
// per-tile barrier of the streaming kernel is gone.
// ---------------------------------------------------------------------------------------
constexpr int kWinRows = 32;
constexpr int kWinMax = 128;   // largest window this kernel takes

template <int D, int NW>
struct WinLds {
  static constexpr int kMaxTiles = (kWinRows + kWinMax - 1 + kPfTile - 1) / kPfTile;
  static constexpr int kTileBytes = kPfTile * D * 2;      // K (or V) of one tile
  static constexpr int kVOff = kMaxTiles * kTileBytes;
  static constexpr int kOkOff = 2 * kMaxTiles * kTileBytes;   // one byte per span key
  // each wave's 32 output rows, staged so that 16-byte lanes store whole rows; a row is
  // padded by 16 bytes to spread the 8-byte writes of the accumulator layout over the banks
  // (not with 4 waves at D = 64, whose 40 KB span area lets four workgroups share a CU)
  static constexpr bool kStageOut = NW == 8 || D != 64;
  static constexpr int kORow = D * 2 + 16;
  static constexpr int kOOff = (kOkOff + kMaxTiles * kPfTile + 15) / 16 * 16;
  static constexpr int kTotal = kStageOut ? kOOff + NW * kWinRows * kORow : kOkOff + kMaxTiles * kPfTile;
};

template <typename QT, int D, int NW>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(prefill_waves_per_eu<QT, D>(), 8)))
void prefill_window_kernel(PrefillParams P) {
  typedef WinLds<D, NW> L;
  typedef typename Op32<QT>::v8 V8;
  constexpr int KC = D / 16;
  constexpr int MT = D / 32;
  constexpr int CHK = D / 8;                        // 16-byte chunks per key row
  constexpr int IPT = kPfTile * CHK / 64;           // DMA instructions per K (or V) tile
  extern __shared__ __align__(16) unsigned char smem[];
  uint8_t* key_ok = smem + L::kOkOff;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // (uniform: scalar)
  const int h = lane >> 5;
  const int l32 = lane & 31;

  // (request, KV head) pair p runs on XCD p % 8, its row blocks in order, so the blocks
  // whose spans overlap share that XCD's L2
  int b, c, rb;
  {
    const int i = blockIdx.x;
    const int x = i & 7, k = i >> 3;
    const int pair = (k / P.n_rt) * 8 + x;
    if (pair >= P.B * P.H_kv) return;
    rb = k - (k / P.n_rt) * P.n_rt;
    c = pair % P.H_kv;
    b = pair / P.H_kv;
  }

  int flags = 0;
  const int c0 = P.cu[b];
  int q_len = P.cu[b + 1] - c0;
  const int kv_len = P.seqlens_k[b] + 1;
  bool dead = false;
  if (q_len < 0 || c0 < 0 || c0 + q_len > P.T) { flags |= SPATTN_STATUS_BAD_CU; q_len = 0; }
  else if (q_len > P.max_q) { flags |= SPATTN_STATUS_Q_BOUND; dead = true; }
  else if (kv_len > P.max_k) { flags |= SPATTN_STATUS_K_BOUND; dead = true; }
  else if (kv_len < q_len) flags |= SPATTN_STATUS_SHORT_KV;
  auto raise = [&]() {
    int wf = 0;
#pragma unroll
    for (int bit = 0; bit < 8; ++bit)
      if (__ballot(flags & (1 << bit))) wf |= 1 << bit;
    if (wf && lane == 0) raise_status(P.status, wf);
  };
  if (dead) {
    // the request's rows are zero; rows past the host bound are covered by striding
    for (int hh = wave; hh < P.group; hh += NW)
      for (int i = rb * kWinRows + l32; i < q_len; i += P.n_rt * kWinRows) {
        QT* o = reinterpret_cast<QT*>(P.out) + ((int64_t)(c0 + i) * P.H_q + c * P.group + hh) * D;
        for (int d = h; d < D; d += 2) o[d] = from_f32<QT>(0.f);
      }
    raise();
    return;
  }
  const int row_base = rb * kWinRows;
  if (row_base >= q_len) { raise(); return; }
  const int rows = min(kWinRows, q_len - row_base);
  const int pos0 = kv_len - q_len;
  const int p_first = pos0 + row_base, p_last = p_first + rows - 1;
  const int j_lo = max(0, p_first - P.window + 1);
  const int j_hi = min(p_last, kv_len - 1);
  const int n_keys = max(0, j_hi - j_lo + 1);
  const int n_tiles = (n_keys + kPfTile - 1) / kPfTile;

  // ---- the span's K and V into LDS: tile t holds keys j_lo + 32 t + kk, row kk with its
  //      16-byte chunks XOR-swizzled by kk (as the streaming kernel's stages) ----
  const QT* kcache = reinterpret_cast<const QT*>(P.k_cache);
  const QT* vcache = reinterpret_cast<const QT*>(P.v_cache);
  const QT* safe = reinterpret_cast<const QT*>(P.q) + ((int64_t)(c0 + row_base) * P.H_q + c * P.group) * D;
  const bool paged = P.cd.block_table != nullptr;
  const int bs = P.cd.block_size;
  const int32_t* table = paged ? P.cd.block_table + (int64_t)b * P.cd.max_blocks : nullptr;
  // the query operands of this wave's first head load under the span's DMA
  const int my_row = row_base + l32;
  const bool row_ok = my_row < q_len;
  auto load_q = [&](int hh, V8 (&qop)[KC]) {
    const QT* qr = reinterpret_cast<const QT*>(P.q) + ((int64_t)(c0 + my_row) * P.H_q + c * P.group + hh) * D;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) qop[kc] = row_ok ? __builtin_bit_cast(V8, load16(qr + kc * 16 + h * 8)) : V8{};
  };
  V8 qop[KC];
  if (wave < P.group) load_q(wave, qop);
  // Block ids: with a power-of-two block size of at least the 64 / CHK keys one DMA
  // instruction covers, an instruction's keys lie in at most two blocks, whose ids are read
  // by scalar loads (the table is read-only here): the DMAs of the span then go out back to
  // back, with no wait for a vector load between them (each such wait would also wait for
  // the DMAs and query loads already in flight).  Other block sizes read ids per lane.
  constexpr int kKeysPerInst = 64 / CHK;
  const bool scalar_ids = paged && P.cd.bs_shift >= 0 && (1 << P.cd.bs_shift) >= kKeysPerInst;
  const __attribute__((address_space(4))) int32_t* ctable =
      (const __attribute__((address_space(4))) int32_t*)table;
  bool all_ok = true;
  auto span_dma = [&](auto scalar_tag) {
    constexpr bool kScalar = decltype(scalar_tag)::value;
    for (int q = wave; q < n_tiles * IPT; q += NW) {
      const int t = q / IPT;
      const int pos = (q - t * IPT) * 64 + lane;
      const int kk = pos / CHK, slot = pos - kk * CHK;
      const int col = (slot ^ pf_swizzle<D>(kk)) * 8;
      const int j = j_lo + t * kPfTile + kk;
      bool ok = j <= j_hi;
      int64_t row = 0;
      int blk_a = -1, blk_b = -1, lb_a = 0;
      if constexpr (kScalar) {
        const int ja = j_lo + t * kPfTile + (q - t * IPT) * kKeysPerInst;   // (uniform)
        lb_a = ja >> P.cd.bs_shift;
        const int lb_b = (ja + kKeysPerInst - 1) >> P.cd.bs_shift;
        blk_a = lb_a < P.cd.max_blocks ? ctable[__builtin_amdgcn_readfirstlane(lb_a)] : -1;
        blk_b = lb_b == lb_a ? blk_a
                             : lb_b < P.cd.max_blocks ? ctable[__builtin_amdgcn_readfirstlane(lb_b)] : -1;
      }
      if (ok) {
        if (paged) {
          const int lb = P.cd.bs_shift >= 0 ? j >> P.cd.bs_shift : j / bs;
          const int blk = kScalar ? (lb == lb_a ? blk_a : blk_b)
                                  : lb < P.cd.max_blocks ? table[lb] : -1;
          if (lb >= P.cd.max_blocks) flags |= SPATTN_STATUS_CAPACITY;
          else if (blk < 0 || blk >= P.cd.num_blocks) flags |= SPATTN_STATUS_BAD_BLOCK;
          ok = lb < P.cd.max_blocks && blk >= 0 && blk < P.cd.num_blocks;
          row = (((int64_t)blk * P.cd.H_kv + c) * bs + (j - lb * bs));
        } else {
          ok = j < bs && b < P.cd.num_blocks;
          if (!ok) flags |= SPATTN_STATUS_CAPACITY;
          row = ((int64_t)b * P.cd.H_kv + c) * bs + j;
        }
      }
      // a missing key reads a finite row (the block's first query row); its weight is 0
      const QT* kp = ok ? kcache + row * D + col : safe + col;
      const QT* vp = ok ? vcache + row * D + col : safe + col;
      pf_dma16(kp, smem + t * L::kTileBytes + (q - t * IPT) * 1024);
      pf_dma16(vp, smem + L::kVOff + t * L::kTileBytes + (q - t * IPT) * 1024);
      if (slot == 0) key_ok[t * kPfTile + kk] = ok ? 1 : 0;
      all_ok = all_ok && (ok || j > j_hi);
    }
  };
  if (scalar_ids) span_dma(std::true_type{});
  else span_dma(std::false_type{});
  // the sink of this wave's first head, by a scalar load (read-only here) issued while the
  // span is in flight instead of at the finalisation
  const __attribute__((address_space(4))) float* csinks =
      (const __attribute__((address_space(4))) float*)P.sinks;
  const float sink_first = P.sinks != nullptr && wave < P.group
      ? csinks[__builtin_amdgcn_readfirstlane(c * P.group + wave)] : kNegInf;
  pf_wait_vm<0>();
  const bool span_ok = __syncthreads_or(!all_ok) == 0;   // every key of the span exists

  // ---- every head of this wave over the span ----
  const float c_scale = fabsf(P.scale_log2);
  const float lazy_raw = kLazyRescaleLog2 / c_scale;   // the rescale threshold in raw scores
  const bool q_neg = P.scale_log2 < 0.f;
  const int my_p = pos0 + my_row;
  const int my_lo = max(0, my_p - P.window + 1);
  // rows of the block: the tiles every row sees whole are those inside
  // [lo(p_last), p_first]
  const int full_lo = max(0, p_last - P.window + 1), full_hi = p_first;
  constexpr bool kPairEnds = !std::is_same<QT, bf16>::value;
  const bool pair_ends = span_ok && rows == kWinRows && p_first - P.window + 1 >= 0 &&
                         (P.window & (kPfTile - 1)) == 0 && n_tiles == P.window / kPfTile + 1;
  auto k_chunk = [&](int kk, int ch) -> int { return kk * D * 2 + ((ch ^ pf_swizzle<D>(kk)) << 4); };
  for (int hh = wave; hh < P.group; hh += NW) {
    const int head = c * P.group + hh;
    const V8 qlo[1] = {V8{}};
    if (hh != wave) load_q(hh, qop);
    if (q_neg) {
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) qop[kc] = -qop[kc];
    }
    f32x16 acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = f32x16{};
    float m_run = kNegInf, l_run = 0.f;
    // a full block of a window that is a multiple of 32 (span W + 31 keys, W / 32 + 1 tiles)
    // takes its first and last tiles in one pass; the tiles between are seen whole
    // (fp16 only: bf16 carries the weights as hi + lo, and two tiles' of them spill)
    int t_begin = 0, t_end = n_tiles;
    if (kPairEnds && pair_ends) {
      pf_tile_math<QT, D, false, kPairEnds>(smem, smem + L::kVOff, k_chunk, k_chunk, qop, qlo,
                                       [](f32x16&) {}, c_scale, lazy_raw, m_run, l_run, acc,
                                       smem + (n_tiles - 1) * L::kTileBytes,
                                       smem + L::kVOff + (n_tiles - 1) * L::kTileBytes);
      t_begin = 1;
      t_end = n_tiles - 1;
    }
    for (int t = t_begin; t < t_end; ++t) {
      const int kt = j_lo + t * kPfTile;
      const bool full = span_ok && kt >= full_lo && kt + kPfTile - 1 <= full_hi;
      auto masks = [&](f32x16& s) {
        if (full) return;
        // key kt + k is visible to this lane's row when lo(p) <= kt + k <= p (k counted
        // from the lane half's first key, 4 h) and it exists
        const int lo_rel = my_lo - kt - 4 * h, hi_rel = my_p - kt - 4 * h;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int k = 8 * (i >> 2) + (i & 3);
          s[i] = (k >= lo_rel && k <= hi_rel) ? s[i] : kNegInf;
        }
        if (!span_ok) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (!key_ok[t * kPfTile + 8 * (i >> 2) + 4 * h + (i & 3)]) s[i] = kNegInf;
        }
      };
      pf_tile_math<QT, D, false>(smem + t * L::kTileBytes, smem + L::kVOff + t * L::kTileBytes,
                                 k_chunk, k_chunk, qop, qlo, masks, c_scale, lazy_raw, m_run, l_run, acc);
    }
    // finalise: sink, normalise, store (lane: row l32, dims 32m + 8(i/4) + 4h + i%4)
    l_run = half_swap_sum(l_run);
    float f = 0.f, inv = 0.f;
    if (row_ok && m_run != kNegInf) {
      const float ms = m_run * c_scale;
      const float sraw = hh == wave ? sink_first : P.sinks != nullptr ? P.sinks[head] : 0.f;
      const float sg = P.sinks != nullptr ? sraw * kLog2e : kNegInf;
      const float M2 = fmaxf(ms, sg);
      f = exp2_safe(ms - M2);
      inv = f / (l_run * f + exp2_safe(sg - M2));
    }
    // the normalised rows go to this wave's LDS rows, then out with 16 bytes a lane and
    // D / 8 lanes a row (an 8-byte piece a lane in the accumulator layout would store each
    // row as D / 4 separate pieces); the wave's LDS accesses complete in order, so the
    // area is free again for its next head
    if constexpr (!L::kStageOut) {
      if (row_ok) {
        QT* o = reinterpret_cast<QT*>(P.out) + ((int64_t)(c0 + my_row) * P.H_q + head) * D;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int d0 = 32 * m + 8 * g4 + 4 * h;
            typename Op32<QT>::v4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = from_f32<QT>(acc[m][4 * g4 + e] * inv);
            *reinterpret_cast<typename Op32<QT>::v4*>(o + d0) = w;
          }
      }
      continue;
    }
    unsigned char* ost = smem + L::kOOff + wave * (kWinRows * L::kORow);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * m + 8 * g4 + 4 * h;
        typename Op32<QT>::v4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = from_f32<QT>(acc[m][4 * g4 + e] * inv);
        *reinterpret_cast<typename Op32<QT>::v4*>(ost + l32 * L::kORow + d0 * 2) = w;
      }
    constexpr int kRowsPerStore = 64 / CHK;
    // (the block's first row of this head as a uniform base, each lane's place as a 32-bit
    // element offset)
    QT* const obase = reinterpret_cast<QT*>(P.out) + ((int64_t)(c0 + row_base) * P.H_q + head) * D;
#pragma unroll
    for (int i = 0; i < kWinRows / kRowsPerStore; ++i) {
      const int r = i * kRowsPerStore + lane / CHK, ch = lane % CHK;
      const i32x4 v = *reinterpret_cast<const i32x4*>(ost + r * L::kORow + ch * 16);
      if (row_base + r < q_len) store16(obase + (r * P.H_q * D + ch * 8), v);
    }
  }
  raise();
}

template <typename QT, typename KT, int D>
static void launch_prefill_typed(const PrefillParams& P, int RW, hipStream_t stream) {
  const size_t lds = PfLds<D, sizeof(KT) == 2>::kTotal;
  dim3 grid(P.total), block(kPfThreads);
  if (RW == 1) hipLaunchKernelGGL((prefill_kernel<QT, KT, D, 1>), grid, block, lds, stream, P);
  else if (RW == 2) hipLaunchKernelGGL((prefill_kernel<QT, KT, D, 2>), grid, block, lds, stream, P);
  else hipLaunchKernelGGL((prefill_kernel<QT, KT, D, 4>), grid, block, lds, stream, P);
}

int launch_prefill_attention(const AttnArgs& a, hipStream_t stream) {
  if (a.T == 0 || a.B == 0) return SPATTN_OK;
  PrefillParams P;
  P.q = a.q; P.k_cache = a.k_cache; P.v_cache = a.v_cache;
  P.key_scale = a.key_scale; P.value_scale = a.value_scale;
  P.cu = a.cu; P.seqlens_k = a.seqlens_k; P.sinks = a.sinks; P.out = a.out; P.status = a.status;
  P.cd.block_table = a.block_table;
  P.cd.max_blocks = a.max_blocks;
  P.cd.block_size = a.block_size;
  P.cd.bs_shift = (a.block_size & (a.block_size - 1)) == 0 ? __builtin_ctz(a.block_size) : -1;
  P.cd.num_blocks = a.num_blocks;
  P.cd.H_kv = a.H_kv;
  P.cd.D = a.D;
  P.B = a.B; P.T = a.T; P.H_q = a.H_q; P.H_kv = a.H_kv; P.D = a.D;
  P.group = a.H_q / a.H_kv;
  P.max_q = a.max_q; P.max_k = a.max_k; P.window = a.window;
  P.scale_log2 = a.scale * kLog2e;
  // a window of at most kWinMax keys over a 16-bit cache, groups of 4 or more heads: the
  // one-span kernel (8 waves for groups of 8 or more, else 4)
  // (the windowed kernel addresses a block's output rows by 32-bit offsets from its first)
  if (a.window > 0 && a.window <= kWinMax && a.cache_dtype == a.dtype && P.group >= 4 &&
      (int64_t)kWinRows * a.H_q * a.D < (int64_t(1) << 31)) {
    P.n_rt = (a.max_q + kWinRows - 1) / kWinRows;
    const long total = ((long)a.B * a.H_kv + 7) / 8 * 8 * P.n_rt;
    if (total <= 0) return SPATTN_OK;
    if (total > 0x7fffffffL) return SPATTN_ERR_SHAPE;
    P.total = (int)total;
    const bool w8 = P.group >= 8;
#define SPATTN_WIN(QT, DD)                                                                      \
  if (w8) hipLaunchKernelGGL((prefill_window_kernel<QT, DD, 8>), dim3(P.total), dim3(512),      \
                             (WinLds<DD, 8>::kTotal), stream, P);                               \
  else hipLaunchKernelGGL((prefill_window_kernel<QT, DD, 4>), dim3(P.total), dim3(256),         \
                          (WinLds<DD, 4>::kTotal), stream, P)
    if (a.D == 64) {
      if (a.dtype == SPATTN_F16) { SPATTN_WIN(f16, 64); } else { SPATTN_WIN(bf16, 64); }
    } else {
      if (a.dtype == SPATTN_F16) { SPATTN_WIN(f16, 128); } else { SPATTN_WIN(bf16, 128); }
    }
#undef SPATTN_WIN
    return hipGetLastError() == hipSuccess ? SPATTN_OK : SPATTN_ERR_LAUNCH;
  }
  // workgroup = RW row blocks x (4 / RW) heads: two row blocks of two heads measured fastest
  // for groups of 4 or more (more rows per K/V tile than four heads of one row block)
  const int RW = P.group == 1 ? 4 : 2;
  const int HW = 4 / RW;
  P.n_hg = (P.group + HW - 1) / HW;
  P.n_rt = (a.max_q + 32 * RW - 1) / (32 * RW);
  const long total = (long)P.n_rt * a.B * a.H_kv * P.n_hg;
  if (total <= 0) return SPATTN_OK;
  if (total > 0x7fffffffL) return SPATTN_ERR_SHAPE;
  P.total = (int)total;
  P.xcd_pairs = (a.B * a.H_kv) % 8 == 0 ? 1 : 0;
  // INT8 caches are int8_t, FP8 E4M3 caches uint8_t
  const bool i8 = a.cache_dtype == SPATTN_I8;
  const bool fp8 = a.cache_dtype == SPATTN_FP8;
#define SPATTN_PREFILL(QT, DD)                                                            \
  if (i8) launch_prefill_typed<QT, int8_t, DD>(P, RW, stream);                            \
  else if (fp8) launch_prefill_typed<QT, uint8_t, DD>(P, RW, stream);                     \
  else launch_prefill_typed<QT, QT, DD>(P, RW, stream)
  if (a.D == 64) {
    if (a.dtype == SPATTN_F16) { SPATTN_PREFILL(f16, 64); } else { SPATTN_PREFILL(bf16, 64); }
  } else {
    if (a.dtype == SPATTN_F16) { SPATTN_PREFILL(f16, 128); } else { SPATTN_PREFILL(bf16, 128); }
  }
#undef SPATTN_PREFILL
  return hipGetLastError() == hipSuccess ? SPATTN_OK : SPATTN_ERR_LAUNCH;
}

}  // namespace spattn
