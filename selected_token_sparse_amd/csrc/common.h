// Device-side helpers shared by the gfx950 kernels of this library: element types and
// conversions, 16-byte vector loads, MFMA operand types, wave reductions, status flags
// and per-row metadata.  Nothing here is shared with the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spattn.h"

namespace spattn {

typedef _Float16 f16;
typedef __bf16 bf16;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();
// Lazy rescaling of the online softmax: a row's reference maximum (log2 domain) moves only
// when a new score exceeds it by more than this, so exp2 arguments stay <= 8 and the
// unnormalised weights <= 256 (exact relative precision in f16 / bf16, no overflow in the
// float32 sums).  Any reference <= the true maximum gives the same softmax once normalised.
constexpr float kLazyRescaleLog2 = 8.0f;

// ---------------------------------------------------------------------------------------
// element conversions
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(f16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(int8_t x) { return (float)x; }

// ---------------------------------------------------------------------------------------
// FP8 E4M3 cache codes (OCP "E4M3FN": sign, 4 exponent bits with bias 7, 3 mantissa bits,
// subnormals m * 2^-9, no infinities, 0x7F / 0xFF NaN).  Caches of this type are uint8_t
// arrays of codes.  Moving the sign to bit 15 and the 7 magnitude bits up by 7 gives the
// f16 whose value is exactly the code's value / 256 (f16 has the wider exponent and
// mantissa, subnormals included), so kernels fold the factor 256 into the per-channel
// scales.
// ---------------------------------------------------------------------------------------
constexpr float kFp8Unit = 256.0f;   // code value = f16 operand value * kFp8Unit

__device__ __forceinline__ uint16_t fp8_to_f16_bits(uint32_t b) {
  const uint32_t mag = b & 0x7Fu;
  return (uint16_t)(((b & 0x80u) << 8) | (mag << 7) | (mag == 0x7Fu ? 0x7C00u : 0u));
}
// Eight codes (the bytes of two 32-bit words, lowest first) as the same f16 operands, code
// value / 256, by the gfx950 conversion instruction with a 2^-8 scale: two codes per
// instruction instead of a few bit operations per code.  (Checked on the device for all
// 256 codes: the values match the construction above exactly; NaN codes give NaN.)
__device__ __forceinline__ f16x8 fp8x8_to_f16(int lo, int hi) {
  const auto a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f / kFp8Unit, false);
  const auto b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f / kFp8Unit, true);
  const auto c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f / kFp8Unit, false);
  const auto d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f / kFp8Unit, true);
  const i32x4 w = {__builtin_bit_cast(int32_t, a), __builtin_bit_cast(int32_t, b),
                   __builtin_bit_cast(int32_t, c), __builtin_bit_cast(int32_t, d)};
  return __builtin_bit_cast(f16x8, w);
}
// Eight INT8 codes (the bytes of two 32-bit words, lowest first) as exact f16 values: with
// the sign bit flipped a code c becomes u = c + 128 in [0, 255], the f16 with bits
// 0x6400 | u is 1024 + u exactly (spacing 1 in [1024, 2048)), and subtracting 1152 leaves
// c exactly.  Two codes per byte permute and per packed f16 subtraction.
__device__ __forceinline__ f16x8 int8x8_to_f16(int lo, int hi) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const uint32_t ul = (uint32_t)lo ^ 0x80808080u, uh = (uint32_t)hi ^ 0x80808080u;
  // byte selectors: result bytes (u_a, 0x64, u_b, 0x64), 0x64 taken from the first source
  const uint32_t w0 = __builtin_amdgcn_perm(0x64646464u, ul, 0x04010400u);
  const uint32_t w1 = __builtin_amdgcn_perm(0x64646464u, ul, 0x04030402u);
  const uint32_t w2 = __builtin_amdgcn_perm(0x64646464u, uh, 0x04010400u);
  const uint32_t w3 = __builtin_amdgcn_perm(0x64646464u, uh, 0x04030402u);
  const h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  const h2 r0 = __builtin_bit_cast(h2, w0) - bias, r1 = __builtin_bit_cast(h2, w1) - bias;
  const h2 r2 = __builtin_bit_cast(h2, w2) - bias, r3 = __builtin_bit_cast(h2, w3) - bias;
  const i32x4 w = {__builtin_bit_cast(int32_t, r0), __builtin_bit_cast(int32_t, r1),
                   __builtin_bit_cast(int32_t, r2), __builtin_bit_cast(int32_t, r3)};
  return __builtin_bit_cast(f16x8, w);
}
// Exact value of a code (NaN codes give NaN).
__device__ __forceinline__ float to_f32(uint8_t code) {
  return (float)__builtin_bit_cast(f16, fp8_to_f16_bits(code)) * kFp8Unit;
}
// Code of x / s: one IEEE float32 division, rounded to the nearest E4M3 value with ties to
// the even mantissa; magnitudes above 448 saturate to 448; a NaN quotient gives code 0.
__device__ __forceinline__ uint8_t quantize_fp8(float x, float s) {
  const float q = x / s;
  if (q != q) return 0;
  const uint32_t sign = (__float_as_uint(q) >> 24) & 0x80u;
  const float a = fabsf(q);
  if (a > 448.0f) return (uint8_t)(sign | 0x7Eu);
  uint32_t mag;
  if (a < 0.015625f) {                       // below 2^-6: multiples of 2^-9 (8 = 2^-6)
    mag = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    const uint32_t bits = __float_as_uint(a);
    int e = (int)(bits >> 23) - 127;
    uint32_t r = (bits >> 20) & 7u;
    const uint32_t rest = bits & 0xFFFFFu;
    if (rest > 0x80000u || (rest == 0x80000u && (r & 1u))) ++r;
    if (r == 8u) { r = 0; ++e; }
    mag = ((uint32_t)(e + 7) << 3) | r;
  }
  return (uint8_t)(sign | mag);
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ f16 from_f32<f16>(float x) { return (f16)x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// ---------------------------------------------------------------------------------------
// status flags (only written when a malformed input is seen)
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ void raise_status(int32_t* status, int bits) {
  if (status != nullptr && bits != 0) atomicOr(status, bits);
}

// ---------------------------------------------------------------------------------------
// wave64 reductions over lanes that differ in bits 4 and 5 (the four 16-lane groups)
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float xor_max(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}
__device__ __forceinline__ float xor_sum(float v, int mask) {
  return v + __shfl_xor(v, mask, 64);
}

// Combine lane l with lane l ^ 32 through v_permlane32_swap (a VALU swap of the two
// 32-lane halves, no LDS round trip): the two results hold v[l] and v[l ^ 32] in some order.
__device__ __forceinline__ float half_swap_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// exp2 that maps -inf to 0 and never produces NaN from (-inf) - (-inf): callers pass
// differences whose minuend is finite or -inf.
__device__ __forceinline__ float exp2_safe(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------------------
// Request lookup for a packed row.  Returns the request b with cu[b] <= r < cu[b+1], found
// by binary search (exact for a well-formed cu), or -1 if the candidate does not own the
// row.  Uniform across the workgroup when r is.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ int find_request(const int32_t* __restrict__ cu, int B, int r) {
  int lo = 0, hi = B - 1;  // largest b in [0, B) with cu[b] <= r
  if (B <= 0 || cu[0] > r) return -1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= r) lo = mid; else hi = mid - 1;
  }
  if (r < cu[lo + 1]) return lo;
  return -1;
}

// Per-row view used by every attention kernel.
struct RowInfo {
  int b;        // request, or -1 when the row is dead (zero output)
  int q_len;
  int kv_len;   // total key count of the request
  int p;        // key position of the row
};

// Resolves row r; applies the host-bound rules (q_len <= max_q, kv_len <= max_k when
// max_k >= 0) and reports malformed rows through `flags` (status bits).
__device__ __forceinline__ RowInfo resolve_row(const int32_t* __restrict__ cu,
                                               const int32_t* __restrict__ seqlens_k, int B,
                                               int r, int max_q, int max_k, int& flags) {
  RowInfo ri;
  ri.b = find_request(cu, B, r);
  ri.q_len = 0; ri.kv_len = 0; ri.p = -1;
  if (ri.b < 0) { flags |= SPATTN_STATUS_BAD_CU; return ri; }
  const int c0 = cu[ri.b];
  ri.q_len = cu[ri.b + 1] - c0;
  ri.kv_len = seqlens_k[ri.b] + 1;
  if (ri.q_len > max_q) { flags |= SPATTN_STATUS_Q_BOUND; ri.b = -1; return ri; }
  if (max_k >= 0 && ri.kv_len > max_k) { flags |= SPATTN_STATUS_K_BOUND; ri.b = -1; return ri; }
  if (ri.kv_len < ri.q_len) flags |= SPATTN_STATUS_SHORT_KV;
  ri.p = ri.kv_len - ri.q_len + (r - c0);
  return ri;
}

// ---------------------------------------------------------------------------------------
// Cache addressing: paged [nb, H_kv, bs, D] through a block table (each block holds its
// slots head by head, so one head's keys of a block are one contiguous run), or contiguous
// [nb >= B, H_kv, cap, D].  Returns the element offset of (position j, KV head c) row, or
// -1 (with a status bit in `flags`) when the slot does not exist.
// ---------------------------------------------------------------------------------------
struct CacheDesc {
  const int32_t* block_table;  // nullptr -> contiguous
  int max_blocks;              // table width
  int block_size;              // block size or capacity
  int bs_shift;                // log2(block_size) when a power of two, else -1
  int num_blocks;
  int H_kv;
  int D;
};

__device__ __forceinline__ int64_t cache_row(const CacheDesc& cd, int b, int j, int c, int& flags) {
  int blk, off;
  if (cd.block_table == nullptr) {
    if (j >= cd.block_size || b >= cd.num_blocks) { flags |= SPATTN_STATUS_CAPACITY; return -1; }
    blk = b; off = j;
  } else {
    int lb, o;
    if (cd.bs_shift >= 0) { lb = j >> cd.bs_shift; o = j & (cd.block_size - 1); }
    else { lb = j / cd.block_size; o = j - lb * cd.block_size; }
    if (lb >= cd.max_blocks) { flags |= SPATTN_STATUS_CAPACITY; return -1; }
    blk = cd.block_table[(int64_t)b * cd.max_blocks + lb];
    if (blk < 0 || blk >= cd.num_blocks) { flags |= SPATTN_STATUS_BAD_BLOCK; return -1; }
    off = o;
  }
  return (((int64_t)blk * cd.H_kv + c) * cd.block_size + off) * cd.D;
}

// Same addressing as cache_row, returned as the index of the D-element cache row (fits
// in 32 bits: the host rejects caches with 2^31 or more rows), or -1.
__device__ __forceinline__ int cache_row_index(const CacheDesc& cd, int b, int j, int c, int& flags) {
  int blk, off;
  if (cd.block_table == nullptr) {
    if (j >= cd.block_size || b >= cd.num_blocks) { flags |= SPATTN_STATUS_CAPACITY; return -1; }
    blk = b; off = j;
  } else {
    int lb, o;
    if (cd.bs_shift >= 0) { lb = j >> cd.bs_shift; o = j & (cd.block_size - 1); }
    else { lb = j / cd.block_size; o = j - lb * cd.block_size; }
    if (lb >= cd.max_blocks) { flags |= SPATTN_STATUS_CAPACITY; return -1; }
    blk = cd.block_table[(int64_t)b * cd.max_blocks + lb];
    if (blk < 0 || blk >= cd.num_blocks) { flags |= SPATTN_STATUS_BAD_BLOCK; return -1; }
    off = o;
  }
  return (blk * cd.H_kv + c) * cd.block_size + off;
}

// ---------------------------------------------------------------------------------------
// 16-byte loads / stores
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ i32x4 load16(const void* p) {
  return *reinterpret_cast<const i32x4*>(p);
}
__device__ __forceinline__ void store16(void* p, i32x4 v) { *reinterpret_cast<i32x4*>(p) = v; }

}  // namespace spattn
