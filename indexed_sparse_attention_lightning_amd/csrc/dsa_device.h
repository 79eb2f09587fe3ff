// Device helpers shared by the DSA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kLatent = 576;     // absorbed MLA key width (512 latent + 64 rope)
constexpr int kValue = 512;      // value width
constexpr int kPage = 64;        // tokens per cache page

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// D = A * B + C on one 32x32x16 bf16 matrix-core tile.
// Operand layout (wave64): lane l holds row/col (l % 32) and the 8 k-slots
// 8*(l/32) .. +7 of A resp. B; C/D lane l holds column l % 32 and rows
// 8*(r/4) + 4*(l/32) + r%4 for accumulator register r = 0..15.
__device__ __forceinline__ f32x16 mfma32(const uint4& a, const uint4& b,
                                         f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
      __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0,
      0);
}

// max(x, 0) as one integer max on the bit pattern: the same value as
// fmaxf(x, 0) for every x that is not a NaN (negative values and -0 give
// +0, +inf stays).  fmaxf on a matrix-core result costs two instructions
// (the operand is first canonicalised for IEEE NaN rules).
__device__ __forceinline__ float relu(float x) {
  return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}

// Value held by lane (l ^ 32): the two wave halves exchange registers.
// (Only one of the instruction's two results is taken per lane: the
// compiler treats the two results of a swap of a register with itself as
// equal, which folds an expression that uses both.)
__device__ __forceinline__ float swap_halves(float x, int lane) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x),
                                            __builtin_bit_cast(int, x), false,
                                            false);
  return __builtin_bit_cast(float, lane < 32 ? r[1] : r[0]);
}
__device__ __forceinline__ float swap_halves(float x) {
  return swap_halves(x, lane_id());
}

// The lane index computed afresh (the compiler cannot reuse an earlier
// value): after a long loop, values derived from it need not stay live.
__device__ __forceinline__ int fresh_lane_id() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0"
               : "=v"(l));
  return l;
}

// Two fp32 -> packed bf16x2 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2v v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Eight e4m3fn codes (little-endian in a uint2) times the power of two whose
// fp32 bit pattern is `pow2_bits` (an e8m0 scale code c gives c << 23) ->
// eight bf16 values (uint4).  The hardware conversion uses only the exponent
// field of its fp32 scale operand.  Exact whenever the result is a normal
// bf16.
__device__ __forceinline__ uint4 dequant8_pow2(uint2 codes,
                                               uint32_t pow2_bits) {
  const float s = __builtin_bit_cast(float, pow2_bits);
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(
                                         codes.x, s, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(
                                         codes.x, s, true));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(
                                         codes.y, s, false));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(
                                         codes.y, s, true));
  return r;
}

// The same with an e8m0 scale code: times 2^(scale_code - 127).
__device__ __forceinline__ uint4 dequant8_e4m3(uint2 codes,
                                               uint32_t scale_code) {
  return dequant8_pow2(codes, scale_code << 23);
}

// Eight bf16 values (a uint4) widened to fp32 (exact).
__device__ __forceinline__ void unpack8(const uint4 v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
    f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
  }
}

// Four e4m3fn codes (nearest, ties to even, sign kept; |y| <= 448) packed
// little-endian by the hardware conversion.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// Exponent X of an MX block-32 scale for the block's largest magnitude amax:
// the smallest X >= -127 with 448 * 2^X >= amax (X = 0 for amax = 0), so no
// element saturates.  amax = m * 2^E, m in [1, 2): 448 * 2^(E-8) = 1.75 * 2^E
// covers it unless m > 1.75 (mantissa field above 0x600000).
__device__ __forceinline__ int mx_exponent(float amax) {
  if (amax == 0.0f) return 0;
  const uint32_t b = __builtin_bit_cast(uint32_t, amax);
  const int X = (int)(b >> 23) - 127 - 8 + ((b & 0x7fffffu) > 0x600000u);
  return max(X, -127);
}

// 2^-X as an fp32 (X in [-127, 126]): multiplying by it is exact.
__device__ __forceinline__ float pow2_neg(int X) {
  return __builtin_bit_cast(float, (uint32_t)(127 - X) << 23);
}

// Split of a non-negative fp32 scale s = 2^e * m for an exact bf16
// dequantisation by the scaled conversion above, which applies only the
// exponent field of its scale operand: returns the exponent part as the
// fp32 bit pattern of 2^e (2^-126 for zero or subnormal s) and sets m = s /
// 2^e (in [1, 2) for normal s; 1 for s = 0, where every code is zero).
__device__ __forceinline__ uint32_t split_scale(uint32_t s_bits, float& m) {
  const uint32_t e = s_bits & 0x7f800000u;
  if (e != 0) {
    m = __builtin_bit_cast(float, (s_bits & 0x007fffffu) | 0x3f800000u);
    return e;
  }
  m = s_bits == 0 ? 1.0f : __builtin_bit_cast(float, s_bits) * 0x1p126f;
  return 0x00800000u;
}

// A raw buffer resource over `bytes` bytes at `base`: a load at an offset
// past `bytes` returns zeros and makes no memory access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t bytes_rsrc(const void* base,
                                                          uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)bytes, 0x00020000);
}
// Cache-policy operand of a buffer load that streams (non-temporal, as
// ld16_stream below).
constexpr int kBufStream = 2;

// 128-bit non-temporal-hint-free global load / LDS access helpers.
__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}
// Loads and stores marked non-temporal, for bytes a launch touches exactly
// once in whole cache lines (the indexer's key stream, the split partials,
// the rows of a cache append): the caches do not keep the lines, and the
// streams run faster (bf16 decode indexer 49.7-51.1 us against 53.2-53.8 us
// per launch; whole-cache append 510-518 us against 531-535 us).  Where an
// instruction reads only part of a line that later ones read again, plain
// loads must stay: the line would be fetched again each time.
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_nt __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st16_stream(void* p, const uint4& v) {
  __builtin_nontemporal_store(u32x4_nt{v.x, v.y, v.z, v.w},
                              reinterpret_cast<u32x4_nt*>(p));
}
__device__ __forceinline__ void st8_stream(void* p, const uint2& v) {
  __builtin_nontemporal_store(u32x2_nt{v.x, v.y}, reinterpret_cast<u32x2_nt*>(p));
}
__device__ __forceinline__ uint2 ld8(const void* p) {
  return *reinterpret_cast<const uint2*>(p);
}

// Physical row index of logical position s of sequence b.
// page_table == nullptr: contiguous [B, L, ...] storage (row = b*L + s).
// A page entry outside [0, num_pages) is clamped into it (num_pages > 0):
// a bad table then reads wrong rows, never memory outside the pool.
__device__ __forceinline__ int64_t cache_row(const int32_t* page_table,
                                             int max_pages, int num_pages,
                                             int L, int b, int s) {
  if (page_table == nullptr) return (int64_t)b * L + s;
  int pg = page_table[(int64_t)b * max_pages + (s >> 6)];
  if (num_pages > 0) pg = min(max(pg, 0), num_pages - 1);
  return (int64_t)pg * kPage + (s & (kPage - 1));
}

// cache_row for a wave-uniform (b, s): the page-table entry is read through
// the scalar cache (the table is read-only for a launch).  A plain load of a
// uniform address becomes a vector load wherever a store precedes it in a
// loop (the compiler cannot rule out aliasing), and waiting for that one
// waits for every vector load in flight.
__device__ __forceinline__ int64_t cache_row_uniform(const int32_t* page_table,
                                                     int max_pages,
                                                     int num_pages, int L,
                                                     int b, int s) {
  if (page_table == nullptr) return (int64_t)b * L + s;
  typedef const __attribute__((address_space(4))) int32_t ConstI32;
  int pg = ((ConstI32*)page_table)[(int64_t)b * max_pages + (s >> 6)];
  if (num_pages > 0) pg = min(max(pg, 0), num_pages - 1);
  return (int64_t)pg * kPage + (s & (kPage - 1));
}

// Order-preserving map float -> uint32: larger float <=> larger key.
// -0 is folded onto +0 and every NaN onto key 1 (below all numbers, whose
// keys start at 0x007fffff for -inf); key 0 is left free as a "no position"
// marker.
__device__ __forceinline__ uint32_t score_key(float x) {
  if (x != x) return 1u;
  const uint32_t u = __builtin_bit_cast(uint32_t, x + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace dsa
