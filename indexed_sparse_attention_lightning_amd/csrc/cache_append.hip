// Cache append: the new tokens' indexer keys and latent rows, given in bf16,
// are stored into the paged pools in each pool's format.
//
// Formats (page "Day-0 Inference Adaptation and Performance Optimization for
// New-Architecture Large Language Models", section "Tiered Quantization":
// per-group dynamic scaling, scale = max|group| / quant_max, then rounding;
// page "Inference Adaptation and Performance Optimization for New Large
// Language Model Architectures", sections 4.2 and 4.3):
//   bf16  the bits are copied;
//   MX32  groups of 32: scale 2^X, X the smallest integer >= -127 with
//         448 * 2^X >= max|group| (X = 0 for an all-zero group), stored as
//         the e8m0 code X + 127; elements as e4m3fn of x * 2^-X;
//   T128  tiles of 128 features (the last of a 576-wide row holds 64): an fp32
//         scale max|tile| / 448, elements as e4m3fn of x / scale, saturated
//         at +-448 (an all-zero tile stores scale 0 and signed-zero codes).
// e4m3fn rounding is to nearest, ties to even, in fp32 with correctly
// rounded divisions, so the codes are a deterministic function of the input.
//
// One wave per token: lane l owns the 8-feature chunks l and 64 + l of a
// row, a group of 32 is four neighbouring lanes and a tile of 128 sixteen, so
// group maxima are butterfly reductions inside the wave.  The work is a few
// KB per token; the launch is latency-bound, not bandwidth-bound.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {
namespace {

constexpr int kTokensPerBlock = 4;
constexpr float kE4m3Max = 448.0f;

// e4m3fn code of y, |y| <= 448: nearest, ties to even; the sign bit is y's.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t u = __builtin_bit_cast(uint32_t, y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t b = u & 0x7fffffffu;
  const float a = __builtin_bit_cast(float, b);
  // below 2^-6 the format steps by 2^-9: scale by 2^9 (exact) and round
  const uint32_t sub = (uint32_t)__builtin_rintf(a * 512.0f);
  // otherwise keep 3 mantissa bits: round half to even at bit 20, a carry
  // moves into the exponent; rebias 127 -> 7
  const uint32_t nrm = ((b + 0x7ffffu + ((b >> 20) & 1u)) >> 20) - (120u << 3);
  return sign | (a < 0x1p-6f ? sub : nrm);
}

// Exponent X of an MX group scale for the group maximum amax (see above).
__device__ __forceinline__ int mx_exponent(float amax) {
  if (amax == 0.0f) return 0;
  const uint32_t b = __builtin_bit_cast(uint32_t, amax);
  // amax = m * 2^E, m in [1, 2): 448 * 2^(E-8) = 1.75 * 2^E covers it
  // unless m > 1.75 (mantissa field above 0x600000)
  const int X = (int)(b >> 23) - 127 - 8 + ((b & 0x7fffffu) > 0x600000u);
  return max(X, -127);
}

__device__ __forceinline__ void unpack8(const uint4 v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
    f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ uint2 pack_codes(const uint32_t (&c)[8]) {
  return make_uint2(c[0] | c[1] << 8 | c[2] << 16 | c[3] << 24,
                    c[4] | c[5] << 8 | c[6] << 16 | c[7] << 24);
}

// Maximum over the `lanes` neighbouring lanes (a power of two) holding x.
template <int LANES>
__device__ __forceinline__ float group_max(float x) {
#pragma unroll
  for (int m = 1; m < LANES; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}

// Store one bf16 row of `width` features (width / 8 <= 128 chunks) at pool
// slot `slot` in format FMT.  Every lane of the wave must call this.
template <int FMT>
__device__ __forceinline__ void store_row(const uint16_t* src, int width,
                                          uint8_t* pool, void* scale,
                                          int64_t slot, int lane) {
  const int nchunk = width / 8;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int c = lane + 64 * half;
    const bool own = c < nchunk;
    if (half == 1 && nchunk <= 64) break;   // wave-uniform
    uint4 v = make_uint4(0, 0, 0, 0);
    if (own) v = reinterpret_cast<const uint4*>(src)[c];
    if constexpr (FMT == kFmtBf16) {
      if (own)
        reinterpret_cast<uint4*>(pool + slot * width * 2)[c] = v;
      continue;
    }
    float f[8];
    unpack8(v, f);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
    uint32_t code[8];
    if constexpr (FMT == kFmtMx32) {
      amax = group_max<4>(amax);
      const int X = mx_exponent(amax);
      const float inv = __builtin_bit_cast(float, (uint32_t)(127 - X) << 23);
#pragma unroll
      for (int i = 0; i < 8; ++i) code[i] = e4m3_code(f[i] * inv);
      if (own) {
        reinterpret_cast<uint2*>(pool + slot * width)[c] = pack_codes(code);
        if ((c & 3) == 0)
          static_cast<uint8_t*>(scale)[slot * (width / 32) + c / 4] =
              (uint8_t)(X + 127);
      }
    } else {
      // tiles of 16 chunks; the 64-feature tail tile is chunks 64..71, and
      // lanes 8..15 of the second half hold no chunk (amax 0)
      amax = group_max<16>(amax);
      const float sc = __fdiv_rn(amax, kE4m3Max);
      const float div = amax > 0.0f ? sc : 1.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float y = __fdiv_rn(f[i], div);
        code[i] = e4m3_code(fminf(fmaxf(y, -kE4m3Max), kE4m3Max));
      }
      if (own) {
        reinterpret_cast<uint2*>(pool + slot * width)[c] = pack_codes(code);
        if ((c & 15) == 0)
          static_cast<float*>(scale)[slot * kT128Tiles + c / 16] = sc;
      }
    }
  }
}

template <int KFMT, int VFMT>
__global__ __launch_bounds__(64 * kTokensPerBlock) void cache_append_kernel(
    AppendLaunch p) {
  const int lane = lane_id();
  const int tok = blockIdx.x * kTokensPerBlock + threadIdx.x / 64;
  if (tok >= p.tokens) return;   // wave-uniform
  const int b = tok / p.T;
  const int pos = p.pos[tok];
  if (pos < 0 || pos / kPage >= p.max_pages) return;
  const int page = p.page_table[(int64_t)b * p.max_pages + pos / kPage];
  if (page < 0 || page >= p.num_pages) return;
  const int64_t slot = (int64_t)page * kPage + pos % kPage;
  if (p.k_new)
    store_row<KFMT>(p.k_new + (int64_t)tok * p.d_I, p.d_I, p.kidx,
                    p.kidx_scale, slot, lane);
  if (p.kv_new)
    store_row<VFMT>(p.kv_new + (int64_t)tok * kLatent, kLatent, p.kv,
                    p.kv_scale, slot, lane);
}

template <int KFMT>
hipError_t launch_v(const AppendLaunch& p, hipStream_t stream) {
  const dim3 grid((p.tokens + kTokensPerBlock - 1) / kTokensPerBlock);
  const dim3 block(64 * kTokensPerBlock);
  switch (p.kv_fmt) {
    case kFmtBf16:
      hipLaunchKernelGGL((cache_append_kernel<KFMT, kFmtBf16>), grid, block, 0,
                         stream, p);
      break;
    case kFmtMx32:
      hipLaunchKernelGGL((cache_append_kernel<KFMT, kFmtMx32>), grid, block, 0,
                         stream, p);
      break;
    default:
      hipLaunchKernelGGL((cache_append_kernel<KFMT, kFmtT128>), grid, block, 0,
                         stream, p);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cache_append(const AppendLaunch& p, hipStream_t stream) {
  return p.kidx_fmt == kFmtMx32 ? launch_v<kFmtMx32>(p, stream)
                                : launch_v<kFmtBf16>(p, stream);
}

}  // namespace dsa
