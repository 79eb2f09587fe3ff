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
// Rows are read and pool bytes written with non-temporal accesses (each is
// touched once).
// e4m3fn rounding is to nearest, ties to even, in fp32 with correctly
// rounded divisions, so the codes are a deterministic function of the input.
//
// A workgroup of four waves stores eight tokens, one 8-feature chunk per
// lane and pass: wave w takes features 0..511 of tokens 2w and 2w+1 (lane =
// chunk, so a group of 32 is four neighbouring lanes and a tile of 128
// sixteen); wave 0 also takes the 64 rope features of all eight tokens (8
// lanes each, one tile), waves 1 and 2 the indexer keys (4 or 8 tokens a
// wave).  Group maxima are butterfly reductions inside the wave; every lane
// is busy in every pass.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {
namespace {

constexpr int kTokensPerBlock = 8;   // per workgroup of four waves
constexpr float kE4m3Max = 448.0f;

// Maximum over the `lanes` neighbouring lanes (a power of two) holding x.
template <int LANES>
__device__ __forceinline__ float group_max(float x) {
#pragma unroll
  for (int m = 1; m < LANES; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}

// Physical pool slot of token `tok`, or -1 when the token is skipped (past
// the batch, negative position, position past the page table, page entry
// outside the pool).
__device__ __forceinline__ int64_t token_slot(const AppendLaunch& p, int tok) {
  if (tok >= p.tokens) return -1;
  const int pos = p.pos[tok];
  if (pos < 0 || pos / kPage >= p.max_pages) return -1;
  const int page = p.page_table[(int64_t)(tok / p.T) * p.max_pages + pos / kPage];
  if (page < 0 || page >= p.num_pages) return -1;
  return (int64_t)page * kPage + pos % kPage;
}

// This lane's chunk c (features 8c..8c+7) of a bf16 row into pool slot
// `slot` (< 0: nothing stored) of a pool of `width`-feature rows in format
// FMT.  GL neighbouring lanes form one scale group (scale index `gidx`,
// written by the group's first lane).  Every lane of the wave must call
// this: the group maximum is exchanged between lanes.
template <int FMT, int GL>
__device__ __forceinline__ void put_chunk(const uint16_t* src, int c,
                                          int64_t slot, int width,
                                          uint8_t* pool, void* scale,
                                          int nscale, int gidx, int lane) {
  const bool own = slot >= 0;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (own) v = ld16_stream(reinterpret_cast<const uint4*>(src) + c);
  if constexpr (FMT == kFmtBf16) {
    if (own) st16_stream(reinterpret_cast<uint4*>(pool + slot * width * 2) + c, v);
  } else {
    float f[8];
    unpack8(v, f);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
    amax = group_max<GL>(amax);
    float y[8];
    float sc;
    if constexpr (FMT == kFmtMx32) {
      const int X = mx_exponent(amax);
      const float inv = pow2_neg(X);
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = f[i] * inv;   // exact
      sc = __builtin_bit_cast(float, (uint32_t)(X + 127));
    } else {
      sc = __fdiv_rn(amax, kE4m3Max);
      const float div = amax > 0.0f ? sc : 1.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        y[i] = fminf(fmaxf(__fdiv_rn(f[i], div), -kE4m3Max), kE4m3Max);
    }
    if (own) {
      st8_stream(reinterpret_cast<uint2*>(pool + slot * width) + c,
                 make_uint2(e4m3x4(y[0], y[1], y[2], y[3]),
                            e4m3x4(y[4], y[5], y[6], y[7])));
      if ((lane & (GL - 1)) == 0) {
        if constexpr (FMT == kFmtMx32)
          static_cast<uint8_t*>(scale)[slot * nscale + gidx] =
              (uint8_t)__builtin_bit_cast(uint32_t, sc);
        else
          static_cast<float*>(scale)[slot * nscale + gidx] = sc;
      }
    }
  }
}

template <int KFMT, int VFMT>
__global__ __launch_bounds__(64 * 4) void cache_append_kernel(AppendLaunch p) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int tok0 = blockIdx.x * kTokensPerBlock;
  constexpr int kVGroup = VFMT == kFmtT128 ? 16 : 4;   // lanes per scale
  constexpr int kVScales = VFMT == kFmtT128 ? kT128Tiles : kLatent / 32;
  if (p.kv_new) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int tok = tok0 + 2 * wave + u;
      const int64_t slot = token_slot(p, tok);   // same for the whole wave
      if (slot >= 0)
        put_chunk<VFMT, kVGroup>(p.kv_new + (int64_t)tok * kLatent, lane, slot,
                                 kLatent, p.kv, p.kv_scale, kVScales,
                                 lane / kVGroup, lane);
    }
    if (wave == 0) {   // the rope features: 8 lanes per token
      const int tok = tok0 + lane / 8;
      const int c = 64 + (lane & 7);
      put_chunk<VFMT, VFMT == kFmtT128 ? 8 : 4>(
          p.kv_new + (int64_t)tok * kLatent, c, token_slot(p, tok), kLatent,
          p.kv, p.kv_scale, kVScales, VFMT == kFmtT128 ? 4 : c / 4, lane);
    }
  }
  if (p.k_new) {
    const int cpt = p.d_I / 8;       // chunks per key row: 16 or 8
    const int tpw = 64 / cpt;        // key rows per wave: 4 or 8
    const int kw = wave - 1;
    if (kw >= 0 && kw * tpw < kTokensPerBlock) {
      const int tok = tok0 + kw * tpw + lane / cpt;
      const int c = lane % cpt;
      put_chunk<KFMT, 4>(p.k_new + (int64_t)tok * p.d_I, c, token_slot(p, tok),
                         p.d_I, p.kidx, p.kidx_scale, p.d_I / 32, c / 4, lane);
    }
  }
}

template <int KFMT>
hipError_t launch_v(const AppendLaunch& p, hipStream_t stream) {
  const dim3 grid((p.tokens + kTokensPerBlock - 1) / kTokensPerBlock);
  const dim3 block(64 * 4);
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
