// Sparse absorbed-MLA attention over the Top-K selected latent rows (gfx950).
//
// Sparse Flash Attention reads only the KV-cache entries at the indices the
// indexer selected (page "Inference Optimization for New Open-Source LLM
// Architectures", "Architectural Overview"; page "Day-0 Inference
// Optimization for a New Sparse Attention Architecture: A Technical Deep
// Dive", section 1).  With MLA absorbed, every query head attends over the
// same 576-wide latent rows (512 latent + 64 rope) as keys and over their
// first 512 features as values.
//
// One workgroup = one query token x one split of its selected rows; four
// waves, wave w owns heads 32w..32w+31.  Per 32-row tile:
//   * gather: direct-to-LDS 16-byte loads, three tiles in flight, the global
//     address of each lane chosen so that the LDS tile lands XOR-swizzled
//     (conflict-free for both read patterns below); FP8 rows land as codes
//     and are dequantised once into a bf16 tile;
//   * S^T = KV_tile . Q^T on the matrix cores (rows = M, heads = N, the 576
//     features = K), Q held as B operands: 27 of its 36 k-steps in
//     registers, the last 9 in LDS (registers are the scarce resource: O
//     takes all 256 accumulation registers);
//   * softmax in the log2 domain against a per-head reference fixed for the
//     pass (the first valid tile's max + 64), so O is never rescaled; a
//     head whose later logits exceed it by more than 64 sends the workgroup
//     through a second pass with the true max as the reference (rare);
//   * O^T += V^T . P^T: P comes straight from the S^T accumulators (its
//     accumulator layout already is a valid B operand after a k-slot
//     permutation), V^T is read with the transposing LDS read
//     (ds_read_b64_tr_b16) using the same row permutation;
//   * O (128 x 512 fp32 per token) lives in the accumulation registers.
// Splits write (O/l, log2-sum-exp) partials that a combine kernel merges.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsT = 32;                      // rows per tile
constexpr int kSlotsRow = kLatent * 2 / 16;     // 72 bf16 chunks per row
constexpr int kTileSlots = kRowsT * kSlotsRow;  // 2304
constexpr int kCodeSegs = 20;                   // 18 code blocks + 2 dummies
constexpr int kStageSlots = kCodeSegs * kWave;  // 1280
constexpr int kMaxSplitRows = 2048;
constexpr int kQRegSteps = 27;                  // Q k-steps kept in registers
constexpr int kQLdsSteps = kLatent / 16 - kQRegSteps;   // 9 in LDS
constexpr int kQLdsStride = 2 * kQLdsSteps + 1; // uint4 per head (padded)
constexpr int kQMaxSlot = 2 * kQLdsSteps;        // the padding slot: the
                                                // head's largest logit
// S^T accumulation chains of the bf16 and MX kernels: 3 and 4 chains (no
// spills in bf16) measured the same as 2 (decode attention 45.2 vs 44.9 us
// with the merge, prefill chunk 2.51 vs 2.51 ms): the chains' latency is not
// what bounds the tile loop
constexpr int kSChains = 2;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRef = 64.0f;     // log2 headroom of the first-pass reference
constexpr float kRange = 64.0f;   // largest logit excess (log2) over the
                                  // reference that the first pass accepts

// A tile is 36 blocks of 64 slots (1 KB), block (g, rg) holding chunks
// 8g..8g+7 of rows 8rg..8rg+7: chunk c of row R sits at slot
// ((c/8)*4 + R/8)*64 + (R%8)*8 + ((c%8) ^ swz(R)).  One direct-to-LDS load
// of 64 lanes fills one block, so a lane loads the same row at 16-byte
// offsets 128g + const for every g; swz spreads the rows of a block over the
// 64 banks for both read patterns of compute_tile.
__device__ __forceinline__ int kv_swz(int R) {
  return (((R >> 1) & 1) << 2) | ((R >> 2) & 3);
}
__device__ __forceinline__ int kv_slot(int R, int c) {
  return ((c >> 3) * 4 + (R >> 3)) * 64 + (R & 7) * 8 + ((c & 7) ^ kv_swz(R));
}

// Direct-to-LDS loads per tile: one builtin call = one instruction.  Tile
// j's loads are known to have landed (for every wave, after the barrier that
// follows) once each wave waits for vmcnt <= kDma(FP8): the loads of tile j+1,
// issued later, are exactly that many instructions, so with in-order
// completion none of tile j's can still be among the outstanding ones.  Any
// other vector-memory instruction (the FP8 scale loads, or anything the
// compiler adds) can only make the wait longer, never shorter; issuing the
// scale loads of a tile before its direct-to-LDS loads keeps it tight.
constexpr int kDmaBf16 = kSlotsRow / 8;         // 9 blocks of 64 x 16 B
constexpr int kDmaFp8 = kCodeSegs / 4;          // 5 code blocks per wave
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  // s_waitcnt vmcnt(N): low bits [3:0], high bits [15:14]; expcnt and
  // lgkmcnt at their maxima (not waited for)
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Workgroup barrier without the memory fence __syncthreads() implies (that
// fence would wait for every in-flight direct-to-LDS load).  `lds` also
// waits for this wave's own LDS writes first.
__device__ __forceinline__ void barrier(bool lds) {
  asm volatile("" ::: "memory");
  if (lds) __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct Split {
  int token, b, r0, r1, ntiles;
  const int32_t* rows;   // LDS: physical row per split row, ~row if invalid
};

// One 16-byte direct-to-LDS load per lane: lane l's bytes land at
// dst + 16*l.  With BUF the load is a buffer load through `rsrc` (pools under
// 4 GiB): the compiler tracks it as a plain vector-memory load, where the
// global (FLAT) form would be treated as possibly touching LDS out of order
// and turn every LDS wait into a full drain.
template <bool BUF>
__device__ __forceinline__ void dma16(const uint8_t* base,
                                      __amdgpu_buffer_rsrc_t rsrc,
                                      uint64_t off, uint4* dst) {
  if constexpr (BUF)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void*)dst, 16, (uint32_t)off,
        0, 0, 0);
  else
    __builtin_amdgcn_global_load_lds(base + off, dst, 16, 0, 0);
}

// Direct-to-LDS loads of blocks G.. of one wave's block row: block g lands 4
// blocks (4 KB) after block g-1 and reads 128 bytes further along the row.
// The step goes into the per-lane offset: the instruction's immediate offset
// would move the LDS destination as well.
template <int G>
__device__ __forceinline__ void block_loads(__amdgpu_buffer_rsrc_t rsrc,
                                            uint32_t voff, uint4* dst) {
  if constexpr (G < kDmaBf16) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void*)(dst + G * 4 * kWave),
        16, voff + G * 128, 0, 0, 0);
    block_loads<G + 1>(rsrc, voff, dst);
  }
}

// The loads of one bf16 tile as nine separate blocks, so that they can be
// spread over the matrix-core work of the tile being computed: prepare()
// looks up this lane's row, block(g) issues block (g, wave).
template <bool BUF>
struct TileLoads {
  const uint8_t* data;
  __amdgpu_buffer_rsrc_t rsrc;
  const int32_t* rows;   // the tile's 32 physical rows (~row if masked)
  uint4* dst;
  int wave;
  uint32_t voff;
  __device__ __forceinline__ void prepare() {
    const int lane = lane_id();
    const int R = wave * 8 + (lane >> 3);
    int ent = rows[R];
    ent ^= ent >> 31;
    const int cpart = ((lane & 7) ^ kv_swz(R)) * 16;
    if constexpr (BUF)
      voff = __umul24((uint32_t)ent, kLatent * 2) + cpart;
    else
      voff = (uint32_t)ent;   // 64-bit offset formed per block
    if constexpr (!BUF) cp = cpart;
  }
  int cp = 0;
  __device__ __forceinline__ void block(int g) const {
    uint4* d = dst + (g * 4 + wave) * kWave;
    if constexpr (BUF)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (__attribute__((address_space(3))) void*)d, 16, voff + g * 128,
          0, 0, 0);
    else
      __builtin_amdgcn_global_load_lds(
          data + (uint64_t)voff * (kLatent * 2) + cp + g * 128, d, 16, 0, 0);
  }
};
struct NoLoads {
  __device__ __forceinline__ void prepare() {}
  __device__ __forceinline__ void block(int) const {}
};

// Issue the direct-to-LDS loads of tile j (bf16 rows straight into a tile):
// wave w fills blocks (g, w), g = 0..8, so lane l always loads row
// 8w + l/8 and its 16-byte chunk 8g + ((l%8) ^ swz(row)): one row lookup and
// one offset per tile, the block index g goes into the instruction offset.
template <bool BUF>
__device__ __forceinline__ void issue_bf16(const AttnLaunch& p, const Split& s,
                                           __amdgpu_buffer_rsrc_t rsrc, int j,
                                           uint4* dst, int wave) {
  const int lane = lane_id();
  const int R = wave * 8 + (lane >> 3);
  int ent = s.rows[j * kRowsT + R];
  ent ^= ent >> 31;   // ~row for masked entries
  const int cpart = ((lane & 7) ^ kv_swz(R)) * 16;
  if constexpr (BUF) {
    // pools under 4 GiB hold fewer than 2^24 rows of 1152 bytes
    const uint32_t voff = __umul24((uint32_t)ent, kLatent * 2) + cpart;
    block_loads<0>(rsrc, voff, dst + wave * kWave);
  } else {
    const uint8_t* src = p.kv.data + (uint64_t)(uint32_t)ent * (kLatent * 2) + cpart;
#pragma unroll
    for (int g = 0; g < kDmaBf16; ++g)
      __builtin_amdgcn_global_load_lds(src + g * 128,
                                       dst + (g * 4 + wave) * kWave, 16, 0, 0);
  }
}

// FP8 code staging: block (cb, hb) of 64 slots holds code chunks
// 4cb..4cb+3 of rows 16hb..16hb+15, chunk c of row R at in-block slot
// (R%16)*4 + ((c%4) ^ ((R/4)%4)), so that one chunk of 16 rows is read
// without bank conflicts.  36 chunks x 32 rows = 18 blocks; wave w loads
// blocks w, w+4, .. (hb = w%2 for all of them: one row per lane), blocks 18
// and 19 are dummies (a copy of 16 and 17 into spare slots) so that every
// wave issues five loads per tile.
__device__ __forceinline__ int code_slot(int R, int c) {
  return ((c >> 2) * 2 + (R >> 4)) * 64 + (R & 15) * 4 + ((c & 3) ^ ((R >> 2) & 3));
}

// FP8: the scales of this lane's conversion slots (row lane%32: MX blocks
// 4k + wave as e8m0 codes, or 128-feature tile k as fp32 bits) into
// registers, then the code blocks by DMA -- in that order (the compiler
// barrier keeps it), so that the last kDmaFp8 vector-memory instructions of
// a tile's loads are its code blocks (see wait_vm).
template <bool BUF, bool T128>
__device__ __forceinline__ void issue_fp8(const AttnLaunch& p, const Split& s,
                                          __amdgpu_buffer_rsrc_t rsrc, int j,
                                          uint4* dst, uint32_t (&sc)[5],
                                          int wave) {
  const int lane = lane_id();
  {
    int ent = s.rows[j * kRowsT + (lane & 31)];
    ent ^= ent >> 31;
    if constexpr (T128) {
      const uint32_t* srow =
          reinterpret_cast<const uint32_t*>(p.kv.scale) + (int64_t)ent * kT128Tiles;
#pragma unroll
      for (int k = 0; k < 5; ++k) sc[k] = srow[k];
    } else {
      const uint8_t* srow = p.kv.scale + (int64_t)ent * (kLatent / 32);
#pragma unroll
      for (int k = 0; k < 5; ++k) {
        const int blk = 4 * k + wave;
        sc[k] = srow[blk < kLatent / 32 ? blk : blk - 4];
      }
    }
  }
  asm volatile("" ::: "memory");
  {
    const int R = 16 * (wave & 1) + (lane >> 2);
    int ent = s.rows[j * kRowsT + R];
    ent ^= ent >> 31;   // ~row for masked entries
    const uint64_t off = (uint64_t)(uint32_t)ent * kLatent +
                         ((lane & 3) ^ ((R >> 2) & 3)) * 16;
    static_assert(kDmaFp8 * 4 == kCodeSegs, "every wave issues kDmaFp8 blocks");
#pragma unroll
    for (int k = 0; k < kDmaFp8; ++k) {
      const int b = wave + 4 * k;                    // 18, 19: dummies
      const int cb = (b < 18 ? b : b - 2) >> 1;
      dma16<BUF>(p.kv.data, rsrc, off + cb * 64, dst + b * kWave);
    }
  }
}

// Tile-scale factors of a 32-row tile (T128), fp32 [9][32] in LDS, row-major
// by tile row: rows 0..3 hold m_t / m_(t+1), row 4 m_4, rows 5..8 m_0..m_3,
// where a row's scale of 128-feature tile t is s_t = 2^(e_t) * m_t and the
// bf16 tile holds the exact code * 2^(e_t).
constexpr int kTmulRows = 9;

// FP8 staging -> bf16 swizzled tile, exact: e4m3 * 2^k fits bf16 (MX: the
// group scale; T128: the exponent part of the tile scale, the mantissa part
// m_t goes to `tmul`).  Lane l of wave w converts row l%32, code chunks c =
// 8k + 2w + l/32 (k = 0..4, c < 36), which lie in 128-feature tile k: 16
// lanes read one chunk of 16 rows and write two chunks of the same rows,
// conflict-free both ways.
template <bool T128>
__device__ __forceinline__ void convert_fp8(const uint4* stg, uint4* tile,
                                            const uint32_t (&sc)[5], int wave,
                                            int lane, float* tmul) {
  const int R = lane & 31;
  float m[5];
  uint32_t e[5];
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    if constexpr (T128) e[k] = split_scale(sc[k], m[k]);
    else e[k] = sc[k] << 23;
  }
  if constexpr (T128) {
    if (wave == 0 && lane < 32) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        tmul[t * 32 + R] = m[t] / m[t + 1];
        tmul[(5 + t) * 32 + R] = m[t];
      }
      tmul[4 * 32 + R] = m[4];
    }
  }
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    const int c = 8 * k + 2 * wave + (lane >> 5);
    if (k < 4 || wave < 2) {   // c < 36 (wave-uniform)
      const uint4 v = stg[code_slot(R, c)];
      tile[kv_slot(R, 2 * c)] = dequant8_pow2(make_uint2(v.x, v.y), e[k]);
      tile[kv_slot(R, 2 * c + 1)] = dequant8_pow2(make_uint2(v.z, v.w), e[k]);
    }
  }
}

struct HeadState {
  uint4 qb[kQRegSteps];     // B operands: this lane's head, 8 features/k-step
  f32x16 o[kValue / 32];    // O^T accumulators, 16 dv tiles of 32
  float m, l;               // softmax reference (log2 units) and partial sum
  int* redo;                // LDS: set when a logit exceeds m by > kRange
};

__device__ __forceinline__ s16x4 lds_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (s16x4 __attribute__((address_space(3)))*)(
          (__attribute__((address_space(3))) char*)(p)));
}

// S^T accumulation in VGPRs.  The O accumulator fills all 256 AGPRs, so the
// S^T chain uses the VGPR form of the 32x32x16 bf16 MFMA, issued directly:
// the first starts from a zero accumulator (its result registers may not
// overlap its operands: early clobber), the chained ones accumulate into
// exactly the same registers (back-to-back dependent accumulation, which the
// hardware forwards), and the last is followed by enough wait states before
// any VALU instruction reads the result.
__device__ __forceinline__ void mfma32_vgpr_first(f32x16& c, const uint4& a,
                                                  const uint4& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
               : "=&v"(c)
               : "v"(__builtin_bit_cast(bf16x8, a)),
                 "v"(__builtin_bit_cast(bf16x8, b)));
}
__device__ __forceinline__ void mfma32_vgpr(f32x16& c, const uint4& a,
                                            const uint4& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
               : "+v"(c)
               : "v"(__builtin_bit_cast(bf16x8, a)),
                 "v"(__builtin_bit_cast(bf16x8, b)));
}
__device__ __forceinline__ void mfma32_vgpr_last(f32x16& c, const uint4& a,
                                                 const uint4& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
      "s_nop 7\n\ts_nop 7\n\ts_nop 7"
      : "+v"(c)
      : "v"(__builtin_bit_cast(bf16x8, a)), "v"(__builtin_bit_cast(bf16x8, b)));
}

// A pair of chained products (one per chain) that start right after VALU
// writes to their accumulators: the leading wait states cover the VALU-write
// to matrix-core-read dependency.
__device__ __forceinline__ void mfma32_pair_after_valu(f32x16& c0, const uint4& a0,
                                                       const uint4& b0, f32x16& c1,
                                                       const uint4& a1,
                                                       const uint4& b1) {
  asm("s_nop 4\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %4, %5, %1"
      : "+v"(c0), "+v"(c1)
      : "v"(__builtin_bit_cast(bf16x8, a0)), "v"(__builtin_bit_cast(bf16x8, b0)),
        "v"(__builtin_bit_cast(bf16x8, a1)), "v"(__builtin_bit_cast(bf16x8, b1)));
}
// The last products of both chains, then enough wait states for VALU reads
// of either accumulator.
__device__ __forceinline__ void mfma32_pair_last(f32x16& c0, const uint4& a0,
                                                 const uint4& b0, f32x16& c1,
                                                 const uint4& a1, const uint4& b1) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %4, %5, %1\n\t"
      "s_nop 7\n\ts_nop 7\n\ts_nop 7"
      : "+v"(c0), "+v"(c1)
      : "v"(__builtin_bit_cast(bf16x8, a0)), "v"(__builtin_bit_cast(bf16x8, b0)),
        "v"(__builtin_bit_cast(bf16x8, a1)), "v"(__builtin_bit_cast(bf16x8, b1)));
}

// Sixteen per-row factors of this lane's S^T rows 8(r/4) + 4h + r%4 from
// row `a` of the T128 factor table.
__device__ __forceinline__ void tile_factors(const float* tmul, int a, int h,
                                             float (&f)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 v = *reinterpret_cast<const float4*>(tmul + a * 32 + 8 * q + 4 * h);
    f[4 * q] = v.x;
    f[4 * q + 1] = v.y;
    f[4 * q + 2] = v.z;
    f[4 * q + 3] = v.w;
  }
}

// One 32-row tile for this wave's 32 heads.  `vmask` bit R says whether tile
// row R is a real selected row.  T128: the tile holds code * 2^(e_t) and
// row R's factor m_t(R) of 128-feature tile t enters exactly: the S^T chains
// are rescaled by m_t / m_(t+1) at each tile boundary (k-step 8t) and by m_4
// at the end, so S^T = sum_t m_t * S^T_t; for O^T the factor multiplies P
// (rounded to bf16 with it) before the products of value tile t.
template <bool T128, class Loads>
__device__ __forceinline__ void compute_tile(const uint4* tile,
                                             const uint4* qrow, uint32_t vmask,
                                             HeadState& st, float sl2,
                                             int lane, Loads& loads,
                                             const float* tmul) {
  const int n = lane & 31, h = lane >> 5;
  const char* tb = reinterpret_cast<const char*>(tile);
  loads.prepare();
  // ---- S^T = KV . Q^T.  Chunk 2ks+h of row n; for ks = 4u + v the slot is
  // that of chunk 2v+h plus u blocks of 4 (4 KB), so four base addresses.
  f32x16 acc;
  {
    int aoff[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) aoff[v] = kv_slot(n, 2 * v + h) * 16;
    auto a_at = [&](int ks) {
      return *reinterpret_cast<const uint4*>(tb + aoff[ks & 3] + 4096 * (ks >> 2));
    };
    auto b_at = [&](int ks) {
      return ks < kQRegSteps ? st.qb[ks < kQRegSteps ? ks : 0]
                             : qrow[(ks - kQRegSteps) * 2];
    };
    // independent accumulation chains (k-step ks feeds chain ks % kChains;
    // T128: two, even / odd) and operands fetched three k-steps ahead keep
    // the matrix core fed
    constexpr int kS = kLatent / 16;   // 36 k-steps
    constexpr int kAhead = 3;
    constexpr int kChains = T128 ? 2 : kSChains;
    static_assert(kS % kChains == 0, "whole chains");
    uint4 aq[kAhead + 1], bq[kAhead + 1];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      aq[i] = a_at(i);
      bq[i] = b_at(i);
    }
    f32x16 accs[kChains - 1];   // chains 1.. (chain 0 is acc)
    uint4 ap, bp;   // T128: the even operands of a pair issued together
#pragma unroll
    for (int ks = 0; ks < kS; ++ks) {
      if (ks + kAhead < kS) {
        aq[(ks + kAhead) % (kAhead + 1)] = a_at(ks + kAhead);
        bq[(ks + kAhead) % (kAhead + 1)] = b_at(ks + kAhead);
      }
      // one block of the next tile's loads every fourth k-step (k-steps 2,
      // 6, ..., 34), so the address unit drains while the matrix core works
      static_assert(kS / 4 == kDmaBf16, "one block per four k-steps");
      if ((ks & 3) == 2) loads.block(ks >> 2);
      const uint4 a = aq[ks % (kAhead + 1)], b = bq[ks % (kAhead + 1)];
      f32x16& c = (ks % kChains) ? accs[(ks % kChains) - 1] : acc;
      // T128: the first and last k-step pairs of each 128-feature tile
      const bool pair_first = T128 && ks >= 8 && (ks & 7) < 2;
      const bool pair_last = T128 && ((ks & 7) >= 6 || ks >= kS - 2);
      if (pair_first || pair_last) {
        f32x16& acc1 = accs[0];
        if ((ks & 1) == 0) {
          ap = a;
          bp = b;
        } else if (pair_first) {
          mfma32_pair_after_valu(acc, ap, bp, acc1, a, b);
        } else {
          mfma32_pair_last(acc, ap, bp, acc1, a, b);
          if (ks < kS - 2) {
            float f[16];
            tile_factors(tmul, ks >> 3, h, f);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              acc[r] *= f[r];
              acc1[r] *= f[r];
            }
          }
        }
      } else if (ks < kChains) {
        mfma32_vgpr_first(c, a, b);
      } else if (T128 || ks + 1 < kS) {
        mfma32_vgpr(c, a, b);
      } else {   // the last product: wait states before the VALU reads
        mfma32_vgpr_last(c, a, b);
      }
    }
    if constexpr (T128) {
      float f[16];
      tile_factors(tmul, 4, h, f);
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = (acc[r] + accs[0][r]) * f[r];
    } else {
#pragma unroll
      for (int k = 0; k < kChains - 1; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] += accs[k][r];
    }
  }
  // ---- online softmax (lane: head n, rows 8(r/4) + 4h + r%4 of the tile).
  // The scale (> 0) is applied once to the max and folded into the exp2
  // argument, fma(s, sl2, -m): masked rows are -inf before scaling.
  if (vmask != 0xffffffffu) {   // some row of the tile is not selected
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int R = 8 * (r >> 2) + 4 * h + (r & 3);
      acc[r] = ((vmask >> R) & 1u) ? acc[r] : -__builtin_inff();
    }
  }
  float tmax = -__builtin_inff();
#pragma unroll
  for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, acc[r]);
  tmax = fmaxf(tmax, swap_halves(tmax)) * sl2;
  // Per-head reference m (log2 units), fixed for the whole pass so that O
  // never needs rescaling (a rescale of the 256 accumulation registers
  // would cost the loop its register allocation): in the first pass, the
  // first valid tile's max + kRef, so later rows up to kRef + kRange above
  // that max stay representable (p <= 2^kRange); `mx` tracks the true max.
  // A head whose logits go past that range is flagged, and the workgroup
  // runs its rows a second time with m = the true max (p <= 1) -- a rare
  // path: N(0,1) inputs stay within a few units of the first tile's max.
  // (Both kept in LDS: the loop has no registers to spare.  The max sits
  // in the padding slot of the head's query row in LDS, so the lanes of
  // the first half reach it at a fixed offset from their query pointer.)
  if (h == 0)
    __hip_atomic_fetch_max(reinterpret_cast<float*>(
                               const_cast<uint4*>(qrow) + kQMaxSlot),
                           tmax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  if (st.m == -__builtin_inff() && tmax != -__builtin_inff()) st.m = tmax + kRef;
  if (tmax > st.m + kRange) *st.redo = 1;
  // no reference yet (no valid row so far): subtracting +inf gives p = 0
  const float mref = st.m != -__builtin_inff() ? st.m : __builtin_inff();
  uint4 pb[2];
  float pr[16];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    float* p = pr + 8 * kk;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[8 * kk + e], sl2, -mref));
      st.l += p[e];
    }
    if constexpr (!T128)
      pb[kk] = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                          pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7]));
  }
  // ---- O^T += V^T . P^T with transposing LDS reads.  Lane (G = lane/16,
  // i = lane%16) supplies the address of row Ra = 16kk + 4h + i/4 (Rb = Ra+8
  // for k-slots 4..7) at features 32t + f0, f0 = 16(G&1) + 4(i&3).  Chunk
  // 4t + c0 of a row sits in block t/2 at in-block chunk 4((t&1) ^ s2) +
  // (c0 ^ s01) with s2, s01 the row's swizzle bits, which gives two bases
  // (even/odd t) per row; rows 16kk + R are 2kk blocks further.
  {
    const int G = lane >> 4, i = lane & 15;
    const int f0 = 16 * (G & 1) + 4 * (i & 3);
    const int c0 = f0 >> 3, e0 = (f0 & 7) * 2;
    const int Ra = 4 * h + (i >> 2), Rb = Ra + 8;
    const int swa = kv_swz(Ra), swb = kv_swz(Rb);
    const int s2 = (swa >> 2) * 64;          // same for Ra and Rb
    const int pa = (Ra & 7) * 128 + (c0 ^ (swa & 3)) * 16 + e0;
    const int pbo = 1024 + (Rb & 7) * 128 + (c0 ^ (swb & 3)) * 16 + e0;
    const int pa_e = pa + s2, pa_o = pa + 64 - s2;
    const int pb_e = pbo + s2, pb_o = pbo + 64 - s2;
    auto rd = [&](int kk, int t) {
      const int off = kk * 2048 + (t >> 1) * 4096;
      const uint2 ua = __builtin_bit_cast(uint2, lds_tr16(tb + ((t & 1) ? pa_o : pa_e) + off));
      const uint2 ub = __builtin_bit_cast(uint2, lds_tr16(tb + ((t & 1) ? pb_o : pb_e) + off));
      return make_uint4(ua.x, ua.y, ub.x, ub.y);
    };
    // V^T operands read seven MFMAs ahead.  Product i covers k-half kk(i)
    // and dv tile t(i); T128 orders them by 128-feature value tile (four dv
    // tiles each) so that one scaled P serves eight products.
    constexpr int kN = 2 * (kValue / 32);   // 32 MFMAs
    constexpr int kAhead = 7;
    auto kk_of = [](int i) { return T128 ? (i >> 2) & 1 : i / (kValue / 32); };
    auto t_of = [](int i) {
      return T128 ? 4 * (i >> 3) + (i & 3) : i % (kValue / 32);
    };
    uint4 vq[kAhead + 1];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) vq[i] = rd(kk_of(i), t_of(i));
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      if (i + kAhead < kN)
        vq[(i + kAhead) % (kAhead + 1)] = rd(kk_of(i + kAhead), t_of(i + kAhead));
      if constexpr (T128) {
        if ((i & 7) == 0) {
          float f[16];
          tile_factors(tmul, 5 + (i >> 3), h, f);
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const float* q = pr + 8 * kk;
            const float* g = f + 8 * kk;
            pb[kk] = make_uint4(pack_bf16x2(q[0] * g[0], q[1] * g[1]),
                                pack_bf16x2(q[2] * g[2], q[3] * g[3]),
                                pack_bf16x2(q[4] * g[4], q[5] * g[5]),
                                pack_bf16x2(q[6] * g[6], q[7] * g[7]));
          }
        }
      }
      const int t = t_of(i);
      st.o[t] = mfma32(vq[i % (kAhead + 1)], pb[kk_of(i)], st.o[t]);
    }
  }
}

template <int FMT, bool BUF>
__global__ __launch_bounds__(kThreads, 1) void sparse_mla_kernel(
    AttnLaunch p, int rows_per_split) {
  constexpr bool FP8 = FMT != kFmtBf16;
  constexpr bool T128 = FMT == kFmtT128;
  constexpr int kBufSlots = FP8 ? kStageSlots : kTileSlots;
  // Separate arrays: the compiler then knows that reads of one tile buffer
  // cannot touch the direct-to-LDS loads in flight into another, and waits
  // only for the loads of the tile it reads.
  __shared__ uint4 buf0[kBufSlots];
  __shared__ uint4 buf1[kBufSlots];
  __shared__ uint4 buf2[kBufSlots];
  __shared__ uint4 ftile[FP8 ? kTileSlots : 1];
  __shared__ int32_t rows[kMaxSplitRows];
  __shared__ int rowcnt[kMaxSplitRows / kThreads][kThreads / kWave];
  __shared__ uint4 qlds[128 * kQLdsStride];
  __shared__ float tmul[T128 ? kTmulRows * 32 : 1];
  __shared__ int redo;   // some head needs the second softmax pass
  static_assert(32 * (128 * 4 + 16) <= kBufSlots * 16 &&
                    32 * (128 * 4 + 16) <=
                        (FP8 ? kTileSlots : 128 * kQLdsStride) * 16,
                "epilogue staging regions");

  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  // Block -> (token, split).  Workgroups are dealt to the 8 XCDs round-robin
  // by linear id; when the token count allows, all splits of a token go to
  // one XCD so that its queries come from that XCD's L2 after the first read.
  const int nsplit = gridDim.x, ntok = gridDim.y;
  const int lin = blockIdx.y * nsplit + blockIdx.x;
  int token = blockIdx.y, split = blockIdx.x;
  if ((ntok & 7) == 0) {
    const int xcd = lin & 7, slot = lin >> 3;
    token = (slot / nsplit) * 8 + xcd;
    split = slot % nsplit;
  }
  // Several queries per sequence (a prefill chunk): take them last to first.
  // Later queries have the longer causal rows, so the longest work items
  // start first and the short ones fill the tail (largest-first list
  // scheduling; measured 1.77 -> 1.73 ms for a 4096-query chunk from
  // position 0, no change when every row is full).
  if (p.T > 1) {
    const int bb = token / p.T, tt = token % p.T;
    token = bb * p.T + (p.T - 1 - tt);
  }
  Split s;
  s.token = token;
  s.b = s.token / p.T;
  s.r0 = split * rows_per_split;
  s.r1 = min(s.r0 + rows_per_split, p.K);
  s.ntiles = (s.r1 - s.r0 + kRowsT - 1) / kRowsT;
  s.rows = rows;
  const int32_t* idx = p.idx + (int64_t)s.token * p.K;

  // physical rows of this split; entries that are -1 or out of range hold
  // ~(row of position 0), a valid and finite row, so that their loads stay in
  // bounds (their logits are masked)
  const int nvalid = p.seq_lens ? p.seq_lens[s.b] : p.kv.L;
  const int dummy = nvalid > 0 ? (int)cache_row(p.kv.page_table,
                                                p.kv.max_pages, p.kv.num_pages, p.kv.L, s.b, 0)
                                 : 0;
  // all index loads of a thread first, then the query loads (in flight
  // while the page-table lookups run), then the row table
  constexpr int kRowIter = kMaxSplitRows / kThreads;   // 8
  int pos[kRowIter];
#pragma unroll
  for (int u = 0; u < kRowIter; ++u) {
    const int i = tid + u * kThreads;
    const int r = s.r0 + i;
    pos[u] = r < s.r1 ? idx[r] : -1;
  }
  const int n = lane & 31, h = lane >> 5;
  const int head = wave * 32 + n;
  const bool active = wave * 32 < p.H;   // wave-uniform
  HeadState st;
  st.m = -__builtin_inff();
  st.l = 0.f;
  st.redo = &redo;
#pragma unroll
  for (int t = 0; t < kValue / 32; ++t) st.o[t] = f32x16{};
  constexpr int kQL = 128 * 2 * kQLdsSteps / kThreads;   // 9 per thread
  uint4 qv[kQL];
  {
    const uint16_t* qh = p.q + ((int64_t)s.token * p.H + min(head, p.H - 1)) * kLatent;
#pragma unroll
    for (int ks = 0; ks < kQRegSteps; ++ks) st.qb[ks] = ld16(qh + ks * 16 + h * 8);
#pragma unroll
    for (int u = 0; u < kQL; ++u) {
      const int i = tid + u * kThreads;
      const int hd = i / (2 * kQLdsSteps), r = i % (2 * kQLdsSteps);
      qv[u] = ld16(p.q + ((int64_t)s.token * p.H + min(hd, p.H - 1)) * kLatent +
                   (kQRegSteps + (r >> 1)) * 16 + (r & 1) * 8);
    }
  }
#pragma unroll
  for (int u = 0; u < kRowIter; ++u)
    if (!(pos[u] >= 0 && pos[u] < nvalid)) pos[u] = -1;
  // The valid entries are compacted, in index order, to the front of the row
  // table and only their tiles are run: padding (-1) and out-of-range entries
  // cost neither loads nor products (a causal row shorter than K, or a short
  // sequence, leaves most of its K entries empty).  A split without valid
  // entries keeps one all-masked tile (out = 0, lse = -inf).
  uint64_t bal[kRowIter];
#pragma unroll
  for (int u = 0; u < kRowIter; ++u) {
    bal[u] = __builtin_amdgcn_ballot_w64(pos[u] >= 0);
    if (lane == 0) rowcnt[u][wave] = __builtin_popcountll(bal[u]);
  }
  // the cache row of every entry, the page-table lookups issued together
  // under one test of the table pointer (a lookup per entry, each behind
  // its own branch, was issued and waited for one at a time); entries
  // without a position look up position 0
  int prow[kRowIter];
  if (p.kv.page_table != nullptr) {
    const int32_t* const pt = p.kv.page_table + (int64_t)s.b * p.kv.max_pages;
    int pg[kRowIter];
#pragma unroll
    for (int u = 0; u < kRowIter; ++u) pg[u] = pt[max(pos[u], 0) >> 6];
#pragma unroll
    for (int u = 0; u < kRowIter; ++u) {
      const int g = p.kv.num_pages > 0 ? min(max(pg[u], 0), p.kv.num_pages - 1) : pg[u];
      prow[u] = g * kPage + (max(pos[u], 0) & (kPage - 1));
    }
  } else {
#pragma unroll
    for (int u = 0; u < kRowIter; ++u) prow[u] = s.b * p.kv.L + max(pos[u], 0);
  }
  barrier(true);
  {
    const uint64_t below = (1ull << lane) - 1;
    int base = 0;
#pragma unroll
    for (int u = 0; u < kRowIter; ++u) {
      int off = base;
#pragma unroll
      for (int w = 0; w < kThreads / kWave; ++w) {
        off += w < wave ? rowcnt[u][w] : 0;
        base += rowcnt[u][w];
      }
      if (pos[u] >= 0)
        rows[off + __builtin_popcountll(bal[u] & below)] = prow[u];
    }
    s.ntiles = max(1, (base + kRowsT - 1) / kRowsT);
    if (base + tid < s.ntiles * kRowsT) rows[base + tid] = ~dummy;
  }
  barrier(true);

  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.kv.data, (short)0,
      (int)(BUF ? (uint32_t)p.kv.bytes : 0u), 0x00020000);
  // the first two tiles go out while the queries are still arriving
  uint32_t sc0[5], sc1[5], sc2[5];
  constexpr int per_tile = FP8 ? kDmaFp8 : kDmaBf16;
  auto issue = [&](int j, uint4* dst, uint32_t (&sc)[5]) {
    if constexpr (FP8) issue_fp8<BUF, T128>(p, s, rsrc, j, dst, sc, wave);
    else issue_bf16<BUF>(p, s, rsrc, j, dst, wave);
  };
  issue(0, buf0, sc0);
  issue(min(1, s.ntiles - 1), buf1, sc1);

  // the last k-steps of every head of this token go to LDS
#pragma unroll
  for (int u = 0; u < kQL; ++u) {
    const int i = tid + u * kThreads;
    const int hd = i / (2 * kQLdsSteps), r = i % (2 * kQLdsSteps);
    qlds[hd * kQLdsStride + r] = hd < p.H ? qv[u] : make_uint4(0, 0, 0, 0);
  }
  if (head >= p.H) {
#pragma unroll
    for (int ks = 0; ks < kQRegSteps; ++ks) st.qb[ks] = make_uint4(0, 0, 0, 0);
  }
  if (tid == 0) redo = 0;
  if (tid < 128)
    *reinterpret_cast<float*>(qlds + tid * kQLdsStride + kQMaxSlot) =
        -__builtin_inff();
  barrier(true);
  const uint4* qrow = qlds + (wave * 32 + n) * kQLdsStride + h;
  const float sl2 = p.scale * kLog2e;

  {
    // Every step issues the loads of tile j+2 (clamped to the last tile, an
    // L2 hit, when past the end) and the step count is padded to a multiple
    // of three: each path then issues the same loads into the same buffers,
    // which keeps the compiler from falling back to waiting for all of them.
    // Step j: wait for tile j (tile j+1 may still be in flight), one barrier
    // (every wave is done with step j-1, so its buffer is free), issue the
    // loads of tile j+2 into that buffer, then compute tile j.  Every step
    // issues the same loads (clamped to the last tile, an L2 hit, past the
    // end) and the step count is padded to a multiple of three, so each path
    // issues the same loads into the same buffers and the compiler keeps its
    // exact per-buffer waits.
    auto step = [&](int j, uint4* cur, uint4* nxt, uint32_t (&scc)[5],
                    uint32_t (&scn)[5]) {
      wait_vm<per_tile>();
      barrier(false);
      const int jn = min(j + 2, s.ntiles - 1);
      // bf16: a wave that computes this step spreads the loads of tile j+2
      // over its S^T products; otherwise they all go out here
      const bool spread = !FP8 && active && j < s.ntiles;   // wave-uniform
      if (!spread) issue(jn, nxt, scn);
      if (j < s.ntiles) {
        const uint4* tile = cur;
        if constexpr (FP8) {
          convert_fp8<T128>(cur, ftile, scc, wave, lane, tmul);
          barrier(true);
          tile = ftile;
        }
        if (active) {
          const uint32_t vmask = (uint32_t)__builtin_amdgcn_ballot_w64(
              s.rows[j * kRowsT + (lane & 31)] >= 0);
          if constexpr (FP8) {
            NoLoads none;
            compute_tile<T128>(tile, qrow, vmask, st, sl2, lane, none, tmul);
          } else {
            TileLoads<BUF> tl{p.kv.data, rsrc, s.rows + jn * kRowsT, nxt, wave, 0u};
            compute_tile<false>(tile, qrow, vmask, st, sl2, lane, tl, tmul);
          }
        }
        // FP8: the barrier at the start of the next step also keeps its
        // conversion from overwriting ftile while a wave still reads it
      }
    };
    const int nsteps = (s.ntiles + 2) / 3 * 3;
    for (int pass = 0;; ++pass) {
      for (int j = 0; j < nsteps; j += 3) {
        step(j, buf0, buf2, sc0, sc2);
        step(j + 1, buf1, buf0, sc1, sc0);
        step(j + 2, buf2, buf1, sc2, sc1);
      }
      wait_vm<0>();
      if (pass == 1) break;
      barrier(true);   // also: every wave is done with the tile buffers
      if (redo == 0) break;
      // second pass: every head of the workgroup restarts with its true
      // max as the reference (all of a tile's loads are shared by the waves)
      const int lane = fresh_lane_id();
      const int n = lane & 31, h = lane >> 5;
      const int head = wave * 32 + n;
#pragma unroll
      for (int t = 0; t < kValue / 32; ++t) st.o[t] = f32x16{};
      st.l = 0.f;
      st.m = *reinterpret_cast<const float*>(qlds + head * kQLdsStride + kQMaxSlot);
      // the query operands are loaded again rather than kept live across
      // the end of the first pass (registers: the loop has none to spare)
      {
        const uint16_t* qh =
            p.q + ((int64_t)s.token * p.H + min(head, p.H - 1)) * kLatent;
#pragma unroll
        for (int ks = 0; ks < kQRegSteps; ++ks)
          st.qb[ks] = head < p.H ? ld16(qh + ks * 16 + h * 8) : make_uint4(0, 0, 0, 0);
      }
      issue(0, buf0, sc0);
      issue(min(1, s.ntiles - 1), buf1, sc1);
    }
  }
  if (!active) return;   // wave-uniform; ended waves leave the barriers

  // lane-derived values afresh: keeping them across the loop costs spills
  const int lane2 = fresh_lane_id();
  const int n2 = lane2 & 31, h2 = lane2 >> 5;
  const int head2 = wave * 32 + n2;
  const float ltot = st.l + swap_halves(st.l, lane2);
  const int dvb = 4 * h2;   // first of this lane2's 4 consecutive dv per group
  if (gridDim.x == 1) {
    // The output rows (fp32) go through LDS a quarter (128 values) at a
    // time, so that every store instruction writes two heads' 512-byte row
    // quarters, whole cache lines (straight from the accumulator layout a
    // store wrote 32 bytes of each of 32 rows).  Each wave stages in a
    // buffer of its own, rows 16 bytes apart beyond their length.
    barrier(true);   // every wave is done reading the tiles and Q
    char* const stg = reinterpret_cast<char*>(
        wave == 0 ? buf0 : wave == 1 ? buf1 : wave == 2 ? buf2 : (FP8 ? ftile : qlds));
    constexpr int kRowQ = 128 * 4 + 16;   // staged row quarter (bytes)
    const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
    float* const o0 = p.out + ((int64_t)s.token * p.H + wave * 32) * kValue;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16& ot = st.o[4 * k + tt];
          *reinterpret_cast<float4*>(stg + n2 * kRowQ + (32 * tt + 8 * g + dvb) * 4) =
              make_float4(ot[4 * g] * inv, ot[4 * g + 1] * inv,
                          ot[4 * g + 2] * inv, ot[4 * g + 3] * inv);
        }
      // a wave's LDS accesses run in order: the next quarter may overwrite
      // this one once its reads are issued
#pragma unroll 4
      for (int i = 0; i < 16; ++i) {
        const int r = 2 * i + (lane2 >> 5);
        const float4 v =
            *reinterpret_cast<const float4*>(stg + r * kRowQ + (lane2 & 31) * 16);
        if (wave * 32 + r < p.H)
          *reinterpret_cast<float4*>(o0 + (int64_t)r * kValue + 128 * k +
                                     (lane2 & 31) * 4) = v;
      }
    }
    if (h2 == 0 && head2 < p.H)
      p.lse[(int64_t)s.token * p.H + head2] =
          ltot > 0.f ? (st.m + __builtin_log2f(ltot)) * kLn2 : -__builtin_inff();
  } else {
    // partial of this split: O / l in bf16 (relative rounding 2^-9, well
    // inside the output tolerance) plus (m, l) in fp32.  The values stay in
    // the accumulator layout: lane (n, h2) writes its 16 values of value
    // block t as two 16-byte pieces, piece q = rows 8q..8q+7, at slot
    // (t, q, lane) of the wave's 32-head block, so every store instruction
    // writes 1 KB contiguous and no LDS staging or barrier is needed; the
    // combine reads the same layout.  Head blocks are 32 heads (padded).
    const int Hp = (p.H + 31) & ~31;
    const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
    const int64_t slot0 = ((int64_t)s.token * gridDim.x + split) * Hp + wave * 32;
    uint4* const o0 = reinterpret_cast<uint4*>(
        reinterpret_cast<uint16_t*>(p.partial) + slot0 * kValue);
#pragma unroll
    for (int t = 0; t < kValue / 32; ++t)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const f32x16& ot = st.o[t];
        st16_stream(o0 + (t * 2 + q) * kWave + lane2,
                    make_uint4(pack_bf16x2(ot[8 * q] * inv, ot[8 * q + 1] * inv),
                               pack_bf16x2(ot[8 * q + 2] * inv, ot[8 * q + 3] * inv),
                               pack_bf16x2(ot[8 * q + 4] * inv, ot[8 * q + 5] * inv),
                               pack_bf16x2(ot[8 * q + 6] * inv, ot[8 * q + 7] * inv)));
      }
    const int64_t slot = slot0 + n2;
    if (h2 == 0 && head2 < p.H) {
      const int64_t nslots = (int64_t)gridDim.y * gridDim.x * Hp;
      float* ml = reinterpret_cast<float*>(
                      reinterpret_cast<uint16_t*>(p.partial) + nslots * kValue) +
                  2 * slot;
      // the split's log2-sum-exp: the combine weighs splits by it
      ml[0] = ltot > 0.f ? st.m + __builtin_log2f(ltot) : -__builtin_inff();
      ml[1] = 0.f;
    }
  }
}

// Merge split partials (written and read non-temporal: each is touched once
// per step).  Split s carries O_s / l_s and its log2-sum-exp
// g_s = m_s + log2(l_s); with G the largest g_s, out = sum_s w_s * (O_s / l_s)
// / sum_s w_s, w_s = 2^(g_s - G) in (0, 1], and lse = ln 2 * (G +
// log2(sum_s w_s)).  The split with the largest sum weighs exactly 1, so no
// split that matters can underflow, however far apart the splits' softmax
// references are.  The partials are in the attention kernel's accumulator
// layout; one wave merges value block t of a 32-head group of a token, lane
// (n, h) the 16 values of head 32g + n at features 32t + 8(r/4) + 4h + r%4,
// r = 0..15, each split's two 16-byte pieces read as 1 KB per instruction.
// Every load of a lane (all splits' g, then all splits' pieces) is issued
// before any is used, so the splits' latencies overlap.
constexpr int kMaxSplits = 32;
constexpr int kCombWaves = 4;   // waves per workgroup
// MAXS: the split count bound the registers are sized for; QPL: 16-byte
// pieces per lane (2: a wave merges a whole value block of its 32 heads;
// 1: half of one, twice the waves -- for many splits over few tokens)
template <int MAXS, int QPL>
__global__ __launch_bounds__(64 * kCombWaves) void combine_kernel(AttnLaunch p,
                                                                  int splits) {
  const int token = blockIdx.x, grp = blockIdx.y;
  const int wave = (int)(threadIdx.x / 64), lane = (int)(threadIdx.x & 63);
  const int unit = blockIdx.z * kCombWaves + wave;   // (block, piece) unit
  const int t = unit / (2 / QPL);                    // value block
  const int q0 = (unit % (2 / QPL)) * QPL;           // first piece
  const int n = lane & 31, h = lane >> 5;
  const int head = grp * 32 + n;
  const int Hp = (p.H + 31) & ~31;
  const int64_t nslots = (int64_t)gridDim.x * splits * Hp;
  const uint16_t* po = reinterpret_cast<const uint16_t*>(p.partial);
  const float* ml = reinterpret_cast<const float*>(po + nslots * kValue);
  // slot of (token, split 0, first head of the group)
  const int64_t slot0 = (int64_t)token * splits * Hp + grp * 32;
  const bool live = head < p.H;
  float g[MAXS];
#pragma unroll
  for (int sp = 0; sp < MAXS; ++sp)
    g[sp] = sp < splits && live ? ml[2 * (slot0 + (int64_t)sp * Hp + n)]
                                : -__builtin_inff();
  uint4 v[MAXS][QPL];
#pragma unroll
  for (int sp = 0; sp < MAXS; ++sp) {
    const uint4* blk = reinterpret_cast<const uint4*>(
        po + (slot0 + (int64_t)sp * Hp) * kValue);
#pragma unroll
    for (int q = 0; q < QPL; ++q)
      v[sp][q] = sp < splits ? ld16_stream(blk + (t * 2 + q0 + q) * kWave + lane)
                             : make_uint4(0u, 0u, 0u, 0u);
  }
  float G = -__builtin_inff();
#pragma unroll
  for (int sp = 0; sp < MAXS; ++sp)
    G = (g[sp] != g[sp] || G != G) ? __builtin_nanf("") : fmaxf(G, g[sp]);
  float wsum = 0.f;
  float acc[8 * QPL];
#pragma unroll
  for (int r = 0; r < 8 * QPL; ++r) acc[r] = 0.f;
  if (G != -__builtin_inff() && G == G) {
#pragma unroll
    for (int sp = 0; sp < MAXS; ++sp) {
      // splits without rows (g = -inf) or beyond `splits` weigh nothing
      const float f = g[sp] == -__builtin_inff() ? 0.f : exp2f(g[sp] - G);
      wsum += f;
      if (f > 0.f) {   // a skipped split's values are never read
#pragma unroll
        for (int q = 0; q < QPL; ++q) {
          const uint32_t w[4] = {v[sp][q].x, v[sp][q].y, v[sp][q].z, v[sp][q].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[8 * q + 2 * i] += f * __builtin_bit_cast(float, w[i] << 16);
            acc[8 * q + 2 * i + 1] +=
                f * __builtin_bit_cast(float, w[i] & 0xffff0000u);
          }
        }
      }
    }
  }
  if (!live) return;
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  // piece q holds accumulator rows 8q..8q+7: features 32t + 8(2q + j) + 4h
  // + 0..3 for j = 0, 1
  float* o = p.out + ((int64_t)token * p.H + head) * kValue + 32 * t + 4 * h;
#pragma unroll
  for (int q = 0; q < QPL; ++q)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      *reinterpret_cast<float4*>(o + 8 * (2 * (q0 + q) + j)) =
          make_float4(acc[8 * q + 4 * j] * inv, acc[8 * q + 4 * j + 1] * inv,
                      acc[8 * q + 4 * j + 2] * inv, acc[8 * q + 4 * j + 3] * inv);
  if (t == 0 && q0 == 0 && h == 0)
    p.lse[(int64_t)token * p.H + head] =
        G != G ? G
               : (wsum > 0.f ? (G + __builtin_log2f(wsum)) * kLn2
                             : -__builtin_inff());
}

}  // namespace

int attn_splits(int tokens, int K) {
  const int tiles = (K + kRowsT - 1) / kRowsT;
  int s = (256 + tokens - 1) / tokens;
  s = s < 1 ? 1 : s;
  s = s > kMaxSplits ? kMaxSplits : s;   // the combine holds up to kMaxSplits
  s = s > tiles ? tiles : s;
  return s;
}

size_t attn_workspace_bytes(int tokens, int H, int K) {
  const int s = attn_splits(tokens, K);
  if (s <= 1) return 0;
  const int Hp = (H + 31) & ~31;   // partials in whole 32-head blocks
  return (size_t)tokens * s * Hp * (kValue * sizeof(uint16_t) + 2 * sizeof(float));
}

hipError_t launch_sparse_mla(const AttnLaunch& p, hipStream_t stream) {
  const int tokens = p.B * p.T;
  const int splits = p.splits;
  // rows per split: whole tiles
  int rps = (p.K + splits - 1) / splits;
  rps = (rps + kRowsT - 1) / kRowsT * kRowsT;
  const int used = (p.K + rps - 1) / rps;   // splits that own rows
  dim3 grid(used, tokens);
  // buffer-form loads address the pool with 32-bit offsets
  const bool buf = p.kv.bytes < (1ull << 32);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, p, rps);
  };
  if (p.kv.t128) {
    if (buf) go(sparse_mla_kernel<kFmtT128, true>);
    else go(sparse_mla_kernel<kFmtT128, false>);
  } else if (p.kv.fp8) {
    if (buf) go(sparse_mla_kernel<kFmtMx32, true>);
    else go(sparse_mla_kernel<kFmtMx32, false>);
  } else {
    if (buf) go(sparse_mla_kernel<kFmtBf16, true>);
    else go(sparse_mla_kernel<kFmtBf16, false>);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || used == 1) return e;
  // units of (value block, pieces): 16 blocks x 2 / QPL, kCombWaves a group
  const int groups = (p.H + 31) / 32;
  if (used <= 8)
    hipLaunchKernelGGL((combine_kernel<8, 2>),
                       dim3(tokens, groups, kValue / 32 / kCombWaves),
                       dim3(64 * kCombWaves), 0, stream, p, used);
  else if (used <= 16)
    hipLaunchKernelGGL((combine_kernel<16, 1>),
                       dim3(tokens, groups, 2 * kValue / 32 / kCombWaves),
                       dim3(64 * kCombWaves), 0, stream, p, used);
  else
    hipLaunchKernelGGL((combine_kernel<kMaxSplits, 1>),
                       dim3(tokens, groups, 2 * kValue / 32 / kCombWaves),
                       dim3(64 * kCombWaves), 0, stream, p, used);
  return hipGetLastError();
}

}  // namespace dsa
