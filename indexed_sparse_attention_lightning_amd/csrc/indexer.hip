// Lightning Indexer score kernels (gfx950).
//
// Score of query t against history position s (page "Day-0 Inference
// Optimization for a New Sparse Attention Architecture: A Technical Deep
// Dive", section 1 -- relevance scoring with head weights; page "Day-0
// Inference Adaptation and Performance Optimization for New-Architecture Large
// Language Models", section "Fusing the Indexer to Reduce Intermediate
// Write-Backs"):
//     I[t,s] = sum_j w[t,j] * max(0, q_I[t,j,:] . k_I[s,:])
//
// Decode is a stream over the key cache: every key row is read exactly once
// per query and scored against all indexer heads of that query on the matrix
// cores (heads form the MFMA M dimension, keys the N dimension, the key
// features the K dimension).  Per wave:
//   * the query's q_I (all heads) sits in registers as MFMA A operands;
//   * keys arrive in 32-key stages: coalesced 16-byte buffer loads into
//     registers (two bf16 stages in flight, four of FP8 codes), then a
//     swizzled write into a wave-private LDS tile and MFMA-layout reads out
//     of it (the transpose a row-major key cache needs; the XOR swizzle keeps
//     both sides free of LDS bank conflicts);
//   * FP8 keys go to LDS as codes and are dequantised when read as operands
//     (e4m3 x 2^(e8m0-127) is exact in bf16), so the products are the bf16
//     ones for both cache formats (the prefill tile kernel dequantises on the
//     way into LDS instead; the quantised kernels further down feed the codes
//     to the scaled FP8 matrix cores as they are);
//   * the ReLU and head-weighted sum run on the accumulators, and the two wave
//     halves combine with one cross-half swap.
// Exactness: integer-valued bf16 inputs with power-of-two weights make every
// partial sum a multiple of 1/8 below 2^24 in magnitude, so fp32 is exact in
// any summation order.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {
namespace {

constexpr int kSub = 32;      // keys per stage == MFMA N
constexpr int kWavesPerWG = 4;
constexpr int kFlush = 1024;  // scores a wave buffers in LDS between writes

template <int DI>
struct KeyLayout {
  static constexpr int kChunks = DI * 2 / 16;            // 16-B bf16 chunks/row
  static constexpr int kRowBytes = DI * 2;                // bf16 row in LDS
  static constexpr int kTileBytes = kSub * kRowBytes;     // one stage in LDS
  static constexpr int kLoadsBf16 = kTileBytes / (16 * kWave);
  static constexpr int kCodeChunks = DI / 16;             // 16-B fp8 chunks/row
  static constexpr int kLoadsFp8 = kSub * DI / (16 * kWave);
  static constexpr int kSteps = DI / 16;                  // MFMA k-steps
  // slot of chunk c of row n (bank-conflict-free writes and reads)
  __device__ static __forceinline__ int slot(int n, int c) {
    return c ^ (kChunks == 16 ? (n & 15) : ((n >> 1) & 7));
  }
};

// FP8 keys (stream path): the e4m3 codes go to LDS as they are (16-byte
// chunk c of key n at chunk slot c ^ swz(n) of the key's DI-byte row) and
// are dequantised when read as MFMA operands.  The features are taken in
// the order that lets a lane read one whole chunk per two k-steps: k-step
// 2j+s, operand half h covers features (2j+h)*16 + 8s .. +8, for the queries
// (A operands) and the keys (B operands) alike.  The chunk of a lane then
// lies in MX block j, whose scale is byte j of the key's scale word.
template <int DI>
struct CodeLayout {
  static constexpr int kChunks = DI / 16;           // 16-B code chunks per key
  static constexpr int kLoads = kSub * DI / (16 * kWave);
  __device__ static __forceinline__ int slot(int n, int c) {
    return c ^ (kChunks == 8 ? ((n >> 1) & 7) : ((n >> 2) & 3));
  }
};

template <int DI>
struct StageF8 {
  uint4 v[CodeLayout<DI>::kLoads];
  uint32_t sc;   // scale codes of key (lane % 32) of the stage, block j in byte j
};

// Past-the-end stages (a wave issues the same loads every step, so its last
// steps load stages beyond its range, whose scores are dropped) load through
// an empty buffer range: the loads return zeros and read no memory.
// A stage's loads go through one buffer resource over its 32 key rows (the
// rows of a stage are consecutive: stages are 32-aligned and pages hold 64
// positions), so a lane's offset is the same every stage and the per-load
// address arithmetic is a scalar base per stage; in the contiguous layout
// the range stops at the cache's last row (the rows past it read zeros).
template <int ROWB>
__device__ __forceinline__ void stage_rows(const CacheView& kc, int b,
                                           int kbase, bool parked,
                                           const uint8_t*& base,
                                           uint32_t& rows, int64_t& row0) {
  rows = 0;
  row0 = 0;
  if (parked) {
    base = kc.data;
    return;
  }
  if (kc.page_table != nullptr) {
    row0 = cache_row_uniform(kc.page_table, kc.max_pages, kc.num_pages, kc.L, b, kbase);
    rows = kSub;
  } else {
    row0 = (int64_t)b * kc.L + kbase;
    rows = (uint32_t)max(0, min(kSub, kc.L - kbase));
  }
  base = kc.data + row0 * ROWB;
  // the resource must be wave-uniform (a divergent one costs a loop of
  // single-value loads per instruction)
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  base = reinterpret_cast<const uint8_t*>(
      ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(a >> 32)) << 32) |
      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a));
  rows = (uint32_t)__builtin_amdgcn_readfirstlane((int)rows);
}

template <int DI>
__device__ __forceinline__ void stage_load_f8(StageF8<DI>& st,
                                              const CacheView& kc, int b,
                                              int kbase, int lane,
                                              bool parked) {
  using CL = CodeLayout<DI>;
  // wave-uniform: the page-table lookup is then a scalar load (a vector one
  // would be waited for with every key load in flight)
  b = __builtin_amdgcn_readfirstlane(b);
  kbase = __builtin_amdgcn_readfirstlane(kbase);
  const uint8_t* base;
  uint32_t rows;
  int64_t row0;
  stage_rows<DI>(kc, b, kbase, parked, base, rows, row0);
  const auto codes = bytes_rsrc(base, rows * DI);
#pragma unroll
  for (int i = 0; i < CL::kLoads; ++i)
    st.v[i] = __builtin_bit_cast(
        uint4, __builtin_amdgcn_raw_buffer_load_b128(
                   codes, (uint32_t)(i * kWave + lane) * 16, 0, kBufStream));
  const auto scales = bytes_rsrc(kc.scale + row0 * (DI / 32), rows * (DI / 32));
  const uint32_t n = lane & 31;
  if constexpr (DI == 128)
    st.sc = __builtin_amdgcn_raw_buffer_load_b32(scales, n * 4, 0, 0);
  else
    st.sc = __builtin_amdgcn_raw_buffer_load_b16(scales, n * 2, 0, 0);
}

// The codes go to the wave's LDS tile and the scale words to `scl` (one per
// key): a scale word kept in a register across the next load of the same
// stage would make the compiler move it at the loop back edge, which waits
// for every load in flight.
template <int DI>
__device__ __forceinline__ void stage_store_f8(const StageF8<DI>& st,
                                               uint4* tile, uint32_t* scl,
                                               int lane) {
  using CL = CodeLayout<DI>;
#pragma unroll
  for (int i = 0; i < CL::kLoads; ++i) {
    const int id = i * kWave + lane;
    const int n = id / CL::kChunks, c = id % CL::kChunks;
    tile[n * CL::kChunks + CL::slot(n, c)] = st.v[i];
  }
  if (lane < kSub) scl[lane] = st.sc;
}

// ReLU and head weighting of a lane's accumulators, then the two wave
// halves: the score of key lane % 32, the sum over heads of
// w * max(0, q.k), accumulated in one running fp32 sum in head order.
// (Four independent partial sums instead, which shorten the chain of
// dependent instructions, measured the same on the prefill chunk.)
template <int MB>
__device__ __forceinline__ float head_weighted_relu(const f32x16 (&acc)[MB],
                                                    const float (&wv)[MB][16]) {
  float s = 0.f;
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += wv[m][r] * relu(acc[m][r]);
  return s + swap_halves(s);
}

// tile_scores for a code tile; `scl` holds the scale words of its keys.
template <int DI, int MB>
__device__ __forceinline__ float tile_scores_f8(const uint4* tile,
                                                const uint4 (&a)[MB][DI / 16],
                                                const float (&wv)[MB][16],
                                                const uint32_t* scl, int lane) {
  using CL = CodeLayout<DI>;
  const int n = lane & 31, h = lane >> 5;
  const uint32_t sc = scl[n];
  f32x16 acc[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) acc[m] = f32x16{};
  // all of the lane's code chunks first: one LDS wait per tile
  uint4 cvs[DI / 32];
#pragma unroll
  for (int j = 0; j < DI / 32; ++j)
    cvs[j] = tile[n * CL::kChunks + CL::slot(n, 2 * j + h)];
#pragma unroll
  for (int j = 0; j < DI / 32; ++j) {
    const uint4 cv = cvs[j];
    const uint32_t e = (sc >> (8 * j)) & 0xffu;
    const uint4 b0 = dequant8_e4m3(make_uint2(cv.x, cv.y), e);
    const uint4 b1 = dequant8_e4m3(make_uint2(cv.z, cv.w), e);
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[m] = mfma32(a[m][2 * j], b0, acc[m]);
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[m] = mfma32(a[m][2 * j + 1], b1, acc[m]);
  }
  return head_weighted_relu<MB>(acc, wv);
}

// The value stored for a score: the score (+0 folds -0), or, for the fused
// path whose Top-K reads keys, its order-preserving key bit pattern.
__device__ __forceinline__ float out_val(const IndexerLaunch& p, float sc) {
  return p.keys_out ? __builtin_bit_cast(float, score_key(sc)) : sc + 0.0f;
}

// Registers holding one 32-key bf16 stage on its way from HBM to LDS.
template <int DI>
struct Stage {
  static constexpr int N = KeyLayout<DI>::kLoadsBf16;
  uint4 v[N];
};

template <int DI>
__device__ __forceinline__ void stage_load(Stage<DI>& st, const CacheView& kc,
                                           int b, int kbase, int lane,
                                           bool parked) {
  // wave-uniform: the page-table lookup is then a scalar load (a vector one
  // would be waited for with every key load in flight)
  b = __builtin_amdgcn_readfirstlane(b);
  kbase = __builtin_amdgcn_readfirstlane(kbase);
  const uint8_t* base;
  uint32_t rows;
  int64_t row0;
  stage_rows<DI * 2>(kc, b, kbase, parked, base, rows, row0);
  const auto keys = bytes_rsrc(base, rows * (DI * 2));
  // lane l of load i takes bytes 16*(64i + l) of the stage's rows:
  // key (64i + l) / chunks, chunk (64i + l) % chunks
#pragma unroll
  for (int i = 0; i < Stage<DI>::N; ++i)
    st.v[i] = __builtin_bit_cast(
        uint4, __builtin_amdgcn_raw_buffer_load_b128(
                   keys, (uint32_t)(i * kWave + lane) * 16, 0, kBufStream));
}

template <int DI>
__device__ __forceinline__ void stage_store(const Stage<DI>& st, uint4* tile,
                                            int lane) {
  using KL = KeyLayout<DI>;
#pragma unroll
  for (int i = 0; i < Stage<DI>::N; ++i) {
    const int id = i * kWave + lane;
    const int n = id / KL::kChunks, c = id % KL::kChunks;
    tile[n * KL::kChunks + KL::slot(n, c)] = st.v[i];
  }
}

// Scores of 32 keys (one LDS tile) for one query held in `a` (A operands)
// with head weights `wv` in accumulator layout.  Returns, in every lane, the
// score of key (lane % 32) of the tile.
template <int DI, int MB>
__device__ __forceinline__ float tile_scores(const uint4* tile,
                                             const uint4 (&a)[MB][DI / 16],
                                             const float (&wv)[MB][16],
                                             int lane) {
  using KL = KeyLayout<DI>;
  const int n = lane & 31, h = lane >> 5;
  f32x16 acc[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) acc[m] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < KL::kSteps; ++ks) {
    const uint4 bop = tile[n * KL::kChunks + KL::slot(n, 2 * ks + h)];
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[m] = mfma32(a[m][ks], bop, acc[m]);
  }
  return head_weighted_relu<MB>(acc, wv);
}

// Loads one query's indexer vectors as MFMA A operands and its head weights
// in accumulator-row layout (heads >= H_I contribute zero).
// CHUNKED: the feature order of the FP8 code tiles (k-step 2j+s, half h =
// features (2j+h)*16 + 8s); otherwise k-step ks, half h = ks*16 + 8h.
template <int DI, int MB, bool CHUNKED = false>
__device__ __forceinline__ void load_query(const uint16_t* q_idx,
                                           const float* w, int H_I, int lane,
                                           uint4 (&a)[MB][DI / 16],
                                           float (&wv)[MB][16]) {
  const int m32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int head = m * 32 + m32;
#pragma unroll
    for (int ks = 0; ks < DI / 16; ++ks) {
      const int f = CHUNKED ? ((ks & ~1) + h) * 16 + (ks & 1) * 8 : ks * 16 + h * 8;
      a[m][ks] = head < H_I ? ld16(q_idx + head * DI + f)
                            : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int hr = m * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      wv[m][r] = hr < H_I ? w[hr] : 0.f;
    }
  }
}

// The (min, max) of the keys a wave wrote, over its lanes, into its span
// entry (lane 0 stores).  Waves without causal positions store nothing (a
// store on their early-exit path cost the page-table lookups their scalar
// loads: the compiler then waited for every key load in flight at each).
__device__ __forceinline__ void span_store(float* span, int64_t qrow,
                                           int entry, uint32_t mn,
                                           uint32_t mx, int lane) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, m));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, m));
  }
  if (lane == 0)
    reinterpret_cast<float2*>(span)[qrow * kSpanMax + entry] =
        make_float2(__builtin_bit_cast(float, mn), __builtin_bit_cast(float, mx));
}

// Streaming indexer: grid (chunks, T, B); each wave scores `kpw`
// consecutive positions of one query.  With `xcd_rows` (a row count that is
// a multiple of 8) the linear workgroup id, which the dispatcher deals to the
// 8 XCDs round-robin, is remapped so that every chunk of query row r runs on
// XCD r % 8: the row's query, weights and score lines stay in one L2.
template <int DI, int MB, bool FP8>
__global__ __launch_bounds__(256, 2) void indexer_stream_kernel(
    IndexerLaunch p, int kpw, int xcd_rows) {
  using KL = KeyLayout<DI>;
  __shared__ uint4 lds[kWavesPerWG][KL::kTileBytes / 16];
  // scores leave in bursts of up to kFlush: a steady trickle of small
  // writes into the key stream costs read bandwidth
  __shared__ float sbuf[kWavesPerWG][kFlush];
  __shared__ uint32_t sscale[kWavesPerWG][FP8 ? kSub : 1];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  int b = blockIdx.z, t = blockIdx.y, chunk = blockIdx.x;
  if (xcd_rows) {
    const int lin = (blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
    const int slot = lin >> 3;
    const int row = (slot / gridDim.x) * 8 + (lin & 7);
    chunk = slot % gridDim.x;
    b = row / p.T;
    t = row % p.T;
  }
  const int k0 = (chunk * kWavesPerWG + wave) * kpw;
  if (k0 >= p.row_len) return;
  const int k1 = min(k0 + kpw, p.row_len);
  const int qpos = __builtin_amdgcn_readfirstlane(query_pos(p.qp, b, t));
  float* srow = p.scores + ((int64_t)b * p.T + t) * p.row_len;

  // positions past the query are masked
  for (int s = max(k0, qpos + 1) + lane; s < k1; s += kWave)
    srow[s] = out_val(p, -__builtin_inff());
  const int kend = min(k1, qpos + 1);
  const int64_t qrow = (int64_t)b * p.T + t;
  if (kend <= k0) return;
  const int nsub = (kend - k0 + kSub - 1) / kSub;

  uint4 a[MB][DI / 16];
  float wv[MB][16];
  load_query<DI, MB, FP8>(p.q_idx + qrow * p.H_I * DI, p.w + qrow * p.H_I,
                          p.H_I, lane, a, wv);

  uint4* tile = lds[wave];
  uint32_t* scl = sscale[wave];
  const auto park_if = [&](int stage) { return stage > nsub - 1; };
  // Every iteration issues the same loads and stores (stages past the end
  // read zeros through an empty range and their scores are dropped), so the
  // compiler can count them and wait only for the stage it consumes.
  const int last = nsub - 1;
  float* sb = sbuf[wave];
  // The flushes also take this lane's (min, max) key over what they write:
  // the wave's causal positions, once each (for the span entry; about 2
  // instructions per 8 keys a lane, where tracking each stage cost the
  // kernel about 1 us).
  uint32_t kmn = ~0u, kmx = 0u;
  const auto flush = [&](int from, int to) {   // positions [from, to)
    for (int s = from + lane; s < to; s += kWave) {
      const float v = sb[(s - k0) % kFlush];
      srow[s] = v;
      kmn = min(kmn, __builtin_bit_cast(uint32_t, v));
      kmx = max(kmx, __builtin_bit_cast(uint32_t, v));
    }
  };
  if constexpr (FP8) {
    // stages are half the bytes of bf16 ones: four in flight
    StageF8<DI> st[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      stage_load_f8<DI>(st[u], p.keys, b, k0 + min(u, last) * kSub, lane,
                        park_if(u));
    for (int i = 0; i < nsub; i += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        stage_store_f8<DI>(st[u], tile, scl, lane);
        stage_load_f8<DI>(st[u], p.keys, b, k0 + min(i + u + 4, last) * kSub,
                          lane, park_if(i + u + 4));
        const float sc = tile_scores_f8<DI, MB>(tile, a, wv, scl, lane);
        // stages past the end (parked) are not buffered
        if (lane < 32 && i + u < nsub)
          sb[((i + u) * kSub + lane) % kFlush] = out_val(p, sc);
      }
      if ((i + 4) * kSub % kFlush == 0 && i + 4 < nsub)   // a full buffer
        flush(k0 + (i + 4) * kSub - kFlush, k0 + (i + 4) * kSub);
    }
  } else {
    Stage<DI> s0, s1;
    stage_load<DI>(s0, p.keys, b, k0, lane, park_if(0));
    stage_load<DI>(s1, p.keys, b, k0 + min(1, last) * kSub, lane,
                        park_if(1));
    for (int i = 0; i < nsub; i += 2) {
      stage_store<DI>(s0, tile, lane);
      stage_load<DI>(s0, p.keys, b, k0 + min(i + 2, last) * kSub, lane,
                          park_if(i + 2));
      {
        const float sc = tile_scores<DI, MB>(tile, a, wv, lane);
        if (lane < 32) sb[(i * kSub + lane) % kFlush] = out_val(p, sc);
      }
      stage_store<DI>(s1, tile, lane);
      stage_load<DI>(s1, p.keys, b, k0 + min(i + 3, last) * kSub, lane,
                          park_if(i + 3));
      {
        const float sc = tile_scores<DI, MB>(tile, a, wv, lane);
        if (lane < 32) sb[((i + 1) * kSub + lane) % kFlush] = out_val(p, sc);
      }
      if ((i + 2) * kSub % kFlush == 0 && i + 2 < nsub)   // a full buffer
        flush(k0 + (i + 2) * kSub - kFlush, k0 + (i + 2) * kSub);
    }
  }
  const int done = (nsub - 1) / (kFlush / kSub) * kFlush;   // flushed so far
  flush(k0 + done, kend);
  if (p.span) span_store(p.span, qrow, k0 / kpw, kmn, kmx, lane);
}

// ------------------------------------------------ quantised indexer (MX32)
// The fully quantised indexer (page "Inference Adaptation and Performance
// Optimization for New Large Language Model Architectures", section 4.2:
// index Q and K in MXFP8, one scale per 32 elements; "Day-0 Inference
// Optimization ...: A Technical Deep Dive", section 2): the bf16 queries are
// quantised per head and 32-feature block on load (the rule of the cache
// append: scale 2^X, X the smallest with 448 * 2^X >= the block maximum),
// and the products run on the 32x32x64 scaled FP8 matrix cores, which take
// the e8m0 block scales of both operands as they are: the key codes are
// never dequantised.  The decode kernel stages them like the FP8-key one
// (coalesced non-temporal loads into the wave's LDS tile, read back in
// operand layout); the prefill kernel shares 128-key LDS stages.
//
// Operand layout of k-step ks (64 features): lane l = n + 32h holds 32 codes
// of row n (query head or key); bytes 0..15 are features 64ks + 16h + 0..15
// (MX block 2ks), bytes 16..31 features 64ks + 32 + 16h + 0..15 (block
// 2ks+1), and its scale operand is row n's e8m0 code of block 2ks + h.  (The
// matrix core takes the 32 values of a scale block 16 from each lane half,
// and the scale of row n's block b from lane n + 32b.)
typedef int v8i __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v8i join8(const uint4& lo, const uint4& hi) {
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

// The query's A operands: quantised codes and the scale operands, plus the
// head weights in accumulator-row layout (heads >= H_I contribute zero).
// One share of a query's A operands -- head block m, k-step ks -- for the
// 64 lanes: the bf16 features 64ks + 32(i/2) + 16h + 8(i%2) of head 32m + n
// (loads first, addresses clamped to a real head), then quantised per MX
// block (scale 2^X, X the smallest with 448 * 2^X >= the block's largest
// magnitude) into the operand codes and this lane's scale operand.  Heads
// past H_I quantise to zero.
template <int DI>
__device__ __forceinline__ void load_share_q8(const uint16_t* q_idx, int H_I,
                                              int m, int ks, int lane,
                                              uint4 (&raw)[4]) {
  const int n = lane & 31, h = lane >> 5;
  const uint16_t* src = q_idx + min(m * 32 + n, H_I - 1) * DI + 64 * ks + 16 * h;
#pragma unroll
  for (int i = 0; i < 4; ++i) raw[i] = ld16(src + 32 * (i >> 1) + 8 * (i & 1));
}

__device__ __forceinline__ void quantise_share_q8(const uint4 (&raw)[4],
                                                  bool valid, int lane,
                                                  v8i& code_out,
                                                  int& scale_out) {
  const int h = lane >> 5;
  uint32_t code[2][4];
  int X[2];
#pragma unroll
  for (int pc = 0; pc < 2; ++pc) {
    float f[16];
    {
      float t[8];
      unpack8(raw[2 * pc], t);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = valid ? t[i] : 0.0f;
      unpack8(raw[2 * pc + 1], t);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[8 + i] = valid ? t[i] : 0.0f;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
    // the block's other 16 features sit in lane n + 32(1-h)
    amax = fmaxf(amax, swap_halves(amax));
    X[pc] = mx_exponent(amax);
    const float inv = pow2_neg(X[pc]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      code[pc][i] = e4m3x4(f[4 * i] * inv, f[4 * i + 1] * inv,
                           f[4 * i + 2] * inv, f[4 * i + 3] * inv);
  }
  code_out = join8(make_uint4(code[0][0], code[0][1], code[0][2], code[0][3]),
                   make_uint4(code[1][0], code[1][1], code[1][2], code[1][3]));
  scale_out = (h ? X[1] : X[0]) + 127;
}

// Head weights in accumulator-row layout 8(r/4) + 4h + r%4 of block m from
// `wl`, the weight of head `lane` (0 past H_I), by lane exchange.
template <int MB>
__device__ __forceinline__ void spread_weights_q8(float wl, int lane,
                                                  float (&wv)[MB][16]) {
  const int h = lane >> 5;
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      wv[m][r] = __shfl(wl, m * 32 + 8 * (r >> 2) + 4 * h + (r & 3));
}


// Scores of 32 keys of an LDS stage (keys 0..31 of `tile`, scale words
// `scl`) against the wave's quantised query: in every lane, the score of key
// lane % 32.
template <int DI, int MB>
__device__ __forceinline__ float tile_scores_q8(const uint4* tile,
                                                const uint32_t* scl,
                                                const v8i (&a)[MB][DI / 64],
                                                const int (&as)[MB][DI / 64],
                                                const float (&wv)[MB][16],
                                                int lane) {
  using CL = CodeLayout<DI>;
  const int n = lane & 31, h = lane >> 5;
  const uint32_t sc = scl[n];
  f32x16 acc[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) acc[m] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < DI / 64; ++ks) {
    const v8i bop = join8(tile[n * CL::kChunks + CL::slot(n, 4 * ks + h)],
                          tile[n * CL::kChunks + CL::slot(n, 4 * ks + 2 + h)]);
    const int bs = (int)((sc >> (8 * (2 * ks + h))) & 0xffu);
#pragma unroll
    for (int m = 0; m < MB; ++m)
      acc[m] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          a[m][ks], bop, acc[m], 0, 0, 0, as[m][ks], 0, bs);
  }
  return head_weighted_relu<MB>(acc, wv);
}

// Streaming indexer with quantised queries over MX keys: the grid, the
// score buffering and the key staging of indexer_stream_kernel for FP8
// keys (four stages in flight, coalesced non-temporal loads into the wave's
// LDS tile, read back in the scaled products' operand layout).  The four
// waves of a workgroup score the same query row, so each quantises one share
// of its operands into LDS (before any wave leaves) and all read them.
template <int DI, int MB>
__global__ __launch_bounds__(256, 2) void indexer_stream_q8_kernel(
    IndexerLaunch p, int kpw, int xcd_rows) {
  constexpr int kShares = MB * (DI / 64);   // (head block, k-step) pairs
  static_assert(kShares <= kWavesPerWG, "one share per wave");
  __shared__ float sbuf[kWavesPerWG][kFlush];
  __shared__ uint4 ktile[kWavesPerWG][kSub * DI / 16];
  __shared__ uint32_t kscl[kWavesPerWG][kSub];
  __shared__ v8i qcode[kShares][kWave];
  __shared__ int qscale[kShares][kWave];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  int b = blockIdx.z, t = blockIdx.y, chunk = blockIdx.x;
  if (xcd_rows) {
    const int lin = (blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
    const int slot = lin >> 3;
    const int row = (slot / gridDim.x) * 8 + (lin & 7);
    chunk = slot % gridDim.x;
    b = row / p.T;
    t = row % p.T;
  }
  const int k0 = (chunk * kWavesPerWG + wave) * kpw;
  const int k1 = min(k0 + kpw, p.row_len);
  const int qpos = __builtin_amdgcn_readfirstlane(query_pos(p.qp, b, t));
  float* srow = p.scores + ((int64_t)b * p.T + t) * p.row_len;
  for (int s = max(k0, qpos + 1) + lane; s < k1; s += kWave)
    srow[s] = out_val(p, -__builtin_inff());
  const int kend = min(k1, qpos + 1);
  const bool work = kend > k0;   // wave-uniform
  const int nsub = work ? (kend - k0 + kSub - 1) / kSub : 1;
  const int last = nsub - 1;
  // Every iteration issues the same loads (stages past the end are parked:
  // they read zeros through an empty range, and their scores are dropped),
  // so the compiler waits only for the stage it consumes.
  // This wave's share of the query first, then the first four key stages,
  // so that the quantisation waits only for the query.  Both are issued by
  // every wave (a wave without a share re-loads share 0, one without keys
  // parks its stages): loads under a branch would make the compiler's wait
  // before the quantisation cover the key loads as well.
  const int64_t qrow = (int64_t)b * p.T + t;
  const int share = wave < kShares ? wave : 0;
  const int qm = share / (DI / 64), qks = share % (DI / 64);
  uint4 raw[4];
  load_share_q8<DI>(p.q_idx + qrow * p.H_I * DI, p.H_I, qm, qks, lane, raw);
  const float wraw = p.w[qrow * p.H_I + min(lane, p.H_I - 1)];
  StageF8<DI> st[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    stage_load_f8<DI>(st[u], p.keys, b, work ? k0 + min(u, last) * kSub : 0,
                      lane, !work || u > last);
  if (wave < kShares) {
    v8i c;
    int sc;
    quantise_share_q8(raw, qm * 32 + (lane & 31) < p.H_I, lane, c, sc);
    qcode[wave][lane] = c;
    qscale[wave][lane] = sc;
  }
  __syncthreads();
  if (!work) return;
  v8i a[MB][DI / 64];
  int as[MB][DI / 64];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int ks = 0; ks < DI / 64; ++ks) {
      a[m][ks] = qcode[m * (DI / 64) + ks][lane];
      as[m][ks] = qscale[m * (DI / 64) + ks][lane];
    }
  float wv[MB][16];
  spread_weights_q8<MB>(lane < p.H_I ? wraw : 0.f, lane, wv);
  float* sb = sbuf[wave];
  // The flushes also take this lane's (min, max) key over what they write:
  // the wave's causal positions, once each (for the span entry; about 2
  // instructions per 8 keys a lane, where tracking each stage cost the
  // kernel about 1 us).
  uint32_t kmn = ~0u, kmx = 0u;
  const auto flush = [&](int from, int to) {   // positions [from, to)
    for (int s = from + lane; s < to; s += kWave) {
      const float v = sb[(s - k0) % kFlush];
      srow[s] = v;
      kmn = min(kmn, __builtin_bit_cast(uint32_t, v));
      kmx = max(kmx, __builtin_bit_cast(uint32_t, v));
    }
  };
  for (int i = 0; i < nsub; i += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      // the products read the stage's registers, then its next load goes
      // into the same registers (no copies: moving a register whose load is
      // in flight would wait for every load)
      stage_store_f8<DI>(st[u], ktile[wave], kscl[wave], lane);
      stage_load_f8<DI>(st[u], p.keys, b, k0 + min(i + u + 4, last) * kSub,
                        lane, i + u + 4 > last);
      const float sc = tile_scores_q8<DI, MB>(ktile[wave], kscl[wave], a, as,
                                              wv, lane);
      if (lane < 32 && i + u < nsub)
        sb[((i + u) * kSub + lane) % kFlush] = out_val(p, sc);
    }
    if ((i + 4) * kSub % kFlush == 0 && i + 4 < nsub)   // a full buffer
      flush(k0 + (i + 4) * kSub - kFlush, k0 + (i + 4) * kSub);
  }
  const int done = (nsub - 1) / (kFlush / kSub) * kFlush;   // flushed so far
  flush(k0 + done, kend);
  if (p.span) span_store(p.span, qrow, k0 / kpw, kmn, kmx, lane);
}

// ---------------------------------------------------------------- prefill
// Query-tiled indexer for many queries per sequence (prefill chunks): a
// workgroup of 8 waves takes 8 consecutive queries (one per wave, two waves
// per SIMD) and one chunk of keys.  The keys are staged once per workgroup
// in 128-key LDS stages of two pages (double-buffered, the next stage's
// loads in flight in registers; one barrier per stage covers four 32-key
// halves of each wave's matrix work) and every wave scores them against its
// own query, so each key byte read from HBM feeds 8 queries x 64 heads of
// MFMA work.  Stages past
// the last query of the tile are skipped (causal), and each wave skips the
// 32-key halves that lie entirely past its own query.
constexpr int kTileQ = 8;          // queries per workgroup (one per wave)
constexpr int kStageKeys = 2 * kPage;   // keys per LDS stage (two pages)

template <int DI, bool FP8>
struct TileStage {
  // 16-byte loads of one stage (bf16 rows are 2*DI bytes, FP8 rows DI codes
  // plus DI/32 scales), spread over the workgroup's threads
  static constexpr int kTotal = kStageKeys * (FP8 ? DI : 2 * DI) / 16;
  static constexpr int kThreads = kTileQ * kWave;
  static constexpr int kLoads = (kTotal + kThreads - 1) / kThreads;
  static constexpr bool kPartial = kTotal % kThreads != 0;
  uint4 v[kLoads];
  uint32_t sc[FP8 ? kLoads : 1];
};

template <int DI, bool FP8>
__device__ __forceinline__ void tile_load(TileStage<DI, FP8>& st,
                                          const CacheView& kc, int b,
                                          int kbase, int tid) {
  using KL = KeyLayout<DI>;
  // wave-uniform: the page-table lookups are then scalar loads (a vector one
  // is waited for together with the other stage's key loads in flight).
  // The stage's two pages (kbase is a multiple of the stage); the second
  // page of the last stage may lie past the table's row: its keys are never
  // scored, so it takes the row's last page, whose rows are in the pool.
  b = __builtin_amdgcn_readfirstlane(b);
  kbase = __builtin_amdgcn_readfirstlane(kbase);
  int64_t row0[2];
  bool clamp = false;
  if (kc.page_table != nullptr) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
      row0[g] = cache_row_uniform(kc.page_table, kc.max_pages, kc.num_pages,
                                  kc.L, b,
                                  min(kbase + g * kPage, (kc.max_pages - 1) * kPage)) -
                g * kPage;
  } else {
    row0[0] = row0[1] = (int64_t)b * kc.L + kbase;
    clamp = kbase + kStageKeys > kc.L;
  }
#pragma unroll
  for (int i = 0; i < TileStage<DI, FP8>::kLoads; ++i) {
    const int id = i * kTileQ * kWave + tid;
    if (TileStage<DI, FP8>::kPartial && id >= TileStage<DI, FP8>::kTotal)
      break;
    if constexpr (!FP8) {
      const int n = id / KL::kChunks, c = id % KL::kChunks;
      int64_t row = row0[n / kPage] + n;
      if (clamp) row = (int64_t)b * kc.L + min(kbase + n, kc.L - 1);
      st.v[i] = ld16(kc.data + row * (DI * 2) + c * 16);
    } else {
      const int n = id / KL::kCodeChunks, c = id % KL::kCodeChunks;
      int64_t row = row0[n / kPage] + n;
      if (clamp) row = (int64_t)b * kc.L + min(kbase + n, kc.L - 1);
      st.v[i] = ld16(kc.data + row * DI + c * 16);
      st.sc[i] = kc.scale[row * (DI / 32) + (c >> 1)];
    }
  }
}

template <int DI, bool FP8>
__device__ __forceinline__ void tile_store(const TileStage<DI, FP8>& st,
                                           uint4* tile, int tid) {
  using KL = KeyLayout<DI>;
#pragma unroll
  for (int i = 0; i < TileStage<DI, FP8>::kLoads; ++i) {
    const int id = i * kTileQ * kWave + tid;
    if (TileStage<DI, FP8>::kPartial && id >= TileStage<DI, FP8>::kTotal)
      break;
    if constexpr (!FP8) {
      const int n = id / KL::kChunks, c = id % KL::kChunks;
      tile[n * KL::kChunks + KL::slot(n, c)] = st.v[i];
    } else {
      const int n = id / KL::kCodeChunks, c = id % KL::kCodeChunks;
      tile[n * KL::kChunks + KL::slot(n, 2 * c)] =
          dequant8_e4m3(make_uint2(st.v[i].x, st.v[i].y), st.sc[i]);
      tile[n * KL::kChunks + KL::slot(n, 2 * c + 1)] =
          dequant8_e4m3(make_uint2(st.v[i].z, st.v[i].w), st.sc[i]);
    }
  }
}

template <int DI, int MB, bool FP8>
__global__ __launch_bounds__(kTileQ * kWave, 2) void indexer_tile_kernel(
    IndexerLaunch p, int keys_per_wg) {
  using KL = KeyLayout<DI>;
  constexpr int kTileU4 = kStageKeys * KL::kRowBytes / 16;
  __shared__ uint4 lds[2][kTileU4];
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int b = blockIdx.z;
  const int t = blockIdx.y * kTileQ + wave;
  const bool has_q = t < p.T;
  const int c0 = blockIdx.x * keys_per_wg;
  const int c1 = min(c0 + keys_per_wg, p.row_len);
  // causal extent of the tile: its last query
  int qmax = -1;
  for (int w = 0; w < kTileQ; ++w) {
    const int tt = blockIdx.y * kTileQ + w;
    if (tt < p.T) qmax = max(qmax, query_pos(p.qp, b, tt));
  }
  const int qpos = has_q ? __builtin_amdgcn_readfirstlane(query_pos(p.qp, b, t)) : -1;
  float* srow = has_q ? p.scores + ((int64_t)b * p.T + t) * p.row_len : nullptr;
  if (has_q)
    for (int s = max(c0, qpos + 1) + lane; s < c1; s += kWave)
      srow[s] = out_val(p, -__builtin_inff());
  const int kend = min(c1, qmax + 1);
  if (kend <= c0) return;   // workgroup-uniform
  const int nst = (kend - c0 + kStageKeys - 1) / kStageKeys;

  uint4 a[MB][DI / 16];
  float wv[MB][16];
  {
    const int64_t qrow = (int64_t)b * p.T + (has_q ? t : 0);
    load_query<DI, MB>(p.q_idx + qrow * p.H_I * DI, p.w + qrow * p.H_I, p.H_I,
                       lane, a, wv);
  }
  // two stages in flight in registers: stage i+2 loads while stage i is
  // computed (the tail re-loads the last stage, whose loads are never stored)
  TileStage<DI, FP8> st[2];
  tile_load<DI, FP8>(st[0], p.keys, b, c0, tid);
  tile_load<DI, FP8>(st[1], p.keys, b, c0 + min(1, nst - 1) * kStageKeys, tid);
  const auto stage = [&](int i, TileStage<DI, FP8>& sr) {
    uint4* tile = lds[i & 1];
    tile_store<DI, FP8>(sr, tile, tid);
    tile_load<DI, FP8>(sr, p.keys, b, c0 + min(i + 2, nst - 1) * kStageKeys, tid);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kStageKeys / kSub; ++u) {
      const int kb = c0 + i * kStageKeys + u * kSub;
      if (has_q && kb <= qpos) {   // wave-uniform
        const float sc = tile_scores<DI, MB>(tile + u * kSub * KL::kChunks, a,
                                             wv, lane);
        const int s = kb + (lane & 31);
        if (lane < 32 && s <= qpos && s < c1) srow[s] = out_val(p, sc);
      }
    }
  };
  int i = 0;
  for (; i + 1 < nst; i += 2) {
    stage(i, st[0]);
    stage(i + 1, st[1]);
  }
  if (i < nst) stage(i, st[0]);
}

// Query-tiled quantised indexer (prefill chunks with quantised queries over
// MX keys): the workgroup shape and causal skipping of indexer_tile_kernel;
// the stages hold the e4m3 codes as they are (16-byte chunk c of key n at
// chunk slot c ^ swz(n), conflict-free for the operand reads) plus the keys'
// scale words, and every wave runs the scaled FP8 products against its own
// query, quantised on load.

template <int DI>
struct TileStageQ8 {
  static constexpr int kChunks = kStageKeys * DI / 16;   // 16-B code chunks
  static constexpr int kThreads = kTileQ * kWave;
  static constexpr int kLoads = (kChunks + kThreads - 1) / kThreads;
  static_assert(kChunks % kThreads == 0 || kLoads == 1, "stage loads");
  uint4 v[kLoads];
  uint32_t sc;   // scale word of key tid (tid < kStageKeys)
};

template <int DI>
__device__ __forceinline__ void tile_load_q8(TileStageQ8<DI>& st,
                                             const CacheView& kc, int b,
                                             int kbase, int tid) {
  using CL = CodeLayout<DI>;
  // wave-uniform (scalar page-table lookups, as in tile_load): the stage's
  // two pages (kbase is a multiple of the stage).  The second page of the
  // last stage may lie past the table's row: its keys are never scored, so
  // it takes the row's last page, whose rows are in the pool.
  b = __builtin_amdgcn_readfirstlane(b);
  kbase = __builtin_amdgcn_readfirstlane(kbase);
  int64_t row0[2];
  bool clamp = false;
  if (kc.page_table != nullptr) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
      row0[g] = cache_row_uniform(kc.page_table, kc.max_pages, kc.num_pages,
                                  kc.L, b,
                                  min(kbase + g * kPage, (kc.max_pages - 1) * kPage)) -
                g * kPage;
  } else {
    row0[0] = row0[1] = (int64_t)b * kc.L + kbase;
    clamp = kbase + kStageKeys > kc.L;
  }
#pragma unroll
  for (int i = 0; i < TileStageQ8<DI>::kLoads; ++i) {
    const int id = min(i * TileStageQ8<DI>::kThreads + tid,
                       TileStageQ8<DI>::kChunks - 1);
    const int n = id / CL::kChunks, c = id % CL::kChunks;
    int64_t row = row0[n / kPage] + n;
    if (clamp) row = (int64_t)b * kc.L + min(kbase + n, kc.L - 1);
    st.v[i] = ld16(kc.data + row * DI + c * 16);
  }
  {
    const int n = tid & (kStageKeys - 1);
    int64_t row = row0[n / kPage] + n;
    if (clamp) row = (int64_t)b * kc.L + min(kbase + n, kc.L - 1);
    if constexpr (DI == 128)
      st.sc = *reinterpret_cast<const uint32_t*>(kc.scale + row * 4);
    else
      st.sc = *reinterpret_cast<const uint16_t*>(kc.scale + row * 2);
  }
}

template <int DI>
__device__ __forceinline__ void tile_store_q8(const TileStageQ8<DI>& st,
                                              uint4* tile, uint32_t* scl,
                                              int tid) {
  using CL = CodeLayout<DI>;
#pragma unroll
  for (int i = 0; i < TileStageQ8<DI>::kLoads; ++i) {
    const int id = i * TileStageQ8<DI>::kThreads + tid;
    if (id < TileStageQ8<DI>::kChunks) {
      const int n = id / CL::kChunks, c = id % CL::kChunks;
      tile[n * CL::kChunks + CL::slot(n, c)] = st.v[i];
    }
  }
  if (tid < kStageKeys) scl[tid] = st.sc;
}

template <int DI, int MB>
__global__ __launch_bounds__(kTileQ * kWave, 2) void indexer_tile_q8_kernel(
    IndexerLaunch p, int keys_per_wg) {
  using CL = CodeLayout<DI>;
  constexpr int kTileU4 = kStageKeys * DI / 16;
  __shared__ uint4 lds[2][kTileU4];
  __shared__ uint32_t scl[2][kStageKeys];
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int b = blockIdx.z;
  const int t = blockIdx.y * kTileQ + wave;
  const bool has_q = t < p.T;
  const int c0 = blockIdx.x * keys_per_wg;
  const int c1 = min(c0 + keys_per_wg, p.row_len);
  // causal extent of the tile: its last query
  int qmax = -1;
  for (int w = 0; w < kTileQ; ++w) {
    const int tt = blockIdx.y * kTileQ + w;
    if (tt < p.T) qmax = max(qmax, query_pos(p.qp, b, tt));
  }
  const int qpos = has_q ? __builtin_amdgcn_readfirstlane(query_pos(p.qp, b, t)) : -1;
  float* srow = has_q ? p.scores + ((int64_t)b * p.T + t) * p.row_len : nullptr;
  if (has_q)
    for (int s = max(c0, qpos + 1) + lane; s < c1; s += kWave)
      srow[s] = out_val(p, -__builtin_inff());
  const int kend = min(c1, qmax + 1);
  if (kend <= c0) return;   // workgroup-uniform
  const int nst = (kend - c0 + kStageKeys - 1) / kStageKeys;

  // this wave's query: every share's loads, the first two key stages, then
  // the quantisation (a query row past T re-reads row 0 and scores nothing)
  const int64_t qrow = (int64_t)b * p.T + (has_q ? t : 0);
  const uint16_t* qsrc = p.q_idx + qrow * p.H_I * DI;
  uint4 raw[MB][DI / 64][4];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int ks = 0; ks < DI / 64; ++ks)
      load_share_q8<DI>(qsrc, p.H_I, m, ks, lane, raw[m][ks]);
  const float wraw = p.w[qrow * p.H_I + min(lane, p.H_I - 1)];
  TileStageQ8<DI> st[2];
  tile_load_q8<DI>(st[0], p.keys, b, c0, tid);
  tile_load_q8<DI>(st[1], p.keys, b, c0 + min(1, nst - 1) * kStageKeys, tid);
  v8i a[MB][DI / 64];
  int as[MB][DI / 64];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int ks = 0; ks < DI / 64; ++ks)
      quantise_share_q8(raw[m][ks], m * 32 + (lane & 31) < p.H_I, lane,
                        a[m][ks], as[m][ks]);
  float wv[MB][16];
  spread_weights_q8<MB>(lane < p.H_I ? wraw : 0.f, lane, wv);

  // two stages in flight in registers: stage i+2 loads while stage i is
  // computed (the tail re-loads the last stage, whose loads are never stored)
  const auto stage = [&](int i, TileStageQ8<DI>& sr) {
    uint4* tile = lds[i & 1];
    uint32_t* sl = scl[i & 1];
    tile_store_q8<DI>(sr, tile, sl, tid);
    tile_load_q8<DI>(sr, p.keys, b, c0 + min(i + 2, nst - 1) * kStageKeys, tid);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kStageKeys / kSub; ++u) {
      const int kb = c0 + i * kStageKeys + u * kSub;
      if (has_q && kb <= qpos) {   // wave-uniform
        const float sc = tile_scores_q8<DI, MB>(tile + u * kSub * CL::kChunks,
                                                sl + u * kSub, a, as, wv, lane);
        const int s = kb + (lane & 31);
        if (lane < 32 && s <= qpos && s < c1) srow[s] = out_val(p, sc);
      }
    }
  };
  int i = 0;
  for (; i + 1 < nst; i += 2) {
    stage(i, st[0]);
    stage(i + 1, st[1]);
  }
  if (i < nst) stage(i, st[0]);
}

// Keys per workgroup of the query-tiled kernels.  Each workgroup loads its
// eight queries and fills its two-stage pipeline once, so long chunks pay
// that over more stages: on the 4096-query prefill chunk (512 query tiles
// of 61K-65K causal keys) 2048 keys per workgroup took 3.61 ms, 8192 3.43,
// 32768 3.31 (quantised indexer 2.70, 2.44, 2.33 ms); from position 0
// (rows up to 4096) 0.198 ms at 2048 against 0.166 at 4096.  The chunk is
// sized for about 512 workgroups (two per CU) and kept within [2048, 32768]
// keys, so that small grids keep the 2048-key chunks.
int tile_kpw(const IndexerLaunch& p) {
  const int64_t tiles = (int64_t)p.B * ((p.T + kTileQ - 1) / kTileQ);
  int64_t kpw = (int64_t)p.row_len * tiles / 512;
  kpw = (kpw + kStageKeys - 1) / kStageKeys * kStageKeys;
  return (int)(kpw < 2048 ? 2048 : (kpw > 32768 ? 32768 : kpw));
}

template <int DI, int MB>
hipError_t launch_tile_q8(const IndexerLaunch& p, hipStream_t stream) {
  const int kpw = tile_kpw(p);
  dim3 grid((p.row_len + kpw - 1) / kpw, (p.T + kTileQ - 1) / kTileQ, p.B);
  hipLaunchKernelGGL((indexer_tile_q8_kernel<DI, MB>), grid,
                     dim3(kTileQ * kWave), 0, stream, p, kpw);
  return hipGetLastError();
}

template <int DI, int MB, bool FP8>
hipError_t launch_tile(const IndexerLaunch& p, hipStream_t stream) {
  const int kpw = tile_kpw(p);
  dim3 grid((p.row_len + kpw - 1) / kpw, (p.T + kTileQ - 1) / kTileQ, p.B);
  hipLaunchKernelGGL((indexer_tile_kernel<DI, MB, FP8>), grid,
                     dim3(kTileQ * kWave), 0, stream, p, kpw);
  return hipGetLastError();
}

// Positions per wave of the stream kernels, for about 1024 waves (one per
// SIMD on 256 CUs) for bf16 keys, or 2048 for FP8 keys (half the bytes per
// stage: a second wave per SIMD keeps as many bytes in flight and hides each
// wave's matrix and dequantisation work).  Longer waves pay their query
// setup less often: the bf16 kernel, with the non-temporal key stream,
// measured 47.7-48.8 us for 1024 waves against 48.7-49.7 us for 2048 (4096:
// 48.2-49.2) on the bf16 decode batch; the quantised one, with its stages in
// LDS, 26.4-26.7 us for 2048 against 28.4-28.7 us for 1024 on the FP8
// decode batch.  Whole 32-key stages, 64..4096.
int stream_kpw(const IndexerLaunch& p) {
  const int64_t total = (int64_t)p.B * p.T * p.row_len;
  const int64_t waves = p.keys.fp8 ? 2048 : 1024;
  int64_t kpw = (total + waves - 1) / waves;
  kpw = (kpw + kSub - 1) / kSub * kSub;
  return (int)(kpw < 64 ? 64 : (kpw > 4096 ? 4096 : kpw));
}

template <int DI, int MB, bool FP8>
hipError_t launch_stream(const IndexerLaunch& p, hipStream_t stream) {
  const int kpw = stream_kpw(p);
  const int per_wg = kpw * kWavesPerWG;
  dim3 grid((p.row_len + per_wg - 1) / per_wg, p.T, p.B);
  const int xcd_rows = ((p.B * p.T) & 7) == 0 ? 1 : 0;
  hipLaunchKernelGGL((indexer_stream_kernel<DI, MB, FP8>), grid, dim3(256), 0,
                     stream, p, (int)kpw, xcd_rows);
  return hipGetLastError();
}

template <int DI, int MB>
hipError_t launch_stream_q8(const IndexerLaunch& p, hipStream_t stream) {
  const int kpw = stream_kpw(p);
  const int per_wg = kpw * kWavesPerWG;
  dim3 grid((p.row_len + per_wg - 1) / per_wg, p.T, p.B);
  const int xcd_rows = ((p.B * p.T) & 7) == 0 ? 1 : 0;
  hipLaunchKernelGGL((indexer_stream_q8_kernel<DI, MB>), grid, dim3(256), 0,
                     stream, p, (int)kpw, xcd_rows);
  return hipGetLastError();
}

template <int DI, int MB, bool FP8>
hipError_t launch_any(const IndexerLaunch& p, hipStream_t stream) {
  // several queries per sequence share every key read: tile them
  return p.T >= kTileQ ? launch_tile<DI, MB, FP8>(p, stream)
                       : launch_stream<DI, MB, FP8>(p, stream);
}

template <int DI, int MB>
hipError_t launch_q8(const IndexerLaunch& p, hipStream_t stream) {
  return p.T >= kTileQ ? launch_tile_q8<DI, MB>(p, stream)
                       : launch_stream_q8<DI, MB>(p, stream);
}

// ------------------------------------------ fused indexer + Top-K (decode)
// Scoring, head weighting and Top-K of one query row in a single kernel that
// reads the paged keys and writes only the selected positions; the scores
// stay in LDS (page "Inference Adaptation and Performance Optimization for
// New Large Language Model Architectures", section 3.1 "Fused Index
// Computation"; page "Day-0 Inference Adaptation and Performance
// Optimization for New-Architecture Large Language Models", "Fusing the
// Indexer to Reduce Intermediate Write-Backs").
// One workgroup of eight waves (two per SIMD) per query row:
//   * stream: stage i of the row's 32-key stages goes to wave i % 8, which
//     loads it as the stream kernel does, transposes it through its LDS tile
//     64 features at a time, scores it with the same products and stores
//     each score's order-preserving key at its position in LDS (32768 keys
//     fill 128 KiB; the eight tiles take the other 32 KiB);
//   * select: a radix select over the LDS keys (digits of up to 11 bits cut
//     from the row's key range, one histogram pass each) finds the K-th
//     largest key; the keys above it and the first keys equal to it in
//     position order go to their ascending output slots.
// A row is one CU's work here, against eight or more CUs in the two-kernel
// path, so the single kernel keeps pace only with about one row per CU.
constexpr int kFusedWaves = 8;
constexpr int kFusedThreads = kFusedWaves * kWave;
constexpr int kFusedDigitBits = 11;
constexpr int kFusedBins = 1 << kFusedDigitBits;
constexpr int kPassDI = 64;   // features of a stage in LDS at a time

// A wave's LDS tile holds 64 features of its stage's 32 keys (a stage of
// 128-feature keys goes through it in two passes), laid out as a whole
// stage of 64-feature keys: bf16 rows, or FP8 codes followed by the stage's
// 32 scale words.  Eight such tiles and 32768 keys fill the 160 KiB.
template <bool FP8>
constexpr int fused_tile_words() {
  return FP8 ? (kSub * kPassDI + kSub * 4) / 16
             : KeyLayout<kPassDI>::kTileBytes / 16;
}

// Pass p of a bf16 stage into the tile: chunks [8p, 8p+8) of every key
// (the lanes holding them store; a lane's chunk index is fixed by its lane).
template <int DI>
__device__ __forceinline__ void stage_store_pass(const Stage<DI>& st,
                                                 uint4* tile, int lane,
                                                 int p) {
  using KL = KeyLayout<DI>;
  using KP = KeyLayout<kPassDI>;
#pragma unroll
  for (int i = 0; i < Stage<DI>::N; ++i) {
    const int id = i * kWave + lane;
    const int n = id / KL::kChunks, c = id % KL::kChunks;
    if (c / KP::kChunks == p)
      tile[n * KP::kChunks + KP::slot(n, c % KP::kChunks)] = st.v[i];
  }
}

// The k-steps [4p, 4p+4) of tile_scores from a pass tile into acc.
template <int DI, int MB>
__device__ __forceinline__ void pass_products(const uint4* tile,
                                              const uint4 (&a)[MB][DI / 16],
                                              f32x16 (&acc)[MB], int lane,
                                              int p) {
  using KP = KeyLayout<kPassDI>;
  const int n = lane & 31, h = lane >> 5;
#pragma unroll
  for (int k = 0; k < KP::kSteps; ++k) {
    const uint4 bop = tile[n * KP::kChunks + KP::slot(n, 2 * k + h)];
#pragma unroll
    for (int m = 0; m < MB; ++m)
      acc[m] = mfma32(a[m][p * KP::kSteps + k], bop, acc[m]);
  }
}

// FP8 codes: pass p stores code chunks [4p, 4p+4) (MX blocks 2p, 2p+1).
template <int DI>
__device__ __forceinline__ void stage_store_f8_pass(const StageF8<DI>& st,
                                                    uint4* tile, int lane,
                                                    int p) {
  using CL = CodeLayout<DI>;
  using CP = CodeLayout<kPassDI>;
#pragma unroll
  for (int i = 0; i < CL::kLoads; ++i) {
    const int id = i * kWave + lane;
    const int n = id / CL::kChunks, c = id % CL::kChunks;
    if (c / CP::kChunks == p)
      tile[n * CP::kChunks + CP::slot(n, c % CP::kChunks)] = st.v[i];
  }
}

template <int DI, int MB>
__device__ __forceinline__ void pass_products_f8(const uint4* tile,
                                                 const uint4 (&a)[MB][DI / 16],
                                                 const uint32_t* scl,
                                                 f32x16 (&acc)[MB], int lane,
                                                 int p) {
  using CP = CodeLayout<kPassDI>;
  const int n = lane & 31, h = lane >> 5;
  const uint32_t sc = scl[n];
  uint4 cvs[kPassDI / 32];
#pragma unroll
  for (int jj = 0; jj < kPassDI / 32; ++jj)
    cvs[jj] = tile[n * CP::kChunks + CP::slot(n, 2 * jj + h)];
#pragma unroll
  for (int jj = 0; jj < kPassDI / 32; ++jj) {
    const int j = p * (kPassDI / 32) + jj;   // MX block of the key row
    const uint32_t e = (sc >> (8 * j)) & 0xffu;
    const uint4 b0 = dequant8_e4m3(make_uint2(cvs[jj].x, cvs[jj].y), e);
    const uint4 b1 = dequant8_e4m3(make_uint2(cvs[jj].z, cvs[jj].w), e);
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[m] = mfma32(a[m][2 * j], b0, acc[m]);
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[m] = mfma32(a[m][2 * j + 1], b1, acc[m]);
  }
}

// Quantised queries: k-step p of the scaled FP8 products (64 features, MX
// blocks 2p and 2p+1) from a pass tile of key codes, as tile_scores_q8.
template <int DI, int MB>
__device__ __forceinline__ void pass_products_q8(const uint4* tile,
                                                 const uint32_t* scl,
                                                 const v8i (&a)[MB][DI / 64],
                                                 const int (&as)[MB][DI / 64],
                                                 f32x16 (&acc)[MB], int lane,
                                                 int p) {
  using CP = CodeLayout<kPassDI>;
  const int n = lane & 31, h = lane >> 5;
  const v8i bop = join8(tile[n * CP::kChunks + CP::slot(n, h)],
                        tile[n * CP::kChunks + CP::slot(n, 2 + h)]);
  const int bs = (int)((scl[n] >> (8 * (2 * p + h))) & 0xffu);
#pragma unroll
  for (int m = 0; m < MB; ++m)
    acc[m] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
        a[m][p], bop, acc[m], 0, 0, 0, as[m][p], 0, bs);
}

template <bool FP8>
struct FusedShared {
  uint32_t key[kFusedMaxLen];   // score keys of positions 0 .. n-1
  union {
    uint4 tile[kFusedWaves][fused_tile_words<FP8>()];       // stream
    struct {   // quantised queries: the (head block, k-step) shares
      v8i code[4][kWave];
      int scale[4][kWave];
    } q;
    struct {                                                // select
      uint32_t hist[kFusedBins];
      uint32_t mn[kFusedWaves], mx[kFusedWaves];   // key range per wave
      uint32_t tot[kFusedWaves];                   // digit pass, per wave
      uint32_t ngt[kFusedWaves], neq[kFusedWaves]; // emit, per wave
      uint32_t pick, above;
    } t;
  } u;
};

__device__ __forceinline__ uint32_t fused_lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

template <int DI, int MB, bool FP8, bool Q8>
__global__ __launch_bounds__(kFusedThreads, 1) void index_topk_kernel(
    IndexerLaunch p, int K, int32_t* idx) {
  static_assert(!Q8 || FP8, "quantised queries take MX keys");
  __shared__ FusedShared<FP8> sm;
  static_assert(sizeof(FusedShared<FP8>) <= 160 * 1024, "LDS");
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int r = blockIdx.x, b = r / p.T, t = r % p.T;
  const int qpos = __builtin_amdgcn_readfirstlane(query_pos(p.qp, b, t));
  const int n = max(0, min(qpos + 1, p.row_len));   // causal positions
  const int kk = min(K, n);
  int32_t* out = idx + (int64_t)r * K;
  for (int i = kk + tid; i < K; i += kFusedThreads) out[i] = -1;
  if (kk == n) {   // every position is selected
    for (int i = tid; i < n; i += kFusedThreads) out[i] = i;
    return;
  }

  // ---- stream: scores of this wave's stages into sm.key
  const int nst = (n + kSub - 1) / kSub;
  const int nsub = nst > wave ? (nst - wave + kFusedWaves - 1) / kFusedWaves : 0;
  uint32_t kmn = ~0u, kmx = 0u;
  const int64_t qrow = (int64_t)b * p.T + t;
  // quantised queries: wave i < MB * DI/64 quantises share i of the query
  // into LDS (as the quantised stream kernel), every wave reads all shares
  // into its operands, and a second barrier frees the space for the tiles
  v8i qa[MB][DI / 64];
  int qas[MB][DI / 64];
  float qwv[MB][16];
  if constexpr (Q8) {
    constexpr int kShares = MB * (DI / 64);
    static_assert(kShares <= 4 && kShares <= kFusedWaves, "query shares");
    if (wave < kShares) {
      const int qm = wave / (DI / 64), qks = wave % (DI / 64);
      uint4 raw[4];
      load_share_q8<DI>(p.q_idx + qrow * p.H_I * DI, p.H_I, qm, qks, lane,
                        raw);
      v8i c;
      int sc;
      quantise_share_q8(raw, qm * 32 + (lane & 31) < p.H_I, lane, c, sc);
      sm.u.q.code[wave][lane] = c;
      sm.u.q.scale[wave][lane] = sc;
    }
    const float wraw = p.w[qrow * p.H_I + min(lane, p.H_I - 1)];
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int ks = 0; ks < DI / 64; ++ks) {
        qa[m][ks] = sm.u.q.code[m * (DI / 64) + ks][lane];
        qas[m][ks] = sm.u.q.scale[m * (DI / 64) + ks][lane];
      }
    spread_weights_q8<MB>(lane < p.H_I ? wraw : 0.f, lane, qwv);
    __syncthreads();
  }
  if (nsub > 0) {
    uint4 a[MB][DI / 16];
    float wv[MB][16];
    if constexpr (!Q8)
      load_query<DI, MB, FP8>(p.q_idx + qrow * p.H_I * DI, p.w + qrow * p.H_I,
                              p.H_I, lane, a, wv);
    uint4* tile = sm.u.tile[wave];
    const int last = nsub - 1;
    // first position of the wave's stage j (stages past the last repeat it
    // and are parked: their loads read nothing)
    const auto at = [&](int j) { return (wave + kFusedWaves * min(j, last)) * kSub; };
    const auto put = [&](int j, float sc) {
      const int s = (wave + kFusedWaves * j) * kSub + lane;
      if (lane < kSub && s < n) {
        const uint32_t k = score_key(sc);
        sm.key[s] = k;
        kmn = min(kmn, k);
        kmx = max(kmx, k);
      }
    };
    constexpr int kPasses = DI / kPassDI;
    if constexpr (FP8) {
      uint32_t* scl = reinterpret_cast<uint32_t*>(tile + kSub * kPassDI / 16);
      StageF8<DI> st[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        stage_load_f8<DI>(st[u], p.keys, b, at(u), lane, u > last);
      for (int i = 0; i < nsub; i += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          f32x16 acc[MB];
#pragma unroll
          for (int m = 0; m < MB; ++m) acc[m] = f32x16{};
          if (lane < kSub) scl[lane] = st[u].sc;
#pragma unroll
          for (int q = 0; q < kPasses; ++q) {
            stage_store_f8_pass<DI>(st[u], tile, lane, q);
            if (q == kPasses - 1)
              stage_load_f8<DI>(st[u], p.keys, b, at(i + u + 4), lane,
                                i + u + 4 > last);
            if constexpr (Q8)
              pass_products_q8<DI, MB>(tile, scl, qa, qas, acc, lane, q);
            else
              pass_products_f8<DI, MB>(tile, a, scl, acc, lane, q);
          }
          const float sc = head_weighted_relu<MB>(acc, Q8 ? qwv : wv);
          if (i + u < nsub) put(i + u, sc);
        }
      }
    } else {
      // two stages in flight: three or four measured no faster
      constexpr int NS = 2;
      Stage<DI> st[NS];
#pragma unroll
      for (int u = 0; u < NS; ++u)
        stage_load<DI>(st[u], p.keys, b, at(u), lane, u > last);
      for (int i = 0; i < nsub; i += NS) {
#pragma unroll
        for (int u = 0; u < NS; ++u) {
          f32x16 acc[MB];
#pragma unroll
          for (int m = 0; m < MB; ++m) acc[m] = f32x16{};
#pragma unroll
          for (int q = 0; q < kPasses; ++q) {
            stage_store_pass<DI>(st[u], tile, lane, q);
            if (q == kPasses - 1)
              stage_load<DI>(st[u], p.keys, b, at(i + u + NS), lane,
                             i + u + NS > last);
            pass_products<DI, MB>(tile, a, acc, lane, q);
          }
          const float sc = head_weighted_relu<MB>(acc, wv);
          if (i + u < nsub) put(i + u, sc);
        }
      }
    }
  }
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    kmn = min(kmn, (uint32_t)__shfl_xor((int)kmn, m));
    kmx = max(kmx, (uint32_t)__shfl_xor((int)kmx, m));
  }
  __syncthreads();   // keys complete; the stage tiles are free
  if (lane == 0) {
    sm.u.t.mn[wave] = kmn;
    sm.u.t.mx[wave] = kmx;
  }
  __syncthreads();
  uint32_t lo = sm.u.t.mn[0], hi = sm.u.t.mx[0];
#pragma unroll
  for (int w = 1; w < kFusedWaves; ++w) {
    lo = min(lo, sm.u.t.mn[w]);
    hi = max(hi, sm.u.t.mx[w]);
  }

  // ---- select: the K-th largest key thr, digit by digit.  Invariant: the
  // window [lo, hi] holds at least `rem` keys, and exactly kk - rem keys
  // lie above it.  Each pass leaves a window below 2^shift wide, so a
  // 32-bit range takes at most three passes (shifts 21, 10, 0).
  uint32_t rem = (uint32_t)kk;
  constexpr int kBinsPT = kFusedBins / kFusedThreads;
  for (int pass = 0; pass < 4 && lo != hi; ++pass) {   // uniform
    const uint32_t range = hi - lo;
    const int shift = max(0, 32 - (int)__builtin_clz(range) - kFusedDigitBits);
    const int nb = (int)(range >> shift) + 1;
    for (int i = tid; i < nb; i += kFusedThreads) sm.u.t.hist[i] = 0u;
    if (tid == 0) {
      sm.u.t.pick = 0u;
      sm.u.t.above = 0u;
    }
    __syncthreads();
    // sixteen keys of a thread are read before their atomics (a read
    // issued after an LDS atomic waits for it); 16-byte reads stay inside
    // the key array (their first position is a multiple of 4 below n)
    for (int s0 = tid * 4; s0 < n; s0 += kFusedThreads * 16) {
      uint4 kv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int s = s0 + u * kFusedThreads * 4;
        kv[u] = s < n ? *reinterpret_cast<const uint4*>(&sm.key[s])
                      : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int s = s0 + u * kFusedThreads * 4;
        const uint32_t ks[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (s + e < n && ks[e] >= lo && ks[e] <= hi)
            atomicAdd(&sm.u.t.hist[(ks[e] - lo) >> shift], 1u);
      }
    }
    __syncthreads();
    // thread tid owns digits tid*kBinsPT .. +kBinsPT-1; keys in the digits
    // of higher threads, by a suffix sum over the threads
    uint32_t c[kBinsPT], own = 0u;
#pragma unroll
    for (int i = 0; i < kBinsPT; ++i) {
      const int d = tid * kBinsPT + i;
      c[i] = d < nb ? sm.u.t.hist[d] : 0u;
      own += c[i];
    }
    uint32_t incl = own;   // inclusive prefix over the wave's lanes
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const uint32_t y = (uint32_t)__shfl_up((int)incl, o);
      if (lane >= o) incl += y;
    }
    const uint32_t wtot = (uint32_t)__shfl((int)incl, kWave - 1);
    if (lane == 0) sm.u.t.tot[wave] = wtot;
    __syncthreads();
    uint32_t run = wtot - incl;   // keys in higher lanes of this wave
    for (int w = wave + 1; w < kFusedWaves; ++w) run += sm.u.t.tot[w];
#pragma unroll
    for (int i = kBinsPT - 1; i >= 0; --i) {
      if (run < rem && rem <= run + c[i]) {
        sm.u.t.pick = (uint32_t)(tid * kBinsPT + i);
        sm.u.t.above = run;
      }
      run += c[i];
    }
    __syncthreads();
    const uint32_t d = sm.u.t.pick;
    rem -= sm.u.t.above;
    const uint32_t nlo = lo + (d << shift);
    hi = (int)d + 1 == nb ? hi : lo + ((d + 1) << shift) - 1u;
    lo = nlo;
    __syncthreads();   // pick and the sums are read before they are reused
  }
  const uint32_t thr = lo, need = rem;

  // ---- emit: wave w takes positions [w*C, (w+1)*C); keys equal to thr
  // are taken in position order, the first `need` of them
  const int C = (n + kFusedThreads - 1) / kFusedThreads * kWave;
  const int s0 = wave * C, s1 = min(s0 + C, n);
  uint32_t ngt = 0u, neq = 0u;
  for (int s = s0; s < s1; s += 4 * kWave) {   // four steps' reads first
    uint32_t k[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = s + u * kWave + lane;
      k[u] = q < s1 ? sm.key[q] : 0u;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ngt += __builtin_popcountll(__ballot(k[u] > thr));
      neq += __builtin_popcountll(__ballot(k[u] == thr));
    }
  }
  if (lane == 0) {
    sm.u.t.ngt[wave] = ngt;
    sm.u.t.neq[wave] = neq;
  }
  __syncthreads();
  uint32_t gt_before = 0u, eq_before = 0u;
  for (int w = 0; w < wave; ++w) {
    gt_before += sm.u.t.ngt[w];
    eq_before += sm.u.t.neq[w];
  }
  uint32_t slot = gt_before + min(need, eq_before), eqr = eq_before;
  for (int s = s0; s < s1; s += 4 * kWave) {
    uint32_t k[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = s + u * kWave + lane;
      k[u] = q < s1 ? sm.key[q] : 0u;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint64_t em = __ballot(k[u] == thr);
      const bool sel =
          k[u] > thr || (k[u] == thr && eqr + fused_lanes_below(em) < need);
      const uint64_t selm = __ballot(sel);
      const uint32_t o = slot + fused_lanes_below(selm);   // < kk
      if (sel && o < (uint32_t)K) out[o] = s + u * kWave + lane;
      eqr += __builtin_popcountll(em);
      slot += __builtin_popcountll(selm);
    }
  }
}

template <int DI, int MB, bool FP8, bool Q8 = false>
hipError_t launch_fused(const IndexerLaunch& p, int K, int32_t* idx,
                        hipStream_t stream) {
  hipLaunchKernelGGL((index_topk_kernel<DI, MB, FP8, Q8>), dim3(p.B * p.T),
                     dim3(kFusedThreads), 0, stream, p, K, idx);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer(const IndexerLaunch& p, hipStream_t stream) {
  const bool mb1 = p.H_I <= 32;
  if (p.q8) {   // quantised queries over MX keys
    if (p.d_I == 128)
      return mb1 ? launch_q8<128, 1>(p, stream) : launch_q8<128, 2>(p, stream);
    return mb1 ? launch_q8<64, 1>(p, stream) : launch_q8<64, 2>(p, stream);
  }
  if (p.d_I == 128) {
    if (p.keys.fp8)
      return mb1 ? launch_any<128, 1, true>(p, stream)
                 : launch_any<128, 2, true>(p, stream);
    return mb1 ? launch_any<128, 1, false>(p, stream)
               : launch_any<128, 2, false>(p, stream);
  }
  if (p.keys.fp8)
    return mb1 ? launch_any<64, 1, true>(p, stream)
               : launch_any<64, 2, true>(p, stream);
  return mb1 ? launch_any<64, 1, false>(p, stream)
             : launch_any<64, 2, false>(p, stream);
}

int indexer_span_kpw(const IndexerLaunch& p) {
  return p.T >= kTileQ ? 0 : stream_kpw(p);
}

hipError_t launch_index_topk(const IndexerLaunch& p, int K, int32_t* idx,
                             hipStream_t stream) {
  const bool mb1 = p.H_I <= 32;
  if (p.q8) {   // quantised queries over MX keys
    if (p.d_I == 128)
      return mb1 ? launch_fused<128, 1, true, true>(p, K, idx, stream)
                 : launch_fused<128, 2, true, true>(p, K, idx, stream);
    return mb1 ? launch_fused<64, 1, true, true>(p, K, idx, stream)
               : launch_fused<64, 2, true, true>(p, K, idx, stream);
  }
  if (p.d_I == 128) {
    if (p.keys.fp8)
      return mb1 ? launch_fused<128, 1, true>(p, K, idx, stream)
                 : launch_fused<128, 2, true>(p, K, idx, stream);
    return mb1 ? launch_fused<128, 1, false>(p, K, idx, stream)
               : launch_fused<128, 2, false>(p, K, idx, stream);
  }
  if (p.keys.fp8)
    return mb1 ? launch_fused<64, 1, true>(p, K, idx, stream)
               : launch_fused<64, 2, true>(p, K, idx, stream);
  return mb1 ? launch_fused<64, 1, false>(p, K, idx, stream)
             : launch_fused<64, 2, false>(p, K, idx, stream);
}

}  // namespace dsa
