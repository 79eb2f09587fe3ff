// Per-row Top-K selection by radix select (gfx950).
//
// The Lightning Indexer keeps the K highest-scoring history positions of each
// query (page "Day-0 Inference Optimization for a New Sparse Attention
// Architecture: A Technical Deep Dive", section 1; page "Day-0 Inference
// Adaptation and Performance Optimization for New-Architecture Large Language
// Models", "Fusing the Indexer to Reduce Intermediate Write-Backs": Top-K
// selection on chip, outputs only the final indices).  Equal scores go to the
// lower position; the chosen positions are written in ascending order.
//
// One 1024-thread workgroup per score row.  Scores become order-preserving
// uint32 keys.  Wave w owns the contiguous positions
// [w*KPT*64, (w+1)*KPT*64), lane l position w*KPT*64 + j*64 + l of step j,
// so one compare-and-ballot covers 64 consecutive positions.  Rows of up to
// 64K positions keep their keys in registers for the whole selection.
//
// The exact K-th largest key `thr` is found digit by digit, with the digits
// cut from the row's own key range [min, max] rather than from fixed bit
// fields: score distributions concentrate in a few exponents, and a fixed
// top-bits digit would pile the row into a handful of bins (slow, conflicting
// LDS atomics).  Each pass histograms the keys still in the window (up to 13
// bits, 8192 bins) and a block scan in descending digit order finds the digit
// holding the K-th key; rows need one to three passes.  Finally the keys
// > thr and the first `need` keys == thr (in position order) are selected and
// written at their ascending output slot, computed from ballots and per-wave
// counts.  All integer work on bit patterns: exact and deterministic.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kDigitBits = 13;
constexpr int kMaxBins = 1 << kDigitBits;
constexpr int kBinsPerThread = kMaxBins / kThreads;   // 8

struct alignas(16) TopkShared {
  uint32_t hist[2][kMaxBins];   // stored in descending digit order
  uint32_t wmin[kWaves], wmax[kWaves];
  uint32_t wsum[kWaves];
  uint32_t gcnt[kWaves], ecnt[kWaves];
  uint32_t pick[4][2];          // per pass: digit, keys in larger digits
};

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf,
                                               true);
}

__device__ __forceinline__ uint32_t readlane(uint32_t x, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)x, l);
}

// Inclusive prefix sum over the 64 lanes: row_shr steps inside each 16-lane
// row, then the row totals added across rows.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x, int lane) {
  x += dpp<0x111>(x);   // row_shr:1
  x += dpp<0x112>(x);   // row_shr:2
  x += dpp<0x114>(x);   // row_shr:4
  x += dpp<0x118>(x);   // row_shr:8
  const uint32_t r0 = readlane(x, 15), r1 = readlane(x, 31),
                 r2 = readlane(x, 47);
  const int row = lane >> 4;
  return x + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) +
         (row >= 3 ? r2 : 0u);
}

// Wave-wide min and max (row rotations, then the four row results).
__device__ __forceinline__ void wave_minmax(uint32_t& mn, uint32_t& mx) {
  mn = min(mn, dpp<0x128>(mn)); mx = max(mx, dpp<0x128>(mx));   // row_ror:8
  mn = min(mn, dpp<0x124>(mn)); mx = max(mx, dpp<0x124>(mx));   // row_ror:4
  mn = min(mn, dpp<0x122>(mn)); mx = max(mx, dpp<0x122>(mx));   // row_ror:2
  mn = min(mn, dpp<0x121>(mn)); mx = max(mx, dpp<0x121>(mx));   // row_ror:1
  mn = min(min(readlane(mn, 0), readlane(mn, 16)),
           min(readlane(mn, 32), readlane(mn, 48)));
  mx = max(max(readlane(mx, 0), readlane(mx, 16)),
           max(readlane(mx, 32), readlane(mx, 48)));
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// The digit holding the `rem`-th largest key of a histogram of `nb` bins kept
// in descending digit order (hist[0] = largest digit): thread t owns slots
// 8t..8t+7.  Returns the digit and the count of keys in larger digits, to
// every thread.  Two barriers.
__device__ __forceinline__ void pick_digit(const uint32_t* hist, int nb,
                                           uint32_t rem, TopkShared& sm,
                                           int pass, int tid, int lane,
                                           int wave, uint32_t& digit,
                                           uint32_t& above) {
  uint32_t c[kBinsPerThread];
  uint32_t s = 0;
  if (kBinsPerThread * tid < nb) {
    const uint4 a = reinterpret_cast<const uint4*>(hist)[2 * tid];
    const uint4 b = reinterpret_cast<const uint4*>(hist)[2 * tid + 1];
    c[0] = a.x; c[1] = a.y; c[2] = a.z; c[3] = a.w;
    c[4] = b.x; c[5] = b.y; c[6] = b.z; c[7] = b.w;
  } else {
#pragma unroll
    for (int u = 0; u < kBinsPerThread; ++u) c[u] = 0;
  }
#pragma unroll
  for (int u = 0; u < kBinsPerThread; ++u) s += c[u];
  const uint32_t incl = wave_incl_scan(s, lane);
  if (lane == kWave - 1) sm.wsum[wave] = incl;
  __syncthreads();
  uint32_t base = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) base += w < wave ? sm.wsum[w] : 0u;
  uint32_t run = base + incl - s;
#pragma unroll
  for (int u = 0; u < kBinsPerThread; ++u) {
    if (c[u] && run < rem && rem <= run + c[u]) {
      sm.pick[pass][0] = (uint32_t)(nb - 1 - (kBinsPerThread * tid + u));
      sm.pick[pass][1] = run;
    }
    run += c[u];
  }
  __syncthreads();
  digit = sm.pick[pass][0];
  above = sm.pick[pass][1];
}

// Keys of one wave step: resident rows hold them in registers, longer rows
// read them again from the score row.  Positions past the row's candidates
// get key 0, which no score maps to: it is below every window and every
// threshold, so no pass needs a separate validity test.
template <int KPT, bool RES>
struct RowKeys {
  uint32_t k[RES ? KPT : 1];
  const float* row;
  int n, base;   // candidate count, this lane's position at step 0

  __device__ __forceinline__ uint32_t at(int j) const {
    if constexpr (RES) {
      return k[j];
    } else {
      const int p = base + j * kWave;
      return p < n ? score_key(row[p]) : 0u;
    }
  }
};

template <int KPT, bool RES>
__global__ __launch_bounds__(kThreads, 1) void topk_kernel(TopkLaunch p) {
  __shared__ TopkShared sm;
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int r = blockIdx.x;
  const int b = r / p.T, t = r % p.T;
  const int qpos = query_pos(p.qp, b, t);
  const int n = max(0, min(qpos + 1, p.L));
  const int kk = min(p.K, n);
  int32_t* out = p.idx + (int64_t)r * p.K;

  for (int i = kk + tid; i < p.K; i += kThreads) out[i] = -1;
  if (kk == n) {  // every candidate is selected
    for (int i = tid; i < n; i += kThreads) out[i] = i;
    return;
  }

  RowKeys<KPT, RES> keys;
  keys.row = p.scores + (int64_t)r * p.L;
  keys.n = n;
  keys.base = wave * KPT * kWave + lane;
  // steps of this wave that hold any candidate (wave-uniform)
  const int nsteps =
      min(KPT, max(0, (n - wave * KPT * kWave + kWave - 1) / kWave));

  // ---- load; min / max over the candidates; clear both histograms
  uint32_t mn = 0xffffffffu, mx = 0u;   // min taken over key - 1
  if constexpr (RES) {
    if (wave * KPT * kWave + KPT * kWave <= n) {   // all candidates
      float v[KPT];
#pragma unroll
      for (int j = 0; j < KPT; ++j) v[j] = keys.row[keys.base + j * kWave];
#pragma unroll
      for (int j = 0; j < KPT; ++j) keys.k[j] = score_key(v[j]);
    } else {
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const int pp = keys.base + j * kWave;
        keys.k[j] = pp < n ? score_key(keys.row[pp]) : 0u;
      }
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      mn = min(mn, keys.k[j] - 1u);
      mx = max(mx, keys.k[j]);
    }
  } else {
#pragma unroll 8
    for (int j = 0; j < nsteps; ++j) {
      const uint32_t k = keys.at(j);
      mn = min(mn, k - 1u);
      mx = max(mx, k);
    }
  }
  {
    uint4* h = reinterpret_cast<uint4*>(&sm.hist[0][0]);
#pragma unroll
    for (int u = 0; u < 2 * kMaxBins / 4 / kThreads; ++u)
      h[u * kThreads + tid] = make_uint4(0, 0, 0, 0);
  }
  wave_minmax(mn, mx);
  if (lane == 0) {
    sm.wmin[wave] = mn;
    sm.wmax[wave] = mx;
  }
  __syncthreads();
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    kmin = min(kmin, sm.wmin[w]);
    kmax = max(kmax, sm.wmax[w]);
  }
  kmin += 1u;   // n >= 2 here, so some key is a candidate (>= 1)

  // ---- digit passes over the window [lo, lo + 2^sh) holding the K-th key
  uint32_t lo = kmin;
  const uint32_t range = kmax - kmin;
  int sh = range ? 32 - __builtin_clz(range) : 0;   // range < 2^sh
  uint32_t rem = (uint32_t)kk;
  for (int pass = 0; sh > 0; ++pass) {
    const int np = (sh + kDigitBits - 1) / kDigitBits;
    const int nbits = (sh + np - 1) / np;
    const int nsh = sh - nbits;
    const int nb = 1 << nbits;
    uint32_t* hist = sm.hist[pass & 1];
    if (pass >= 1) {   // the other buffer feeds the pass after this one
      uint4* h = reinterpret_cast<uint4*>(sm.hist[(pass + 1) & 1]);
#pragma unroll
      for (int u = 0; u < kMaxBins / 4 / kThreads; ++u)
        h[u * kThreads + tid] = make_uint4(0, 0, 0, 0);
    }
    // key 0 (no position) is below every window: lo >= kmin >= 1
    const uint64_t win = 1ull << sh;
    const auto count = [&](uint32_t k) {
      const uint32_t off = k - lo;
      if ((uint64_t)off < win && k >= lo)
        atomicAdd(&hist[nb - 1 - (int)(off >> nsh)], 1u);
    };
    if constexpr (RES) {
#pragma unroll
      for (int j = 0; j < KPT; ++j) count(keys.k[j]);
    } else {
#pragma unroll 8
      for (int j = 0; j < nsteps; ++j) count(keys.at(j));
    }
    __syncthreads();
    uint32_t d, above;
    pick_digit(hist, nb, rem, sm, pass, tid, lane, wave, d, above);
    lo += d << nsh;
    rem -= above;
    sh = nsh;
  }
  const uint32_t thr = lo;     // >= 1, so key 0 never counts below
  const uint32_t need = rem;   // keys equal to thr that are taken

  // ---- per-wave counts of keys > thr and == thr
  uint32_t gc = 0, ec = 0;
  if constexpr (RES) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      gc += __builtin_popcountll(__ballot(keys.k[j] > thr));
      ec += __builtin_popcountll(__ballot(keys.k[j] == thr));
    }
  } else {
    for (int j = 0; j < nsteps; ++j) {
      const uint32_t k = keys.at(j);
      gc += __builtin_popcountll(__ballot(k > thr));
      ec += __builtin_popcountll(__ballot(k == thr));
    }
  }
  if (lane == 0) {
    sm.gcnt[wave] = gc;
    sm.ecnt[wave] = ec;
  }
  __syncthreads();
  // equal keys before this wave, and its first output slot
  uint32_t erun = 0, slot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave) {
      const uint32_t e = sm.ecnt[w];
      const uint32_t take = erun >= need ? 0u : min(e, need - erun);
      slot += sm.gcnt[w] + take;
      erun += e;
    }
  }

  // ---- emit: keys > thr, and equal keys while fewer than `need` precede
  const auto emit = [&](int j, uint32_t k) {
    const uint64_t e = __ballot(k == thr);
    const bool sel = k > thr || (k == thr && erun + lanes_below(e) < need);
    const uint64_t sm_ = __ballot(sel);
    const uint32_t o = slot + lanes_below(sm_);
    if (sel && o < (uint32_t)kk) out[o] = keys.base + j * kWave;
    slot += __builtin_popcountll(sm_);
    erun += __builtin_popcountll(e);
  };
  if constexpr (RES) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) emit(j, keys.k[j]);
  } else {
    for (int j = 0; j < nsteps; ++j) emit(j, keys.at(j));
  }
}

template <int KPT, bool RES>
void launch_kpt(const TopkLaunch& p, hipStream_t stream) {
  hipLaunchKernelGGL((topk_kernel<KPT, RES>), dim3(p.rows), dim3(kThreads), 0,
                     stream, p);
}

}  // namespace

hipError_t launch_topk(const TopkLaunch& p, hipStream_t stream) {
  // positions per row a workgroup covers: 1024 * KPT
  if (p.L <= 4 * kThreads)
    launch_kpt<4, true>(p, stream);
  else if (p.L <= 16 * kThreads)
    launch_kpt<16, true>(p, stream);
  else if (p.L <= 32 * kThreads)
    launch_kpt<32, true>(p, stream);
  else if (p.L <= 64 * kThreads)
    launch_kpt<64, true>(p, stream);
  else
    launch_kpt<128, false>(p, stream);
  return hipGetLastError();
}

}  // namespace dsa
