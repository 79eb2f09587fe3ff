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
// Longer rows, given a workspace, go in two launches: one workgroup per
// 16K-position chunk selects the chunk's own Top-K into a candidate list,
// then one workgroup per row selects from its chunks' lists (the row's Top-K
// lies in their union, and list order is position order); without the
// workspace one workgroup streams the whole row through each pass.
//
// The exact K-th largest key `thr` is found digit by digit, with the digits
// cut from the row's own key range [min, max] rather than from fixed bit
// fields: score distributions concentrate in a few exponents, and a fixed
// top-bits digit would pile the row into a handful of bins (slow, conflicting
// LDS atomics).  Each pass histograms the keys still in the window (up to 13
// bits, 8192 bins) and a block scan in descending digit order finds the digit
// holding the K-th key; rows need one to three passes, except that when the
// first pass leaves at most 64 keys in that digit one wave sorts them.
// Finally the keys > thr and the first `need` keys == thr (in position
// order) are selected and written at their ascending output slot, computed
// from ballots and per-wave counts.  All integer work on bit patterns: exact
// and deterministic.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kDigitBits = 13;
constexpr int kMaxBins = 1 << kDigitBits;
constexpr int kBinsPerThread = kMaxBins / kThreads;   // 8

constexpr int kSlab = 512;                  // candidates a wave may keep
constexpr int kMaxWords = 131072 / 32;      // bitmap words of the longest row

struct alignas(16) TopkShared {
  uint32_t hist[kMaxBins + 4];   // hist[d]: keys with digit d; the slot past
                                 // the last digit is a sink
  uint2 slab[kWaves][kSlab];     // per wave: (position, key) of candidates
  uint32_t gtw[kMaxWords];       // bitmap: selected keys above thr
  uint32_t eqw[kMaxWords];       // bitmap: keys equal to thr
  uint32_t wmin[kWaves], wmax[kWaves];
  uint32_t wsum[kWaves];
  uint32_t scnt[kWaves];         // candidates per wave
  uint32_t pick[4][3];           // per pass: digit, keys above, keys in it
  uint32_t overflow;
};

// Unsigned compare predicates of __builtin_amdgcn_uicmpl (LLVM's ICmp codes).
constexpr int kCmpUgt = 34, kCmpUge = 35, kCmpUle = 37;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf,
                                               true);
}

__device__ __forceinline__ uint32_t readlane(uint32_t x, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)x, l);
}

// Lane l of `reg` takes the wave-uniform value v (v_writelane_b32).
__device__ __forceinline__ uint32_t writelane(uint32_t reg, uint32_t v,
                                              int l) {
  asm("s_nop 4\n\tv_writelane_b32 %0, %1, %2" : "+v"(reg) : "s"(v), "i"(l));
  return reg;
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

// Keeps the scheduler from hoisting work of later key steps over earlier
// ones (register pressure: one live temporary per step otherwise).
#define TOPK_STEP_FENCE(j) \
  if (((j) & 7) == 7) __builtin_amdgcn_sched_barrier(0)

// Exclusive prefix of v over the block in thread order, and the block
// total.  Two barriers (the second frees wsum for the next use).
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v,
                                                   struct TopkShared& sm,
                                                   int tid, int lane,
                                                   uint32_t& total);

// Per-wave values arr[0..kWaves): the sum over waves before `wave` and the
// total, with one LDS read per lane (not one register per wave).
__device__ __forceinline__ void waves_prefix(const uint32_t* arr, int lane,
                                             int wave, uint32_t& before,
                                             uint32_t& total) {
  const uint32_t incl = wave_incl_scan(lane < kWaves ? arr[lane] : 0u, lane);
  total = readlane(incl, kWaves - 1);
  before = wave ? readlane(incl, wave - 1) : 0u;
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// The digit holding the `rem`-th largest key of a histogram of `nb` bins
// (hist[d] counts digit d): thread t owns the digits nb-1-8t .. nb-8-8t, in
// descending order.  Returns the digit, the count of keys in larger digits
// and the count in the digit itself, to every thread.  Two barriers.
__device__ __forceinline__ void pick_digit(const uint32_t* hist, int nb,
                                           uint32_t rem, TopkShared& sm,
                                           int pass, int tid, int lane,
                                           int wave, uint32_t& digit,
                                           uint32_t& above, uint32_t& count) {
  uint32_t c[kBinsPerThread];
  const int top = nb - kBinsPerThread * tid;   // one past this thread's digits
  if (top >= kBinsPerThread) {
    const uint4 a = reinterpret_cast<const uint4*>(hist)[top / 4 - 2];
    const uint4 b = reinterpret_cast<const uint4*>(hist)[top / 4 - 1];
    c[0] = b.w; c[1] = b.z; c[2] = b.y; c[3] = b.x;
    c[4] = a.w; c[5] = a.z; c[6] = a.y; c[7] = a.x;
  } else {
#pragma unroll
    for (int u = 0; u < kBinsPerThread; ++u)
      c[u] = top - 1 - u >= 0 ? hist[top - 1 - u] : 0u;
  }
  uint32_t s = 0;
#pragma unroll
  for (int u = 0; u < kBinsPerThread; ++u) s += c[u];
  const uint32_t incl = wave_incl_scan(s, lane);
  if (lane == kWave - 1) sm.wsum[wave] = incl;
  __syncthreads();
  uint32_t base, total;
  waves_prefix(sm.wsum, lane, wave, base, total);
  uint32_t run = base + incl - s;
#pragma unroll
  for (int u = 0; u < kBinsPerThread; ++u) {
    if (c[u] && run < rem && rem <= run + c[u]) {
      sm.pick[pass][0] = (uint32_t)(top - 1 - u);
      sm.pick[pass][1] = run;
      sm.pick[pass][2] = c[u];
    }
    run += c[u];
  }
  __syncthreads();
  digit = sm.pick[pass][0];
  above = sm.pick[pass][1];
  count = sm.pick[pass][2];
}

__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v,
                                                   TopkShared& sm, int tid,
                                                   int lane, uint32_t& total) {
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const uint32_t incl = wave_incl_scan(v, lane);
  if (lane == kWave - 1) sm.wsum[wave] = incl;
  __syncthreads();
  uint32_t base;
  waves_prefix(sm.wsum, lane, wave, base, total);
  __syncthreads();
  return base + incl - v;
}

// Keys of one wave step.  Once the row's smallest key is known they are kept
// relative to it minus one (r = key - kmin >= 1, so a pass's digit is a
// shift of r); resident rows hold them in registers, longer rows read them
// again from the score row.  Lanes past the row's n candidates get r = 0,
// which the histograms and candidate lists skip (one compare; no position
// test).
// A loaded row value as a key: the scores' keys, or the value itself when
// the row already holds keys (the fused path's indexer writes them).
__device__ __forceinline__ uint32_t as_key(uint32_t raw, bool keys_in) {
  return keys_in ? raw : score_key(__builtin_bit_cast(float, raw));
}

template <int KPT, bool RES>
struct RowKeys {
  uint32_t k[RES ? KPT : 1];
  const float* row;
  int n;            // candidate count
  int wbase;        // first position of the wave (uniform)
  int lane;
  uint32_t kmin;
  bool keys_in;

  // compares the lane against a uniform bound: no per-step registers
  __device__ __forceinline__ bool valid(int j) const {
    return lane < n - wbase - j * kWave;
  }
  __device__ __forceinline__ int pos(int j) const {
    return wbase + j * kWave + lane;
  }
  __device__ __forceinline__ uint32_t rel(int j) const {
    if constexpr (RES) {
      return k[j];
    } else {
      return valid(j) ? as_key(__builtin_bit_cast(uint32_t, row[pos(j)]), keys_in) - kmin : 0u;
    }
  }

  // Rows read again from memory: f(j, key) for steps 0..nsteps-1 in chunks
  // of kChunk steps, every load of a chunk issued together and the next
  // chunk's loads in flight while this one is processed.  Buffer loads
  // bounded by the candidate count read 0 past n.
  static constexpr int kChunk = 16;
  template <class F>
  __device__ __forceinline__ void stream(int nsteps, F&& f) const {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(row), 0, n * 4, 0x00020000);
    const uint32_t voff = (uint32_t)(wbase + lane) * 4;
    uint32_t cur[kChunk], nxt[kChunk];
#pragma unroll
    for (int u = 0; u < kChunk; ++u)
      cur[u] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
          rs, voff + u * kWave * 4, 0, 0);
    for (int j0 = 0; j0 < nsteps; j0 += kChunk) {
#pragma unroll
      for (int u = 0; u < kChunk; ++u)
        nxt[u] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
            rs, voff + (j0 + kChunk + u) * kWave * 4, 0, 0);
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        const int j = j0 + u;
        if (j < nsteps)   // wave-uniform
          f(j, valid(j) ? as_key(cur[u], keys_in) - kmin : 0u);
      }
#pragma unroll
      for (int u = 0; u < kChunk; ++u) cur[u] = nxt[u];
    }
  }
};

// What one workgroup selects from:
//   kRow     a whole score row (positions 0..n-1, n from the query position);
//   kChunk   chunk c of a row (its positions c*chunk ..), writing the chunk's
//            own Top-K as row positions (-1 padded) to the candidate lists;
//   kGather  a row's candidate lists (nchunks * K slots of positions in
//            ascending order, -1 holes), each slot's key read from the row
//            at its position.  A row's Top-K lies in the union of its chunks'
//            Top-Ks (an entry of the row's Top-K has fewer than K entries
//            above it in its own chunk), and slot order is position order,
//            so ties still go to the lower position.
//   kRowSpan as kRow, for rows whose keys the indexer wrote together with
//            each of its waves' (min, max) key: the row's range is known
//            before the keys arrive, so the first histogram counts each key
//            step as its load completes (no pass and barrier for the range)
enum TopkMode { kRow = 0, kChunk = 1, kGather = 2, kRowSpan = 3 };

template <int KPT, bool RES, int MODE = kRow>
__global__ __launch_bounds__(kThreads, 1) void topk_kernel(TopkLaunch p) {
  __shared__ TopkShared sm;
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int r = MODE == kChunk ? blockIdx.x / p.nchunks : blockIdx.x;
  const int b = r / p.T, t = r % p.T;
  const int qpos = query_pos(p.qp, b, t);
  const int nrow = max(0, min(qpos + 1, p.L));   // causal candidates of the row
  int n, kk, pbase = 0;
  const float* rowp = p.scores + (int64_t)r * p.L;
  const int32_t* cand = nullptr;
  int32_t* out;
  if constexpr (MODE == kRow || MODE == kRowSpan) {
    n = nrow;
    kk = min(p.K, n);
    out = p.idx + (int64_t)r * p.K;
  } else if constexpr (MODE == kChunk) {
    const int c = blockIdx.x % p.nchunks;
    pbase = c * p.chunk;
    n = max(0, min(nrow - pbase, p.chunk));
    kk = min(p.K, n);
    rowp += pbase;
    out = p.cand + (int64_t)blockIdx.x * p.K;
  } else {
    n = p.nchunks * p.K;   // candidate slots
    kk = min(p.K, nrow);
    cand = p.cand + (int64_t)r * n;
    out = p.idx + (int64_t)r * p.K;
  }

  for (int i = kk + tid; i < p.K; i += kThreads) out[i] = -1;
  if (kk == n) {  // every candidate is selected
    for (int i = tid; i < n; i += kThreads)
      out[i] = MODE == kGather ? cand[i] : pbase + i;
    return;
  }
  if (MODE == kGather && kk == 0) return;

  // the row's key range from the indexer's span entries 0 .. ns-1 (those
  // that cover its causal positions 0 .. n-1), loaded before the keys: the
  // wait counter retires loads in issue order
  uint32_t smn = 0xffffffffu, smx = 0u;
  if constexpr (MODE == kRowSpan) {
    const int ns = (n + p.span_kpw - 1) / p.span_kpw;
    const uint2 v = reinterpret_cast<const uint2*>(
        p.span)[(int64_t)r * kSpanMax + min(lane, ns - 1)];
    if (lane < ns) {
      smn = v.x;
      smx = v.y;
    }
  }

  RowKeys<KPT, RES> keys;
  keys.row = rowp;
  keys.keys_in = p.keys_in != 0;
  keys.n = n;
  keys.wbase = wave * KPT * kWave;
  keys.lane = lane;
  keys.kmin = 0;
  // steps of this wave that hold any candidate (wave-uniform)
  const int nsteps =
      min(KPT, max(0, (n - wave * KPT * kWave + kWave - 1) / kWave));

  // ---- load; min / max over the candidates; clear histogram and bitmap
  uint32_t mn = 0xffffffffu, mx = 0u;   // min taken over key - 1
  if constexpr (RES) {
    // buffer loads bounded by the candidate count: positions past n read 0
    // without branches, and all loads share one offset register
    if constexpr (MODE == kGather) {
      // slot positions first (slots past n are holes), then the scores at
      // those positions (a hole's offset is out of the row's range: the
      // bounded load reads 0 without touching memory); a hole gets key 0
      const __amdgpu_buffer_rsrc_t cs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<int32_t*>(cand), 0, n * 4, 0x00020000);
      int32_t ps[KPT];
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const int32_t v = __builtin_amdgcn_raw_buffer_load_b32(
            cs, (keys.wbase + lane) * 4, j * kWave * 4, 0);
        ps[j] = keys.valid(j) ? v : -1;
      }
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(keys.row), 0, nrow * 4, 0x00020000);
#pragma unroll
      for (int j = 0; j < KPT; ++j)
        keys.k[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
            rs, (uint32_t)ps[j] * 4u, 0, 0);
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        keys.k[j] = ps[j] >= 0 ? as_key(keys.k[j], keys.keys_in) : 0u;
        mn = min(mn, keys.k[j] - 1u);
        mx = max(mx, keys.k[j]);
      }
    } else {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(keys.row), 0, n * 4, 0x00020000);
#pragma unroll
      for (int j = 0; j < KPT; ++j)
        keys.k[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
            rs, (keys.wbase + lane) * 4, j * kWave * 4, 0);
      // keys of candidates are >= 1 (NaN maps to 1): 0 marks a lane past n
      // (only waves that reach past n test positions; the conversion is
      // skipped when the row holds keys).  kRowSpan rows hold keys and
      // the bounded loads read 0 past n: nothing to convert, and the range
      // comes from the span entries.
      if constexpr (MODE != kRowSpan) {
        const bool padded = keys.wbase + KPT * kWave > n;   // wave-uniform
        const bool kin = keys.keys_in;
        if (padded) {
#pragma unroll
          for (int j = 0; j < KPT; ++j)
            keys.k[j] = keys.valid(j) ? as_key(keys.k[j], kin) : 0u;
        } else if (!kin) {
#pragma unroll
          for (int j = 0; j < KPT; ++j)
            keys.k[j] = score_key(__builtin_bit_cast(float, keys.k[j]));
        }
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
          mn = min(mn, keys.k[j] - 1u);
          mx = max(mx, keys.k[j]);
        }
      }
    }
  } else {
    // kmin is still 0: absolute keys, 0 past n
    keys.stream(nsteps, [&](int, uint32_t k) {
      mn = min(mn, k - 1u);
      mx = max(mx, k);
    });
  }
  {
    uint4* h = reinterpret_cast<uint4*>(sm.hist);
    for (int i = tid; i < (kMaxBins + 4) / 4; i += kThreads)
      h[i] = make_uint4(0, 0, 0, 0);
    uint4* e = reinterpret_cast<uint4*>(sm.eqw);
    for (int i = tid; i < kMaxWords / 4; i += kThreads)
      e[i] = make_uint4(0, 0, 0, 0);
    if (tid == 0) sm.overflow = 0u;
  }
  uint32_t kmin, kmax;
  if constexpr (MODE == kRowSpan) {
    // every wave reduces the span entries itself: no exchange
    kmin = smn != 0xffffffffu ? smn - 1u : 0xffffffffu;
    kmax = smx;
    wave_minmax(kmin, kmax);
    __syncthreads();   // the cleared histogram and bitmap
  } else {
    wave_minmax(mn, mx);
    if (lane == 0) {
      sm.wmin[wave] = mn;
      sm.wmax[wave] = mx;
    }
    __syncthreads();
    kmin = lane < kWaves ? sm.wmin[lane] : 0xffffffffu;
    kmax = lane < kWaves ? sm.wmax[lane] : 0u;
    wave_minmax(kmin, kmax);
  }
  // some lane holds a candidate (n >= 2 here).  kmin is the smallest
  // candidate key minus one: candidates have relative keys >= 1 and lanes
  // past n (or holes between candidate slots) the relative key 0, which no
  // histogram, candidate list or bitmap takes.
  keys.kmin = kmin;
  if constexpr (RES && MODE != kRowSpan) {   // kRowSpan: in the first count
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      keys.k[j] = keys.k[j] ? keys.k[j] - kmin : 0u;
  }

  // ---- first digit over all keys: digit(r) = r >> nsh, r <= range
  const uint32_t range = kmax - kmin;
  const int sh0 = 32 - __builtin_clz(range);   // range >= 1, < 2^sh0
  uint32_t rem = (uint32_t)kk;
  uint32_t d0 = 0, cnt0 = 0;
  int nsh = 0;
  if (sh0 > 0) {
    const int np = (sh0 + kDigitBits - 1) / kDigitBits;
    const int nbits = (sh0 + np - 1) / np;
    nsh = sh0 - nbits;
    const int nb = 1 << nbits;
    const auto count = [&](int j, uint32_t rk) {
      (void)j;
      if (rk != 0u) atomicAdd(&sm.hist[rk >> nsh], 1u);   // rk <= range < 2^sh0
    };
    // only waves that reach past n (or hold candidate-slot holes) have
    // keys to skip; the others count without the test
    const bool padded = MODE == kGather || keys.wbase + KPT * kWave > n;
    if constexpr (MODE == kRowSpan) {
      // each key step is made relative and counted as its load completes
      if (padded) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
          const uint32_t k = keys.k[j];
          const uint32_t rk = k ? k - kmin : 0u;
          keys.k[j] = rk;
          if (rk != 0u) atomicAdd(&sm.hist[rk >> nsh], 1u);
          TOPK_STEP_FENCE(j);
        }
      } else {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
          const uint32_t rk = keys.k[j] - kmin;   // keys >= 1 > kmin
          keys.k[j] = rk;
          atomicAdd(&sm.hist[rk >> nsh], 1u);
          TOPK_STEP_FENCE(j);
        }
      }
    } else if constexpr (RES) {
      if (padded) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
          count(j, keys.k[j]);
          TOPK_STEP_FENCE(j);
        }
      } else {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
          atomicAdd(&sm.hist[keys.k[j] >> nsh], 1u);
          TOPK_STEP_FENCE(j);
        }
      }
    } else {
      keys.stream(nsteps, count);
    }
    __syncthreads();
    uint32_t above;
    pick_digit(sm.hist, nb, rem, sm, 0, tid, lane, wave, d0, above, cnt0);
    rem -= above;
  }
  // digit d0 spans relative keys [blo, bhi]; blo1 leaves out the key 0 of
  // lanes past n
  const uint32_t blo = d0 << nsh;
  const uint32_t bhi = blo | ((1u << nsh) - 1u);
  const uint32_t blo1 = blo > 1u ? blo : 1u;

  // ---- sweep: bitmap of keys in larger digits; keys in digit d0 are
  // final (nsh == 0: they all equal the threshold) or go to the wave's
  // candidate list, in position order
  uint32_t ns = 0;
  // resident rows gather the wave's 2*KPT mask words in registers (word i
  // in lane i % 64 of register i / 64) and store them once
  constexpr int kMaskRegs = RES ? (2 * KPT + kWave - 1) / kWave : 1;
  uint32_t gwr[kMaskRegs], ewr[kMaskRegs];
#pragma unroll
  for (int i = 0; i < kMaskRegs; ++i) gwr[i] = ewr[i] = 0u;
  const auto sweep = [&](int j, uint32_t rk) {
    // lane masks straight from the compares (a ballot of a flag is lowered
    // through a vector register: two more instructions every step); the
    // 64-step kernel, short of registers, spills more with them and keeps
    // the ballots
    uint64_t g, c;
    if constexpr (KPT <= 32) {
      g = __builtin_amdgcn_uicmpl(rk, bhi, kCmpUgt);
      c = __builtin_amdgcn_uicmpl(rk, blo1, kCmpUge) &
          __builtin_amdgcn_uicmpl(rk, bhi, kCmpUle);
    } else {
      g = __ballot(rk > bhi);
      c = __ballot(rk >= blo1 && rk <= bhi);
    }
    if constexpr (RES) {
      const int i0 = (2 * j) / kWave, l0 = (2 * j) % kWave;
      gwr[i0] = writelane(gwr[i0], (uint32_t)g, l0);
      gwr[i0] = writelane(gwr[i0], (uint32_t)(g >> 32), l0 + 1);
      if (nsh == 0) {
        ewr[i0] = writelane(ewr[i0], (uint32_t)c, l0);
        ewr[i0] = writelane(ewr[i0], (uint32_t)(c >> 32), l0 + 1);
      }
    } else {
      const int wd = 2 * (wave * KPT + j);
      if (lane == 0) {
        sm.gtw[wd] = (uint32_t)g;
        sm.gtw[wd + 1] = (uint32_t)(g >> 32);
        if (nsh == 0) {
          sm.eqw[wd] = (uint32_t)c;
          sm.eqw[wd + 1] = (uint32_t)(c >> 32);
        }
      }
    }
    if (nsh != 0 && c != 0ull) {   // (the digit test again: rarely taken)
      const uint32_t at = ns + lanes_below(c);
      if (rk >= blo1 && rk <= bhi && at < (uint32_t)kSlab)
        sm.slab[wave][at] = make_uint2((uint32_t)keys.pos(j), rk);
      ns += __builtin_popcountll(c);
    }
  };
  if constexpr (RES) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      sweep(j, keys.k[j]);
      TOPK_STEP_FENCE(j);
    }
  } else {
    keys.stream(nsteps, sweep);
  }
  if constexpr (RES) {
#pragma unroll
    for (int i = 0; i < kMaskRegs; ++i) {
      const int wd = i * kWave + lane;
      if (wd < 2 * KPT) {
        sm.gtw[2 * wave * KPT + wd] = gwr[i];
        if (nsh == 0) sm.eqw[2 * wave * KPT + wd] = ewr[i];
      }
    }
  }
  if (lane == 0) {
    sm.scnt[wave] = min(ns, (uint32_t)kSlab);
    if (ns > (uint32_t)kSlab) sm.overflow = 1u;
  }
  __syncthreads();

  uint32_t thr = blo;            // relative threshold
  uint32_t eq_total = cnt0;
  uint32_t ctot, cbefore;        // keys listed in the threshold digit
  waves_prefix(sm.scnt, lane, wave, cbefore, ctot);
  if (nsh > 0 && sm.overflow == 0u && ctot <= (uint32_t)kWave) {
    // ---- few keys in the threshold digit (the usual case: about ten in a
    // 32K-position decode row): wave 0 orders them by key, then position,
    // and marks the first `rem` in the above-threshold bitmap, in place of
    // the remaining digit passes (each a histogram clear, a count and a
    // block scan, with four barriers)
    if (wave == 0) {
      // lane i takes candidate i of the waves' lists, in wave order
      const uint32_t c = lane < kWaves ? sm.scnt[lane] : 0u;
      const uint32_t incl = wave_incl_scan(c, lane);
      int w = 0;
#pragma unroll
      for (int x = 0; x < kWaves; ++x)
        w += readlane(incl, x) <= (uint32_t)lane ? 1 : 0;
      // list entries before wave w (read with every lane active: a lane
      // reading an inactive lane's register gets 0)
      const int ws = min(w, kWaves - 1);
      const uint32_t ew = (uint32_t)__shfl((int)incl, ws) -
                          (uint32_t)__shfl((int)c, ws);
      uint64_t v = 0;   // (key << 32) | ~position; 0 for lanes past the list
      if ((uint32_t)lane < ctot) {
        const uint2 cd = sm.slab[w][lane - ew];
        v = ((uint64_t)cd.y << 32) | (uint32_t)~cd.x;
      }
      // bitonic sort across the lanes, descending: larger keys first, equal
      // keys by ascending position (relative keys of candidates are >= 1)
#pragma unroll
      for (int k = 2; k <= kWave; k <<= 1)
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
          const uint64_t o =
              ((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), j) << 32) |
              (uint32_t)__shfl_xor((int)(uint32_t)v, j);
          const bool keep_max = ((lane & k) == 0) == ((lane & j) == 0);
          v = keep_max ? (v > o ? v : o) : (v < o ? v : o);
        }
      if ((uint32_t)lane < rem) {
        const uint32_t pos = ~(uint32_t)v;
        atomicOr(&sm.gtw[pos >> 5], 1u << (pos & 31));
      }
    }
    rem = 0;        // the taken keys are all in the bitmap
    eq_total = 0;
    __syncthreads();
  } else if (nsh > 0) {
    // ---- the remaining digits, on the candidates only (or, if a wave's
    // list overflowed, on all keys again)
    const bool ovf = sm.overflow != 0u;
    uint32_t lo = blo;
    int sh = nsh;
    for (int pass = 1; sh > 0; ++pass) {
      const int np = (sh + kDigitBits - 1) / kDigitBits;
      const int nbits = (sh + np - 1) / np;
      const int psh = sh - nbits;
      const int nb = 1 << nbits;
      {
        uint4* h = reinterpret_cast<uint4*>(sm.hist);
        for (int i = tid; i < kMaxBins / 4; i += kThreads)
          h[i] = make_uint4(0, 0, 0, 0);
      }
      __syncthreads();
      const uint32_t win = 1u << sh;   // window [lo, lo + 2^sh)
      if (!ovf) {   // each wave counts its own candidates
        const int nc = (int)sm.scnt[wave];
        for (int e = lane; e < nc; e += kWave) {
          const uint32_t rk = sm.slab[wave][e].y;
          if (rk >= lo && rk - lo < win)
            atomicAdd(&sm.hist[(rk - lo) >> psh], 1u);
        }
      } else {
        const auto count = [&](int j, uint32_t rk) {
          (void)j;
          const bool in = rk >= (lo > 1u ? lo : 1u) && rk - lo < win;
          if (__ballot(in) != 0ull && in)
            atomicAdd(&sm.hist[(rk - lo) >> psh], 1u);
        };
        if constexpr (RES) {
#pragma unroll
          for (int j = 0; j < KPT; ++j) {
            count(j, keys.k[j]);
            TOPK_STEP_FENCE(j);
          }
        } else {
          keys.stream(nsteps, count);
        }
      }
      __syncthreads();
      uint32_t d, above, cnt;
      pick_digit(sm.hist, nb, rem, sm, pass, tid, lane, wave, d, above, cnt);
      lo += d << psh;
      rem -= above;
      sh = psh;
      eq_total = cnt;
    }
    thr = lo;
    // ---- keys of digit d0 above thr join the bitmap; those equal to thr
    // form the equal-key bitmap
    if (!ovf) {
      const int nc = (int)sm.scnt[wave];
      for (int e = lane; e < nc; e += kWave) {
        const uint2 c = sm.slab[wave][e];
        if (c.y > thr) atomicOr(&sm.gtw[c.x >> 5], 1u << (c.x & 31));
        else if (c.y == thr) atomicOr(&sm.eqw[c.x >> 5], 1u << (c.x & 31));
      }
    } else {
      const auto marks = [&](int j, uint32_t rk) {
        const uint64_t g = __ballot(rk > thr);
        const uint64_t e = __ballot(rk == thr);
        const int wd = 2 * (wave * KPT + j);
        if (lane == 0) {
          sm.gtw[wd] = (uint32_t)g;
          sm.gtw[wd + 1] = (uint32_t)(g >> 32);
          sm.eqw[wd] = (uint32_t)e;
          sm.eqw[wd + 1] = (uint32_t)(e >> 32);
        }
      };
      if constexpr (RES) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
          marks(j, keys.k[j]);
          TOPK_STEP_FENCE(j);
        }
      } else {
        keys.stream(nsteps, marks);
      }
    }
    __syncthreads();
  }
  const uint32_t need = rem;   // keys equal to thr that are taken

  // ---- thread t owns bitmap words [t*q, t*q + q): keep the first `need`
  // equal keys in position order, then emit in ascending order
  const int nw = (n + 31) / 32;
  const int q = (nw + kThreads - 1) / kThreads;
  const int w0 = tid * q, w1 = min(nw, w0 + q);
  const bool ties = need < eq_total;   // keep only the lowest equal keys
  uint32_t ebefore = 0;
  if (ties) {
    uint32_t ecount = 0;
    for (int w = w0; w < w1; ++w) ecount += __builtin_popcount(sm.eqw[w]);
    uint32_t total;
    ebefore = block_excl_scan(ecount, sm, tid, lane, total);
  }
  uint32_t scount = 0;
  for (int w = w0; w < w1; ++w) {
    uint32_t e = sm.eqw[w];
    if (ties) {
      const uint32_t ce = __builtin_popcount(e);
      if (ebefore >= need) {
        e = 0u;
      } else if (ebefore + ce > need) {
        uint32_t keep = need - ebefore, m = e;   // the lowest `keep` bits
        e = 0u;
        while (keep--) {
          const uint32_t lowbit = m & (0u - m);
          e |= lowbit;
          m ^= lowbit;
        }
      }
      ebefore += ce;
    }
    const uint32_t sel = sm.gtw[w] | e;
    sm.eqw[w] = sel;
    scount += __builtin_popcount(sel);
  }
  uint32_t stotal;
  uint32_t slot = block_excl_scan(scount, sm, tid, lane, stotal);
  for (int w = w0; w < w1; ++w) {
    uint32_t m = sm.eqw[w];
    while (m) {
      const int bit = __builtin_ctz(m);
      m &= m - 1;
      if (slot < (uint32_t)kk)
        out[slot] = MODE == kGather ? cand[w * 32 + bit] : pbase + w * 32 + bit;
      ++slot;
    }
  }
}

template <int KPT, bool RES, int MODE = kRow>
void launch_kpt(const TopkLaunch& p, hipStream_t stream) {
  hipLaunchKernelGGL((topk_kernel<KPT, RES, MODE>), dim3(p.rows),
                     dim3(kThreads), 0, stream, p);
}

constexpr int kChunkLen = 16 * kThreads;   // positions per chunk workgroup

}  // namespace

int topk_chunks(int L) {
  return L > 64 * kThreads ? (L + kChunkLen - 1) / kChunkLen : 0;
}

size_t topk_workspace_bytes(int rows, int L, int K) {
  return (size_t)rows * topk_chunks(L) * K * sizeof(int32_t);
}

hipError_t launch_topk(const TopkLaunch& p0, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  // Rows past 64K positions: one workgroup per 16K-position chunk selects
  // the chunk's Top-K (keys in registers), then one workgroup per row
  // selects from the chunks' candidates.  Without the workspace for the
  // candidate lists, one workgroup streams the whole row.
  const int nch = topk_chunks(p0.L);
  const size_t need = topk_workspace_bytes(p0.rows, p0.L, p0.K);
  if (nch > 0 && workspace && workspace_bytes >= need) {
    TopkLaunch p = p0;
    p.nchunks = nch;
    p.chunk = kChunkLen;
    p.cand = static_cast<int32_t*>(workspace);
    hipLaunchKernelGGL((topk_kernel<16, true, kChunk>), dim3(p.rows * nch),
                       dim3(kThreads), 0, stream, p);
    const int slots = nch * p.K;   // <= 8 * 2048
    if (slots <= 4 * kThreads)
      hipLaunchKernelGGL((topk_kernel<4, true, kGather>), dim3(p.rows),
                         dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((topk_kernel<16, true, kGather>), dim3(p.rows),
                         dim3(kThreads), 0, stream, p);
    return hipGetLastError();
  }
  return launch_topk(p0, stream);
}

hipError_t launch_topk(const TopkLaunch& p, hipStream_t stream) {
  // positions per row a workgroup covers: 1024 * KPT
  if (p.span != nullptr && p.keys_in && p.span_kpw > 0 &&
      (p.L + p.span_kpw - 1) / p.span_kpw <= kSpanMax && p.L <= 64 * kThreads) {
    if (p.L <= 4 * kThreads)
      launch_kpt<4, true, kRowSpan>(p, stream);
    else if (p.L <= 16 * kThreads)
      launch_kpt<16, true, kRowSpan>(p, stream);
    else if (p.L <= 32 * kThreads)
      launch_kpt<32, true, kRowSpan>(p, stream);
    else
      launch_kpt<64, true, kRowSpan>(p, stream);
    return hipGetLastError();
  }
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
