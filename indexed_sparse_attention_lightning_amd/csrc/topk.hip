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
// uint32 keys (cached in LDS when the row fits).  The exact K-th largest key
// `thr` is found digit by digit, 12 + 12 + 8 bits from the top: each pass
// histograms the keys that share the digits fixed so far, and a block scan in
// descending digit order finds the digit holding the K-th key.  A last pass
// marks, with one wave ballot per 64 positions, a bitmap of keys > thr and one
// of keys == thr; the first `need` set bits of the second (in position order)
// join the first, and word-level prefix popcounts give every selected
// position its ascending output slot.  All of it is integer work on bit
// patterns: exact and deterministic.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kCacheKeys = 32768;          // rows up to this length live in LDS
constexpr int kBins = 4096;                // 12-bit digits
constexpr int kMaxRow = 131072;            // longest row of the uncached path
constexpr int kMaxWords = kMaxRow / 32;    // bitmap words for that row

struct alignas(16) Small {
  uint32_t wsum[kWaves];
  uint32_t pick[2];      // chosen digit, keys in larger digits
};

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

// Exclusive prefix of v over the block in thread order; also returns the
// block total.  Two barriers.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, Small& sm,
                                                   int tid, int lane,
                                                   uint32_t& total) {
  const int wave = tid / kWave;
  const uint32_t incl = wave_incl_scan(v, lane);
  if (lane == kWave - 1) sm.wsum[wave] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t x = sm.wsum[w];
    base += w < wave ? x : 0u;
    tot += x;
  }
  total = tot;
  __syncthreads();
  return base + incl - v;
}

// The digit holding the `remaining`-th largest key: thread tid owns digits
// nbins-1-4*tid .. nbins-4-4*tid (descending order across the block).
// Returns the digit and the count of keys in larger digits, to every thread.
__device__ __forceinline__ void pick_digit(const uint32_t* hist, int nbins,
                                           uint32_t remaining, Small& sm,
                                           int tid, int lane,
                                           uint32_t& digit, uint32_t& above) {
  uint32_t c[4];
  uint32_t s = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int d = nbins - 1 - 4 * tid - u;
    c[u] = d >= 0 ? hist[d] : 0u;
    s += c[u];
  }
  uint32_t total;
  uint32_t run = block_excl_scan(s, sm, tid, lane, total);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int d = nbins - 1 - 4 * tid - u;
    if (c[u] && run < remaining && remaining <= run + c[u]) {
      sm.pick[0] = (uint32_t)d;
      sm.pick[1] = run;
    }
    run += c[u];
  }
  __syncthreads();
  digit = sm.pick[0];
  above = sm.pick[1];
  __syncthreads();
}

template <bool CACHED>
__device__ __forceinline__ uint32_t key_at(const uint32_t* keys,
                                           const float* row, int i) {
  if constexpr (CACHED) return keys[i];
  return score_key(row[i]);
}

template <bool CACHED>
__global__ __launch_bounds__(kThreads, 1) void topk_kernel(TopkLaunch p) {
  // LDS: key cache | histogram, reused afterwards for the two bitmaps
  constexpr int kHist = CACHED ? kBins : 2 * kMaxWords;
  __shared__ __attribute__((aligned(16))) uint32_t keys[CACHED ? kCacheKeys : 4];
  __shared__ __attribute__((aligned(16))) uint32_t hist[kHist];
  __shared__ Small sm;
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = tid / kWave;
  const int r = blockIdx.x;
  const int b = r / p.T, t = r % p.T;
  const int qpos = query_pos(p.qp, b, t);
  const int n = max(0, min(qpos + 1, p.L));
  const int kk = min(p.K, n);
  int32_t* out = p.idx + (int64_t)r * p.K;
  const float* row = p.scores + (int64_t)r * p.L;

  for (int i = kk + tid; i < p.K; i += kThreads) out[i] = -1;
  if (kk == n) {  // every candidate is selected
    for (int i = tid; i < n; i += kThreads) out[i] = i;
    return;
  }

  // ---- pass 1: keys (cached), histogram of the top 12 bits
  for (int i = tid; i < kBins; i += kThreads) hist[i] = 0;
  __syncthreads();
  {
    const bool vec = ((reinterpret_cast<uintptr_t>(row) & 15) == 0);
    const int n4 = vec ? n / 4 : 0;
    for (int base = 0; base < n4; base += 8 * kThreads) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i4 = base + u * kThreads + tid;
        v[u] = i4 < n4 ? reinterpret_cast<const float4*>(row)[i4]
                       : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i4 = base + u * kThreads + tid;
        if (i4 < n4) {
          const uint32_t k0 = score_key(v[u].x), k1 = score_key(v[u].y);
          const uint32_t k2 = score_key(v[u].z), k3 = score_key(v[u].w);
          if constexpr (CACHED)
            reinterpret_cast<uint4*>(keys)[i4] = make_uint4(k0, k1, k2, k3);
          atomicAdd(&hist[k0 >> 20], 1u);
          atomicAdd(&hist[k1 >> 20], 1u);
          atomicAdd(&hist[k2 >> 20], 1u);
          atomicAdd(&hist[k3 >> 20], 1u);
        }
      }
    }
    for (int i = 4 * n4 + tid; i < n; i += kThreads) {
      const uint32_t k = score_key(row[i]);
      if constexpr (CACHED) keys[i] = k;
      atomicAdd(&hist[k >> 20], 1u);
    }
  }
  __syncthreads();
  uint32_t d1, above;
  pick_digit(hist, kBins, (uint32_t)kk, sm, tid, lane, d1, above);
  uint32_t remaining = (uint32_t)kk - above;

  // ---- pass 2: the next 12 bits among keys whose top 12 bits are d1
  for (int i = tid; i < kBins; i += kThreads) hist[i] = 0;
  __syncthreads();
#pragma unroll 8
  for (int i = tid; i < n; i += kThreads) {
    const uint32_t k = key_at<CACHED>(keys, row, i);
    if ((k >> 20) == d1) atomicAdd(&hist[(k >> 8) & 0xfffu], 1u);
  }
  __syncthreads();
  uint32_t d2;
  pick_digit(hist, kBins, remaining, sm, tid, lane, d2, above);
  remaining -= above;
  const uint32_t pre24 = (d1 << 12) | d2;

  // ---- pass 3: the last 8 bits
  for (int i = tid; i < 256; i += kThreads) hist[i] = 0;
  __syncthreads();
#pragma unroll 8
  for (int i = tid; i < n; i += kThreads) {
    const uint32_t k = key_at<CACHED>(keys, row, i);
    if ((k >> 8) == pre24) atomicAdd(&hist[k & 0xffu], 1u);
  }
  __syncthreads();
  uint32_t d3;
  pick_digit(hist, 256, remaining, sm, tid, lane, d3, above);
  const uint32_t thr = (pre24 << 8) | d3;
  const uint32_t need = remaining - above;   // keys equal to thr that are taken

  // ---- pass 4: bitmaps of keys > thr and keys == thr (one ballot per 64)
  const int nwords = (n + 31) / 32;
  uint32_t* gtw = hist;
  uint32_t* eqw = hist + kHist / 2;
#pragma unroll 4
  for (int base = wave * kWave; base < n; base += kThreads) {
    const int i = base + lane;
    const uint32_t k = i < n ? key_at<CACHED>(keys, row, i) : 0u;
    const uint64_t g = __ballot(i < n && k > thr);
    const uint64_t e = __ballot(i < n && k == thr);
    if (lane == 0) {
      const int w = base / 32;
      gtw[w] = (uint32_t)g;
      eqw[w] = (uint32_t)e;
      if (w + 1 < nwords) {
        gtw[w + 1] = (uint32_t)(g >> 32);
        eqw[w + 1] = (uint32_t)(e >> 32);
      }
    }
  }
  __syncthreads();

  // ---- keep the first `need` equal keys in position order, then emit the
  // selected positions in ascending order
  constexpr int kWPT = kHist / 2 / kThreads;   // bitmap words per thread
  uint32_t ew[kWPT], sw[kWPT];
  uint32_t ecount = 0;
#pragma unroll
  for (int u = 0; u < kWPT; ++u) {
    const int w = tid * kWPT + u;
    ew[u] = w < nwords ? eqw[w] : 0u;
    ecount += __builtin_popcount(ew[u]);
  }
  uint32_t etotal;
  uint32_t ebefore = block_excl_scan(ecount, sm, tid, lane, etotal);
  uint32_t scount = 0;
#pragma unroll
  for (int u = 0; u < kWPT; ++u) {
    const int w = tid * kWPT + u;
    uint32_t e = ew[u];
    const uint32_t c = __builtin_popcount(e);
    if (ebefore >= need) {
      e = 0;
    } else if (ebefore + c > need) {
      uint32_t keep = need - ebefore, m = e;   // the lowest `keep` set bits
      e = 0;
      while (keep--) {
        const uint32_t lo = m & (0u - m);
        e |= lo;
        m ^= lo;
      }
    }
    ebefore += c;
    sw[u] = (w < nwords ? gtw[w] : 0u) | e;
    scount += __builtin_popcount(sw[u]);
  }
  uint32_t stotal;
  uint32_t slot = block_excl_scan(scount, sm, tid, lane, stotal);
#pragma unroll
  for (int u = 0; u < kWPT; ++u) {
    const int w = tid * kWPT + u;
    uint32_t m = sw[u];
    while (m) {
      const int bit = __builtin_ctz(m);
      m &= m - 1;
      if (slot < (uint32_t)kk) out[slot] = w * 32 + bit;
      ++slot;
    }
  }
}

}  // namespace

hipError_t launch_topk(const TopkLaunch& p, hipStream_t stream) {
  if (p.L <= kCacheKeys)
    hipLaunchKernelGGL(topk_kernel<true>, dim3(p.rows), dim3(kThreads), 0,
                       stream, p);
  else
    hipLaunchKernelGGL(topk_kernel<false>, dim3(p.rows), dim3(kThreads), 0,
                       stream, p);
  return hipGetLastError();
}

}  // namespace dsa
