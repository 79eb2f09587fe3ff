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
// One 1024-thread workgroup per score row:
//   1. scores become order-preserving uint32 keys (cached in LDS when the row
//      fits), with the row's min and max key;
//   2. radix passes of up to 11 bits, starting just below the common prefix
//      of min and max, narrow down the exact K-th largest key `thr` and how
//      many keys equal to it are taken (`need`);
//   3. an ordered pass over the row: every wave owns a contiguous range of
//      positions, ranks its keys with ballot/mbcnt prefix counts, and writes
//      each position with key > thr, plus the first `need` positions with
//      key == thr, at its final ascending slot.
// Everything is integer work on bit patterns, so the result is exact and
// deterministic.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kCacheKeys = 32768;   // rows up to this length live in LDS
constexpr int kBins = 2048;         // 11-bit digits

struct TopkShared {
  uint32_t hist[kBins];
  uint32_t red[2][kWaves];
  uint32_t wtot[kWaves];
  uint32_t gt_w[kWaves];
  uint32_t eq_w[kWaves];
  uint32_t pick[2];       // chosen digit, keys above it
};

__device__ __forceinline__ uint32_t prefix_below(uint64_t mask) {
  // number of set bits of `mask` in lanes below this one
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

template <bool CACHED>
__device__ __forceinline__ uint32_t key_at(const uint32_t* keys,
                                           const float* row, int i) {
  if constexpr (CACHED) return keys[i];
  return score_key(row[i]);
}

template <bool CACHED>
__global__ __launch_bounds__(kThreads, 1) void topk_kernel(TopkLaunch p) {
  __shared__ TopkShared sh;
  __shared__ __attribute__((aligned(16))) uint32_t keys[CACHED ? kCacheKeys : 4];
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

  // ---- keys, min and max (16-byte loads, eight in flight per thread)
  uint32_t kmin = 0xffffffffu, kmax = 0u;
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
        kmin = min(min(kmin, min(k0, k1)), min(k2, k3));
        kmax = max(max(kmax, max(k0, k1)), max(k2, k3));
      }
    }
  }
  for (int i = 4 * n4 + tid; i < n; i += kThreads) {
    const uint32_t k = score_key(row[i]);
    if constexpr (CACHED) keys[i] = k;
    kmin = min(kmin, k);
    kmax = max(kmax, k);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor(kmin, off, kWave));
    kmax = max(kmax, (uint32_t)__shfl_xor(kmax, off, kWave));
  }
  if (lane == 0) {
    sh.red[0][wave] = kmin;
    sh.red[1][wave] = kmax;
  }
  __syncthreads();
  kmin = sh.red[0][0];
  kmax = sh.red[1][0];
  for (int w = 1; w < kWaves; ++w) {
    kmin = min(kmin, sh.red[0][w]);
    kmax = max(kmax, sh.red[1][w]);
  }

  // ---- radix passes below the common prefix of kmin and kmax
  uint32_t prefix = 0;   // value of the fixed top `plen` bits
  int plen = 0;
  uint32_t remaining = kk;
  const uint32_t diff = kmin ^ kmax;
  if (diff == 0) {
    prefix = kmax;
    plen = 32;
  } else {
    plen = __builtin_clz(diff);
    prefix = plen ? (kmax >> (32 - plen)) : 0u;
  }
  while (plen < 32) {
    const int width = min(11, 32 - plen);
    const int shift = 32 - plen - width;
    const uint32_t dmask = (1u << width) - 1u;
    for (int i = tid; i < kBins; i += kThreads) sh.hist[i] = 0;
    __syncthreads();
#pragma unroll 8
    for (int i = tid; i < n; i += kThreads) {
      const uint32_t k = key_at<CACHED>(keys, row, i);
      const bool match = plen == 0 || (k >> (32 - plen)) == prefix;
      if (match) atomicAdd(&sh.hist[(k >> shift) & dmask], 1u);
    }
    __syncthreads();
    // thread tid owns digits (2047 - 2*tid) and (2046 - 2*tid): a scan in
    // descending digit order gives, per digit, the count of larger digits
    const int d0 = kBins - 1 - 2 * tid, d1 = d0 - 1;
    const uint32_t c0 = sh.hist[d0], c1 = sh.hist[d1];
    const uint32_t incl = wave_incl_scan(c0 + c1, lane);
    if (lane == kWave - 1) sh.wtot[wave] = incl;
    __syncthreads();
    uint32_t base = 0;
    for (int w = 0; w < wave; ++w) base += sh.wtot[w];
    const uint32_t above0 = base + incl - (c0 + c1);   // keys in digits > d0
    const uint32_t above1 = above0 + c0;
    if (c0 && above0 < remaining && remaining <= above0 + c0) {
      sh.pick[0] = d0;
      sh.pick[1] = above0;
    }
    if (c1 && above1 < remaining && remaining <= above1 + c1) {
      sh.pick[0] = d1;
      sh.pick[1] = above1;
    }
    __syncthreads();
    const uint32_t dsel = sh.pick[0];
    remaining -= sh.pick[1];
    prefix = (plen == 0 ? 0u : (prefix << width)) | dsel;
    plen += width;
    __syncthreads();   // hist and pick are rewritten by the next pass
  }
  const uint32_t thr = prefix;
  const uint32_t need = remaining;   // keys equal to thr that are taken

  // ---- ordered output
  const int seg = ((n + kWaves - 1) / kWaves + kWave - 1) / kWave * kWave;
  const int lo = wave * seg, hi = min(n, lo + seg);
  uint32_t gt = 0, eq = 0;
#pragma unroll 8
  for (int base = lo; base < hi; base += kWave) {
    const int i = base + lane;
    const uint32_t k = i < hi ? key_at<CACHED>(keys, row, i) : 0u;
    gt += (i < hi && k > thr);
    eq += (i < hi && k == thr);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    gt += __shfl_xor(gt, off, kWave);
    eq += __shfl_xor(eq, off, kWave);
  }
  if (lane == 0) {
    sh.gt_w[wave] = gt;
    sh.eq_w[wave] = eq;
  }
  __syncthreads();
  uint32_t eq_before = 0, sel_before = 0;
  for (int w = 0; w < wave; ++w) {
    const uint32_t take = eq_before >= need ? 0u : min(sh.eq_w[w], need - eq_before);
    sel_before += sh.gt_w[w] + take;
    eq_before += sh.eq_w[w];
  }
  for (int base = lo; base < hi; base += kWave) {
    const int i = base + lane;
    const bool valid = i < hi;
    const uint32_t k = valid ? key_at<CACHED>(keys, row, i) : 0u;
    const bool is_gt = valid && k > thr;
    const bool is_eq = valid && k == thr;
    const uint64_t eq_mask = __ballot(is_eq);
    const uint32_t eq_rank = eq_before + prefix_below(eq_mask);
    const bool sel = is_gt || (is_eq && eq_rank < need);
    const uint64_t sel_mask = __ballot(sel);
    const uint32_t slot = sel_before + prefix_below(sel_mask);
    if (sel && slot < (uint32_t)kk) out[slot] = i;
    eq_before += __popcll(eq_mask);
    sel_before += __popcll(sel_mask);
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
