// Internal launch interface between the C-ABI layer (dsa_api.cpp) and the
// kernel translation units.  Every function only enqueues work on `stream`
// and returns hipGetLastError()'s result.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// Storage formats of a cache row: bf16; e4m3 codes with one e8m0 scale per
// 32 features; e4m3 codes with one fp32 scale per 128-feature tile (a
// 576-wide row has 5 tiles, the last of 64 features).
constexpr int kFmtBf16 = 0, kFmtMx32 = 1, kFmtT128 = 2;
constexpr int kT128Tiles = 5;

// Where a query's history lives: either a contiguous [B, L, width] tensor
// (page_table == nullptr) or a paged pool read through a page table.
struct CacheView {
  const uint8_t* data;        // rows of `row_bytes` bytes
  const uint8_t* scale;       // e8m0 codes (width/32 per row), fp32 tile
                              // scales (5 per row, t128) or nullptr
  const int32_t* page_table;  // [B, max_pages] or nullptr (contiguous)
  int max_pages;
  int L;                      // contiguous length (rows per sequence)
  bool fp8;                   // e4m3 codes + scales, else bf16
  uint64_t bytes;             // size of `data` in bytes
  bool t128;                  // fp8 with fp32 scales per 128-feature tile
  int num_pages;              // pages in the pool (paged); page entries are
                              // clamped to [0, num_pages)
};

// Query positions: q_pos[b*T + t] if given, else seq_lens[b] - 1; with
// seq_lens given, a position is clamped to seq_lens[b] - 1.
struct QueryPos {
  const int32_t* q_pos;
  const int32_t* seq_lens;
  int T;
};

__device__ __forceinline__ int query_pos(const QueryPos& qp, int b, int t) {
  int p = qp.q_pos ? qp.q_pos[(int64_t)b * qp.T + t] : qp.seq_lens[b] - 1;
  if (qp.seq_lens) p = min(p, qp.seq_lens[b] - 1);
  return p;
}

struct IndexerLaunch {
  int B, T, H_I, d_I;
  const uint16_t* q_idx;   // [B, T, H_I, d_I] bf16
  const float* w;          // [B, T, H_I]
  CacheView keys;          // width d_I
  QueryPos qp;
  float* scores;           // [B*T, row_len]
  int row_len;             // positions written per row (L or max_seq_len)
  int keys_out;            // store score_key(score) bit patterns, not scores
  int q8;                  // quantise q_idx to MX block-32 and use the scaled
                           // FP8 matrix cores (keys must be MX32)
  float* span;             // keys_out only, or nullptr: per query row
                           // kSpanMax (min, max) key pairs, one per wave of
                           // the row (wave c covers positions c*kpw ..);
                           // waves past the row's causal positions write
                           // nothing.  The uint32 keys are stored as float bit
                           // patterns: stores of an integer type could alias
                           // the page table, whose loads then could not be
                           // scalar loads
};
constexpr int kSpanMax = 64;   // waves per row with a key-range entry
hipError_t launch_indexer(const IndexerLaunch& a, hipStream_t stream);
// Positions per wave (and per span entry) of the stream kernel a launch
// runs, or 0 when it keeps no key ranges (a tile kernel for several queries
// per sequence, or the FP8-key kernel with bf16 queries).
int indexer_span_kpw(const IndexerLaunch& a);
// Indexer and Top-K of each query row in one kernel (bf16 or, with a.q8,
// quantised queries): one workgroup per row holds the row's score keys in
// LDS, so rows are limited to
// kFusedMaxLen positions (a.row_len <= kFusedMaxLen); writes idx [B*T, K]
// (ascending positions, -1 padded), no scores.
constexpr int kFusedMaxLen = 32768;
hipError_t launch_index_topk(const IndexerLaunch& a, int K, int32_t* idx,
                             hipStream_t stream);

struct TopkLaunch {
  int rows, T, L, K;       // rows = B*T; scores row stride = L
  const float* scores;
  QueryPos qp;
  int32_t* idx;            // [rows, K]
  int nchunks, chunk;      // long rows: chunks per row, positions per chunk
  int32_t* cand;           // long rows: [rows, nchunks, K] candidate lists
  int keys_in;             // scores holds score_key bit patterns already
  const uint32_t* span;    // keys_in rows only, or nullptr: the indexer's
  int span_kpw;            // per-row key ranges, one per span_kpw positions
                           // (entries past a row's causal positions unused)
};
// One workgroup per row.
hipError_t launch_topk(const TopkLaunch& a, hipStream_t stream);
// Rows longer than 64K positions go through per-chunk candidate lists when
// the workspace holds topk_workspace_bytes(); otherwise as above.
hipError_t launch_topk(const TopkLaunch& a, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);
int topk_chunks(int L);
size_t topk_workspace_bytes(int rows, int L, int K);

struct AttnLaunch {
  int B, T, H, K;
  const uint16_t* q;       // [B, T, H, 576] bf16
  CacheView kv;            // width 576
  const int32_t* idx;      // [B*T, K]
  const int32_t* seq_lens; // [B] valid positions per sequence, or nullptr
                           // (contiguous: kv.L)
  float scale;             // softmax scale
  float* out;              // [B*T, H, 512]
  float* lse;              // [B*T, H]
  float* partial;          // workspace for split partials (may be unused)
  int splits;              // row splits per token (>= 1)
};
// Number of row splits the attention uses for a shape, and the workspace
// bytes its partials need.
int attn_splits(int tokens, int K);
size_t attn_workspace_bytes(int tokens, int H, int K);
hipError_t launch_sparse_mla(const AttnLaunch& a, hipStream_t stream);

struct AppendLaunch {
  int tokens, T;               // tokens = B*T, T per sequence
  const int32_t* pos;          // [tokens] logical positions; < 0 skipped
  const int32_t* page_table;   // [B, max_pages]
  int max_pages, num_pages;
  int d_I, kidx_fmt;           // indexer keys: width, kFmtBf16 or kFmtMx32
  const uint16_t* k_new;       // [tokens, d_I] bf16, or nullptr
  uint8_t* kidx;               // pool [num_pages, 64, d_I]
  void* kidx_scale;            // pool [num_pages, 64, d_I/32] e8m0
  int kv_fmt;                  // latent rows: any format
  const uint16_t* kv_new;      // [tokens, 576] bf16, or nullptr
  uint8_t* kv;                 // pool [num_pages, 64, 576]
  void* kv_scale;              // pool [num_pages, 64, 18] e8m0 or [.., 5] fp32
};
// One wave per token; tokens whose page is unmapped are skipped.
hipError_t launch_cache_append(const AppendLaunch& a, hipStream_t stream);

}  // namespace dsa
