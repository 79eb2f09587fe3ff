// C ABI of the DSA hot path: argument validation (host only, before any HIP
// call), workspace carving and the launch sequence on the caller's stream.
// The operations and their semantics are documented in include/dsa.h.
#include "../../include/dsa.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "dsa_launch.h"

namespace {

thread_local char g_last_error[256] = "";

dsa_status fail(dsa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

dsa_status ok() {
  g_last_error[0] = '\0';
  return DSA_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Indexer keys: bf16 or MX block-32; latent KV: any of the three formats.
bool valid_key_dtype(int d) { return d == DSA_BF16 || d == DSA_E4M3_MX32; }
bool valid_kv_dtype(int d) { return valid_key_dtype(d) || d == DSA_E4M3_T128; }

dsa::CacheView kv_view(const void* data, const void* scale, int dtype,
                       const int32_t* page_table, int max_pages, int L,
                       uint64_t rows, int num_pages) {
  const bool fp8 = dtype != DSA_BF16;
  return dsa::CacheView{static_cast<const uint8_t*>(data),
                        static_cast<const uint8_t*>(scale), page_table,
                        max_pages, L, fp8,
                        rows * DSA_LATENT_DIM * (fp8 ? 1 : 2),
                        dtype == DSA_E4M3_T128, num_pages};
}

// Grid limits: B*T query tokens index a grid dimension capped at 65535.
constexpr int kMaxTokens = 65535;

dsa_status check_indexer_dims(int B, int T, int H_I, int d_I) {
  if (B < 1 || T < 1) return fail(DSA_ERR_SHAPE, "B and T must be >= 1");
  if ((long long)B * T > kMaxTokens)
    return fail(DSA_ERR_UNSUPPORTED, "B*T must be <= %d", kMaxTokens);
  if (H_I < 1 || H_I > 64)
    return fail(DSA_ERR_UNSUPPORTED, "H_I must be in [1, 64], got %d", H_I);
  if (d_I != 64 && d_I != 128)
    return fail(DSA_ERR_UNSUPPORTED, "d_I must be 64 or 128, got %d", d_I);
  return DSA_OK;
}

dsa_status check_attn_dims(int B, int T, int H, int K) {
  if (B < 1 || T < 1) return fail(DSA_ERR_SHAPE, "B and T must be >= 1");
  if ((long long)B * T > kMaxTokens)
    return fail(DSA_ERR_UNSUPPORTED, "B*T must be <= %d", kMaxTokens);
  if (H < 1 || H > 128)
    return fail(DSA_ERR_UNSUPPORTED, "H must be in [1, 128], got %d", H);
  if (K < 1 || K > DSA_MAX_TOPK)
    return fail(DSA_ERR_UNSUPPORTED, "K must be in [1, %d], got %d",
                DSA_MAX_TOPK, K);
  return DSA_OK;
}

size_t decode_ws(int B, int T, int L, int H, int K) {
  const size_t tokens = (size_t)B * T;
  return align_up(tokens * (size_t)L * sizeof(float)) +
         align_up(tokens * (size_t)K * sizeof(int32_t)) +
         align_up(dsa::topk_workspace_bytes((int)tokens, L, K)) +
         align_up(dsa::attn_workspace_bytes((int)tokens, H, K)) +
         align_up(tokens * dsa::kSpanMax * 2 * sizeof(uint32_t));
}

// Quantised queries need MX keys: both operands of the scaled FP8 products.
dsa_status check_q_mode(int q_mode, bool mx_keys) {
  if (q_mode != DSA_Q_BF16 && q_mode != DSA_Q_MX32)
    return fail(DSA_ERR_UNSUPPORTED, "unknown q_mode %d", q_mode);
  if (q_mode == DSA_Q_MX32 && !mx_keys)
    return fail(DSA_ERR_UNSUPPORTED, "q_mode DSA_Q_MX32 needs MX32 keys");
  return DSA_OK;
}

dsa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Scratch of dsa_decode_step_static: device memory of the library itself, one
// copy per GPU, held until the process ends.  In host code `scratch` only
// names the symbol; its device address (different on every GPU) comes from
// hipGetSymbolAddress with that GPU current, looked up once per device and
// kept in g_scratch.  Nothing in it needs to start at zero: every byte a
// decode step reads from its workspace was written earlier in the same step.
constexpr size_t kScratchBytes = DSA_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

dsa_status static_scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "dsa_decode_step_static: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DSA_ERR_UNSUPPORTED, "device %d beyond the %d the library tracks",
                dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol,
                        "dsa_decode_step_static: hipGetSymbolAddress(scratch)");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return DSA_OK;
}

}  // namespace

extern "C" {

const char* dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_NULL: return "DSA_ERR_NULL: a required pointer is NULL";
    case DSA_ERR_SHAPE: return "DSA_ERR_SHAPE: invalid or inconsistent size";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED: outside the support set";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace too small";
    case DSA_ERR_HIP: return "DSA_ERR_HIP: HIP launch failed";
    default: return "unknown dsa_status";
  }
}

const char* dsa_last_error(void) { return g_last_error; }

size_t dsa_workspace_size(int op, int B, int T, int L, int H, int K) {
  if (B < 1 || T < 1 || L < 1 || H < 1 || K < 1) return 0;
  switch (op) {
    case DSA_OP_INDEXER_SCORES: return 0;
    case DSA_OP_TOPK: return dsa::topk_workspace_bytes(B * T, L, K);
    case DSA_OP_SPARSE_MLA: return dsa::attn_workspace_bytes(B * T, H, K);
    case DSA_OP_DECODE_STEP: return decode_ws(B, T, L, H, K);
    default: return 0;
  }
}

dsa_status dsa_indexer_scores(int B, int T, int L, int H_I, int d_I,
                              const void* q_idx, int q_mode, const float* w,
                              const void* k_idx, int k_dtype,
                              const uint8_t* k_scale, const int32_t* q_pos,
                              float* scores, void* stream) {
  if (!q_idx || !w || !k_idx || !q_pos || !scores)
    return fail(DSA_ERR_NULL, "dsa_indexer_scores: NULL tensor pointer");
  if (dsa_status s = check_indexer_dims(B, T, H_I, d_I)) return s;
  if (L < 1) return fail(DSA_ERR_SHAPE, "L must be >= 1");
  if ((long long)B * L > 0x7fffffffLL)
    return fail(DSA_ERR_UNSUPPORTED, "B*L must fit in int32");
  if (!valid_key_dtype(k_dtype))
    return fail(DSA_ERR_UNSUPPORTED, "unsupported key dtype %d", k_dtype);
  const bool fp8 = k_dtype == DSA_E4M3_MX32;
  if (fp8 && !k_scale) return fail(DSA_ERR_NULL, "MX keys need k_scale");
  if (dsa_status st = check_q_mode(q_mode, fp8)) return st;
  dsa::IndexerLaunch a{};
  a.q8 = q_mode == DSA_Q_MX32;
  a.B = B; a.T = T; a.H_I = H_I; a.d_I = d_I;
  a.q_idx = static_cast<const uint16_t*>(q_idx);
  a.w = w;
  a.keys = dsa::CacheView{static_cast<const uint8_t*>(k_idx), k_scale, nullptr,
                          0, L, fp8,
                          (uint64_t)B * L * d_I * (fp8 ? 1 : 2), false};
  a.qp = dsa::QueryPos{q_pos, nullptr, T};
  a.scores = scores;
  a.row_len = L;
  return hip_status(dsa::launch_indexer(a, (hipStream_t)stream),
                    "dsa_indexer_scores");
}

dsa_status dsa_topk(int B, int T, int L, int K, const float* scores,
                    const int32_t* q_pos, int32_t* idx, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (!scores || !q_pos || !idx)
    return fail(DSA_ERR_NULL, "dsa_topk: NULL tensor pointer");
  if (B < 1 || T < 1 || L < 1) return fail(DSA_ERR_SHAPE, "B, T, L must be >= 1");
  if (L > DSA_MAX_CONTEXT)
    return fail(DSA_ERR_UNSUPPORTED, "L must be <= %d", DSA_MAX_CONTEXT);
  if ((long long)B * T > 0x7fffffffLL)
    return fail(DSA_ERR_UNSUPPORTED, "B*T too large");
  if (K < 1 || K > DSA_MAX_TOPK)
    return fail(DSA_ERR_UNSUPPORTED, "K must be in [1, %d], got %d",
                DSA_MAX_TOPK, K);
  dsa::TopkLaunch a{};
  a.rows = B * T; a.T = T; a.L = L; a.K = K;
  a.scores = scores;
  a.qp = dsa::QueryPos{q_pos, nullptr, T};
  a.idx = idx;
  return hip_status(dsa::launch_topk(a, workspace, workspace_bytes,
                                     (hipStream_t)stream), "dsa_topk");
}

dsa_status dsa_sparse_mla_attn(int B, int T, int L, int H, int K,
                               const void* q, const void* kv, int kv_dtype,
                               const void* kv_scale, const int32_t* idx,
                               float softmax_scale, float* out, float* lse,
                               void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (!q || !kv || !idx || !out || !lse)
    return fail(DSA_ERR_NULL, "dsa_sparse_mla_attn: NULL tensor pointer");
  if (dsa_status s = check_attn_dims(B, T, H, K)) return s;
  if (!(softmax_scale > 0.f) || softmax_scale == __builtin_inff())
    return fail(DSA_ERR_SHAPE, "softmax_scale must be positive and finite");
  if (L < 1) return fail(DSA_ERR_SHAPE, "L must be >= 1");
  if ((long long)B * L > 0x7fffffffLL)
    return fail(DSA_ERR_UNSUPPORTED, "B*L must fit in int32");
  if (!valid_kv_dtype(kv_dtype))
    return fail(DSA_ERR_UNSUPPORTED, "unknown kv dtype %d", kv_dtype);
  if (kv_dtype != DSA_BF16 && !kv_scale)
    return fail(DSA_ERR_NULL, "FP8 KV needs kv_scale");
  const size_t need = dsa::attn_workspace_bytes(B * T, H, K);
  if (need && (!workspace || workspace_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  dsa::AttnLaunch a{};
  a.B = B; a.T = T; a.H = H; a.K = K;
  a.q = static_cast<const uint16_t*>(q);
  a.kv = kv_view(kv, kv_scale, kv_dtype, nullptr, 0, L, (uint64_t)B * L, 0);
  a.idx = idx;
  a.seq_lens = nullptr;
  a.scale = softmax_scale;
  a.out = out;
  a.lse = lse;
  a.partial = static_cast<float*>(workspace);
  a.splits = dsa::attn_splits(B * T, K);
  return hip_status(dsa::launch_sparse_mla(a, (hipStream_t)stream),
                    "dsa_sparse_mla_attn");
}

}  // extern "C"

namespace {

// The decode step's sparse attention over the paged latent cache.
dsa_status launch_attention(const dsa_paged_cache* cache, int B, int T, int H,
                            int K, float softmax_scale, const void* q,
                            float* out, float* lse, const int32_t* idx,
                            float* partial, hipStream_t st) {
  dsa::AttnLaunch aa{};
  aa.B = B; aa.T = T; aa.H = H; aa.K = K;
  aa.q = static_cast<const uint16_t*>(q);
  aa.kv = kv_view(cache->kv, cache->kv_scale, cache->kv_dtype,
                  cache->page_table, cache->max_pages_per_seq, 0,
                  (uint64_t)cache->num_pages * DSA_PAGE_SIZE, cache->num_pages);
  aa.idx = idx;
  aa.seq_lens = cache->seq_lens;
  aa.scale = softmax_scale;
  aa.out = out;
  aa.lse = lse;
  aa.partial = partial;
  aa.splits = dsa::attn_splits(B * T, K);
  return hip_status(dsa::launch_sparse_mla(aa, st),
                    "dsa_decode_step: sparse attention");
}

dsa_status decode_step_impl(int B, int T, int H_I, int d_I, int H, int K,
                           float softmax_scale, const dsa_paged_cache* cache,
                           int max_seq_len, const void* q_idx, int q_mode,
                           const float* w,
                           const void* q, const int32_t* q_pos, float* out,
                           float* lse, int32_t* idx_out, void* workspace,
                           size_t workspace_bytes, void* stream,
                           bool static_scratch) {
  if (!cache || !q_idx || !w || !q || !out || !lse)
    return fail(DSA_ERR_NULL, "dsa_decode_step: NULL pointer");
  if (!cache->kidx || !cache->kv || !cache->page_table || !cache->seq_lens)
    return fail(DSA_ERR_NULL, "dsa_decode_step: NULL cache pointer");
  if (dsa_status s = check_indexer_dims(B, T, H_I, d_I)) return s;
  if (dsa_status s = check_attn_dims(B, T, H, K)) return s;
  if (!(softmax_scale > 0.f) || softmax_scale == __builtin_inff())
    return fail(DSA_ERR_SHAPE, "softmax_scale must be positive and finite");
  if (!q_pos && T != 1)
    return fail(DSA_ERR_NULL, "q_pos may be NULL only when T == 1");
  if (cache->page_size != DSA_PAGE_SIZE)
    return fail(DSA_ERR_UNSUPPORTED, "page_size must be %d", DSA_PAGE_SIZE);
  if (cache->num_pages < 1 || cache->max_pages_per_seq < 1)
    return fail(DSA_ERR_SHAPE, "num_pages and max_pages_per_seq must be >= 1");
  if ((long long)cache->num_pages * DSA_PAGE_SIZE > 0x7fffffffLL)
    return fail(DSA_ERR_UNSUPPORTED, "num_pages * 64 must fit in int32");
  if (max_seq_len > DSA_MAX_CONTEXT)
    return fail(DSA_ERR_UNSUPPORTED, "max_seq_len must be <= %d",
                DSA_MAX_CONTEXT);
  if (max_seq_len < 1 ||
      (long long)max_seq_len > (long long)cache->max_pages_per_seq * DSA_PAGE_SIZE)
    return fail(DSA_ERR_SHAPE,
                "max_seq_len must be in [1, max_pages_per_seq * 64]");
  if (!valid_key_dtype(cache->kidx_dtype) || !valid_kv_dtype(cache->kv_dtype))
    return fail(DSA_ERR_UNSUPPORTED, "unsupported cache dtype");
  const bool kfp8 = cache->kidx_dtype == DSA_E4M3_MX32;
  if (kfp8 && !cache->kidx_scale)
    return fail(DSA_ERR_NULL, "MX indexer keys need kidx_scale");
  if (dsa_status st = check_q_mode(q_mode, kfp8)) return st;
  if (cache->kv_dtype != DSA_BF16 && !cache->kv_scale)
    return fail(DSA_ERR_NULL, "FP8 KV needs kv_scale");
  const size_t need = decode_ws(B, T, max_seq_len, H, K);
  if (static_scratch) {
    if (need > kScratchBytes)
      return fail(DSA_ERR_WORKSPACE,
                  "dsa_decode_step_static: these sizes need %zu bytes of "
                  "scratch, the library's static scratch holds %zu",
                  need, kScratchBytes);
    if (dsa_status st = static_scratch_ptr(&workspace)) return st;
    workspace_bytes = kScratchBytes;
  }
  if (!workspace || workspace_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);

  const size_t tokens = (size_t)B * T;
  char* ws = static_cast<char*>(workspace);
  float* scores = reinterpret_cast<float*>(ws);
  ws += align_up(tokens * (size_t)max_seq_len * sizeof(float));
  int32_t* idx = reinterpret_cast<int32_t*>(ws);
  ws += align_up(tokens * (size_t)K * sizeof(int32_t));
  void* topk_ws = ws;
  const size_t topk_bytes = dsa::topk_workspace_bytes((int)tokens, max_seq_len, K);
  ws += align_up(topk_bytes);
  float* partial = reinterpret_cast<float*>(ws);
  ws += align_up(dsa::attn_workspace_bytes((int)tokens, H, K));
  uint32_t* span = reinterpret_cast<uint32_t*>(ws);
  if (idx_out) idx = idx_out;

  const hipStream_t st = (hipStream_t)stream;
  const dsa::QueryPos qp{q_pos, cache->seq_lens, T};

  dsa::IndexerLaunch ia{};
  ia.B = B; ia.T = T; ia.H_I = H_I; ia.d_I = d_I;
  ia.q_idx = static_cast<const uint16_t*>(q_idx);
  ia.w = w;
  ia.keys = dsa::CacheView{static_cast<const uint8_t*>(cache->kidx),
                           cache->kidx_scale, cache->page_table,
                           cache->max_pages_per_seq, 0, kfp8,
                           (uint64_t)cache->num_pages * DSA_PAGE_SIZE * d_I *
                               (kfp8 ? 1 : 2), false, cache->num_pages};
  ia.qp = qp;
  ia.scores = scores;
  ia.row_len = max_seq_len;
  ia.keys_out = 1;   // the Top-K below reads keys: no conversion there
  ia.q8 = q_mode == DSA_Q_MX32;
  // With a row for every CU, the single kernel that keeps each row's scores
  // in LDS matches or beats the score stream plus the Top-K launch (256 rows
  // of 4096 positions: 56 us against 47.5 + 9.7 us and a launch with bf16
  // keys, 38 against 32 + 9.7 us with MX keys, 36 against 38 us through the
  // entry points with quantised queries; 256 of 32768: 377 against 365 + 15
  // us); with fewer rows it leaves CUs idle (128 rows of 8192: 70 against
  // 50 + 10 us).  Several queries per sequence share key reads in the
  // query-tiled indexer instead.
  if (T < 8 && tokens >= 256 && max_seq_len <= dsa::kFusedMaxLen) {
    ia.row_len = max_seq_len;
    if (hipError_t e = dsa::launch_index_topk(ia, K, idx, st))
      return hip_status(e, "dsa_decode_step: fused indexer and Top-K");
    return launch_attention(cache, B, T, H, K, softmax_scale, q, out, lse,
                            idx, partial, st);
  }
  // the stream kernels also leave each wave's key range for the Top-K
  const int span_kpw = dsa::indexer_span_kpw(ia);
  const bool spans = span_kpw > 0 &&
                     (max_seq_len + span_kpw - 1) / span_kpw <= dsa::kSpanMax;
  ia.span = spans ? reinterpret_cast<float*>(span) : nullptr;
  if (hipError_t e = dsa::launch_indexer(ia, st))
    return hip_status(e, "dsa_decode_step: indexer");

  dsa::TopkLaunch ta{};
  ta.rows = (int)tokens; ta.T = T; ta.L = max_seq_len; ta.K = K;
  ta.scores = scores;
  ta.qp = qp;
  ta.keys_in = 1;
  ta.span = reinterpret_cast<const uint32_t*>(ia.span);
  ta.span_kpw = spans ? span_kpw : 0;
  ta.idx = idx;
  if (hipError_t e = dsa::launch_topk(ta, topk_ws, topk_bytes, st))
    return hip_status(e, "dsa_decode_step: topk");

  return launch_attention(cache, B, T, H, K, softmax_scale, q, out, lse, idx,
                          partial, st);
}

}  // namespace

extern "C" {

dsa_status dsa_decode_step(int B, int T, int H_I, int d_I, int H, int K,
                           float softmax_scale, const dsa_paged_cache* cache,
                           int max_seq_len, const void* q_idx, int q_mode,
                           const float* w,
                           const void* q, const int32_t* q_pos, float* out,
                           float* lse, int32_t* idx_out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return decode_step_impl(B, T, H_I, d_I, H, K, softmax_scale, cache,
                          max_seq_len, q_idx, q_mode, w, q, q_pos, out, lse,
                          idx_out, workspace, workspace_bytes, stream, false);
}

dsa_status dsa_decode_step_static(int B, int T, int H_I, int d_I, int H, int K,
                                  float softmax_scale,
                                  const dsa_paged_cache* cache,
                                  int max_seq_len, const void* q_idx,
                                  int q_mode, const float* w, const void* q,
                                  const int32_t* q_pos, float* out, float* lse,
                                  int32_t* idx_out, void* stream) {
  return decode_step_impl(B, T, H_I, d_I, H, K, softmax_scale, cache,
                          max_seq_len, q_idx, q_mode, w, q, q_pos, out, lse,
                          idx_out, nullptr, 0, stream, true);
}

dsa_status dsa_indexer_topk(int B, int T, int H_I, int d_I, int K,
                            const dsa_paged_cache* cache, int max_seq_len,
                            const void* q_idx, int q_mode, const float* w,
                            const int32_t* q_pos, int32_t* idx, void* stream) {
  if (!cache || !q_idx || !w || !idx)
    return fail(DSA_ERR_NULL, "dsa_indexer_topk: NULL pointer");
  if (!cache->kidx || !cache->page_table || !cache->seq_lens)
    return fail(DSA_ERR_NULL, "dsa_indexer_topk: NULL cache pointer");
  if (dsa_status s = check_indexer_dims(B, T, H_I, d_I)) return s;
  if (K < 1 || K > DSA_MAX_TOPK)
    return fail(DSA_ERR_UNSUPPORTED, "K must be in [1, %d], got %d",
                DSA_MAX_TOPK, K);
  if (!q_pos && T != 1)
    return fail(DSA_ERR_NULL, "q_pos may be NULL only when T == 1");
  if (cache->page_size != DSA_PAGE_SIZE)
    return fail(DSA_ERR_UNSUPPORTED, "page_size must be %d", DSA_PAGE_SIZE);
  if (cache->num_pages < 1 || cache->max_pages_per_seq < 1)
    return fail(DSA_ERR_SHAPE, "num_pages and max_pages_per_seq must be >= 1");
  if ((long long)cache->num_pages * DSA_PAGE_SIZE > 0x7fffffffLL)
    return fail(DSA_ERR_UNSUPPORTED, "num_pages * 64 must fit in int32");
  if (max_seq_len > DSA_FUSED_MAX_CONTEXT)
    return fail(DSA_ERR_UNSUPPORTED,
                "dsa_indexer_topk: max_seq_len must be <= %d (one row's "
                "scores in one workgroup's LDS)", DSA_FUSED_MAX_CONTEXT);
  if (max_seq_len < 1 ||
      (long long)max_seq_len > (long long)cache->max_pages_per_seq * DSA_PAGE_SIZE)
    return fail(DSA_ERR_SHAPE,
                "max_seq_len must be in [1, max_pages_per_seq * 64]");
  if (!valid_key_dtype(cache->kidx_dtype))
    return fail(DSA_ERR_UNSUPPORTED, "unsupported key dtype %d",
                cache->kidx_dtype);
  const bool kfp8 = cache->kidx_dtype == DSA_E4M3_MX32;
  if (kfp8 && !cache->kidx_scale)
    return fail(DSA_ERR_NULL, "MX indexer keys need kidx_scale");
  if (dsa_status st = check_q_mode(q_mode, kfp8)) return st;
  static_assert(DSA_FUSED_MAX_CONTEXT == dsa::kFusedMaxLen, "LDS row bound");
  dsa::IndexerLaunch a{};
  a.B = B; a.T = T; a.H_I = H_I; a.d_I = d_I;
  a.q_idx = static_cast<const uint16_t*>(q_idx);
  a.w = w;
  a.keys = dsa::CacheView{static_cast<const uint8_t*>(cache->kidx),
                          cache->kidx_scale, cache->page_table,
                          cache->max_pages_per_seq, 0, kfp8,
                          (uint64_t)cache->num_pages * DSA_PAGE_SIZE * d_I *
                              (kfp8 ? 1 : 2), false, cache->num_pages};
  a.qp = dsa::QueryPos{q_pos, cache->seq_lens, T};
  a.row_len = max_seq_len;
  a.q8 = q_mode == DSA_Q_MX32;
  return hip_status(dsa::launch_index_topk(a, K, idx, (hipStream_t)stream),
                    "dsa_indexer_topk");
}

dsa_status dsa_cache_append(int B, int T, int d_I, int num_pages,
                            int max_pages_per_seq, const int32_t* page_table,
                            const int32_t* pos, const void* k_new,
                            int kidx_dtype, void* kidx, uint8_t* kidx_scale,
                            const void* kv_new, int kv_dtype, void* kv,
                            void* kv_scale, void* stream) {
  if (!page_table || !pos)
    return fail(DSA_ERR_NULL, "dsa_cache_append: NULL page_table or pos");
  if (!k_new && !kv_new)
    return fail(DSA_ERR_NULL, "dsa_cache_append: neither k_new nor kv_new");
  if (B < 1 || T < 1) return fail(DSA_ERR_SHAPE, "B and T must be >= 1");
  if ((long long)B * T > 0x7fffffffLL)
    return fail(DSA_ERR_UNSUPPORTED, "B*T too large");
  if (num_pages < 1 || max_pages_per_seq < 1)
    return fail(DSA_ERR_SHAPE, "num_pages and max_pages_per_seq must be >= 1");
  if ((long long)max_pages_per_seq * DSA_PAGE_SIZE > 0x7fffffffLL)
    return fail(DSA_ERR_UNSUPPORTED, "max_pages_per_seq * 64 must fit in int32");
  dsa::AppendLaunch a{};
  a.tokens = B * T; a.T = T;
  a.pos = pos;
  a.page_table = page_table;
  a.max_pages = max_pages_per_seq;
  a.num_pages = num_pages;
  if (k_new) {
    if (d_I != 64 && d_I != 128)
      return fail(DSA_ERR_UNSUPPORTED, "d_I must be 64 or 128, got %d", d_I);
    if (!valid_key_dtype(kidx_dtype))
      return fail(DSA_ERR_UNSUPPORTED, "unsupported key dtype %d", kidx_dtype);
    if (!kidx) return fail(DSA_ERR_NULL, "k_new given without kidx pool");
    if (kidx_dtype == DSA_E4M3_MX32 && !kidx_scale)
      return fail(DSA_ERR_NULL, "MX indexer keys need kidx_scale");
    a.d_I = d_I;
    a.kidx_fmt = kidx_dtype == DSA_E4M3_MX32 ? dsa::kFmtMx32 : dsa::kFmtBf16;
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.kidx = static_cast<uint8_t*>(kidx);
    a.kidx_scale = kidx_scale;
  }
  if (kv_new) {
    if (!valid_kv_dtype(kv_dtype))
      return fail(DSA_ERR_UNSUPPORTED, "unknown kv dtype %d", kv_dtype);
    if (!kv) return fail(DSA_ERR_NULL, "kv_new given without kv pool");
    if (kv_dtype != DSA_BF16 && !kv_scale)
      return fail(DSA_ERR_NULL, "FP8 KV needs kv_scale");
    a.kv_fmt = kv_dtype == DSA_E4M3_T128   ? dsa::kFmtT128
               : kv_dtype == DSA_E4M3_MX32 ? dsa::kFmtMx32
                                           : dsa::kFmtBf16;
    a.kv_new = static_cast<const uint16_t*>(kv_new);
    a.kv = static_cast<uint8_t*>(kv);
    a.kv_scale = kv_scale;
  }
  return hip_status(dsa::launch_cache_append(a, (hipStream_t)stream),
                    "dsa_cache_append");
}

}  // extern "C"
