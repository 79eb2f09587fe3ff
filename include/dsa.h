/*
 * dsa.h -- C ABI of the indexed sparse attention (DSA) hot path for AMD
 * Instinct MI355X (gfx950).
 *
 * For each query token the path runs three steps (pages: "Day-0 Inference
 * Optimization for a New Sparse Attention Architecture: A Technical Deep
 * Dive", section 1, Lightning Indexer and Sparse Flash Attention; "Inference
 * Adaptation and Performance Optimization for New Large Language Model
 * Architectures", the illustrative pseudocode in which a lightning indexer
 * returns indices and sparse flash attention consumes them):
 *
 *   1. Lightning Indexer score of every causal history position s <= q_pos:
 *        I[t,s] = sum_j w[t,j] * max(0, q_I[t,j,:] . k_I[s,:])
 *      (one indexer key per position, shared by all H_I indexer heads);
 *   2. Top-K: the K highest-scoring positions, ties to the lower position;
 *   3. sparse absorbed-MLA attention of the token's H query heads over only
 *      the selected latent rows: keys are the full 576-wide rows (512 latent
 *      + 64 rope), values their first 512 features, softmax scale given.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensor pointers are DEVICE pointers, 16-byte aligned, row-major and
 *   densely packed in the layouts stated per argument.  Scalars are host
 *   values.  The caller owns every buffer; the library never allocates,
 *   frees or synchronises (dsa_decode_step_static works in the library's
 *   own static device scratch instead of a caller workspace).
 * - bf16 tensors hold IEEE bfloat16 bit patterns (uint16).  FP8 tensors hold
 *   OCP e4m3fn codes (uint8) with one OCP e8m0 scale code per 32 consecutive
 *   features of a row (the "MX block-32" layout: page "Optimizing Inference
 *   for New Model Architectures", section 4, one shared scale per group of
 *   32; the "Technical Deep Dive" page, section 2, names it MXFP8).  The
 *   value of element i of a row is e4m3(code[i]) * 2^(scale[i/32] - 127).
 *   Dequantisation is exact while the product is a normal bf16 number.
 * - The latent KV may instead use the "tile" layout DSA_E4M3_T128 (page
 *   "Inference Adaptation and Performance Optimization for New Large
 *   Language Model Architectures", section 4.3: FP8 per token and head in
 *   blocks of 128 elements; page "Day-0 Inference Adaptation and Performance
 *   Optimization for New-Architecture Large Language Models", section
 *   "Tiered Quantization", whose scale is max|tile| / quant_max): a row's
 *   576 codes form tiles [0,128) [128,256) [256,384) [384,512) [512,576),
 *   each with one fp32 scale, and element i is e4m3(code[i]) * scale[tile].
 *   The attention rounds that fp32 product to bf16.
 * - `stream` is a hipStream_t (NULL = the legacy default stream).  Every call
 *   only enqueues kernels on it and returns.
 * - Errors: argument and shape checks run on the host before any HIP call and
 *   return a non-zero dsa_status without touching any buffer.  A launch
 *   failure returns DSA_ERR_HIP.  Faults inside kernels surface at the
 *   caller's next synchronisation.  dsa_last_error() gives a message for the
 *   last failing call on the calling thread.
 * - The library is stateless and thread-safe; calls that share an output or
 *   workspace buffer on different streams race.
 *
 * Support set: indexer heads 1 <= H_I <= 64; indexer dim d_I in {64, 128};
 * MLA heads 1 <= H <= 128; latent width 576, value width 512; 1 <= K <= 2048;
 * page size 64; Top-K rows (and decode-step sequences) up to 131072 tokens.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_NULL = 1,         /* a required pointer is NULL                  */
  DSA_ERR_SHAPE = 2,        /* a size is negative, zero or inconsistent    */
  DSA_ERR_UNSUPPORTED = 3,  /* a size or dtype outside the support set     */
  DSA_ERR_WORKSPACE = 4,    /* workspace missing or smaller than required  */
  DSA_ERR_HIP = 5           /* a HIP launch failed                          */
} dsa_status;

typedef enum dsa_dtype {
  DSA_BF16 = 0,             /* bfloat16 values                              */
  DSA_E4M3_MX32 = 1,        /* e4m3fn codes + one e8m0 scale per 32 values  */
  DSA_E4M3_T128 = 2         /* e4m3fn codes + one fp32 scale per 128-value
                               tile of a 576-wide latent row (latent KV only) */
} dsa_dtype;

/* Operation selector for dsa_workspace_size. */
/* Precision of the indexer queries (step 1). */
typedef enum dsa_q_mode {
  DSA_Q_BF16 = 0,           /* bf16 queries; keys dequantised to bf16       */
  DSA_Q_MX32 = 1            /* queries quantised on the fly to e4m3 with one
                               e8m0 scale per 32 features of each head, the
                               products on the scaled FP8 matrix cores (keys
                               must be DSA_E4M3_MX32)                      */
} dsa_q_mode;

typedef enum dsa_op {
  DSA_OP_INDEXER_SCORES = 0,
  DSA_OP_TOPK = 1,
  DSA_OP_SPARSE_MLA = 2,
  DSA_OP_DECODE_STEP = 3
} dsa_op;

#define DSA_LATENT_DIM 576
#define DSA_VALUE_DIM 512
#define DSA_PAGE_SIZE 64
#define DSA_MAX_TOPK 2048
#define DSA_MAX_CONTEXT 131072   /* longest score row / sequence */
#define DSA_FUSED_MAX_CONTEXT 32768   /* longest row of dsa_indexer_topk */
/* Bytes of device scratch that dsa_decode_step_static owns on each GPU. */
#define DSA_STATIC_SCRATCH_BYTES (64ull << 20)

/*
 * One layer's paged cache: indexer keys and latent KV in two page pools that
 * share one page table (page "Optimizing Inference for New Model
 * Architectures", section 3: the fused indexer reads the paged key cache
 * directly).  Logical position s of sequence b lives in physical page
 * page_table[b * max_pages_per_seq + s / 64], row s % 64.  Entries past a
 * sequence's last page are never read.  Every entry that is read (the
 * pages of positions 0 .. seq_lens[b]-1) must lie in [0, num_pages): the
 * kernels clamp an entry outside that range into it, so a bad table reads
 * wrong rows but never outside the pools.
 */
typedef struct dsa_paged_cache {
  int32_t page_size;          /* tokens per page; must be 64                */
  int32_t num_pages;          /* pages in each pool                          */
  int32_t max_pages_per_seq;  /* columns of page_table                       */
  int32_t kidx_dtype;         /* dsa_dtype of the indexer-key pool           */
  int32_t kv_dtype;           /* dsa_dtype of the latent-KV pool             */
  const void* kidx;           /* [num_pages, 64, d_I] bf16 or e4m3 codes     */
  const uint8_t* kidx_scale;  /* [num_pages, 64, d_I/32] e8m0; NULL if bf16  */
  const void* kv;             /* [num_pages, 64, 576] bf16 or e4m3 codes     */
  const void* kv_scale;       /* [num_pages, 64, 18] e8m0 (MX32), [num_pages,
                                 64, 5] fp32 (T128); NULL if bf16           */
  const int32_t* page_table;  /* [B, max_pages_per_seq] int32               */
  const int32_t* seq_lens;    /* [B] tokens in the cache, current ones incl. */
} dsa_paged_cache;

/*
 * Lightning Indexer scores over a contiguous key cache (step 1).
 *   q_idx   [B, T, H_I, d_I] bf16   indexer queries
 *   q_mode  dsa_q_mode.  DSA_Q_MX32 is the fully quantised indexer (page
 *           "Inference Adaptation and Performance Optimization for New Large
 *           Language Model Architectures", section 4.2: index Q and K in
 *           MXFP8, per-group dynamic scales, groups of 32; page "Day-0
 *           Inference Optimization for a New Sparse Attention Architecture:
 *           A Technical Deep Dive", section 2): each head's 32-feature
 *           blocks of q_idx take the scale 2^X, X the smallest integer
 *           >= -127 with 448 * 2^X >= the block's largest magnitude (X = 0
 *           for a zero block), codes are the nearest e4m3fn (ties to even)
 *           of q * 2^-X, and the scores use those dequantised queries
 *   w       [B, T, H_I] fp32        head weights
 *   k_idx   [B, L, d_I]             bf16, or e4m3 codes if k_dtype is MX
 *   k_scale [B, L, d_I/32] e8m0     (NULL unless k_dtype == DSA_E4M3_MX32)
 *   q_pos   [B, T] int32            position of each query, 0 <= q_pos < L
 *   scores  [B, T, L] fp32 out      I[t,s] for s <= q_pos, -inf beyond
 * Scores are summed in fp32; for integer-valued q/k and power-of-two
 * weights they are exact.  -0 is written as +0.
 */
dsa_status dsa_indexer_scores(int B, int T, int L, int H_I, int d_I,
                              const void* q_idx, int q_mode, const float* w,
                              const void* k_idx, int k_dtype,
                              const uint8_t* k_scale, const int32_t* q_pos,
                              float* scores, void* stream);

/*
 * Top-K per score row (step 2): the indexer's selection of the most relevant
 * history positions (page "Day-0 Inference Optimization for a New Sparse
 * Attention Architecture: A Technical Deep Dive", section 1, Lightning
 * Indexer; page "Inference Optimization for New Open-Source LLM
 * Architectures", "Architectural Overview": the Top-K most relevant
 * positions).  The pages give no tie rule; ties go to the lower position.
 *   scores [B, T, L] fp32; candidates of row (b,t) are positions
 *          0..min(q_pos[b,t], L-1); NaN ranks below every number
 *   q_pos  [B, T] int32
 *   idx    [B, T, K] int32 out: the min(K, q_pos+1) positions with the
 *          largest scores (equal scores: lower position first), in ascending
 *          order, then -1 padding
 *   workspace: dsa_workspace_size(DSA_OP_TOPK, ...) bytes: candidate lists
 *          for rows longer than 65536 positions (each 16384-position chunk
 *          selects its own Top-K, then each row selects from its chunks'
 *          candidates).  It is 0 for shorter rows and may be NULL / too
 *          small: long rows then run on one workgroup each (same result,
 *          slower).
 */
dsa_status dsa_topk(int B, int T, int L, int K, const float* scores,
                    const int32_t* q_pos, int32_t* idx, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * Sparse absorbed-MLA attention over selected latent rows of a contiguous
 * KV cache (step 3): Sparse Flash Attention reads only the cache entries at
 * the selected indices (page "Inference Optimization for New Open-Source LLM
 * Architectures", "Architectural Overview"; page "Day-0 Inference
 * Optimization for a New Sparse Attention Architecture: A Technical Deep
 * Dive", section 1, Sparse Flash Attention), with MLA absorbed: keys are
 * the 576-wide latent rows, values their first 512 features.
 *   q        [B, T, H, 576] bf16    absorbed queries (512 latent + 64 rope)
 *   kv       [B, L, 576]            bf16, or e4m3 codes (MX32 / T128)
 *   kv_scale [B, L, 18] e8m0 (MX32), [B, L, 5] fp32 (T128); NULL for bf16
 *   idx      [B, T, K] int32        selected positions; -1 entries skipped;
 *                                   valid entries must lie in [0, L)
 *   softmax_scale > 0, finite (else DSA_ERR_SHAPE)
 *   out      [B, T, H, 512] fp32    softmax-weighted sum of value rows
 *   lse      [B, T, H] fp32         natural-log sum of exp(scale * q.k);
 *                                   a row with no valid index gets out = 0,
 *                                   lse = -inf
 * Logits may span any range that fp32 holds: a head whose logits rise more
 * than 128 (in log2 units) above its first tile's max takes a second pass
 * with its true max as the softmax reference, and split partial sums are
 * merged by their log-sum-exp.  Inputs whose scaled logits overflow fp32
 * are outside the support set.
 *   workspace: dsa_workspace_size(DSA_OP_SPARSE_MLA, ...) bytes
 */
dsa_status dsa_sparse_mla_attn(int B, int T, int L, int H, int K,
                               const void* q, const void* kv, int kv_dtype,
                               const void* kv_scale, const int32_t* idx,
                               float softmax_scale, float* out, float* lse,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * Steps 1 and 2 as one kernel over the paged key cache: scoring, head
 * weighting and Top-K of each query row without the scores leaving the chip
 * (page "Inference Adaptation and Performance Optimization for New Large
 * Language Model Architectures", section 3.1 "Fused Index Computation": the
 * three steps in one kernel that reads the paged keys and outputs only the
 * final indices; page "Day-0 Inference Adaptation and Performance
 * Optimization for New-Architecture Large Language Models", "Fusing the
 * Indexer to Reduce Intermediate Write-Backs"; both name a bf16 and a
 * quantised path).  One workgroup per query row keeps the row's scores in
 * its LDS, so rows are limited to DSA_FUSED_MAX_CONTEXT positions.  The same
 * scores and the same selection as dsa_indexer_scores followed by dsa_topk
 * (ties to the lower position).
 *   cache         page pools as for dsa_decode_step; only the indexer-key
 *                 fields, page_table and seq_lens are read (kv, kv_scale
 *                 may be NULL)
 *   max_seq_len   host upper bound of seq_lens, 1 .. DSA_FUSED_MAX_CONTEXT
 *                 (else DSA_ERR_UNSUPPORTED) and <= max_pages_per_seq * 64
 *   q_idx [B, T, H_I, d_I] bf16; q_mode as for dsa_indexer_scores
 *                 (DSA_Q_MX32 needs MX keys)
 *   w [B, T, H_I] fp32
 *   q_pos [B, T] int32, or NULL when T == 1: then q_pos = seq_lens[b] - 1;
 *                 positions are clamped to seq_lens[b] - 1
 *   idx [B, T, K] int32 out, as dsa_topk's idx
 * Needs no workspace and allocates nothing.
 */
dsa_status dsa_indexer_topk(int B, int T, int H_I, int d_I, int K,
                            const dsa_paged_cache* cache, int max_seq_len,
                            const void* q_idx, int q_mode, const float* w,
                            const int32_t* q_pos, int32_t* idx, void* stream);

/*
 * The whole path for T query tokens per sequence over a paged cache:
 * indexer -> Top-K -> sparse attention, enqueued on one stream (page
 * "Optimizing Inference for New Model Architectures", section 3: the index
 * stage reads the paged key cache, the sparse attention kernel then reads
 * the KV cache by index; page "Inference Adaptation and Performance
 * Optimization for New Large Language Model Architectures", section 3.1).
 *   cache         see dsa_paged_cache; seq_lens[b] <= max_seq_len
 *   max_seq_len   host upper bound of seq_lens (sizes the score workspace)
 *   q_idx [B, T, H_I, d_I] bf16; q_mode as for dsa_indexer_scores
 *   w [B, T, H_I] fp32; q [B, T, H, 576] bf16
 *   q_pos [B, T] int32, or NULL when T == 1: then q_pos = seq_lens[b] - 1
 *   out [B, T, H, 512] fp32; lse [B, T, H] fp32
 *   idx_out [B, T, K] int32 or NULL: the selected positions (as dsa_topk)
 *   workspace: dsa_workspace_size(DSA_OP_DECODE_STEP, B, T, max_seq_len,
 *              H, K) bytes
 */
dsa_status dsa_decode_step(int B, int T, int H_I, int d_I, int H, int K,
                           float softmax_scale, const dsa_paged_cache* cache,
                           int max_seq_len, const void* q_idx, int q_mode,
                           const float* w,
                           const void* q, const int32_t* q_pos, float* out,
                           float* lse, int32_t* idx_out, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * dsa_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the workspace is the library's
 * own static device scratch of DSA_STATIC_SCRATCH_BYTES per GPU, held from
 * the first call on a device until the process ends.  Arguments and results
 * as for dsa_decode_step.  Sizes whose workspace
 * (dsa_workspace_size(DSA_OP_DECODE_STEP, ...)) exceeds the scratch return
 * DSA_ERR_WORKSPACE before any launch.  The call itself allocates nothing;
 * its first call on a device looks up the scratch's address there.  All
 * calls on one GPU share that scratch: calls that may overlap on one GPU
 * (different streams, or different threads without ordering) race.
 */
dsa_status dsa_decode_step_static(int B, int T, int H_I, int d_I, int H, int K,
                                  float softmax_scale,
                                  const dsa_paged_cache* cache,
                                  int max_seq_len, const void* q_idx,
                                  int q_mode, const float* w, const void* q,
                                  const int32_t* q_pos, float* out, float* lse,
                                  int32_t* idx_out, void* stream);

/*
 * Store new tokens' indexer keys and latent rows into the paged pools -- the
 * write that precedes the path for every new token -- quantising each row
 * into its pool's format (pages: "Day-0 Inference Adaptation and
 * Performance Optimization for New-Architecture Large Language Models",
 * section "Tiered Quantization", per-group dynamic scaling with the scale
 * max|group| / quant_max; "Inference Adaptation and Performance
 * Optimization for New Large Language Model Architectures", sections 4.2
 * and 4.3, groups of 32 for the index keys and 128-element tiles for the
 * KV).
 *   page_table [B, max_pages_per_seq] int32 (as in dsa_paged_cache)
 *   pos        [B, T] int32: logical position of each new token; the row
 *              goes to page page_table[b, pos / 64], row pos % 64.  Tokens
 *              with pos < 0, pos >= 64 * max_pages_per_seq or a page entry
 *              outside [0, num_pages) are skipped (nothing is written).
 *   k_new      [B, T, d_I] bf16 or NULL (keys not appended); d_I in {64, 128}
 *   kidx       [num_pages, 64, d_I] pool of dtype kidx_dtype (BF16 or MX32)
 *   kidx_scale [num_pages, 64, d_I/32] e8m0 (MX32) or NULL
 *   kv_new     [B, T, 576] bf16 or NULL (latent rows not appended)
 *   kv         [num_pages, 64, 576] pool of dtype kv_dtype (any)
 *   kv_scale   [num_pages, 64, 18] e8m0 (MX32), [num_pages, 64, 5] fp32
 *              (T128), or NULL (BF16)
 * BF16 pools receive the bits unchanged.  MX32 groups of 32 take the scale
 * 2^X with X the smallest integer >= -127 such that 448 * 2^X >= the
 * group's largest magnitude (X = 0 for an all-zero group); T128 tiles take
 * the fp32 scale max|tile| / 448 (0 for an all-zero tile).  Codes are the
 * nearest e4m3fn (ties to even) of x * 2^-X, resp. of x / scale computed
 * with correctly rounded fp32 division and saturated at +-448; the sign bit
 * is x's, also for zero.  Inputs must be finite.  The written bytes are a
 * deterministic function of the inputs.  Tokens that map to the same slot
 * race.  seq_lens is not touched: the caller advances it.
 */
dsa_status dsa_cache_append(int B, int T, int d_I, int num_pages,
                            int max_pages_per_seq, const int32_t* page_table,
                            const int32_t* pos, const void* k_new,
                            int kidx_dtype, void* kidx, uint8_t* kidx_scale,
                            const void* kv_new, int kv_dtype, void* kv,
                            void* kv_scale, void* stream);

/* Bytes of workspace an operation needs for these sizes (L = the context
 * length, or max_seq_len for DSA_OP_DECODE_STEP).  0 for an unknown op. */
size_t dsa_workspace_size(int op, int B, int T, int L, int H, int K);

/* Static text for a status code. */
const char* dsa_status_string(int status);

/* Message describing the last failing call on this thread ("" if none). */
const char* dsa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H_ */
