/*
 * topidx.h - C ABI of libtopidx.so: indexer-driven Top-K sparse attention over a paged
 * latent (MLA-style) KV cache, for MI355X (gfx950).
 *
 * The method: "Day 0 Support for New LLM Architectures", Step 1 (sparse attention modules:
 * a light indexer scores every earlier position, the Top-K positions are selected, and an
 * exact sparse-attention kernel reads only those entries of the low-rank KV cache) and Key
 * Optimization 1 (scoring, head weighting and Top-K fused into one kernel that reads the
 * paged K cache directly; the chain ends as two kernels: indexer and sparse attention).
 * "Day-0 Support for Large Model Inference", Core Operator Optimization items 1-2 (index
 * stays resident on the device; selected rows are gathered, then attention is computed
 * blockwise with fused normalisation).  "Achieving Day-0 Readiness ... Million-Token
 * Context", section 2.2 (the cache is split into fixed-size blocks with a block index table).
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless the name ends in _host.  The caller owns every
 *    buffer; the library never allocates device memory, never synchronises the stream and
 *    keeps no pointer after returning.  All work is enqueued on `stream` (a hipStream_t,
 *    NULL = the null stream).
 *  - Arguments are validated on the host before anything is enqueued.  On any status other
 *    than TIS_OK nothing has been launched and no output has been written, except
 *    TIS_ERR_HIP (a launch failed part-way; outputs are then unspecified).  The message of
 *    the last failing call on the calling thread is returned by tis_last_error().
 *  - Calls are reentrant; calls that share a workspace on overlapping streams race.
 *  - Layouts are row-major and contiguous.  Caches are paged with 64 tokens per page:
 *    pool[n_pages][64][D] (+ per-slot scales: one fp32 per token slot for e4m3,
 *    scale[n_pages][64], or D/32 bytes for MXFP8, scale[n_pages][64][D/32]).  The logical
 *    position s of request b lives in slot s % 64 of page page_table[b][s / 64].
 *  - Request b holds seq_lens[b] positions.  Its query tokens are its LAST
 *    q_len_b = cu_q[b+1] - cu_q[b] positions (the caller has already appended them to both
 *    caches); flattened token t of request b sits at position p_t = seq_lens[b] - q_len_b +
 *    (t - cu_q[b]) and attends causally to positions 0..p_t (n_t = p_t + 1 candidates).
 *    cache_append writes those rows.
 *  - Page-table entries read by the library (logical pages below ceil(seq_lens[b]/64)) must
 *    lie in [0, n_pages); a position whose page is out of range is never read: it scores
 *    -inf and is skipped by attention.  Scales must be positive and finite (MXFP8 scale
 *    bytes below 255); caches hold no NaN/Inf codes.
 */
#ifndef TOPIDX_H
#define TOPIDX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TIS_ABI_VERSION 6
#define TIS_PAGE_SIZE 64

typedef enum {
  TIS_OK = 0,
  TIS_ERR_INVALID = 1,      /* bad argument (null, size, alignment, workspace too small) */
  TIS_ERR_UNSUPPORTED = 2,  /* valid but not implemented dtype/shape combination */
  TIS_ERR_HIP = 3           /* a HIP launch failed; see tis_last_error() */
} tis_status_t;

/* Storage formats.  TIS_E4M3 caches carry one fp32 scale per token slot.  TIS_MXFP8 ("Day 0
 * Support for New LLM Architectures", Key Optimization 2: the indexer fully quantised as MXFP8,
 * every 32 consecutive elements sharing one scale) is E4M3FN codes with one scale byte per 32
 * consecutive elements of a row: byte b stands for 2^(b - 127) (b = 255 is not allowed), the
 * element's value is code * 2^(b - 127); scale bytes are laid out [n_pages][64][D / 32]. */
typedef enum {
  TIS_F32 = 0,
  TIS_BF16 = 1,
  TIS_E4M3 = 2,  /* OCP E4M3FN */
  TIS_MXFP8 = 3  /* E4M3FN codes + one power-of-two scale byte per 32 elements */
} tis_dtype_t;

/* Indexer query handling ("Day 0 Support for New LLM Architectures", Key Optimization 1: a
 * BF16 and a quantised implementation are kept side by side; Key Optimization 2: the indexer
 * query is quantised dynamically, as MXFP8 with group 32):
 *   TIS_QMODE_FP8   - quantise each (token, head) row of q_I to e4m3 with the smallest
 *                     power-of-two scale s that keeps max|q_I|/s <= 448 (round to nearest
 *                     even), fold s into the head weight, and score on FP8 matrix cores;
 *   TIS_QMODE_BF16  - use q_I as stored: bf16 queries are multiplied on bf16 matrix cores with
 *                     the e4m3 keys widened to bf16 (exactly: every e4m3 value is a bf16
 *                     value); fp32 queries with fp32 keys use the fp32 kernel;
 *   TIS_QMODE_MXFP8 - with TIS_MXFP8 keys: quantise q_I per (token, head, 32 consecutive
 *                     dims) with the shared exponent X = floor(log2 amax) - 8 (clamped to
 *                     [-127, 127]; -127 for an all-zero group) and codes RNE(q / 2^X) clamped
 *                     to +-448; both sides' scales enter the FP8 matrix products exactly. */
typedef enum { TIS_QMODE_FP8 = 0, TIS_QMODE_BF16 = 1, TIS_QMODE_MXFP8 = 2 } tis_qmode_t;

/* A ragged, paged batch ("Achieving Day-0 Readiness ... Million-Token Context", section 2.2:
 * the cache is cut into fixed-size blocks located through a block index table; "Day-0
 * Support for Large Model Inference", Core Operator Optimization item 2: requests of
 * different lengths share one launch).  Host copies of seq_lens and cu_q size the launch
 * grids without a device round trip; they must equal the device copies. */
typedef struct {
  int32_t B;                     /* requests, >= 1 */
  int32_t T;                     /* flattened query tokens = cu_q[B], >= 1 */
  const int32_t* seq_lens;       /* [B]     positions held by each request (>= its q_len) */
  const int32_t* cu_q;           /* [B+1]   query-token offsets, cu_q[0] = 0, nondecreasing */
  const int32_t* seq_lens_host;  /* [B]     host copy */
  const int32_t* cu_q_host;      /* [B+1]   host copy */
  const int32_t* page_table;     /* [B][pt_stride] physical page of each logical page */
  int32_t pt_stride;             /* >= ceil(max seq_len / 64) */
  int32_t page_size;             /* must be TIS_PAGE_SIZE (64) */
  int32_t n_pages;               /* pages in each pool (bounds page-table entries) */
} tis_batch_t;

/* index_score - indexer scores of every causal candidate ("Day 0 Support for New LLM
 * Architectures", Step 1: the light indexer scores each earlier position; Key Optimization 1:
 * relevance scores and head weights computed reading the paged K cache directly).
 *   score[t][s] = sum_h w[t][h] * max(0, q_I[t][h] . k_I[s]) for s in [0, p_t], where
 *   k_I[s] = k_code[s] * k_scale[s] (e4m3 keys), the MXFP8 row's values (see tis_dtype_t) or
 *   the fp32 key.  With TIS_QMODE_FP8 or TIS_QMODE_MXFP8 the query is first quantised as
 *   described at tis_qmode_t.  Accumulation is fp32.
 * q_idx   [T][H_I][D_I]  q_dt = TIS_BF16 (with k_dt = TIS_E4M3 and qmode FP8 or BF16, or with
 *                        k_dt = TIS_MXFP8 and qmode MXFP8; H_I = 64, D_I = 128) or TIS_F32
 *                        (with k_dt = TIS_F32, qmode BF16; H_I * D_I <= 8192)
 * w       [T][H_I] fp32 head weights
 * k_pool  [n_pages][64][D_I]; k_scale: [n_pages][64] fp32 (e4m3 keys), [n_pages][64][D_I/32]
 *         scale bytes (MXFP8 keys; 16-byte aligned) or NULL (fp32 keys)
 * scores  [T][ld_scores] fp32, ld_scores >= max p_t + 1 and a multiple of 4; entries
 *         s > p_t are not written.
 * ws      unused by this call (pass NULL, 0).
 */
tis_status_t index_score(const tis_batch_t* batch, const void* q_idx, tis_dtype_t q_dt,
                         const float* w, const void* k_pool, tis_dtype_t k_dt,
                         const void* k_scale, int32_t H_I, int32_t D_I, tis_qmode_t qmode,
                         float* scores, int64_t ld_scores, void* ws, size_t ws_bytes,
                         void* stream);

/* topk_select - per-token Top-K over the scores of positions 0..p_t ("Day 0 Support for New
 * LLM Architectures", Step 1 and Key Optimization 1: the Top-K positions of the relevance
 * scores are kept; "Achieving Day-0 Readiness ... Million-Token Context", section 2.1:
 * selection is an operator of its own on the device, the index never leaving it).
 *   Selects the k_t = min(K, p_t + 1) positions that are largest under the total order
 *   (score descending, position ascending); -0.0 and +0.0 are equal.  Scores must not be NaN.
 * topk_idx [T][K] int32: the selected positions in ascending order, then -1 up to K.
 * topk_val [T][K] fp32 or NULL: the score of each emitted position (0 where idx = -1).
 * ws       workspace of topk_select_workspace_size() bytes, 16-byte aligned: nonzero for a
 *          batch of at most 64 tokens with rows longer than 32768 positions and K <= 4096,
 *          which are selected by several workgroups per row (otherwise 0 / NULL).  Returns
 *          TIS_ERR_INVALID when it is too small.
 */
tis_status_t topk_select(const tis_batch_t* batch, const float* scores, int64_t ld_scores,
                         int32_t K, int32_t* topk_idx, float* topk_val, void* ws,
                         size_t ws_bytes, void* stream);

/* index_score_topk - index_score followed by topk_select with no score tensor owned by the
 * caller; identical results to the two calls ("Day 0 Support for New LLM Architectures", Key
 * Optimization 1: scoring, head weighting and Top-K fused into one kernel chain).  ws: index_score_topk_workspace_size() bytes,
 * 16-byte aligned (the score rows of one chunk of tokens, then the selection's workspace as for
 * topk_select over that chunk). */
tis_status_t index_score_topk(const tis_batch_t* batch, const void* q_idx, tis_dtype_t q_dt,
                              const float* w, const void* k_pool, tis_dtype_t k_dt,
                              const void* k_scale, int32_t H_I, int32_t D_I,
                              tis_qmode_t qmode, int32_t K, int32_t* topk_idx,
                              float* topk_val, void* ws, size_t ws_bytes, void* stream);

/* index_score_topk_noalloc - index_score_topk for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).  The
 * same arguments and results as index_score_topk without ws/ws_bytes: the workspace is a
 * 64 MiB scratch array that the library holds on each device until the process ends (its
 * address is looked up on the first call on a device; no call allocates or frees anything).
 * The score rows of one chunk of tokens must fit it: a batch whose longest causal range exceeds
 * about 15.5M positions returns TIS_ERR_INVALID before anything is enqueued.  Every call on a
 * device shares that device's scratch, so calls that overlap on one device (on other streams
 * or threads) race; calls ordered on one stream do not. */
tis_status_t index_score_topk_noalloc(const tis_batch_t* batch, const void* q_idx,
                                      tis_dtype_t q_dt, const float* w, const void* k_pool,
                                      tis_dtype_t k_dt, const void* k_scale, int32_t H_I,
                                      int32_t D_I, tis_qmode_t qmode, int32_t K,
                                      int32_t* topk_idx, float* topk_val, void* stream);

/* sparse_mla_attn - exact attention of each token over its selected latent rows ("Day 0
 * Support for New LLM Architectures", Step 1: the sparse-attention kernel reads only the
 * selected entries of the low-rank KV cache and computes exact attention over them; "Day-0
 * Support for Large Model Inference", Core Operator Optimization item 2: the scattered rows
 * are gathered and attention is computed blockwise with the normalisation fused in).
 *   For token t, head h and each valid entry s of topk_idx[t] (0 <= s < seq_lens[b]; other
 *   entries, e.g. -1 padding, are skipped; duplicates count as given; causality is not
 *   checked):  c_s = kv_code[s] * kv_scale[s] (e4m3) or the stored row,
 *   z_s = softmax_scale * (q[t][h] . c_s[0:D_qk]),  out[t][h] = sum_s softmax(z)_s *
 *   c_s[0:D_v],  lse[t][h] = ln sum_s exp(z_s)  (natural log).  A token with no valid entry
 *   gets out = 0 and lse = -inf.  The value vector is the first D_v dims of the same row.
 * q        [T][H][D_qk]  TIS_BF16 (H = 128, D_qk = 576, D_v = 512, kv TIS_BF16 or TIS_E4M3
 *                        with kv_scale) or TIS_F32 (kv TIS_F32, kv_scale NULL,
 *                        D_qk <= 1024, H <= 1024)
 * kv_pool  [n_pages][64][D_qk]; kv_scale [n_pages][64] fp32 or NULL
 * topk_idx [T][K] int32 logical positions
 * out      [T][H][D_v] out_dt = TIS_BF16 or TIS_F32 with bf16 q; TIS_F32 with fp32 inputs.
 *          (bf16 output rounds to 2^-9 relative; rows of large magnitude need TIS_F32.)
 * lse      [T][H] fp32 or NULL
 * ws       workspace of sparse_mla_attn_workspace_size() bytes (split-K partials).
 */
tis_status_t sparse_mla_attn(const tis_batch_t* batch, const void* q, tis_dtype_t q_dt,
                             const void* kv_pool, tis_dtype_t kv_dt, const float* kv_scale,
                             const int32_t* topk_idx, int32_t K, int32_t H, int32_t D_qk,
                             int32_t D_v, float softmax_scale, void* out, tis_dtype_t out_dt,
                             float* lse, void* ws, size_t ws_bytes, void* stream);

/* sparse_mla_attn_dense - the same attention as sparse_mla_attn, computed the dense-masked way
 * ("Achieving Day-0 Readiness ... Million-Token Context", section 2.3: the prefill path treats
 * sparse attention as a dense matrix product over the full key range with a row-wise sparse
 * mask): every causal position 0..p_t of the token is read and multiplied, and the selection
 * topk_idx[t] (K entries) only decides which positions keep their softmax weight.  Results
 * equal sparse_mla_attn's up to rounding for selections without repeated positions (here a
 * position listed twice counts once).  Arguments as sparse_mla_attn; matrix-core shapes only
 * (H = 128, D_qk = 576, D_v = 512, bf16 q, bf16 or e4m3 cache), else TIS_ERR_UNSUPPORTED.
 * ws: sparse_mla_attn_dense_workspace_size() bytes (split partials of one chunk of tokens). */
tis_status_t sparse_mla_attn_dense(const tis_batch_t* batch, const void* q, tis_dtype_t q_dt,
                                   const void* kv_pool, tis_dtype_t kv_dt,
                                   const float* kv_scale, const int32_t* topk_idx, int32_t K,
                                   int32_t H, int32_t D_qk, int32_t D_v, float softmax_scale,
                                   void* out, tis_dtype_t out_dt, float* lse, void* ws,
                                   size_t ws_bytes, void* stream);

/* cache_append - write the rows of the batch's query tokens into their slots of one paged
 * cache, the step before the path ("Day-0 Support for Large Model Inference", Core Operator
 * Optimization item 1: the index stays on the device and is updated incrementally; "Day 0
 * Support for New LLM Architectures", Key Optimization 2: FP8 caches whose scale factors are
 * computed online: one fp32 scale per token over the whole row, or MXFP8 with one scale per
 * 32 elements for the indexer keys).
 *   Row t of `rows` goes to position p_t of its request (see the conventions above), i.e.
 *   slot page_table[b][p_t / 64] * 64 + p_t % 64, and is stored as
 *     TIS_E4M3: pool_scale[slot] = amax / 448 rounded to fp32 (amax = the largest |x| of the
 *               row; a scale of 0 is replaced by 1), and each code is the e4m3 round-to-
 *               nearest-even of the fp32 quotient x / pool_scale[slot], clamped to +-448
 *               (the sign of zero is kept);
 *     TIS_MXFP8: per 32 consecutive elements, pool_scale byte [slot][g] = X + 127 and each
 *               code the e4m3 round-to-nearest-even of x / 2^X clamped to +-448, with X as at
 *               TIS_QMODE_MXFP8 (D must be a multiple of 32);
 *     TIS_BF16: x rounded to bf16, to nearest even (pool_scale unused, must be NULL).
 *   A token whose page-table entry lies outside [0, n_pages) is not written.  Rows must be
 *   finite.  Call it once per cache (indexer keys: D = D_I; latent rows: D = D_qk).
 * rows        [T][D] TIS_F32 or TIS_BF16, 16-byte aligned
 * D           a multiple of 16, 16 <= D <= 2048
 * pool        [n_pages][64][D] of pool_dt (TIS_E4M3, TIS_MXFP8 or TIS_BF16), 16-byte aligned
 * pool_scale  [n_pages][64] fp32 (TIS_E4M3), [n_pages][64][D/32] bytes (TIS_MXFP8) or NULL
 *             (TIS_BF16)
 * Other slots of pool and pool_scale are left as they are.  Tokens of one call must not
 * share a slot (two writes of one slot race).
 */
tis_status_t cache_append(const tis_batch_t* batch, const void* rows, tis_dtype_t rows_dt,
                          int32_t D, void* pool, tis_dtype_t pool_dt, void* pool_scale,
                          void* stream);

/* Block-granular selection ("Day-0 Adaptation for Trillion-Parameter Models": the index
 * selection returns blocks of the cache layout, which the attention fetches whole; "Achieving
 * Day-0 Readiness ... Million-Token Context", section 2.2: fixed-size blocks located through a
 * block index table).  A block is one 64-position page of the request; block j of token t
 * covers positions [64j, min(64j + 64, n_t)), nb_t = ceil(n_t / 64) blocks in all.
 *
 * index_score_block - block scores: bscore[t][j] = the largest index_score of token t over the
 *   causal positions of block j (the same fp32 values index_score would write), -inf for a block
 *   whose page-table entry is out of range.  Arguments as index_score (matrix-core paths only:
 *   bf16 queries; fp32 queries return TIS_ERR_UNSUPPORTED).
 * block_scores [T][ld_blocks] fp32, ld_blocks >= max nb_t and a multiple of 4, 16-byte aligned;
 *              entries j >= nb_t are not written. */
tis_status_t index_score_block(const tis_batch_t* batch, const void* q_idx, tis_dtype_t q_dt,
                               const float* w, const void* k_pool, tis_dtype_t k_dt,
                               const void* k_scale, int32_t H_I, int32_t D_I, tis_qmode_t qmode,
                               float* block_scores, int64_t ld_blocks, void* stream);

/* topk_block_select - per token, the kb_t = min(K_blocks, nb_t) blocks with the largest block
 *   scores under (score descending, block ascending), as topk_select orders positions.
 * block_idx [T][K_blocks] int32: the kept blocks ascending, then -1 up to K_blocks.
 * block_val [T][K_blocks] fp32 or NULL: their block scores (0 where block_idx = -1).
 * topk_idx  [T][64 * K_blocks] int32 or NULL (16-byte aligned): the positions the attention
 *           reads: entry 64i + r is 64 * block_idx[t][i] + r when that position is causal
 *           (<= p_t), else -1 (also for padding blocks); it can be passed to sparse_mla_attn
 *           with K = 64 * K_blocks.
 * ws        topk_block_select_workspace_size() bytes (nonzero only for rows above 32768
 *           blocks, i.e. contexts above 2M positions, with K_blocks <= 4096), 16-byte aligned.
 * K_blocks  >= 1, K_blocks * 64 <= 2^24. */
tis_status_t topk_block_select(const tis_batch_t* batch, const float* block_scores,
                               int64_t ld_blocks, int32_t K_blocks, int32_t* block_idx,
                               float* block_val, int32_t* topk_idx, void* ws, size_t ws_bytes,
                               void* stream);

/* index_score_topk_block - index_score_block followed by topk_block_select with the block
 * scores in the workspace (index_score_topk_block_workspace_size() bytes, 16-byte aligned);
 * identical results to the two calls. */
tis_status_t index_score_topk_block(const tis_batch_t* batch, const void* q_idx,
                                    tis_dtype_t q_dt, const float* w, const void* k_pool,
                                    tis_dtype_t k_dt, const void* k_scale, int32_t H_I,
                                    int32_t D_I, tis_qmode_t qmode, int32_t K_blocks,
                                    int32_t* block_idx, float* block_val, int32_t* topk_idx,
                                    void* ws, size_t ws_bytes, void* stream);

/* Workspace sizes in bytes for the calls above, from the host fields of `batch` only (the
 * caller owns every buffer).  index_score needs none and returns 0.  topk_select: nonzero only
 * for the several-workgroups-per-row selection (see topk_select).  index_score_topk: one chunk
 * of score rows plus that selection's workspace.  sparse_mla_attn: the split partials, nonzero
 * when a token's keys are split across workgroups. */
size_t index_score_workspace_size(const tis_batch_t* batch, int32_t H_I, int32_t D_I);
size_t topk_select_workspace_size(const tis_batch_t* batch, int32_t K);
size_t index_score_topk_workspace_size(const tis_batch_t* batch, int32_t H_I, int32_t D_I,
                                       int32_t K);
size_t sparse_mla_attn_workspace_size(const tis_batch_t* batch, int32_t K, int32_t H,
                                      int32_t D_qk, int32_t D_v, tis_dtype_t kv_dt);
size_t sparse_mla_attn_dense_workspace_size(const tis_batch_t* batch, int32_t K, int32_t H,
                                            int32_t D_qk, int32_t D_v, tis_dtype_t kv_dt);
size_t topk_block_select_workspace_size(const tis_batch_t* batch, int32_t K_blocks);
size_t index_score_topk_block_workspace_size(const tis_batch_t* batch, int32_t H_I, int32_t D_I,
                                             int32_t K_blocks);

/* Message of the last non-OK status returned on the calling thread ("" if none). */
const char* tis_last_error(void);

/* TIS_ABI_VERSION of the loaded library. */
int32_t tis_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TOPIDX_H */
