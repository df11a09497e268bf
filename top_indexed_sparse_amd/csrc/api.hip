// C ABI of libtopidx: host-side validation, workspace sizing and kernel dispatch.
// Every check runs on the host before anything is enqueued; the library never allocates
// device memory and never synchronises the caller's stream.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "launch.h"
#include "topidx.h"

#define TIS_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_err;

tis_status_t fail(tis_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

tis_status_t hip_fail(hipError_t e, const char* what) {
  return fail(TIS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Size limits that keep every position, slot and byte offset the kernels form in 32-bit
// arithmetic in range: a score row of kMaxSeqLen fp32 values spans 2^30 bytes, and a slot
// (page * 64 + offset) stays below 2^30.
constexpr int kMaxSeqLen = 1 << 28;
constexpr int kMaxPages = 1 << 24;

// Scores that do not stay on chip go to a workspace of at most this many bytes; longer
// batches are processed in row chunks.
constexpr size_t kScoreScratchBudget = size_t(1) << 30;
// ... unless that holds fewer than kMinChunkRows rows (long rows): then up to kMinChunkRows
// rows within kScoreScratchMax bytes, since each chunk's launches end in a partly idle tail
// (ragged, rows up to 252K positions: 49 chunks of 1,065 rows took the fused call 26.4 ms, 13
// of 4,096 rows 25.0 ms; prefill64k keeps its 4,096-row chunks, which larger ones slowed).
constexpr size_t kScoreScratchMax = size_t(1) << 32;
constexpr int64_t kMinChunkRows = 4096;

struct HostInfo {
  int max_n = 0;   // longest causal range of any query token (= max seq_len with q_len > 0)
  int max_q = 0;   // longest query run of a request
  bool prefill_like = false;
};

tis_status_t check_batch(const tis_batch_t* b, HostInfo* hi) {
  if (!b) return fail(TIS_ERR_INVALID, "batch is NULL");
  if (b->B < 1 || b->T < 1) return fail(TIS_ERR_INVALID, "batch needs B >= 1 and T >= 1");
  if (!b->seq_lens || !b->cu_q || !b->seq_lens_host || !b->cu_q_host || !b->page_table)
    return fail(TIS_ERR_INVALID, "batch has a NULL array");
  if (b->page_size != TIS_PAGE_SIZE)
    return fail(TIS_ERR_INVALID, "page_size must be %d (got %d)", TIS_PAGE_SIZE, b->page_size);
  if (b->pt_stride < 1 || b->n_pages < 1)
    return fail(TIS_ERR_INVALID, "pt_stride and n_pages must be >= 1");
  if (b->n_pages > kMaxPages)
    return fail(TIS_ERR_INVALID, "n_pages must be <= %d (got %d)", kMaxPages, b->n_pages);
  if (b->cu_q_host[0] != 0) return fail(TIS_ERR_INVALID, "cu_q[0] must be 0");
  if (b->cu_q_host[b->B] != b->T) return fail(TIS_ERR_INVALID, "cu_q[B] must equal T");
  HostInfo h;
  for (int r = 0; r < b->B; ++r) {
    const int q = b->cu_q_host[r + 1] - b->cu_q_host[r];
    const int L = b->seq_lens_host[r];
    if (q < 0) return fail(TIS_ERR_INVALID, "cu_q must be nondecreasing (request %d)", r);
    if (L < q) return fail(TIS_ERR_INVALID, "seq_lens[%d]=%d < its %d query tokens", r, L, q);
    if ((int64_t)L > (int64_t)b->pt_stride * TIS_PAGE_SIZE)
      return fail(TIS_ERR_INVALID, "seq_lens[%d]=%d exceeds pt_stride*64", r, L);
    if (L > kMaxSeqLen)
      return fail(TIS_ERR_INVALID, "seq_lens[%d]=%d exceeds %d", r, L, kMaxSeqLen);
    if (q > 0) h.max_n = std::max(h.max_n, L);
    h.max_q = std::max(h.max_q, q);
  }
  h.prefill_like = (int64_t)b->T >= 4 * (int64_t)b->B;
  if (hi) *hi = h;
  return TIS_OK;
}

tis::DevBatch dev_batch(const tis_batch_t* b) {
  tis::DevBatch d;
  d.seq_lens = b->seq_lens;
  d.cu_q = b->cu_q;
  d.page_table = b->page_table;
  d.B = b->B;
  d.T = b->T;
  d.pt_stride = b->pt_stride;
  d.n_pages = b->n_pages;
  d.row_shift = 0;
  return d;
}

// fp32 kernel; matrix-core scorer with an e4m3 / bf16 query over per-token-scaled e4m3 keys,
// or MXFP8 query and keys
enum class IdxPath { F32, FP8, BF16, MX };

tis_status_t check_index_args(const void* q_idx, tis_dtype_t q_dt, const float* w,
                              const void* k_pool, tis_dtype_t k_dt, const void* k_scale,
                              int32_t H_I, int32_t D_I, tis_qmode_t qmode, IdxPath* path) {
  if (!q_idx || !w || !k_pool) return fail(TIS_ERR_INVALID, "q_idx, w and k_pool must be set");
  if (!aligned16(q_idx) || !aligned16(k_pool) || !aligned16(w))
    return fail(TIS_ERR_INVALID, "q_idx, w and k_pool must be 16-byte aligned");
  if (H_I < 1 || D_I < 1) return fail(TIS_ERR_INVALID, "H_I and D_I must be >= 1");
  if (q_dt == TIS_F32 && k_dt == TIS_F32 && qmode == TIS_QMODE_BF16) {
    if (k_scale) return fail(TIS_ERR_INVALID, "fp32 keys take no k_scale");
    if ((int64_t)H_I * D_I > 8192)
      return fail(TIS_ERR_UNSUPPORTED, "fp32 indexer supports H_I*D_I <= 8192");
    *path = IdxPath::F32;
    return TIS_OK;
  }
  if (q_dt == TIS_BF16 && k_dt == TIS_E4M3 &&
      (qmode == TIS_QMODE_FP8 || qmode == TIS_QMODE_BF16)) {
    if (!k_scale || !aligned16(k_scale))
      return fail(TIS_ERR_INVALID, "e4m3 keys need a 16-byte aligned k_scale");
    if (H_I != 64 || D_I != 128)
      return fail(TIS_ERR_UNSUPPORTED, "e4m3 indexer supports H_I=64, D_I=128");
    *path = qmode == TIS_QMODE_FP8 ? IdxPath::FP8 : IdxPath::BF16;
    return TIS_OK;
  }
  if (q_dt == TIS_BF16 && k_dt == TIS_MXFP8 && qmode == TIS_QMODE_MXFP8) {
    if (!k_scale || !aligned16(k_scale))
      return fail(TIS_ERR_INVALID, "MXFP8 keys need 16-byte aligned scale bytes");
    if (H_I != 64 || D_I != 128)
      return fail(TIS_ERR_UNSUPPORTED, "MXFP8 indexer supports H_I=64, D_I=128");
    *path = IdxPath::MX;
    return TIS_OK;
  }
  return fail(TIS_ERR_UNSUPPORTED,
              "indexer supports (f32, f32, BF16), (bf16, e4m3, FP8 or BF16) and (bf16, MXFP8, "
              "MXFP8) for (q, k, qmode)");
}

// The matrix-core scorer's work list ("Day 0 Support for New LLM Architectures", Key
// Optimization 3: balance the causal work of long inputs; "Day-0 Support for Large Model
// Inference", Core Operator Optimization 2: requests of different lengths share the device).
// A launch covers a token range with a grid of (token group) x (key chunk) units sized by the
// range's longest causal length; a unit past its tokens' range only looks its tokens up and
// exits.  Batches that mix short and long requests, and a long prefill's causal triangle,
// therefore run as a few launches over runs of consecutive tokens, each sized by its own longest
// causal length: the cuts (at request boundaries and every few thousand tokens within a
// request) minimise the units launched plus a per-launch cost, by dynamic programming.
struct Segment {
  int t0, tc, max_n;
};

std::vector<Segment> plan_segments(const tis_batch_t* b, int t0, int tc, bool prefill_like) {
  const int tok = prefill_like ? 4 : 1;  // tokens per unit
  const int chunk = 4096;                // keys per unit
  // a launch's fixed cost, in units (a prefill unit scores four tokens)
  const double kLaunchUnits = prefill_like ? 750.0 : 3000.0;
  if (tc < 1) return {};
  // intervals between consecutive cut points lie within one request; each interval's longest
  // causal length is that of its last token
  // Within a request the causal length grows by one per token (a prefill's triangle), so a
  // request's range is also cut every `step` tokens (a multiple of the group; enough to keep
  // the plan at about 128 intervals besides the request boundaries).
  std::vector<int> cut{t0};
  std::vector<int> imax;
  const int t1 = t0 + tc;
  const int step = std::max(2048, (tc / 128 + tok - 1) / tok * tok);
  for (int r = 0; r < b->B; ++r) {
    const int a = std::max(b->cu_q_host[r], t0), e = std::min(b->cu_q_host[r + 1], t1);
    if (a >= e) continue;
    for (int c = a; c < e; c += step) {
      const int ce = std::min(e, c + step);
      const int n_last = b->seq_lens_host[r] - (b->cu_q_host[r + 1] - (ce - 1)) + 1;
      cut.push_back(ce);
      imax.push_back(n_last);
    }
  }
  const int m = (int)cut.size() - 1;  // intervals
  std::vector<Segment> segs;
  if (m <= 0) return segs;
  auto units = [&](int ntok, int maxn) {
    return (double)((ntok + tok - 1) / tok) * (double)((maxn + chunk - 1) / chunk);
  };
  if (m == 1 || m > 512) {  // one launch (beyond 512 intervals the plan is not worth its cost)
    int mx = 0;
    for (int v : imax) mx = std::max(mx, v);
    segs.push_back({t0, tc, mx});
    return segs;
  }
  std::vector<double> best(m + 1, 0.0);
  std::vector<int> from(m + 1, 0);
  for (int j = 1; j <= m; ++j) {
    best[j] = 1e300;
    int mx = 0;
    for (int i = j - 1; i >= 0; --i) {
      mx = std::max(mx, imax[i]);
      const double c = best[i] + kLaunchUnits + units(cut[j] - cut[i], mx);
      if (c < best[j]) {
        best[j] = c;
        from[j] = i;
      }
    }
  }
  for (int j = m; j > 0; j = from[j]) {
    const int i = from[j];
    int mx = 0;
    for (int k = i; k < j; ++k) mx = std::max(mx, imax[k]);
    segs.push_back({cut[i], cut[j] - cut[i], mx});
  }
  std::reverse(segs.begin(), segs.end());
  return segs;
}

// Pages per wave of the decode scorer over tokens t0 .. t0+tc-1 (a workgroup scores a chunk
// of 512 * np keys of one token, one workgroup per compute unit at a time): of 8, 16 and 32,
// the one with the fewest rounds of workgroups over the 256 units, each round costing its
// chunk plus the workgroup's set-up (the request lookup, the query quantisation and the
// filling of the page ring, about two pages per wave).  Few long rows thus take large chunks
// and pay the set-up once per chunk instead of once per 4,096 keys, while batches whose
// 4,096-key chunks already fill the chip keep them.  (The kernel takes up to 64; 32 already
// brings the set-up below 6% of a workgroup's time.)
int decode_pages_per_wave(const tis_batch_t* b, int t0, int tc) {
  constexpr int kUnits = 256, kSetup = 2;
  // the requests that hold tokens t0 .. t0+tc-1: from the last r with cu_q[r] <= t0
  const int r0 = std::max(
      0, (int)(std::upper_bound(b->cu_q_host, b->cu_q_host + b->B + 1, t0) - b->cu_q_host) - 1);
  int best = 8;
  int64_t best_cost = INT64_MAX;
  for (int np = 8; np <= 32; np *= 2) {
    const int64_t ck = 512 * (int64_t)np;
    int64_t units = 0;
    for (int r = r0; r < b->B && b->cu_q_host[r] < t0 + tc; ++r) {
      const int a = std::max(b->cu_q_host[r], t0), e = std::min(b->cu_q_host[r + 1], t0 + tc);
      for (int t = a; t < e; ++t) {
        const int64_t n = (int64_t)b->seq_lens_host[r] - (b->cu_q_host[r + 1] - t) + 1;
        units += (n + ck - 1) / ck;
      }
    }
    const int64_t cost = (units + kUnits - 1) / kUnits * (np + kSetup);
    if (cost < best_cost) {
      best_cost = cost;
      best = np;
    }
  }
  return best;
}

// block: one score per 64-key page (rows of ld entries) instead of one per key; the fp32
// scorer has no block form (callers check).  Rows of scores are those of tokens t0 .. t0+tc-1.
tis_status_t run_index(const tis_batch_t* batch, const HostInfo& hi, IdxPath path, int t0,
                       int tc, const void* q_idx, const float* w, const void* k_pool,
                       const void* k_scale, int H_I, int D_I, float* scores, int64_t ld,
                       hipStream_t st, bool block = false) {
  const tis::DevBatch d = dev_batch(batch);
  hipError_t e;
  if (path == IdxPath::F32) {
    e = tis::launch_index_score_f32(d, t0, tc, hi.max_n, (const float*)q_idx, w,
                                    (const float*)k_pool, H_I, D_I, scores, ld, st);
    return e == hipSuccess ? TIS_OK : hip_fail(e, "index_score launch");
  }
  for (const Segment& sg : plan_segments(batch, t0, tc, hi.prefill_like)) {
    if (sg.max_n < 1) continue;
    const int np = hi.prefill_like ? 0 : decode_pages_per_wave(batch, sg.t0, sg.tc);
    e = tis::launch_index_score_fp8(d, sg.t0, sg.tc, sg.max_n, hi.prefill_like, np,
                                    path == IdxPath::BF16 ? 1 : path == IdxPath::MX ? 2 : 0,
                                    block, (const uint16_t*)q_idx, w, (const uint8_t*)k_pool,
                                    k_scale, scores + (int64_t)(sg.t0 - t0) * ld, ld, st);
    if (e != hipSuccess) return hip_fail(e, "index_score launch");
  }
  return TIS_OK;
}

int64_t round4(int64_t x) { return (x + 3) & ~int64_t(3); }

// the fused call's workspace: the score rows of one chunk, then the selection's workspace
size_t fused_scores_bytes(int rows, const HostInfo& hi) {
  return ((size_t)rows * (size_t)round4(hi.max_n) * sizeof(float) + 255) & ~(size_t)255;
}

// score rows per chunk under a byte budget for the score rows (0 if one row does not fit)
// Rows of scores per chunk of the fused call: within `budget` bytes, or (long rows) up to
// kMinChunkRows rows within `cap` bytes.
int fused_rows_per_chunk(const tis_batch_t* b, const HostInfo& hi,
                         size_t budget = kScoreScratchBudget, size_t cap = kScoreScratchMax) {
  const int64_t row_bytes = std::max<int64_t>(round4(hi.max_n) * 4, 1);
  int64_t r = (int64_t)budget / row_bytes;
  if (r < kMinChunkRows) r = std::max(r, std::min<int64_t>(kMinChunkRows, (int64_t)cap / row_bytes));
  return (int)std::min<int64_t>(r, b->T);
}

enum class AttnPath { F32, MFMA };

tis_status_t check_attn_args(const void* q, tis_dtype_t q_dt, const void* kv_pool,
                             tis_dtype_t kv_dt, const float* kv_scale, const int32_t* topk_idx,
                             int32_t K, int32_t H, int32_t D_qk, int32_t D_v,
                             float softmax_scale, const void* out, tis_dtype_t out_dt,
                             AttnPath* path) {
  if (!q || !kv_pool || !topk_idx || !out)
    return fail(TIS_ERR_INVALID, "q, kv_pool, topk_idx and out must be set");
  if (!aligned16(q) || !aligned16(kv_pool) || !aligned16(out) || !aligned16(topk_idx))
    return fail(TIS_ERR_INVALID, "q, kv_pool, topk_idx and out must be 16-byte aligned");
  if (K < 1 || H < 1 || D_qk < 1 || D_v < 1) return fail(TIS_ERR_INVALID, "K, H, D must be >= 1");
  if (D_v > D_qk) return fail(TIS_ERR_INVALID, "D_v (%d) > D_qk (%d)", D_v, D_qk);
  if (!std::isfinite(softmax_scale)) return fail(TIS_ERR_INVALID, "softmax_scale not finite");
  if (q_dt == TIS_F32 && kv_dt == TIS_F32 && out_dt == TIS_F32) {
    if (kv_scale) return fail(TIS_ERR_INVALID, "fp32 cache takes no kv_scale");
    if (D_qk > 1024 || H > 1024 || (int64_t)(D_qk + 2 * K) * 4 > 64 * 1024)
      return fail(TIS_ERR_UNSUPPORTED, "fp32 attention supports D_qk<=1024, H<=1024, small K");
    *path = AttnPath::F32;
    return TIS_OK;
  }
  if (q_dt == TIS_BF16 && (out_dt == TIS_BF16 || out_dt == TIS_F32) &&
      (kv_dt == TIS_BF16 || kv_dt == TIS_E4M3)) {
    if (kv_dt == TIS_E4M3 && (!kv_scale || !aligned16(kv_scale)))
      return fail(TIS_ERR_INVALID, "e4m3 cache needs a 16-byte aligned kv_scale");
    if (kv_dt == TIS_BF16 && kv_scale) return fail(TIS_ERR_INVALID, "bf16 cache takes no kv_scale");
    if (H != 128 || D_qk != 576 || D_v != 512)
      return fail(TIS_ERR_UNSUPPORTED, "bf16 attention supports H=128, D_qk=576, D_v=512");
    *path = AttnPath::MFMA;
    return TIS_OK;
  }
  return fail(TIS_ERR_UNSUPPORTED, "attention supports all-fp32 or bf16 q/out with bf16|e4m3 cache");
}

size_t attn_ws_bytes(const tis_batch_t* b, int32_t K, AttnPath path) {
  if (path == AttnPath::F32) return 0;
  const int ns = tis::attn_split_count(b->T, K);
  if (ns == 1) return 0;
  return (size_t)b->T * ns * 128 * (512 + 4) * sizeof(float);
}

}  // namespace

// ============================================================================ C ABI
TIS_API int32_t tis_abi_version(void) { return TIS_ABI_VERSION; }

TIS_API const char* tis_last_error(void) { return g_err.c_str(); }

TIS_API size_t index_score_workspace_size(const tis_batch_t* batch, int32_t H_I, int32_t D_I) {
  (void)batch; (void)H_I; (void)D_I;
  return 0;
}

TIS_API size_t topk_select_workspace_size(const tis_batch_t* batch, int32_t K) {
  HostInfo hi;
  if (check_batch(batch, &hi) != TIS_OK || K < 1) return 0;
  return tis::topk_ws_bytes(batch->T, hi.max_n, K);
}

TIS_API size_t index_score_topk_workspace_size(const tis_batch_t* batch, int32_t H_I,
                                               int32_t D_I, int32_t K) {
  (void)H_I; (void)D_I;
  HostInfo hi;
  if (check_batch(batch, &hi) != TIS_OK || K < 1) return 0;
  const int rows = std::max(1, fused_rows_per_chunk(batch, hi));
  return fused_scores_bytes(rows, hi) + tis::topk_ws_bytes(rows, hi.max_n, K);
}

TIS_API size_t sparse_mla_attn_workspace_size(const tis_batch_t* batch, int32_t K, int32_t H,
                                              int32_t D_qk, int32_t D_v, tis_dtype_t kv_dt) {
  if (check_batch(batch, nullptr) != TIS_OK || K < 1) return 0;
  const bool mfma = (kv_dt == TIS_BF16 || kv_dt == TIS_E4M3) && H == 128 && D_qk == 576 &&
                    D_v == 512;
  return attn_ws_bytes(batch, K, mfma ? AttnPath::MFMA : AttnPath::F32);
}

TIS_API tis_status_t index_score(const tis_batch_t* batch, const void* q_idx, tis_dtype_t q_dt,
                                 const float* w, const void* k_pool, tis_dtype_t k_dt,
                                 const void* k_scale, int32_t H_I, int32_t D_I,
                                 tis_qmode_t qmode, float* scores, int64_t ld_scores, void* ws,
                                 size_t ws_bytes, void* stream) {
  (void)ws; (void)ws_bytes;
  HostInfo hi;
  tis_status_t st = check_batch(batch, &hi);
  if (st != TIS_OK) return st;
  IdxPath path;
  st = check_index_args(q_idx, q_dt, w, k_pool, k_dt, k_scale, H_I, D_I, qmode, &path);
  if (st != TIS_OK) return st;
  if (!scores || !aligned16(scores)) return fail(TIS_ERR_INVALID, "scores must be 16-byte aligned");
  if (ld_scores < hi.max_n || (ld_scores & 3))
    return fail(TIS_ERR_INVALID, "ld_scores must be >= %d and a multiple of 4", hi.max_n);
  return run_index(batch, hi, path, 0, batch->T, q_idx, w, k_pool, k_scale, H_I, D_I, scores,
                   ld_scores, (hipStream_t)stream);
}

TIS_API tis_status_t topk_select(const tis_batch_t* batch, const float* scores,
                                 int64_t ld_scores, int32_t K, int32_t* topk_idx,
                                 float* topk_val, void* ws, size_t ws_bytes, void* stream) {
  HostInfo hi;
  tis_status_t st = check_batch(batch, &hi);
  if (st != TIS_OK) return st;
  if (K < 1) return fail(TIS_ERR_INVALID, "K must be >= 1");
  if (!scores || !topk_idx) return fail(TIS_ERR_INVALID, "scores and topk_idx must be set");
  const size_t need = tis::topk_ws_bytes(batch->T, hi.max_n, K);
  if (ws_bytes < need || (need && (!ws || !aligned16(ws))))
    return fail(TIS_ERR_INVALID, "workspace needs %zu bytes, 16-byte aligned", need);
  if (!aligned16(scores)) return fail(TIS_ERR_INVALID, "scores must be 16-byte aligned");
  if (ld_scores < hi.max_n || (ld_scores & 3))
    return fail(TIS_ERR_INVALID, "ld_scores must be >= %d and a multiple of 4", hi.max_n);
  hipError_t e = tis::launch_topk(dev_batch(batch), 0, batch->T, hi.max_n, scores, ld_scores, K,
                                  topk_idx, topk_val, ws, (hipStream_t)stream);
  return e == hipSuccess ? TIS_OK : hip_fail(e, "topk_select launch");
}

namespace {

// The fused chain over `rows`-token chunks with its workspace at ws (score rows, then the
// selection's workspace); the arguments have been checked.
tis_status_t fused_run(const tis_batch_t* batch, const HostInfo& hi, IdxPath path,
                       const void* q_idx, const float* w, const void* k_pool,
                       const void* k_scale, int32_t H_I, int32_t D_I, int32_t K,
                       int32_t* topk_idx, float* topk_val, int rows, void* ws, hipStream_t s) {
  const int64_t ld = round4(hi.max_n);
  const size_t sbytes = fused_scores_bytes(rows, hi);
  float* sc = (float*)ws;
  void* tws = (char*)ws + sbytes;
  const tis::DevBatch d = dev_batch(batch);
  for (int t0 = 0; t0 < batch->T; t0 += rows) {
    const int tc = std::min(rows, batch->T - t0);
    tis_status_t st =
        run_index(batch, hi, path, t0, tc, q_idx, w, k_pool, k_scale, H_I, D_I, sc, ld, s);
    if (st != TIS_OK) return st;
    hipError_t e = tis::launch_topk(d, t0, tc, hi.max_n, sc, ld, K, topk_idx, topk_val, tws, s);
    if (e != hipSuccess) return hip_fail(e, "index_score_topk select launch");
  }
  return TIS_OK;
}

tis_status_t fused_checks(const tis_batch_t* batch, HostInfo* hi, const void* q_idx,
                          tis_dtype_t q_dt, const float* w, const void* k_pool,
                          tis_dtype_t k_dt, const void* k_scale, int32_t H_I, int32_t D_I,
                          tis_qmode_t qmode, int32_t K, const int32_t* topk_idx,
                          IdxPath* path) {
  tis_status_t st = check_batch(batch, hi);
  if (st != TIS_OK) return st;
  st = check_index_args(q_idx, q_dt, w, k_pool, k_dt, k_scale, H_I, D_I, qmode, path);
  if (st != TIS_OK) return st;
  if (K < 1) return fail(TIS_ERR_INVALID, "K must be >= 1");
  if (!topk_idx) return fail(TIS_ERR_INVALID, "topk_idx must be set");
  return TIS_OK;
}

// ---- the allocation-free variant's scratch: one array per device, held until the process
// ends.  Host code never passes the array's name to a kernel (in host code it only stands in
// for the symbol): its device address is looked up once per device and used instead.
constexpr size_t kNoAllocScratch = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratch];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device (or null)

tis_status_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(TIS_ERR_UNSUPPORTED, "device %d beyond the %d the library tracks", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(TIS_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TIS_OK;
}

}  // namespace

TIS_API tis_status_t index_score_topk(const tis_batch_t* batch, const void* q_idx,
                                      tis_dtype_t q_dt, const float* w, const void* k_pool,
                                      tis_dtype_t k_dt, const void* k_scale, int32_t H_I,
                                      int32_t D_I, tis_qmode_t qmode, int32_t K,
                                      int32_t* topk_idx, float* topk_val, void* ws,
                                      size_t ws_bytes, void* stream) {
  HostInfo hi;
  IdxPath path;
  tis_status_t st = fused_checks(batch, &hi, q_idx, q_dt, w, k_pool, k_dt, k_scale, H_I, D_I,
                                 qmode, K, topk_idx, &path);
  if (st != TIS_OK) return st;
  const int rows = std::max(1, fused_rows_per_chunk(batch, hi));
  const size_t need = fused_scores_bytes(rows, hi) + tis::topk_ws_bytes(rows, hi.max_n, K);
  if (ws_bytes < need || (need && (!ws || !aligned16(ws))))
    return fail(TIS_ERR_INVALID, "workspace needs %zu bytes, 16-byte aligned", need);
  return fused_run(batch, hi, path, q_idx, w, k_pool, k_scale, H_I, D_I, K, topk_idx, topk_val,
                   rows, ws, (hipStream_t)stream);
}

TIS_API tis_status_t index_score_topk_noalloc(const tis_batch_t* batch, const void* q_idx,
                                              tis_dtype_t q_dt, const float* w,
                                              const void* k_pool, tis_dtype_t k_dt,
                                              const void* k_scale, int32_t H_I, int32_t D_I,
                                              tis_qmode_t qmode, int32_t K, int32_t* topk_idx,
                                              float* topk_val, void* stream) {
  HostInfo hi;
  IdxPath path;
  tis_status_t st = fused_checks(batch, &hi, q_idx, q_dt, w, k_pool, k_dt, k_scale, H_I, D_I,
                                 qmode, K, topk_idx, &path);
  if (st != TIS_OK) return st;
  // the selection's workspace is bounded by its 64-row limit; the rest holds score rows
  const size_t sel = tis::topk_ws_bytes(64, hi.max_n, K);
  const int rows = fused_rows_per_chunk(batch, hi, kNoAllocScratch - sel - 256,
                                        kNoAllocScratch - sel - 256);
  if (rows < 1)
    return fail(TIS_ERR_INVALID,
                "index_score_topk_noalloc: a score row of %d positions does not fit its %zu-byte "
                "scratch (at most %zu positions)", hi.max_n, kNoAllocScratch,
                (kNoAllocScratch - sel - 256) / 4);
  const size_t need = fused_scores_bytes(rows, hi) + tis::topk_ws_bytes(rows, hi.max_n, K);
  if (need > kNoAllocScratch)
    return fail(TIS_ERR_INVALID, "index_score_topk_noalloc: needs %zu bytes of scratch, has %zu",
                need, kNoAllocScratch);
  void* ptr = nullptr;
  st = scratch_address(&ptr);
  if (st != TIS_OK) return st;
  return fused_run(batch, hi, path, q_idx, w, k_pool, k_scale, H_I, D_I, K, topk_idx, topk_val,
                   rows, ptr, (hipStream_t)stream);
}

// ============================================================================ block selection
namespace {

constexpr int kBlockShift = 6;  // one block = one 64-position page

int blocks_of(int n) { return (n + (1 << kBlockShift) - 1) >> kBlockShift; }

tis::DevBatch block_batch(const tis_batch_t* b) {
  tis::DevBatch d = dev_batch(b);
  d.row_shift = kBlockShift;
  return d;
}

size_t block_rows_bytes(int rows, const HostInfo& hi) {
  return ((size_t)rows * (size_t)round4(blocks_of(hi.max_n)) * sizeof(float) + 255) &
         ~(size_t)255;
}

// selection over block rows, then the optional expansion to positions
tis_status_t run_block_select(const tis_batch_t* batch, const HostInfo& hi, int t0, int tc,
                              const float* bs, int64_t ld, int32_t K_blocks, int32_t* block_idx,
                              float* block_val, int32_t* topk_idx, void* ws, hipStream_t s) {
  hipError_t e = tis::launch_topk(block_batch(batch), t0, tc, blocks_of(hi.max_n), bs, ld,
                                  K_blocks, block_idx, block_val, ws, s);
  if (e != hipSuccess) return hip_fail(e, "block selection launch");
  if (topk_idx) {
    e = tis::launch_expand_blocks(dev_batch(batch), t0, tc, block_idx, K_blocks, topk_idx, s);
    if (e != hipSuccess) return hip_fail(e, "block expansion launch");
  }
  return TIS_OK;
}

tis_status_t check_block_outputs(int32_t K_blocks, const int32_t* block_idx,
                                 const int32_t* topk_idx) {
  if (K_blocks < 1) return fail(TIS_ERR_INVALID, "K_blocks must be >= 1");
  if ((int64_t)K_blocks * TIS_PAGE_SIZE > (int64_t)1 << 24)
    return fail(TIS_ERR_INVALID, "K_blocks * 64 must be <= 2^24");
  if (!block_idx) return fail(TIS_ERR_INVALID, "block_idx must be set");
  if (topk_idx && !aligned16(topk_idx))
    return fail(TIS_ERR_INVALID, "topk_idx must be 16-byte aligned");
  return TIS_OK;
}

}  // namespace

TIS_API tis_status_t index_score_block(const tis_batch_t* batch, const void* q_idx,
                                       tis_dtype_t q_dt, const float* w, const void* k_pool,
                                       tis_dtype_t k_dt, const void* k_scale, int32_t H_I,
                                       int32_t D_I, tis_qmode_t qmode, float* block_scores,
                                       int64_t ld_blocks, void* stream) {
  HostInfo hi;
  tis_status_t st = check_batch(batch, &hi);
  if (st != TIS_OK) return st;
  IdxPath path;
  st = check_index_args(q_idx, q_dt, w, k_pool, k_dt, k_scale, H_I, D_I, qmode, &path);
  if (st != TIS_OK) return st;
  if (path == IdxPath::F32)
    return fail(TIS_ERR_UNSUPPORTED, "block scores need the matrix-core scorer (bf16 queries)");
  if (!block_scores || !aligned16(block_scores))
    return fail(TIS_ERR_INVALID, "block_scores must be 16-byte aligned");
  if (ld_blocks < blocks_of(hi.max_n) || (ld_blocks & 3))
    return fail(TIS_ERR_INVALID, "ld_blocks must be >= %d and a multiple of 4",
                blocks_of(hi.max_n));
  return run_index(batch, hi, path, 0, batch->T, q_idx, w, k_pool, k_scale, H_I, D_I,
                   block_scores, ld_blocks, (hipStream_t)stream, true);
}

TIS_API size_t topk_block_select_workspace_size(const tis_batch_t* batch, int32_t K_blocks) {
  HostInfo hi;
  if (check_batch(batch, &hi) != TIS_OK || K_blocks < 1) return 0;
  return tis::topk_ws_bytes(batch->T, blocks_of(hi.max_n), K_blocks);
}

TIS_API tis_status_t topk_block_select(const tis_batch_t* batch, const float* block_scores,
                                       int64_t ld_blocks, int32_t K_blocks, int32_t* block_idx,
                                       float* block_val, int32_t* topk_idx, void* ws,
                                       size_t ws_bytes, void* stream) {
  HostInfo hi;
  tis_status_t st = check_batch(batch, &hi);
  if (st != TIS_OK) return st;
  st = check_block_outputs(K_blocks, block_idx, topk_idx);
  if (st != TIS_OK) return st;
  if (!block_scores || !aligned16(block_scores))
    return fail(TIS_ERR_INVALID, "block_scores must be 16-byte aligned");
  if (ld_blocks < blocks_of(hi.max_n) || (ld_blocks & 3))
    return fail(TIS_ERR_INVALID, "ld_blocks must be >= %d and a multiple of 4",
                blocks_of(hi.max_n));
  const size_t need = tis::topk_ws_bytes(batch->T, blocks_of(hi.max_n), K_blocks);
  if (ws_bytes < need || (need && (!ws || !aligned16(ws))))
    return fail(TIS_ERR_INVALID, "workspace needs %zu bytes, 16-byte aligned", need);
  return run_block_select(batch, hi, 0, batch->T, block_scores, ld_blocks, K_blocks, block_idx,
                          block_val, topk_idx, ws, (hipStream_t)stream);
}

TIS_API size_t index_score_topk_block_workspace_size(const tis_batch_t* batch, int32_t H_I,
                                                     int32_t D_I, int32_t K_blocks) {
  (void)H_I; (void)D_I;
  HostInfo hi;
  if (check_batch(batch, &hi) != TIS_OK || K_blocks < 1) return 0;
  const int rows = std::max(1, std::min<int>(batch->T, (int)(kScoreScratchBudget /
                                                        (round4(blocks_of(hi.max_n)) * 4))));
  return block_rows_bytes(rows, hi) + tis::topk_ws_bytes(rows, blocks_of(hi.max_n), K_blocks);
}

TIS_API tis_status_t index_score_topk_block(const tis_batch_t* batch, const void* q_idx,
                                            tis_dtype_t q_dt, const float* w,
                                            const void* k_pool, tis_dtype_t k_dt,
                                            const void* k_scale, int32_t H_I, int32_t D_I,
                                            tis_qmode_t qmode, int32_t K_blocks,
                                            int32_t* block_idx, float* block_val,
                                            int32_t* topk_idx, void* ws, size_t ws_bytes,
                                            void* stream) {
  HostInfo hi;
  tis_status_t st = check_batch(batch, &hi);
  if (st != TIS_OK) return st;
  IdxPath path;
  st = check_index_args(q_idx, q_dt, w, k_pool, k_dt, k_scale, H_I, D_I, qmode, &path);
  if (st != TIS_OK) return st;
  if (path == IdxPath::F32)
    return fail(TIS_ERR_UNSUPPORTED, "block scores need the matrix-core scorer (bf16 queries)");
  st = check_block_outputs(K_blocks, block_idx, topk_idx);
  if (st != TIS_OK) return st;
  const int nb = blocks_of(hi.max_n);
  const int rows = std::max(1, std::min<int>(batch->T, (int)(kScoreScratchBudget /
                                                        (round4(nb) * 4))));
  const size_t sbytes = block_rows_bytes(rows, hi);
  const size_t need = sbytes + tis::topk_ws_bytes(rows, nb, K_blocks);
  if (ws_bytes < need || (need && (!ws || !aligned16(ws))))
    return fail(TIS_ERR_INVALID, "workspace needs %zu bytes, 16-byte aligned", need);
  hipStream_t s = (hipStream_t)stream;
  float* bs = (float*)ws;
  void* tws = (char*)ws + sbytes;
  const int64_t ld = round4(nb);
  for (int t0 = 0; t0 < batch->T; t0 += rows) {
    const int tc = std::min(rows, batch->T - t0);
    st = run_index(batch, hi, path, t0, tc, q_idx, w, k_pool, k_scale, H_I, D_I, bs, ld, s,
                   true);
    if (st != TIS_OK) return st;
    // (the chunk's rows start at bs: the selection indexes its rows from t0)
    st = run_block_select(batch, hi, t0, tc, bs, ld, K_blocks, block_idx, block_val, topk_idx,
                          tws, s);
    if (st != TIS_OK) return st;
  }
  return TIS_OK;
}

// ============================================================================ dense-masked form
namespace {

constexpr size_t kDenseScratchBudget = size_t(1) << 30;

// Token chunk and split count of the dense form: every chunk uses the same split count (that
// of a full chunk), so the partials of one chunk fit the workspace.
void dense_plan(const tis_batch_t* b, const HostInfo& hi, int* chunk, int* nsplit) {
  int c = std::min(b->T, 256);
  int ns = tis::attn_split_count(c, std::max(hi.max_n, 1));
  const size_t per_tok = (size_t)ns * 128 * (512 + 4) * sizeof(float);
  if (ns > 1) c = (int)std::max<size_t>(1, std::min<size_t>(c, kDenseScratchBudget / per_tok));
  *chunk = c;
  *nsplit = ns;
}

size_t dense_ws_bytes(const tis_batch_t* b, const HostInfo& hi) {
  int c, ns;
  dense_plan(b, hi, &c, &ns);
  return ns > 1 ? (size_t)c * ns * 128 * (512 + 4) * sizeof(float) : 0;
}

}  // namespace

TIS_API size_t sparse_mla_attn_dense_workspace_size(const tis_batch_t* batch, int32_t K,
                                                    int32_t H, int32_t D_qk, int32_t D_v,
                                                    tis_dtype_t kv_dt) {
  (void)K; (void)H; (void)D_qk; (void)D_v; (void)kv_dt;
  HostInfo hi;
  if (check_batch(batch, &hi) != TIS_OK) return 0;
  return dense_ws_bytes(batch, hi);
}

TIS_API tis_status_t sparse_mla_attn_dense(const tis_batch_t* batch, const void* q,
                                           tis_dtype_t q_dt, const void* kv_pool,
                                           tis_dtype_t kv_dt, const float* kv_scale,
                                           const int32_t* topk_idx, int32_t K, int32_t H,
                                           int32_t D_qk, int32_t D_v, float softmax_scale,
                                           void* out, tis_dtype_t out_dt, float* lse, void* ws,
                                           size_t ws_bytes, void* stream) {
  HostInfo hi;
  tis_status_t st = check_batch(batch, &hi);
  if (st != TIS_OK) return st;
  AttnPath path;
  st = check_attn_args(q, q_dt, kv_pool, kv_dt, kv_scale, topk_idx, K, H, D_qk, D_v,
                       softmax_scale, out, out_dt, &path);
  if (st != TIS_OK) return st;
  if (path != AttnPath::MFMA)
    return fail(TIS_ERR_UNSUPPORTED, "the dense-masked form runs on the matrix-core kernel only");
  const size_t need = dense_ws_bytes(batch, hi);
  if (ws_bytes < need || (need && (!ws || !aligned16(ws))))
    return fail(TIS_ERR_INVALID, "workspace needs %zu bytes, 16-byte aligned", need);
  int chunk, ns;
  dense_plan(batch, hi, &chunk, &ns);
  hipStream_t s = (hipStream_t)stream;
  const tis::DevBatch d = dev_batch(batch);
  float* part_o = ns > 1 ? (float*)ws : nullptr;
  float* part_ml = ns > 1 ? part_o + (size_t)chunk * ns * 128 * 512 : nullptr;
  for (int t0 = 0; t0 < batch->T; t0 += chunk) {
    const int tc = std::min(chunk, batch->T - t0);
    hipError_t e = tis::launch_mla_attn(d, t0, tc, kv_dt == TIS_E4M3, (const uint16_t*)q,
                                        (const uint8_t*)kv_pool, kv_scale, topk_idx, K,
                                        softmax_scale, ns, out, out_dt == TIS_F32, lse, part_o,
                                        part_ml, s, std::max(hi.max_n, 1));
    if (e != hipSuccess) return hip_fail(e, "sparse_mla_attn_dense launch");
  }
  return TIS_OK;
}

TIS_API tis_status_t cache_append(const tis_batch_t* batch, const void* rows,
                                  tis_dtype_t rows_dt, int32_t D, void* pool, tis_dtype_t pool_dt,
                                  void* pool_scale, void* stream) {
  tis_status_t st = check_batch(batch, nullptr);
  if (st != TIS_OK) return st;
  if (!rows || !pool) return fail(TIS_ERR_INVALID, "rows and pool must be set");
  if (!aligned16(rows) || !aligned16(pool))
    return fail(TIS_ERR_INVALID, "rows and pool must be 16-byte aligned");
  if (D < 16 || D > 2048 || D % 16)
    return fail(TIS_ERR_INVALID, "D must be a multiple of 16 in [16, 2048] (got %d)", D);
  if (rows_dt != TIS_F32 && rows_dt != TIS_BF16)
    return fail(TIS_ERR_UNSUPPORTED, "cache_append takes fp32 or bf16 rows");
  int fmt;
  if (pool_dt == TIS_E4M3) {
    if (!pool_scale || ((uintptr_t)pool_scale & 3))
      return fail(TIS_ERR_INVALID, "an e4m3 cache needs a 4-byte aligned pool_scale");
    fmt = 1;
  } else if (pool_dt == TIS_MXFP8) {
    if (!pool_scale) return fail(TIS_ERR_INVALID, "an MXFP8 cache needs pool_scale");
    if (D % 32) return fail(TIS_ERR_INVALID, "an MXFP8 cache needs D a multiple of 32 (got %d)", D);
    fmt = 2;
  } else if (pool_dt == TIS_BF16) {
    if (pool_scale) return fail(TIS_ERR_INVALID, "a bf16 cache takes no pool_scale");
    fmt = 0;
  } else {
    return fail(TIS_ERR_UNSUPPORTED, "cache_append writes e4m3, MXFP8 or bf16 caches");
  }
  hipError_t e = tis::launch_cache_append(dev_batch(batch), rows, rows_dt == TIS_BF16, D, pool,
                                          fmt, pool_scale, (hipStream_t)stream);
  return e == hipSuccess ? TIS_OK : hip_fail(e, "cache_append launch");
}

TIS_API tis_status_t sparse_mla_attn(const tis_batch_t* batch, const void* q, tis_dtype_t q_dt,
                                     const void* kv_pool, tis_dtype_t kv_dt,
                                     const float* kv_scale, const int32_t* topk_idx, int32_t K,
                                     int32_t H, int32_t D_qk, int32_t D_v, float softmax_scale,
                                     void* out, tis_dtype_t out_dt, float* lse, void* ws,
                                     size_t ws_bytes, void* stream) {
  HostInfo hi;
  tis_status_t st = check_batch(batch, &hi);
  if (st != TIS_OK) return st;
  AttnPath path;
  st = check_attn_args(q, q_dt, kv_pool, kv_dt, kv_scale, topk_idx, K, H, D_qk, D_v,
                       softmax_scale, out, out_dt, &path);
  if (st != TIS_OK) return st;
  const size_t need = attn_ws_bytes(batch, K, path);
  if (ws_bytes < need || (need && (!ws || !aligned16(ws))))
    return fail(TIS_ERR_INVALID, "workspace needs %zu bytes, 16-byte aligned", need);
  hipStream_t s = (hipStream_t)stream;
  const tis::DevBatch d = dev_batch(batch);
  hipError_t e;
  if (path == AttnPath::F32) {
    e = tis::launch_mla_attn_f32(d, 0, batch->T, (const float*)q, (const float*)kv_pool, topk_idx,
                                 K, H, D_qk, D_v, softmax_scale, (float*)out, lse, s);
  } else {
    const int ns = tis::attn_split_count(batch->T, K);
    float* part_o = ns > 1 ? (float*)ws : nullptr;
    float* part_ml = ns > 1 ? part_o + (size_t)batch->T * ns * 128 * 512 : nullptr;
    e = tis::launch_mla_attn(d, 0, batch->T, kv_dt == TIS_E4M3, (const uint16_t*)q,
                             (const uint8_t*)kv_pool, kv_scale, topk_idx, K, softmax_scale, ns,
                             out, out_dt == TIS_F32, lse, part_o, part_ml, s);
  }
  return e == hipSuccess ? TIS_OK : hip_fail(e, "sparse_mla_attn launch");
}
