// C ABI of the indexer library (include/dsa_indexer.h): argument validation, workspace planning
// and kernel launches.  Host code only; validation returns before any HIP call.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/dsa_indexer.h"
#include "attn.h"
#include "internal.h"

namespace {

using namespace dsa;

constexpr size_t kAlign = 256;
// Recommended workspace cap: query chunks are sized so that one chunk's head-reduced scores
// stay within this bound, whatever the batch (the 8192 x 5632 long-prefill chunk needs 185 MB).
constexpr size_t kWorkspaceCap = size_t(256) << 20;
// Key chunk per wave of the split (decode) kernel: 512 keys while the launch still has at least
// kMinWaves (row, chunk) work items (two per SIMD), else down to 256.
constexpr int64_t kMinWaves = 2048;
constexpr int32_t kMaxChunkKeys = 512;
constexpr int32_t kMinChunkKeys = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Workspaces hold 16-byte vectors and 8-byte atomics: the base must be 16-byte aligned.
bool misaligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Batches with several queries per sequence on average (prefill chunks) use the kernel whose
// workgroups share key pages between 4 query rows; decode-shaped batches (about one query per
// sequence) and small batches, where 4 rows per workgroup would leave most of the 256 CUs idle,
// split each row's keys over many waves instead.
bool prefill_shaped(int64_t n_rows, int32_t n_seq) {
  return n_rows >= 1024 && n_rows >= 4 * static_cast<int64_t>(n_seq > 0 ? n_seq : 1);
}

hipError_t score_launch(const ScoreArgs& a, int dtype, hipStream_t s) {
  if (a.q8) return launch_score_fp8q(a, s);   // fp8 x fp8: one kernel for every batch shape
  // the rows kernel stages pages unconditionally, so it needs at least one page in the pool
  return prefill_shaped(a.n_rows, a.n_seq) && a.n_pages_pool > 0
             ? launch_score_rows(a, dtype, s)
             : launch_score(a, dtype, s);
}

RopeFreq rope_table() {
  RopeFreq t;
  for (int j = 0; j < 32; ++j) t.f[j] = static_cast<float>(std::pow(10000.0, -(2.0 * j) / 64.0));
  return t;
}

int hip_status(hipError_t e) { return e == hipSuccess ? IDX_OK : IDX_EHIP; }

bool dtype_ok(int dtype) {
  return dtype == IDX_KV_FP8_E4M3 || dtype == IDX_KV_BF16 || dtype == IDX_KV_FP4_E2M1;
}

// Decode-shaped chunks (the split scoring kernel) are selected with the per-workgroup histograms
// the scoring kernel writes: its workgroups cover 4 chunks of 128, 256 or 512 keys of one row.
// Rows of at least kBucketMinCols key columns are selected from the workgroups' keys bucketed by
// bin (launch_topk_list: the selection reads little more than its winners, at the cost of a
// sort in every scoring workgroup), shorter ones from the scores in segments (launch_topk_hist:
// the scoring workgroups only count, and a selection workgroup covers seg_len scores).  Rows of
// more than kMaxHistWgPerRow such workgroups are selected in segments and passes (run_topk).
// (Measured, one box: 32 rows of 32768 keys 41.5 -> 39.0 us with the lists (fp8), 64 rows of
// 1024..5632 keys 25.3 -> 27.4 us.)
constexpr int32_t kBucketMinCols = 16384;

struct HistPlan {
  int32_t chunk_keys, n_chunks, wg_per_row, seg_len, n_seg;
  bool bucket;
};

void plan_chunks(int64_t n_rows, int32_t n_cols, int32_t* chunk_keys, int32_t* n_chunks);

HistPlan hist_plan(int64_t rows, int32_t cols) {
  HistPlan h{};
  int32_t ck, nc;
  plan_chunks(rows, cols, &ck, &nc);
  h.chunk_keys = ck >= 512 ? 512 : 256;
  // batches too small for two 256-key work items per SIMD take 128-key chunks, where the row
  // still fits the histogram selection
  const int64_t fill = static_cast<int64_t>(cols) * rows / kMinWaves;
  if (h.chunk_keys == 256 && fill < 256 &&
      (cols + 128 * kHistChunks - 1) / (128 * kHistChunks) <= kMaxHistWgPerRow)
    h.chunk_keys = 128;
  h.n_chunks = (cols + h.chunk_keys - 1) / h.chunk_keys;
  h.wg_per_row = (h.n_chunks + kHistChunks - 1) / kHistChunks;
  const int64_t segs4k = (static_cast<int64_t>(cols) + 4095) / 4096;
  h.seg_len = rows * segs4k >= 256 ? 4096 : 2048;
  h.n_seg = (cols + h.seg_len - 1) / h.seg_len;
  h.bucket = cols >= kBucketMinCols;
  return h;
}

// The selection a chunk of `rows` query rows gets: from histograms for decode-shaped chunks
// scored by the split kernel (not for fp8 x fp8 scoring, whose rows kernel serves every shape).
bool use_hist(int64_t rows, int32_t n_seq, int32_t cols, bool q8) {
  if (q8 || cols <= 0 || prefill_shaped(rows, n_seq)) return false;
  return hist_plan(rows, cols).wg_per_row <= kMaxHistWgPerRow;
}

// Workspace layout for a chunk of `rows` query rows:
//   [row_nvis int32 x rows | pad] then one of
//   [scores fp32 rows x cols | pad][selection candidates] (segments and passes);
//   [scores fp32 rows x cols | pad][histograms u16 rows x wg_per_row x kHistBins | pad]
//     [row counters int32 x rows | pad][candidates u64 rows x cols] (histograms and scores);
//   [bucketed keys u64 rows x wg_per_row x wg_keys | pad][histograms | pad][bucket starts u16,
//     like the histograms] (histograms and bucketed keys)
struct WsLayout {
  size_t nvis, scores, topk, hist, ctr, cand, list, off, total;
  bool hist_path, bucket;
};

WsLayout workspace_layout(int64_t rows, int32_t max_pages, int32_t k, int32_t n_seq, bool q8) {
  WsLayout L{};
  const size_t cols = static_cast<size_t>(max_pages) * IDX_PAGE_KEYS;
  L.nvis = 0;
  L.hist_path = use_hist(rows, n_seq, static_cast<int32_t>(cols), q8);
  const HistPlan h = L.hist_path ? hist_plan(rows, static_cast<int32_t>(cols)) : HistPlan{};
  L.bucket = L.hist_path && h.bucket;
  const size_t lists = static_cast<size_t>(rows) * h.wg_per_row;
  if (L.bucket) {
    L.list = align_up(static_cast<size_t>(rows) * sizeof(int32_t));
    L.hist = align_up(L.list + lists * kHistChunks * h.chunk_keys * 8);
    L.off = align_up(L.hist + lists * kHistBins * 2);
    L.total = L.off + lists * kHistBins * 2;
    return L;
  }
  L.scores = align_up(static_cast<size_t>(rows) * sizeof(int32_t));
  L.topk = align_up(L.scores + static_cast<size_t>(rows) * cols * sizeof(float));
  if (!L.hist_path) {
    L.total = L.topk + topk_workspace_bytes(rows, static_cast<int64_t>(cols), k);
    return L;
  }
  L.hist = L.topk;
  L.ctr = align_up(L.hist + lists * kHistBins * 2);
  L.cand = align_up(L.ctr + static_cast<size_t>(rows) * sizeof(int32_t));
  L.total = L.cand + static_cast<size_t>(rows) * cols * 8;
  return L;
}

// A bound on workspace_layout(n).total for every n <= rows, every n_seq and every selection,
// that never decreases with `rows`: the exact size is not monotone (a batch of few rows is
// selected by one workgroup per row with no candidates, more rows in segments with candidate
// buffers, decode-shaped chunks from histograms), so every row reserves the most any of them
// needs per row, and the alignment slack of each region is counted.
size_t workspace_upper(int64_t rows, int32_t max_pages, int32_t k) {
  const size_t cols = static_cast<size_t>(max_pages) * IDX_PAGE_KEYS;
  const size_t cand = static_cast<size_t>(topk_cand_bound(static_cast<int64_t>(cols), k));
  const size_t passes_row = cols * sizeof(float) + 2 * cand * 8;
  // histogram workgroups of kHistChunks chunks of 128 keys at the least; bucketed keys cover the
  // columns rounded up to one workgroup of the widest chunks
  const size_t wg_max = (cols + kHistChunks * 128 - 1) / (kHistChunks * 128);
  const size_t scores_row = cols * sizeof(float) + wg_max * kHistBins * 2 + sizeof(int32_t) +
                            cols * 8;
  const size_t bucket_row = (cols + kHistWgKeysMax) * 8 + wg_max * kHistBins * 2 * 2;
  size_t sel_row = passes_row > scores_row ? passes_row : scores_row;
  sel_row = sel_row > bucket_row ? sel_row : bucket_row;
  return static_cast<size_t>(rows) * (sizeof(int32_t) + sel_row) + 6 * kAlign;
}

// Query rows per chunk for a workspace of `bytes`: all of them if they fit, else the largest
// count whose upper bound fits, so that every chunk (the last one has fewer rows) fits too.
int64_t rows_fitting(size_t bytes, int32_t max_pages, int32_t k, int64_t n_q, int32_t n_seq,
                     bool q8) {
  if (workspace_layout(n_q, max_pages, k, n_seq, q8).total <= bytes) return n_q;
  int64_t lo = 0, hi = n_q;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo + 1) / 2;
    if (workspace_upper(mid, max_pages, k) <= bytes) lo = mid; else hi = mid - 1;
  }
  return lo;
}

void plan_chunks(int64_t n_rows, int32_t n_cols, int32_t* chunk_keys, int32_t* n_chunks) {
  const int64_t cols32 = (static_cast<int64_t>(n_cols) + 31) / 32 * 32;
  int64_t ck = static_cast<int64_t>(n_cols) * n_rows / kMinWaves / 32 * 32;
  if (ck > kMaxChunkKeys) ck = kMaxChunkKeys;
  if (ck < kMinChunkKeys) ck = kMinChunkKeys;
  if (ck > cols32) ck = cols32;
  if (ck < 32) ck = 32;
  *chunk_keys = static_cast<int32_t>(ck);
  *n_chunks = static_cast<int32_t>((cols32 + ck - 1) / ck);
}

int validate_logits_common(const void* q, const float* w, const void* kcache, int dtype,
                           int64_t n_pages_pool, const int32_t* page_table, int32_t n_seq,
                           int32_t max_pages, const int32_t* seq_lens, const int32_t* cu_q,
                           int64_t n_q, int32_t n_heads) {
  if (n_q < 0 || n_seq < 0 || max_pages < 0 || n_pages_pool < 0) return IDX_EINVAL;
  if (!dtype_ok(dtype)) return IDX_EUNSUPPORTED;
  if (n_heads != IDX_N_HEADS) return IDX_EUNSUPPORTED;
  if (n_q > INT32_MAX || static_cast<int64_t>(max_pages) * IDX_PAGE_KEYS > INT32_MAX / 2)
    return IDX_EINVAL;
  if (n_q > 0 && (!q || !w || !cu_q || (n_seq > 0 && (!seq_lens || !page_table))))
    return IDX_EINVAL;
  if (n_q > 0 && n_seq > 0 && max_pages > 0 && n_pages_pool > 0 && !kcache) return IDX_EINVAL;
  // q rows and key pages are read in 16-byte vectors
  if (n_q > 0 && (misaligned16(q) || misaligned16(kcache))) return IDX_EINVAL;
  return IDX_OK;
}

ScoreArgs score_args(const void* q, const float* w, const void* kcache, int64_t n_pages_pool,
                     const int32_t* page_table, int32_t n_seq, int32_t max_pages,
                     const int32_t* seq_lens, const int32_t* cu_q) {
  ScoreArgs s{};
  s.q = static_cast<const uint16_t*>(q);
  s.w = w;
  s.kcache = static_cast<const uint8_t*>(kcache);
  s.n_pages_pool = n_pages_pool;
  s.page_table = page_table;
  s.n_seq = n_seq;
  s.max_pages = max_pages;
  s.seq_lens = seq_lens;
  s.cu_q = cu_q;
  return s;
}

int logits_topk_impl(const void* q, const float* q_scale, const float* w, const void* kcache,
                     int dtype, int64_t n_pages_pool, const int32_t* page_table, int32_t n_seq,
                     int32_t max_pages, const int32_t* seq_lens, const int32_t* cu_q, int64_t n_q,
                     int32_t n_heads, int32_t k, int32_t* out_idx, float* out_val,
                     void* workspace, size_t workspace_bytes, void* ev_begin, void* ev_end,
                     void* stream) {
  int st = validate_logits_common(q, w, kcache, dtype, n_pages_pool, page_table, n_seq, max_pages,
                                  seq_lens, cu_q, n_q, n_heads);
  if (st != IDX_OK) return st;
  if (k < 1 || k > IDX_MAX_TOPK) return IDX_EINVAL;
  if (n_q > 0 && !out_idx) return IDX_EINVAL;
  if (n_q == 0) return IDX_OK;
  if (!workspace) return IDX_EWORKSPACE;
  if (misaligned16(workspace)) return IDX_EINVAL;
  const bool q8 = q_scale != nullptr;
  const int64_t rows_per_chunk = rows_fitting(workspace_bytes, max_pages, k, n_q, n_seq, q8);
  if (rows_per_chunk < 1) return IDX_EWORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t cols = max_pages * IDX_PAGE_KEYS;
  char* ws = static_cast<char*>(workspace);
  ScoreArgs sa = score_args(q, w, kcache, n_pages_pool, page_table, n_seq, max_pages, seq_lens,
                            cu_q);
  if (q_scale) {   // fp8 x fp8: q is codes
    sa.q = nullptr;
    sa.q8 = static_cast<const uint8_t*>(q);
    sa.q_scale = q_scale;
  }
  sa.n_cols = cols;
  sa.out_stride = cols;
  sa.fill_invisible = 0;

  for (int64_t q0 = 0; q0 < n_q; q0 += rows_per_chunk) {
    const int64_t rows = (n_q - q0 < rows_per_chunk) ? n_q - q0 : rows_per_chunk;
    const WsLayout L = workspace_layout(rows, max_pages, k, n_seq, q8);
    int32_t* nvis = reinterpret_cast<int32_t*>(ws + L.nvis);
    float* scores = L.bucket ? nullptr : reinterpret_cast<float*>(ws + L.scores);
    sa.q_begin = q0;
    sa.n_rows = rows;
    sa.out = scores;
    sa.row_nvis = nvis;
    sa.wg_hist = nullptr;
    sa.row_ctr = nullptr;
    sa.wg_off = nullptr;
    sa.wg_list = nullptr;
    sa.wg_per_row = 0;
    sa.sel_k = k;
    HistPlan hp{};
    if (L.hist_path) {
      hp = hist_plan(rows, cols);
      sa.chunk_keys = hp.chunk_keys;
      sa.n_chunks = hp.n_chunks;
      sa.wg_per_row = hp.wg_per_row;
      sa.wg_hist = reinterpret_cast<uint16_t*>(ws + L.hist);
      if (L.bucket) {
        sa.wg_list = reinterpret_cast<uint64_t*>(ws + L.list);
        sa.wg_off = reinterpret_cast<uint16_t*>(ws + L.off);
      } else {
        sa.row_ctr = reinterpret_cast<int32_t*>(ws + L.ctr);
      }
    } else if (cols > 0) {
      plan_chunks(rows, cols, &sa.chunk_keys, &sa.n_chunks);
    } else {
      sa.chunk_keys = 32;
      sa.n_chunks = 1;
    }
    if (ev_begin && q0 == 0 && hipEventRecord(static_cast<hipEvent_t>(ev_begin), s) != hipSuccess)
      return IDX_EHIP;
    if (score_launch(sa, dtype, s) != hipSuccess) return IDX_EHIP;
    if (ev_end && q0 + rows >= n_q &&
        hipEventRecord(static_cast<hipEvent_t>(ev_end), s) != hipSuccess)
      return IDX_EHIP;
    if (L.bucket) {
      ListSelArgs h{};
      h.wg_list = sa.wg_list;
      h.wg_hist = sa.wg_hist;
      h.wg_off = sa.wg_off;
      h.row_nvis = nvis;
      h.cols = cols;
      h.n_rows = rows;
      h.k = k;
      h.wg_per_row = hp.wg_per_row;
      h.wg_keys = kHistChunks * hp.chunk_keys;
      h.out_idx = out_idx + q0 * k;
      h.out_val = out_val ? out_val + q0 * k : nullptr;
      if (launch_topk_list(h, s) != hipSuccess) return IDX_EHIP;
    } else if (L.hist_path) {
      HistSelArgs h{};
      h.scores = scores;
      h.cols = cols;
      h.row_nvis = nvis;
      h.n_rows = rows;
      h.k = k;
      h.wg_hist = sa.wg_hist;
      h.wg_per_row = hp.wg_per_row;
      h.wg_keys = kHistChunks * hp.chunk_keys;
      h.row_ctr = sa.row_ctr;
      h.n_seg = hp.n_seg;
      h.seg_len = hp.seg_len;
      h.cand = reinterpret_cast<uint64_t*>(ws + L.cand);
      h.out_idx = out_idx + q0 * k;
      h.out_val = out_val ? out_val + q0 * k : nullptr;
      if (launch_topk_hist(h, s) != hipSuccess) return IDX_EHIP;
    } else if (run_topk(scores, cols > 0 ? cols : 1, nvis, rows, k, out_idx + q0 * k,
                        out_val ? out_val + q0 * k : nullptr, ws + L.topk, s) != hipSuccess) {
      return IDX_EHIP;
    }
  }
  return IDX_OK;
}

// Workspace of idx_logits_topk_noalloc: device memory that belongs to the loaded library (each
// GPU holds its own copy until the process ends), so that the call allocates nothing.  In host
// code `scratch` only names the symbol; its device address on each GPU comes from
// hipGetSymbolAddress, taken once per device with that device current and kept below.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current GPU's scratch, or null when it cannot be had.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int idx_abi_version(void) { return IDX_ABI_VERSION; }

const char* idx_status_string(int status) {
  switch (status) {
    case IDX_OK: return "ok";
    case IDX_EINVAL: return "invalid argument";
    case IDX_EUNSUPPORTED: return "unsupported configuration";
    case IDX_EWORKSPACE: return "workspace too small";
    case IDX_EHIP: return "HIP launch error";
    default: return "unknown status";
  }
}

size_t idx_page_bytes(int dtype) {
  if (dtype == IDX_KV_FP8_E4M3) return static_cast<size_t>(kFp8PageBytes);
  if (dtype == IDX_KV_BF16) return static_cast<size_t>(kBf16PageBytes);
  if (dtype == IDX_KV_FP4_E2M1) return static_cast<size_t>(kFp4PageBytes);
  return 0;
}

static int store_keys(const float* x, const float* gamma, float eps, const int32_t* key_idx,
                      const int32_t* key_seq, int64_t n_keys, const int32_t* page_table,
                      int32_t n_seq, int32_t max_pages, int dtype, void* kcache,
                      int64_t n_pages_pool, void* stream, bool hadamard) {
  if (n_keys < 0 || n_seq < 0 || max_pages < 0 || n_pages_pool < 0) return IDX_EINVAL;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return IDX_EINVAL;
  if (!dtype_ok(dtype)) return IDX_EUNSUPPORTED;
  if (n_keys == 0) return IDX_OK;
  if (!x || !gamma || !key_idx || !page_table || !kcache) return IDX_EINVAL;
  if (misaligned16(x) || misaligned16(gamma) || misaligned16(kcache)) return IDX_EINVAL;
  if (n_keys > (static_cast<int64_t>(INT32_MAX) - 255) / 8 * 8) return IDX_EINVAL;
  StoreArgs a{};
  a.x = x;
  a.gamma = gamma;
  a.eps = eps;
  a.key_idx = key_idx;
  a.key_seq = key_seq;
  a.n_keys = n_keys;
  a.page_table = page_table;
  a.n_seq = n_seq;
  a.max_pages = max_pages;
  a.kcache = static_cast<uint8_t*>(kcache);
  a.n_pages_pool = n_pages_pool;
  a.rope = rope_table();
  return hip_status(launch_store(a, dtype, hadamard, static_cast<hipStream_t>(stream)));
}

int idx_store_keys(const float* x, const float* gamma, float eps, const int32_t* key_idx,
                   const int32_t* key_seq, int64_t n_keys, const int32_t* page_table,
                   int32_t n_seq, int32_t max_pages, int dtype, void* kcache,
                   int64_t n_pages_pool, void* stream) {
  return store_keys(x, gamma, eps, key_idx, key_seq, n_keys, page_table, n_seq, max_pages, dtype,
                    kcache, n_pages_pool, stream, false);
}

int idx_store_keys_rotated(const float* x, const float* gamma, float eps, const int32_t* key_idx,
                           const int32_t* key_seq, int64_t n_keys, const int32_t* page_table,
                           int32_t n_seq, int32_t max_pages, int dtype, void* kcache,
                           int64_t n_pages_pool, void* stream) {
  return store_keys(x, gamma, eps, key_idx, key_seq, n_keys, page_table, n_seq, max_pages, dtype,
                    kcache, n_pages_pool, stream, true);
}

int idx_rotate_q(const void* q, void* out, int64_t n_vec, void* stream) {
  if (n_vec < 0) return IDX_EINVAL;
  if (n_vec == 0) return IDX_OK;
  if (!q || !out) return IDX_EINVAL;
  if (misaligned16(q) || misaligned16(out)) return IDX_EINVAL;
  if (n_vec > (static_cast<int64_t>(INT32_MAX) - 255) / 8) return IDX_EINVAL;
  return hip_status(launch_rotate_q(static_cast<const uint16_t*>(q), static_cast<uint16_t*>(out),
                                    n_vec, static_cast<hipStream_t>(stream)));
}

size_t idx_logits_topk_workspace_size(int64_t n_q, int32_t n_seq, int32_t max_pages, int32_t k) {
  if (k < 1) k = 1;
  if (max_pages < 0) max_pages = 0;
  if (n_q <= 0) return align_up(sizeof(int32_t));
  // enough for the selection either scoring path (bf16-q or fp8-q) takes for the whole batch
  const size_t a = workspace_layout(n_q, max_pages, k, n_seq, false).total;
  const size_t b = workspace_layout(n_q, max_pages, k, n_seq, true).total;
  const size_t all = a > b ? a : b;
  if (all <= kWorkspaceCap) return all;
  const int64_t cap_rows = rows_fitting(kWorkspaceCap, max_pages, k, n_q, n_seq, false);
  return workspace_upper(cap_rows < 1 ? 1 : cap_rows, max_pages, k);
}

size_t idx_logits_topk_min_workspace(int32_t n_seq, int32_t max_pages, int32_t k) {
  (void)n_seq;
  return workspace_upper(1, max_pages < 0 ? 0 : max_pages, k < 1 ? 1 : k);
}

int idx_logits_topk_plan(int64_t n_q, int32_t n_seq, int32_t max_pages, int32_t k,
                         size_t workspace_bytes, int64_t* rows_per_chunk,
                         size_t* max_chunk_bytes) {
  if (n_q < 1 || n_seq < 0 || max_pages < 0 || k < 1 || k > IDX_MAX_TOPK || !rows_per_chunk ||
      !max_chunk_bytes)
    return IDX_EINVAL;
  if (n_q > INT32_MAX || static_cast<int64_t>(max_pages) * IDX_PAGE_KEYS > INT32_MAX / 2)
    return IDX_EINVAL;
  *rows_per_chunk = 0;
  *max_chunk_bytes = 0;
  // the plan of the bf16 / fp8 / fp4-q call, and of the fp8 x fp8 one: report the larger
  size_t most = 0;
  int64_t rows_min = n_q;
  for (int v = 0; v < 2; ++v) {
    const bool q8 = v == 1;
    const int64_t rows = rows_fitting(workspace_bytes, max_pages, k, n_q, n_seq, q8);
    if (rows < 1) return IDX_EWORKSPACE;
    rows_min = rows < rows_min ? rows : rows_min;
    // every chunk has `rows` rows except the last, which has the remainder
    size_t m = workspace_layout(rows, max_pages, k, n_seq, q8).total;
    const int64_t tail = n_q % rows;
    if (tail > 0) {
      const size_t t = workspace_layout(tail, max_pages, k, n_seq, q8).total;
      m = t > m ? t : m;
    }
    most = m > most ? m : most;
  }
  *rows_per_chunk = rows_min;
  *max_chunk_bytes = most;
  return IDX_OK;
}

int idx_logits_topk(const void* q, const float* w, const void* kcache, int dtype,
                    int64_t n_pages_pool, const int32_t* page_table, int32_t n_seq,
                    int32_t max_pages, const int32_t* seq_lens, const int32_t* cu_q, int64_t n_q,
                    int32_t n_heads, int32_t k, int32_t* out_idx, float* out_val,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return logits_topk_impl(q, nullptr, w, kcache, dtype, n_pages_pool, page_table, n_seq,
                          max_pages, seq_lens, cu_q, n_q, n_heads, k, out_idx, out_val, workspace,
                          workspace_bytes, nullptr, nullptr, stream);
}

int idx_logits_topk_noalloc(const void* q, const float* w, const void* kcache, int dtype,
                            int64_t n_pages_pool, const int32_t* page_table, int32_t n_seq,
                            int32_t max_pages, const int32_t* seq_lens, const int32_t* cu_q,
                            int64_t n_q, int32_t n_heads, int32_t k, int32_t* out_idx,
                            float* out_val, void* stream) {
  // the checks the workspace entry point makes, before the scratch is looked up
  int st = validate_logits_common(q, w, kcache, dtype, n_pages_pool, page_table, n_seq, max_pages,
                                  seq_lens, cu_q, n_q, n_heads);
  if (st != IDX_OK) return st;
  if (k < 1 || k > IDX_MAX_TOPK) return IDX_EINVAL;
  if (n_q > 0 && !out_idx) return IDX_EINVAL;
  if (n_q == 0) return IDX_OK;
  if (rows_fitting(kScratchBytes, max_pages, k, n_q, n_seq, false) < 1) return IDX_EWORKSPACE;
  void* ws = scratch_on_current_device();
  if (!ws) return IDX_EHIP;
  return logits_topk_impl(q, nullptr, w, kcache, dtype, n_pages_pool, page_table, n_seq,
                          max_pages, seq_lens, cu_q, n_q, n_heads, k, out_idx, out_val, ws,
                          kScratchBytes, nullptr, nullptr, stream);
}

size_t idx_logits_topk_noalloc_scratch_bytes(void) { return kScratchBytes; }

int idx_logits_topk_timed(const void* q, const float* w, const void* kcache, int dtype,
                          int64_t n_pages_pool, const int32_t* page_table, int32_t n_seq,
                          int32_t max_pages, const int32_t* seq_lens, const int32_t* cu_q,
                          int64_t n_q, int32_t n_heads, int32_t k, int32_t* out_idx,
                          float* out_val, void* workspace, size_t workspace_bytes,
                          void* ev_score_begin, void* ev_score_end, void* stream) {
  return logits_topk_impl(q, nullptr, w, kcache, dtype, n_pages_pool, page_table, n_seq,
                          max_pages, seq_lens, cu_q, n_q, n_heads, k, out_idx, out_val, workspace,
                          workspace_bytes, ev_score_begin, ev_score_end, stream);
}

int idx_quantize_q(const void* q, void* q_codes, float* q_scales, int64_t n_vec, void* stream) {
  if (n_vec < 0) return IDX_EINVAL;
  if (n_vec == 0) return IDX_OK;
  if (!q || !q_codes || !q_scales) return IDX_EINVAL;
  if (misaligned16(q) || misaligned16(q_codes)) return IDX_EINVAL;
  if (n_vec > (static_cast<int64_t>(INT32_MAX) - 255) / 8) return IDX_EINVAL;
  return hip_status(launch_quantize_q(static_cast<const uint16_t*>(q),
                                      static_cast<uint8_t*>(q_codes), q_scales, n_vec,
                                      static_cast<hipStream_t>(stream)));
}

int idx_logits_topk_fp8q(const void* q_codes, const float* q_scales, const float* w,
                         const void* kcache, int64_t n_pages_pool, const int32_t* page_table,
                         int32_t n_seq, int32_t max_pages, const int32_t* seq_lens,
                         const int32_t* cu_q, int64_t n_q, int32_t n_heads, int32_t k,
                         int32_t* out_idx, float* out_val, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (n_q > 0 && !q_scales) return IDX_EINVAL;
  return logits_topk_impl(q_codes, n_q > 0 ? q_scales : nullptr, w, kcache, IDX_KV_FP8_E4M3,
                          n_pages_pool, page_table, n_seq, max_pages, seq_lens, cu_q, n_q,
                          n_heads, k, out_idx, out_val, workspace, workspace_bytes, nullptr,
                          nullptr, stream);
}

int idx_logits_topk_fp8q_timed(const void* q_codes, const float* q_scales, const float* w,
                               const void* kcache, int64_t n_pages_pool,
                               const int32_t* page_table, int32_t n_seq, int32_t max_pages,
                               const int32_t* seq_lens, const int32_t* cu_q, int64_t n_q,
                               int32_t n_heads, int32_t k, int32_t* out_idx, float* out_val,
                               void* workspace, size_t workspace_bytes, void* ev_score_begin,
                               void* ev_score_end, void* stream) {
  if (n_q > 0 && !q_scales) return IDX_EINVAL;
  return logits_topk_impl(q_codes, n_q > 0 ? q_scales : nullptr, w, kcache, IDX_KV_FP8_E4M3,
                          n_pages_pool, page_table, n_seq, max_pages, seq_lens, cu_q, n_q,
                          n_heads, k, out_idx, out_val, workspace, workspace_bytes,
                          ev_score_begin, ev_score_end, stream);
}

static int logits_dense_impl(const void* q, const float* q_scale, const float* w,
                             const void* kcache, int dtype, int64_t n_pages_pool,
                             const int32_t* page_table, int32_t n_seq, int32_t max_pages,
                             const int32_t* seq_lens, const int32_t* cu_q, int64_t n_q,
                             int32_t n_heads, float* out_logits, int32_t max_keys, void* stream) {
  int st = validate_logits_common(q, w, kcache, dtype, n_pages_pool, page_table, n_seq, max_pages,
                                  seq_lens, cu_q, n_q, n_heads);
  if (st != IDX_OK) return st;
  if (max_keys < 1) return IDX_EINVAL;
  if (n_q > 0 && !out_logits) return IDX_EINVAL;
  if (n_q == 0) return IDX_OK;
  ScoreArgs sa = score_args(q, w, kcache, n_pages_pool, page_table, n_seq, max_pages, seq_lens,
                            cu_q);
  if (q_scale) {   // fp8 x fp8: q is codes
    sa.q = nullptr;
    sa.q8 = static_cast<const uint8_t*>(q);
    sa.q_scale = q_scale;
  }
  sa.q_begin = 0;
  sa.n_rows = n_q;
  sa.n_cols = max_keys;
  plan_chunks(n_q, max_keys, &sa.chunk_keys, &sa.n_chunks);
  sa.out = out_logits;
  sa.out_stride = max_keys;
  sa.fill_invisible = 1;
  sa.row_nvis = nullptr;
  return hip_status(score_launch(sa, dtype, static_cast<hipStream_t>(stream)));
}

int idx_logits_dense(const void* q, const float* w, const void* kcache, int dtype,
                     int64_t n_pages_pool, const int32_t* page_table, int32_t n_seq,
                     int32_t max_pages, const int32_t* seq_lens, const int32_t* cu_q, int64_t n_q,
                     int32_t n_heads, float* out_logits, int32_t max_keys, void* stream) {
  return logits_dense_impl(q, nullptr, w, kcache, dtype, n_pages_pool, page_table, n_seq,
                           max_pages, seq_lens, cu_q, n_q, n_heads, out_logits, max_keys, stream);
}

int idx_logits_dense_fp8q(const void* q_codes, const float* q_scales, const float* w,
                          const void* kcache, int64_t n_pages_pool, const int32_t* page_table,
                          int32_t n_seq, int32_t max_pages, const int32_t* seq_lens,
                          const int32_t* cu_q, int64_t n_q, int32_t n_heads, float* out_logits,
                          int32_t max_keys, void* stream) {
  if (n_q > 0 && !q_scales) return IDX_EINVAL;
  return logits_dense_impl(q_codes, n_q > 0 ? q_scales : nullptr, w, kcache, IDX_KV_FP8_E4M3,
                           n_pages_pool, page_table, n_seq, max_pages, seq_lens, cu_q, n_q,
                           n_heads, out_logits, max_keys, stream);
}

size_t idx_topk_rows_workspace_size(int64_t n_rows, int64_t row_stride, int32_t k) {
  if (n_rows <= 0 || row_stride < 1 || k < 1) return 0;
  return topk_workspace_bytes(n_rows, row_stride, k);
}

int idx_topk_rows(const float* scores, int64_t n_rows, int64_t row_stride, const int32_t* row_len,
                  int32_t k, int32_t* out_idx, float* out_val, void* workspace,
                  size_t workspace_bytes, void* stream) {
  if (n_rows < 0 || row_stride < 1 || k < 1 || k > IDX_MAX_TOPK) return IDX_EINVAL;
  if (n_rows > INT32_MAX || row_stride > INT32_MAX) return IDX_EINVAL;
  if (n_rows == 0) return IDX_OK;
  if (!scores || !out_idx) return IDX_EINVAL;
  const size_t need = topk_workspace_bytes(n_rows, row_stride, k);
  if (need > 0 && (!workspace || workspace_bytes < need)) return IDX_EWORKSPACE;
  if (need > 0 && misaligned16(workspace)) return IDX_EINVAL;
  return hip_status(run_topk(scores, row_stride, row_len, n_rows, k, out_idx, out_val, workspace,
                             static_cast<hipStream_t>(stream)));
}

size_t idx_sparse_attn_workspace_size(int64_t n_q, int32_t n_heads, int32_t k) {
  if (n_q <= 0 || k < 1 || (n_heads != 32 && n_heads != 64 && n_heads != 128)) return 0;
  return attn_workspace_bytes(n_q, n_heads, k);
}

int idx_sparse_attn(const void* q, const void* kv, int64_t n_slots, const int32_t* kv_slot,
                    int32_t n_seq, int32_t max_keys, const int32_t* cu_q, const int32_t* idx,
                    int64_t n_q, int32_t n_heads, int32_t k, float softmax_scale, void* out,
                    float* out_lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (n_q < 0 || n_seq < 1 || max_keys < 1 || n_slots < 0 || k < 1) return IDX_EINVAL;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.0f)) return IDX_EINVAL;
  if (n_heads != 32 && n_heads != 64 && n_heads != 128) return IDX_EUNSUPPORTED;
  if (n_q == 0) return IDX_OK;
  if (!q || !kv || !kv_slot || !cu_q || !idx || !out) return IDX_EINVAL;
  if (misaligned16(q) || misaligned16(kv) || misaligned16(out)) return IDX_EINVAL;
  AttnArgs a{};
  attn_plan(n_q, n_heads, k, &a.n_split, &a.split_keys);
  if (n_q * a.n_split * 2 > INT32_MAX || n_q * n_heads > INT64_C(4) * INT32_MAX) return IDX_EINVAL;
  const size_t need = attn_workspace_bytes(n_q, n_heads, k);
  if (need > 0 && (!workspace || workspace_bytes < need)) return IDX_EWORKSPACE;
  if (need > 0 && misaligned16(workspace)) return IDX_EINVAL;
  a.q = static_cast<const uint16_t*>(q);
  a.kv = static_cast<const uint16_t*>(kv);
  a.n_slots = n_slots;
  a.kv_slot = kv_slot;
  a.n_seq = n_seq;
  a.max_keys = max_keys;
  a.cu_q = cu_q;
  a.idx = idx;
  a.n_q = n_q;
  a.n_heads = n_heads;
  a.k = k;
  a.scale_log2 = static_cast<float>(static_cast<double>(softmax_scale) * 1.4426950408889634);
  a.out = static_cast<uint16_t*>(out);
  a.lse = out_lse;
  if (a.n_split > 1) {
    const size_t parts = static_cast<size_t>(n_q) * a.n_split * n_heads;
    a.part_o = static_cast<float*>(workspace);
    a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + parts * kLatentDim * 4);
  }
  return hip_status(launch_sparse_attn(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
