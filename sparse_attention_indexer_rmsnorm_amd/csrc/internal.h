// Internal declarations shared by the HIP translation units of the indexer library.
// The exported C ABI is include/dsa_indexer.h; nothing here crosses it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

constexpr int kHeadDim = 128;        // index-key head dim
constexpr int kHeads = 64;           // indexer heads
constexpr int kPageKeys = 64;        // keys per cache page
constexpr int kRatio = 4;            // tokens per compressed key
constexpr int kFp8 = 0;
constexpr int kBf16 = 1;
constexpr int kFp4 = 2;
constexpr int64_t kFp8PageBytes = kPageKeys * (kHeadDim + 4);   // 8448: codes, then scales
constexpr int64_t kBf16PageBytes = kPageKeys * kHeadDim * 2;    // 16384
constexpr int kFp8ScaleOffset = kPageKeys * kHeadDim;           // 8192
constexpr int64_t kFp4PageBytes = kPageKeys * (kHeadDim / 2 + 4);   // 4352: codes, then scales
constexpr int kFp4ScaleOffset = kPageKeys * kHeadDim / 2;           // 4096

// RoPE inverse frequencies, rounded to fp32 on the host and passed by value.
struct RopeFreq {
  float f[32];
};

struct StoreArgs {
  const float* x;
  const float* gamma;
  float eps;
  const int32_t* key_idx;
  const int32_t* key_seq;   // may be null
  int64_t n_keys;
  const int32_t* page_table;
  int32_t n_seq;
  int32_t max_pages;
  uint8_t* kcache;
  int64_t n_pages_pool;
  RopeFreq rope;
};

hipError_t launch_store(const StoreArgs& a, int dtype, bool hadamard, hipStream_t stream);
hipError_t launch_rotate_q(const uint16_t* in, uint16_t* out, int64_t n_vec, hipStream_t stream);

// One launch scores rows [q_begin, q_begin + n_rows) of the query batch against key columns
// [0, n_cols).  Each wave owns one (row, chunk of chunk_keys columns) work item.
struct ScoreArgs {
  const uint16_t* q;         // [n_q, 64, 128] bf16 bit patterns
  const float* w;            // [n_q, 64]
  const uint8_t* kcache;
  int64_t n_pages_pool;
  const int32_t* page_table; // [n_seq, max_pages]
  int32_t n_seq;
  int32_t max_pages;
  const int32_t* seq_lens;   // [n_seq]
  const int32_t* cu_q;       // [n_seq + 1]
  int64_t q_begin;
  int64_t n_rows;
  int32_t n_cols;            // columns covered by the chunks
  int32_t chunk_keys;        // multiple of 32
  int32_t n_chunks;
  float* out;                // [n_rows, out_stride]
  int64_t out_stride;
  int32_t fill_invisible;    // 1: write -inf to invisible columns < n_cols
  int32_t* row_nvis;         // [n_rows] visible-key count per row, or null
  const uint8_t* q8;         // fp8 x fp8 scoring: q e4m3 codes [n_q, 64, 128], or null
  const float* q_scale;      // [n_q, 64] scales of q8
  // Histogram modes of the split kernel (set by the decode-shaped selections): workgroup
  // (row r, j) scores chunks 4j .. 4j + 3 of row r (keys [j * wg_keys, (j + 1) * wg_keys),
  // wg_keys = 4 * chunk_keys) and writes a kHistBins-bin histogram of their scores (16-bit
  // counts) to wg_hist[L * kHistBins ..], L = r * wg_per_row + j.  Then either
  //   - scores mode (wg_list null): the scores go to out like plain mode, and workgroup (r, 0)
  //     zeroes row_ctr[r] for the selection; or
  //   - bucket mode (wg_list set): nothing goes to out; the workgroup writes
  //       wg_off[L * kHistBins + b]  its number of keys in bins above b (16-bit), and
  //       wg_list[L * wg_keys + p]   its keys bucketed by bin, highest bin first: the keys of
  //                                  bin b at positions [wg_off[b], wg_off[b] + count) in no
  //                                  set order, each as (order key << 32 | key index).  When
  //                                  the workgroup holds more than sel_k keys, the bins below
  //                                  its own sel_k-th largest key are counted, not written.
  // Null wg_hist: plain mode (any four work items per workgroup, scores to out).
  uint16_t* wg_hist;
  int32_t* row_ctr;
  uint16_t* wg_off;
  uint64_t* wg_list;
  int32_t wg_per_row;
  int32_t sel_k;
};

// Selection histogram: bins are the top kHistBits bits of a score's order-preserving key, so a
// bin is the same set of values in every workgroup of a row.
constexpr int kHistBits = 11;
constexpr int kHistBins = 1 << kHistBits;
constexpr int kHistShift = 32 - kHistBits;
// Chunks of one row per histogram workgroup (one per wave), and the most keys such a workgroup
// covers (4 chunks of at most 512 keys).
constexpr int kHistChunks = 4;
constexpr int kXcds = 8;   // MI355X: 8 XCDs, each with its own L2
constexpr int kHistWgKeysMax = 2048;
// Most histogram workgroups per row (the selection keeps one entry per workgroup in LDS) and the
// longest row that the selection covers (its winner bitmap is held in LDS).
constexpr int kMaxHistWgPerRow = 64;
constexpr int kHistMaxCols = kMaxHistWgPerRow * kHistWgKeysMax;

// Order-preserving uint32 key of a score that is not a NaN: adding +0 turns -0 into +0 (fp32
// denormals are kept), then the sign selects the mask.
__device__ __forceinline__ uint32_t score_order_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return u ^ (static_cast<uint32_t>(static_cast<int32_t>(u) >> 31) | 0x80000000u);
}

hipError_t launch_score(const ScoreArgs& a, int dtype, hipStream_t stream);
// Prefill-shaped variant: 4 query rows per workgroup share LDS-staged key pages; covers all
// columns [0, n_cols) of each row (chunk_keys / n_chunks unused).
hipError_t launch_score_rows(const ScoreArgs& a, int dtype, hipStream_t stream);
// fp8 x fp8 scoring (q8 / q_scale set, fp8 cache): every batch shape, 4 rows per workgroup.
hipError_t launch_score_fp8q(const ScoreArgs& a, hipStream_t stream);
// q quantised per 128-dim vector: e4m3 codes and one fp32 scale each.
hipError_t launch_quantize_q(const uint16_t* q, uint8_t* codes, float* scales, int64_t n_vec,
                             hipStream_t stream);

struct TopkArgs {
  const float* scores;       // [n_rows, row_stride]
  int64_t row_stride;
  const int32_t* row_len;    // [n_rows] or null (= row_stride)
  int64_t n_rows;
  int32_t k;
  int32_t* out_idx;          // [n_rows * n_seg, k]
  float* out_val;            // [n_rows * n_seg, k] or null
  int32_t n_seg;             // segments per row, each selected by its own wave (1 = whole row)
  int32_t seg_len;           // elements per segment when n_seg > 1
  const int32_t* src_idx;    // [n_rows, row_stride] reported indices (< 0: padding), or null
  int32_t pad_bits;          // 1: pad short outputs with a NaN pattern (intermediate candidate
                             //    lists, read back by a later pass), 0: with -inf (final output)
};

// Largest row segment one wave selects from (64 lanes x 96 keys in registers).
constexpr int32_t kMaxSegment = 96 * 64;

struct TopkPlan {
  int passes;                // selection passes (1: each row in one wave)
  int64_t cand_elems;        // widest candidate row between passes
};

// Selection over a score matrix written by the split kernel in scores mode (few rows of moderate
// length: decode batches).  Row r is cut into n_seg segments of seg_len scores, one workgroup
// each; the workgroup sums the row's histograms, finds the bin holding the k-th largest score,
// and writes the keys of higher bins straight to their output positions (the histograms of the
// earlier segments give the offset) and the threshold bin's keys to the row's candidate list;
// the last workgroup of the row to finish refines the candidates to the exact threshold.
struct HistSelArgs {
  const float* scores;       // [n_rows, cols]
  int64_t cols;
  const int32_t* row_nvis;   // [n_rows] visible keys per row
  int64_t n_rows;
  int32_t k;
  const uint16_t* wg_hist;   // [n_rows, wg_per_row, kHistBins]
  int32_t wg_per_row;
  int32_t wg_keys;           // scores per histogram workgroup; divides seg_len
  int32_t* row_ctr;          // [n_rows], zero on entry
  int32_t n_seg;
  int32_t seg_len;           // 2048 or 4096
  uint64_t* cand;            // [n_rows, cols] (order key << 32 | index), index order
  int32_t* out_idx;          // [n_rows, k]
  float* out_val;            // [n_rows, k] or null
};

hipError_t launch_topk_hist(const HistSelArgs& a, hipStream_t stream);

// Selection from the bucketed lists the split kernel writes in bucket mode (few long rows: long-
// context decode batches), one workgroup per row: the sum of the row's histograms gives the bin
// B that holds the k-th largest score; every key of a higher bin is a winner and is read from
// the front of its list, bin B's keys are read from behind them and refined to the exact
// threshold, and a bitmap of the winners' indices gives each its output position (the output
// is sorted by index).
struct ListSelArgs {
  const uint64_t* wg_list;   // [n_rows, wg_per_row, wg_keys]
  const uint16_t* wg_hist;   // [n_rows, wg_per_row, kHistBins]
  const uint16_t* wg_off;    // [n_rows, wg_per_row, kHistBins]
  const int32_t* row_nvis;   // [n_rows] visible keys per row
  int64_t cols;              // key columns scored per row (<= kHistMaxCols)
  int64_t n_rows;
  int32_t k;
  int32_t wg_per_row;        // <= kMaxHistWgPerRow
  int32_t wg_keys;           // keys per scoring workgroup (<= kHistWgKeysMax)
  int32_t* out_idx;          // [n_rows, k]
  float* out_val;            // [n_rows, k] or null
};

hipError_t launch_topk_list(const ListSelArgs& a, hipStream_t stream);

TopkPlan topk_plan(int64_t n_rows, int64_t cols, int32_t k);
// Workspace the selection of n_rows rows of `cols` scores needs (0 for one pass).
size_t topk_workspace_bytes(int64_t n_rows, int64_t cols, int32_t k);
// Widest candidate row any batch of rows of `cols` scores can need, whatever its row count:
// topk_workspace_bytes(n, cols, k) <= 2 * (n * topk_cand_bound(cols, k) * 8 + 256) for every n.
int64_t topk_cand_bound(int64_t cols, int32_t k);
// Top-k of every row (ties to the lower index, output sorted by index, -1 / -inf padding).
hipError_t run_topk(const float* scores, int64_t row_stride, const int32_t* row_len,
                    int64_t n_rows, int32_t k, int32_t* out_idx, float* out_val, void* ws,
                    hipStream_t stream);

}  // namespace dsa
