// S2: indexer scores of queries against causally visible compressed keys.
//
//   logit(i, s) = sum_h w[i,h] * max(0, sum_d q[i,h,d] * k[s,d])
//
// The scores are a batched q.k product followed by ReLU and a combination over heads ("The Crash
// That Changed Direction", Assumptions and Input Knowledge Required); fp8 keys are widened exactly
// to bf16 before a bf16 product ("The Crash That Changed Direction", Experiment).  Per query, the
// product q[64 x 128] . K^T[128 x n] is a dense contraction, so it runs on the bf16 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation) with heads as the 32-row M tiles and keys as the
// 32-column N tiles.  The head-reduction epilogue is in-lane: in the 32x32 accumulator layout a lane
// holds 16 rows (heads) of one column (key), so 2 head tiles leave 32 heads per lane and a single
// cross-half exchange finishes the sum.  The per-head [q x n x H] tensor, the transient behind the
// 22K-token out-of-memory ("When the Fused Kernel Isn't Enough", Message), never exists: only the
// head-reduced fp32 logit of each (query, key) pair is written.
//
// fp8 keys: the e4m3 codes are widened to bf16 (exact: every e4m3 value is a bf16 value), and the
// per-key scale multiplies the head-reduced sum, which equals scaling inside the ReLU because the
// scale is non-negative.
//
// The K (head_dim) order inside the MFMA is a permutation that q and k share ("The Fused Kernel
// Decision", Assumptions: q and k must use the same element order): lane group g = lane / 32 of
// k-step jj holds dims 64g + 8jj .. 64g + 8jj + 7, so each lane reads 128 contiguous bytes of its
// key (bf16) or 64 contiguous code bytes (fp8).
#include "internal.h"

namespace dsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
// 16-byte moves use a native vector type: HIP's uint4 is a struct whose copies lower to memcpy,
// which keeps staging arrays from being promoted to registers.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

union Frag {
  bf16x8 v;
  u32x4 u;
  bf16x2 p[4];
};

// Read a wave-uniform int32 through the constant address space: a scalar load whose completion
// is tracked apart from the vector-memory counter (which also counts outstanding stores).  Only for
// read-only metadata at addresses that are the same in every lane.
__device__ __forceinline__ int32_t load_uniform(const int32_t* p) {
  return *reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
      reinterpret_cast<uintptr_t>(p));
}

// Raw buffer view of n floats at p (p wave-uniform).  Stores whose (vector + immediate) offset
// lies at or past the end are dropped by the hardware, so a wave can store whole tiles without
// clamping; the scalar offset is not range-checked and stays 0.  Word 3 of a gfx9-family
// descriptor selects 32-bit elements.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_view(float* p, int64_t n) {
  const uint64_t addr = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(addr));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(addr >> 32));
  void* base = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(n * 4), 0x00020000);
}

// Sequence of flattened query row i: the last b with cu_q[b] <= i (binary search), or -1 when i
// lies outside every [cu_q[b], cu_q[b+1]).
__device__ __forceinline__ int32_t seq_of_row(const int32_t* cu_q, int32_t n_seq, int64_t i) {
  int32_t lo = 0, hi = n_seq;   // find last b in [0, n_seq) with cu_q[b] <= i
  if (n_seq <= 0 || cu_q[0] > i) return -1;
  while (hi - lo > 1) {
    const int32_t mid = (lo + hi) >> 1;
    if (cu_q[mid] <= i) lo = mid; else hi = mid;
  }
  return i < cu_q[lo + 1] ? lo : -1;
}

// Sequence b of flattened query row i and its context length, for the split kernel: with at most
// 256 sequences every lane loads its share of cu_q and seq_lens at once and a ballot counts the
// sequences starting at or before i (one memory round trip instead of a dependent binary
// search); longer batches take the binary search.  b = -1 when i lies in no sequence.
__device__ __forceinline__ void row_sequence(const int32_t* cu_q, const int32_t* seq_lens,
                                             int32_t n_seq, int64_t i, int32_t* b_out,
                                             int64_t* q_len_out, int64_t* row_in_seq,
                                             int32_t* len_out) {
  if (n_seq > 256) {
    const int32_t b = seq_of_row(cu_q, n_seq, i);
    *b_out = b;
    if (b >= 0) {
      *q_len_out = cu_q[b + 1] - cu_q[b];
      *row_in_seq = i - cu_q[b];
      *len_out = seq_lens[b];
    }
    return;
  }
  const int lane = threadIdx.x & 63;
  int32_t c[4], nxt[4], len[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = lane + 64 * u;
    c[u] = e < n_seq ? cu_q[e] : INT32_MAX;
    nxt[u] = e < n_seq ? cu_q[e + 1] : 0;
    len[u] = e < n_seq ? seq_lens[e] : 0;
  }
  int32_t count = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) count += __popcll(__ballot(static_cast<int64_t>(c[u]) <= i));
  const int32_t b = count - 1;           // cu_q is non-decreasing: the last b with cu_q[b] <= i
  if (b < 0) {
    *b_out = -1;
    return;
  }
  const int src = b & 63, u_b = b >> 6;
  int32_t cb = 0, cn = 0, lb = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int32_t vc = __builtin_amdgcn_readlane(c[u], src);
    const int32_t vn = __builtin_amdgcn_readlane(nxt[u], src);
    const int32_t vl = __builtin_amdgcn_readlane(len[u], src);
    cb = u == u_b ? vc : cb;
    cn = u == u_b ? vn : cn;
    lb = u == u_b ? vl : lb;
  }
  *b_out = i < cn ? b : -1;
  *q_len_out = cn - cb;
  *row_in_seq = i - cb;
  *len_out = lb;
}

// Inclusive sum over the lanes of a wave with DPP (no LDS round trips): row_shr 1, 2, 4, 8 within
// each 16-lane row, then row_bcast 15 and 31 across rows.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_or_zero(uint32_t x) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, ROW_MASK, 0xF, false));
}
__device__ __forceinline__ uint32_t wave_add_scan(uint32_t x) {
  x += dpp_or_zero<0x111, 0xF>(x);
  x += dpp_or_zero<0x112, 0xF>(x);
  x += dpp_or_zero<0x114, 0xF>(x);
  x += dpp_or_zero<0x118, 0xF>(x);
  x += dpp_or_zero<0x142, 0xA>(x);
  x += dpp_or_zero<0x143, 0xC>(x);
  return x;
}

// ReLU of a finite float as one integer max: a set sign bit makes the pattern a negative int32,
// which max(., 0) maps to +0; non-negative floats are unchanged.  (A float max would first have
// to quieten NaNs in IEEE mode, costing a second instruction.)
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// Weighted ReLU sum over the 64 heads of one key column.  acc0 / acc1 are the two 32-head MFMA
// tiles; lane (m, g) holds heads 32*ht + 8*(rr/4) + 4*g + rr%4 of key m in acc_ht[rr].  Four
// independent fma chains keep the VALU pipeline full.  The summation order is fixed, so every
// kernel that uses this returns bit-identical logits.
__device__ __forceinline__ float head_sum(const floatx16& acc0, const floatx16& acc1,
                                          const float (&wv)[2][16]) {
  float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int rr = 0; rr < 16; ++rr)
    p[rr & 3] = fmaf(relu(acc0[rr]), wv[0][rr], p[rr & 3]);
#pragma unroll
  for (int rr = 0; rr < 16; ++rr)
    p[rr & 3] = fmaf(relu(acc1[rr]), wv[1][rr], p[rr & 3]);
  const float part = (p[0] + p[1]) + (p[2] + p[3]);
  // v_permlane32_swap with both operands = part: the first result holds the low half's partial
  // sums in both halves, the second the high half's, so their sum is the key's total in every
  // lane (one VALU op; fp32 addition is commutative, so both halves get identical bits).
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part),
                                                   false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// fp4 (e2m1) keys: like fp8, widened exactly to bf16 (every e2m1 value is a bf16 value) with
// v_cvt_scalef32_pk_bf16_fp4 at scale 1, which converts the two codes of one byte, low nibble
// first.

// Load a 32-key column block of B fragments for the split kernel: lane (m, g) reads key s (its
// column) at dims 64g.. from the pool; zeros when the key is not to be read.
template <int DT>
struct KeyBlock;

template <>
struct KeyBlock<kBf16> {
  u32x4 raw[8];
  float scale;
  // Unconditional load (the caller passes an in-range page and slot for keys it will not use, so
  // that no branch separates the loads of successive blocks).
  __device__ __forceinline__ void load_any(const uint8_t* kcache, int32_t page, int slot, int g) {
    const u32x4* src = reinterpret_cast<const u32x4*>(
        kcache + page * kBf16PageBytes + slot * (kHeadDim * 2) + 128 * g);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) raw[jj] = src[jj];
    scale = 1.0f;
  }
  __device__ __forceinline__ void load(const uint8_t* kcache, int32_t page, int slot, int g, bool ok) {
    if (ok) {
      const u32x4* src = reinterpret_cast<const u32x4*>(
          kcache + page * kBf16PageBytes + slot * (kHeadDim * 2) + 128 * g);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) raw[jj] = src[jj];
    } else {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) raw[jj] = u32x4{0u, 0u, 0u, 0u};
    }
    scale = 1.0f;
  }
  __device__ __forceinline__ void frags(Frag (&kb)[8]) const {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) kb[jj].u = raw[jj];
  }
};

template <>
struct KeyBlock<kFp8> {
  u32x4 raw[4];
  float scale;
  __device__ __forceinline__ void load_any(const uint8_t* kcache, int32_t page, int slot, int g) {
    const uint8_t* pg = kcache + page * kFp8PageBytes;
    const u32x4* src = reinterpret_cast<const u32x4*>(pg + slot * kHeadDim + 64 * g);
#pragma unroll
    for (int c = 0; c < 4; ++c) raw[c] = src[c];
    scale = *reinterpret_cast<const float*>(pg + kFp8ScaleOffset + slot * 4);
  }
  __device__ __forceinline__ void load(const uint8_t* kcache, int32_t page, int slot, int g, bool ok) {
    if (ok) {
      const uint8_t* pg = kcache + page * kFp8PageBytes;
      const u32x4* src = reinterpret_cast<const u32x4*>(pg + slot * kHeadDim + 64 * g);
#pragma unroll
      for (int c = 0; c < 4; ++c) raw[c] = src[c];
      scale = *reinterpret_cast<const float*>(pg + kFp8ScaleOffset + slot * 4);
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) raw[c] = u32x4{0u, 0u, 0u, 0u};
      scale = 0.0f;
    }
  }
  // k-step jj uses code bytes 8jj..8jj+7 of this lane's 64: words 2jj and 2jj+1.
  __device__ __forceinline__ void frags(Frag (&kb)[8]) const {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const uint32_t w0 = (jj & 1) ? raw[jj >> 1].z : raw[jj >> 1].x;
      const uint32_t w1 = (jj & 1) ? raw[jj >> 1].w : raw[jj >> 1].y;
      kb[jj].p[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
      kb[jj].p[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
      kb[jj].p[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
      kb[jj].p[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
    }
  }
};

template <>
struct KeyBlock<kFp4> {
  u32x4 raw[2];
  float scale;
  __device__ __forceinline__ void load_any(const uint8_t* kcache, int32_t page, int slot, int g) {
    const uint8_t* pg = kcache + page * kFp4PageBytes;
    const u32x4* src = reinterpret_cast<const u32x4*>(pg + slot * (kHeadDim / 2) + 32 * g);
    raw[0] = src[0];
    raw[1] = src[1];
    scale = *reinterpret_cast<const float*>(pg + kFp4ScaleOffset + slot * 4);
  }
  __device__ __forceinline__ void load(const uint8_t* kcache, int32_t page, int slot, int g, bool ok) {
    if (ok) {
      const uint8_t* pg = kcache + page * kFp4PageBytes;
      const u32x4* src = reinterpret_cast<const u32x4*>(pg + slot * (kHeadDim / 2) + 32 * g);
      raw[0] = src[0];
      raw[1] = src[1];
      scale = *reinterpret_cast<const float*>(pg + kFp4ScaleOffset + slot * 4);
    } else {
      raw[0] = u32x4{0u, 0u, 0u, 0u};
      raw[1] = u32x4{0u, 0u, 0u, 0u};
      scale = 0.0f;
    }
  }
  // k-step jj uses code bytes 4jj..4jj+3 of this lane's 32 (dims 8jj..8jj+7): word jj.
  __device__ __forceinline__ void frags(Frag (&kb)[8]) const {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const u32x4 r = raw[jj >> 2];
      const uint32_t w = (jj & 3) == 0 ? r.x : (jj & 3) == 1 ? r.y : (jj & 3) == 2 ? r.z : r.w;
      kb[jj].p[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
      kb[jj].p[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
      kb[jj].p[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
      kb[jj].p[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
    }
  }
};

// Scores of keys [c_begin, s_end) of query row i (sequence b): lane (m, g) holds key s0 + m of
// each 32-key block; in histogram mode the lanes of group 0 also count their keys' scores.
// A operand of query row i (q for two 32-head tiles, resident for the whole key loop) and the
// head weights of the accumulator rows lane (m, g) holds: row = 8 (rr / 4) + 4 g + rr % 4.
__device__ __forceinline__ void load_query(const ScoreArgs& a, int64_t i, Frag (&qa)[2][8],
                                           float (&wv)[2][16]) {
  const int lane = threadIdx.x & 63;
  const int m = lane & 31, g = lane >> 5;
  const uint16_t* qrow = a.q + i * (kHeads * kHeadDim);
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const u32x4* src = reinterpret_cast<const u32x4*>(qrow + (32 * ht + m) * kHeadDim + 64 * g);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) qa[ht][jj].u = src[jj];
  }
  const float* wrow = a.w + i * kHeads;
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) wv[ht][rr] = wrow[32 * ht + 8 * (rr >> 2) + 4 * g + (rr & 3)];
}

// Modes of the split kernel: scores to out only; scores to out and per-workgroup histograms;
// histograms and the workgroup's keys bucketed by bin (see ScoreArgs).
constexpr int kModePlain = 0;
constexpr int kModeHist = 1;
constexpr int kModeBucket = 2;

template <int DT, int MODE>
__device__ __forceinline__ void score_chunk(const ScoreArgs& a, int32_t b, int32_t c_begin,
                                            int32_t s_end, float* out_row, uint32_t* hist,
                                            float* sc, int32_t wg_begin,
                                            const Frag (&qa)[2][8], const float (&wv)[2][16]) {
  const int lane = threadIdx.x & 63;
  const int m = lane & 31;      // MFMA row (A) / column (B, D) index
  const int g = lane >> 5;      // lane group: which 64 dims of head_dim this lane feeds

  const int32_t* pt_row = a.page_table + static_cast<int64_t>(b) * a.max_pages;
  auto page_ok = [&](int32_t page) { return page >= 0 && page < a.n_pages_pool; };
  // Key block s0 .. s0+31 (32-aligned, so inside one page): lane (m, g) holds key s0 + m.  Two
  // blocks are in flight while one is multiplied (decode batches are bound by the key bytes in
  // flight); page ids (wave-uniform scalar loads) run one block further ahead.  The three block
  // buffers and page ids rotate by unrolling the loop three times: copying a register whose load
  // is still in flight would make the wave wait for every load it has outstanding.
  // Every load is issued unconditionally: page ids at a clamped in-range table index, key rows
  // that are not used (past the chunk, or on a page outside the pool) from page 0, slot 0.  A
  // branch around some loads would make the compiler's wait for one block conservative enough to
  // wait for the blocks behind it.  The scores of unused keys are never stored, and a block on an
  // invalid page scores -inf whatever its data.
  KeyBlock<DT> kb0, kb1, kb2;
  bool ok[3];
  int32_t pid[3];
  auto pg_of = [&](int32_t s0) { return load_uniform(pt_row + min(s0, s_end - 1) / kPageKeys); };
  auto load_block = [&](KeyBlock<DT>& blk, int32_t s0, int32_t page, bool& okb) {
    okb = page_ok(page);
    const bool use = okb && s0 + m < s_end;
    blk.load_any(a.kcache, use ? page : 0, use ? (s0 + m) % kPageKeys : 0, g);
  };
  // One block: score block s0 from `cur`, request block s0 + 64 into `nxt` (its page id was read
  // a block ago into pid[in]) and read the page id of block s0 + 96 into pid[out].
  auto step = [&](int32_t s0, const KeyBlock<DT>& cur, bool ok_cur, KeyBlock<DT>& nxt,
                  bool& ok_nxt, int in, int out) {
    load_block(nxt, s0 + 64, pid[in], ok_nxt);
    pid[out] = pg_of(s0 + 96);
    Frag kb[8];
    cur.frags(kb);
    floatx16 acc0 = {}, acc1 = {};
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][jj].v, kb[jj].v, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][jj].v, kb[jj].v, acc1, 0, 0, 0);
    }
    float tot = head_sum(acc0, acc1, wv);
    if constexpr (DT != kBf16) tot *= cur.scale;
    const int32_t s = s0 + m;
    const float v = ok_cur ? tot : -INFINITY;
    if (g == 0 && s < s_end) {
      if constexpr (MODE == kModeBucket) {
        sc[s - wg_begin] = v;
      } else {
        out_row[s] = v;
      }
      if constexpr (MODE != kModePlain) atomicAdd(&hist[score_order_key(v) >> kHistShift], 1u);
    }
  };
  pid[0] = pg_of(c_begin);
  pid[1] = pg_of(c_begin + 32);
  load_block(kb0, c_begin, pid[0], ok[0]);
  load_block(kb1, c_begin + 32, pid[1], ok[1]);
  pid[2] = pg_of(c_begin + 64);
  for (int32_t s0 = c_begin; s0 < s_end; s0 += 96) {
    step(s0, kb0, ok[0], kb2, ok[2], 2, 0);
    if (s0 + 32 >= s_end) break;
    step(s0 + 32, kb1, ok[1], kb0, ok[0], 0, 1);
    if (s0 + 64 >= s_end) break;
    step(s0 + 64, kb2, ok[2], kb1, ok[1], 1, 2);
  }
}

// One wave owns one (query row, chunk of chunk_keys keys) work item.  In histogram mode the four
// waves of a workgroup own consecutive chunks of one row and count their scores into a shared
// LDS histogram, which the workgroup writes out for the selection.
// q rows staged in LDS for histogram mode: 16 chunks of 16 bytes per head, each head row padded
// to 17 chunks so that the fragment reads (32 heads of one read 272 bytes apart) fall on distinct
// banks.
constexpr int kQRowChunks = kHeadDim * 2 / 16 + 1;   // 17

template <int DT, int MODE>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
  constexpr bool HIST = MODE != kModePlain;
  constexpr bool BUCKET = MODE == kModeBucket;
  __shared__ __attribute__((aligned(16))) uint32_t hist[HIST ? kHistBins : 1];
  __shared__ __attribute__((aligned(16))) u32x4 qs[HIST ? kHeads * kQRowChunks : 1];
  __shared__ float wsh[HIST ? kHeads : 1];
  __shared__ float sc[BUCKET ? kHistWgKeysMax : 1];   // the workgroup's scores, by key
  __shared__ uint32_t wsum[4];
  __shared__ uint32_t blo_sh;
  const int lane = threadIdx.x & 63;
  // the wave index is uniform within a wave; say so, so that everything derived from it
  // (row, sequence, page-table row) lives in scalar registers
  const int wid = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  int64_t r;
  int32_t chunk;
  int32_t wg_j = 0;   // histogram modes: which of its row's workgroups this is
  if constexpr (HIST) {
    r = blockIdx.x / a.wg_per_row;
    wg_j = static_cast<int32_t>(blockIdx.x % a.wg_per_row);
    chunk = wg_j * kHistChunks + wid;
  } else {
    const int64_t wave = static_cast<int64_t>(blockIdx.x) * 4 + wid;
    r = wave / a.n_chunks;
    chunk = static_cast<int32_t>(wave % a.n_chunks);
    if (r >= a.n_rows) return;
  }
  const int64_t i = a.q_begin + r;
  // q and the head weights depend on the row alone: requested first, they load while the
  // sequence lookup below makes its round trip.  In histogram mode the four waves share the row,
  // so the workgroup reads it once (each thread a quarter) and the waves take their operands
  // from LDS: every wave reading the whole row made the start of the kernel a read of 16.5 KB
  // per wave.
  Frag qa[2][8];
  float wv[2][16];
  u32x4 qv[4];
  float wt = 0.0f;
  if constexpr (HIST) {
    const u32x4* qsrc = reinterpret_cast<const u32x4*>(a.q + i * (kHeads * kHeadDim));
#pragma unroll
    for (int c = 0; c < 4; ++c) qv[c] = qsrc[threadIdx.x + 256 * c];
    if (threadIdx.x < kHeads) wt = a.w[i * kHeads + threadIdx.x];
  } else {
    load_query(a, i, qa, wv);
  }

  // Query position and visible-key count.
  int32_t b, len = 0;
  int64_t q_len = 0, row_in_seq = 0;
  row_sequence(a.cu_q, a.seq_lens, a.n_seq, i, &b, &q_len, &row_in_seq, &len);
  b = __builtin_amdgcn_readfirstlane(b);
  if constexpr (HIST) {
#pragma unroll
    for (int c = 0; c < kHistBins / 1024; ++c)
      reinterpret_cast<u32x4*>(hist)[threadIdx.x + 256 * c] = u32x4{0u, 0u, 0u, 0u};
    if (threadIdx.x == 0) blo_sh = 0u;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = threadIdx.x + 256 * c;          // chunk e of the row: head e / 16
      qs[(e >> 4) * kQRowChunks + (e & 15)] = qv[c];
    }
    if (threadIdx.x < kHeads) wsh[threadIdx.x] = wt;
    __syncthreads();
    const int m = lane & 31, g = lane >> 5;
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) qa[ht][jj].u = qs[(32 * ht + m) * kQRowChunks + 8 * g + jj];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) wv[ht][rr] = wsh[32 * ht + 8 * (rr >> 2) + 4 * g + (rr & 3)];
  }
  int64_t n_vis = 0;
  if (b >= 0) {
    const int64_t t = static_cast<int64_t>(len) - q_len + row_in_seq;
    if (t >= 0) {
      n_vis = (t + 1) / kRatio;
      const int64_t cap = static_cast<int64_t>(a.max_pages) * kPageKeys;
      n_vis = n_vis < cap ? n_vis : cap;
    }
  }
  if (a.row_nvis && chunk == 0 && lane == 0) a.row_nvis[r] = static_cast<int32_t>(n_vis);

  const int32_t c_begin = chunk * a.chunk_keys;
  const int32_t c_end = min(c_begin + a.chunk_keys, a.n_cols);
  const int32_t s_end = static_cast<int32_t>(min<int64_t>(c_end, n_vis));
  // histogram mode: keys [wg_begin, wg_begin + 4 * chunk_keys) of the row are this workgroup's
  const int32_t wg_begin = HIST ? wg_j * kHistChunks * a.chunk_keys : 0;
  float* out_row = BUCKET ? nullptr : a.out + r * a.out_stride;
  if (!HIST && a.fill_invisible) {
    for (int32_t s = max(c_begin, s_end) + lane; s < c_end; s += 64) out_row[s] = -INFINITY;
  }
  if (c_begin < s_end) {
    if (a.n_pages_pool > 0) {
      score_chunk<DT, MODE>(a, b, c_begin, s_end, out_row, hist, sc, wg_begin, qa, wv);
    } else {   // no page in the pool: every visible key scores -inf
      for (int32_t s = c_begin + lane; s < s_end; s += 64) {
        if constexpr (BUCKET) {
          sc[s - wg_begin] = -INFINITY;
        } else {
          out_row[s] = -INFINITY;
        }
        if constexpr (HIST) atomicAdd(&hist[score_order_key(-INFINITY) >> kHistShift], 1u);
      }
    }
  }

  if constexpr (MODE == kModeHist) {
    __syncthreads();
    // bins 8 t .. 8 t + 7 of thread t as 16-bit counts (at most 4 x 512 scores per workgroup)
    const u32x4 lo = reinterpret_cast<const u32x4*>(hist)[2 * threadIdx.x];
    const u32x4 hi = reinterpret_cast<const u32x4*>(hist)[2 * threadIdx.x + 1];
    const u32x4 packed = {lo.x | (lo.y << 16), lo.z | (lo.w << 16), hi.x | (hi.y << 16),
                          hi.z | (hi.w << 16)};
    reinterpret_cast<u32x4*>(a.wg_hist + static_cast<int64_t>(blockIdx.x) * kHistBins)
        [threadIdx.x] = packed;
    if (threadIdx.x == 0 && wg_j == 0) a.row_ctr[r] = 0;
  }
  if constexpr (BUCKET) {
    // The workgroup's keys, bucketed by histogram bin (a counting sort in LDS): the histogram,
    // then for every bin the number of keys in higher bins (where its bucket starts), then each
    // key to the next free place of its bucket.  The selection reads only the buckets at and
    // above the bin of the row's k-th largest key; that bin is at or above the bin of this
    // workgroup's own k-th largest key whenever the workgroup holds more than k keys (the row
    // holds those k keys too), so the keys of lower bins are never read and are not written.
    __syncthreads();
    const int tid = threadIdx.x;
    const int64_t list = r * a.wg_per_row + wg_j;
    // bins 8 t .. 8 t + 7 of thread t
    const u32x4 lo = reinterpret_cast<const u32x4*>(hist)[2 * tid];
    const u32x4 hi = reinterpret_cast<const u32x4*>(hist)[2 * tid + 1];
    const uint32_t c[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    // 16-bit counts: at most 4 x 512 keys per workgroup
    reinterpret_cast<u32x4*>(a.wg_hist + list * kHistBins)[tid] =
        u32x4{c[0] | (c[1] << 16), c[2] | (c[3] << 16), c[4] | (c[5] << 16), c[6] | (c[7] << 16)};
    uint32_t mine = 0;
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) mine += c[bb];
    const uint32_t incl = wave_add_scan(mine);
    if (lane == 63) wsum[threadIdx.x >> 6] = incl;
    __syncthreads();
    // keys above thread t's bins: those of the later lanes of its wave and of the later waves
    const int wv_id = threadIdx.x >> 6;
    uint32_t later = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), 63)) - incl;
    uint32_t total = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      total += wsum[w];
      later += w > wv_id ? wsum[w] : 0u;
    }
    uint32_t e[8];
    e[7] = later;
#pragma unroll
    for (int bb = 6; bb >= 0; --bb) e[bb] = e[bb + 1] + c[bb + 1];
    const uint32_t k = static_cast<uint32_t>(a.sel_k);
    if (total > k) {
#pragma unroll
      for (int bb = 0; bb < 8; ++bb)
        if (e[bb] < k && e[bb] + c[bb] >= k) blo_sh = 8 * tid + bb;
    }
    reinterpret_cast<u32x4*>(a.wg_off + list * kHistBins)[tid] =
        u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
    reinterpret_cast<u32x4*>(hist)[2 * tid] = u32x4{e[0], e[1], e[2], e[3]};
    reinterpret_cast<u32x4*>(hist)[2 * tid + 1] = u32x4{e[4], e[5], e[6], e[7]};
    __syncthreads();
    const uint32_t blo = blo_sh;
    const int32_t wg_keys = kHistChunks * a.chunk_keys;
    const int64_t wg_end =
        min<int64_t>(min<int64_t>(wg_begin + static_cast<int64_t>(wg_keys), a.n_cols), n_vis);
    const int32_t n_valid = wg_end > wg_begin ? static_cast<int32_t>(wg_end - wg_begin) : 0;
    uint64_t* lst = a.wg_list + list * wg_keys;
    // every score read, then every bucket place taken, then every store: no LDS round trip
    // waits on another
    constexpr int kPer = kHistWgKeysMax / 256;
    const int32_t upto = (n_valid + 255) / 256;   // groups of 256 keys the workgroup holds
    uint32_t key[kPer], slot[kPer];
    bool take[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int32_t el = tid + 256 * u;
      key[u] = 0u;
      take[u] = false;
      if (u < upto) {   // uniform
        key[u] = score_order_key(sc[el]);
        take[u] = el < n_valid && (key[u] >> kHistShift) >= blo;
      }
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      slot[u] = take[u] ? atomicAdd(&hist[key[u] >> kHistShift], 1u) : 0u;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      if (take[u] && slot[u] < static_cast<uint32_t>(wg_keys))
        lst[slot[u]] =
            (static_cast<uint64_t>(key[u]) << 32) | static_cast<uint32_t>(wg_begin + tid + 256 * u);
    }
  }
}

// One thread's share of a 64-key page staged through LDS: key kk, dims 32qq..32qq+31, i.e. 64 B
// of a bf16 row or 32 code bytes of an fp8 row (plus the key's scale, held by qq == 0).
template <int DT>
struct Stage;

template <>
struct Stage<kBf16> {
  u32x4 v[4];
  __device__ __forceinline__ void load(const uint8_t* kcache, int32_t page, int kk, int qq) {
    const u32x4* src = reinterpret_cast<const u32x4*>(
        kcache + page * kBf16PageBytes + kk * (kHeadDim * 2) + qq * 64);
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] = src[c];
  }
  __device__ __forceinline__ void commit(uint8_t* dst, float* scale_slot, int qq) const {
#pragma unroll
    for (int c = 0; c < 4; ++c) reinterpret_cast<u32x4*>(dst)[c] = v[c];
    (void)scale_slot;
    (void)qq;
  }
};

template <>
struct Stage<kFp8> {
  u32x4 v[2];
  float scale;
  __device__ __forceinline__ void load(const uint8_t* kcache, int32_t page, int kk, int qq) {
    const uint8_t* pg = kcache + page * kFp8PageBytes;
    const u32x4* src = reinterpret_cast<const u32x4*>(pg + kk * kHeadDim + qq * 32);
#pragma unroll
    for (int c = 0; c < 2; ++c) v[c] = src[c];
    scale = qq == 0 ? *reinterpret_cast<const float*>(pg + kFp8ScaleOffset + kk * 4) : 0.0f;
  }
  // 32 codes -> 32 bf16 (64 B), natural dim order
  __device__ __forceinline__ void commit(uint8_t* dst, float* scale_slot, int qq) const {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint32_t wds[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
      Frag f0, f1;
      f0.p[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wds[0], 1.0f, false);
      f0.p[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wds[0], 1.0f, true);
      f0.p[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wds[1], 1.0f, false);
      f0.p[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wds[1], 1.0f, true);
      f1.p[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wds[2], 1.0f, false);
      f1.p[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wds[2], 1.0f, true);
      f1.p[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wds[3], 1.0f, false);
      f1.p[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wds[3], 1.0f, true);
      reinterpret_cast<u32x4*>(dst)[2 * c] = f0.u;
      reinterpret_cast<u32x4*>(dst)[2 * c + 1] = f1.u;
    }
    if (qq == 0) *scale_slot = scale;
  }
};

template <>
struct Stage<kFp4> {
  u32x4 v;
  float scale;
  __device__ __forceinline__ void load(const uint8_t* kcache, int32_t page, int kk, int qq) {
    const uint8_t* pg = kcache + page * kFp4PageBytes;
    v = *reinterpret_cast<const u32x4*>(pg + kk * (kHeadDim / 2) + qq * 16);
    scale = qq == 0 ? *reinterpret_cast<const float*>(pg + kFp4ScaleOffset + kk * 4) : 0.0f;
  }
  // 32 codes (16 B) -> 32 bf16 (64 B), natural dim order
  __device__ __forceinline__ void commit(uint8_t* dst, float* scale_slot, int qq) const {
    const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      Frag f;
      f.p[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wds[c], 1.0f, 0);
      f.p[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wds[c], 1.0f, 1);
      f.p[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wds[c], 1.0f, 2);
      f.p[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wds[c], 1.0f, 3);
      reinterpret_cast<u32x4*>(dst)[c] = f.u;
    }
    if (qq == 0) *scale_slot = scale;
  }
};

// Prefill-shaped batches: a workgroup scores 4 consecutive query rows (one per wave) against
// their sequence's keys, one 64-key page at a time.  The page is staged once per workgroup into
// LDS (fp8 codes widened to bf16 while staging) and each wave reads its B fragments from there, so
// the L2 -> CU traffic is shared by 4 queries.  Rows are padded to 272 B in LDS so that the 16 B
// fragment reads of consecutive lanes (consecutive keys) fall in distinct banks.  The next page is
// fetched into registers while the current one is being scored (double-buffered LDS).
constexpr int kTileKeys = 64;
constexpr int kLdsRow = kHeadDim * 2 + 16;

template <int DT>
__global__ __launch_bounds__(256) void score_rows_kernel(ScoreArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[2][kTileKeys * kLdsRow];
  __shared__ float tscale[2][kTileKeys];
  __shared__ int32_t seg_b[4];
  __shared__ int32_t seg_nvis[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 31;
  const int g = lane >> 5;
  // rows in reverse, longest workgroups first (as in score_rows_bf16_kernel)
  const int64_t r = (static_cast<int64_t>(gridDim.x) - 1 - blockIdx.x) * 4 + wid;
  const bool row_ok = r < a.n_rows;
  const int64_t i = a.q_begin + (row_ok ? r : a.n_rows - 1);

  int32_t b = seq_of_row(a.cu_q, a.n_seq, i);
  int64_t n_vis = 0;
  if (b >= 0) {
    const int64_t q_len = a.cu_q[b + 1] - a.cu_q[b];
    const int64_t t = static_cast<int64_t>(a.seq_lens[b]) - q_len + (i - a.cu_q[b]);
    if (t >= 0) {
      n_vis = (t + 1) / kRatio;
      const int64_t cap = static_cast<int64_t>(a.max_pages) * kPageKeys;
      n_vis = n_vis < cap ? n_vis : cap;
    }
  }
  if (!row_ok) {
    b = -1;
    n_vis = 0;
  }
  const int32_t nv_own = static_cast<int32_t>(min<int64_t>(n_vis, a.n_cols));
  float* out_row = a.out + (row_ok ? r : 0) * a.out_stride;
  if (row_ok) {
    if (a.row_nvis && lane == 0) a.row_nvis[r] = static_cast<int32_t>(n_vis);
    if (a.fill_invisible)
      for (int32_t s = nv_own + lane; s < a.n_cols; s += 64) out_row[s] = -INFINITY;
  }
  if (lane == 0) {
    seg_b[wid] = nv_own > 0 ? b : -1;
    seg_nvis[wid] = nv_own;
  }

  // A operand (this wave's query, both 32-head tiles) and the head weights of its rows.
  Frag qa[2][8];
  float wv[2][16];
  if (nv_own > 0) {
    const uint16_t* qrow = a.q + i * (kHeads * kHeadDim);
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const u32x4* src = reinterpret_cast<const u32x4*>(qrow + (32 * ht + m) * kHeadDim + 64 * g);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) qa[ht][jj].u = src[jj];
    }
    const float* wrow = a.w + i * kHeads;
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) wv[ht][rr] = wrow[32 * ht + 8 * (rr >> 2) + 4 * g + (rr & 3)];
  }
  __syncthreads();

  // Staging assignment: thread -> (key kk of the page, quarter qq of its 128 dims).
  const int kk = tid >> 2;
  const int qq = tid & 3;

  for (int j = 0; j < 4; ++j) {
    const int32_t bj = seg_b[j];
    if (bj < 0) continue;
    bool seen = false;
    int32_t nmax = 0;
    for (int jj = 0; jj < 4; ++jj) {
      if (jj < j && seg_b[jj] == bj) seen = true;
      if (seg_b[jj] == bj) nmax = max(nmax, seg_nvis[jj]);
    }
    if (seen) continue;
    const bool mine = (b == bj) && nv_own > 0;
    // bj comes from LDS: make it visibly wave-uniform so that page-table reads are scalar loads.
    const int32_t bu = __builtin_amdgcn_readfirstlane(bj);
    const int32_t* pt_row = a.page_table + static_cast<int64_t>(bu) * a.max_pages;
    const int n_tiles = (nmax + kTileKeys - 1) / kTileKeys;

    // Page t (id `page`) into this thread's staging registers.  The load is unconditional so that
    // the staging registers stay registers: an invalid page id reads page 0 instead (its scores
    // are then replaced by -inf; the host never sends an empty pool here) and key slots past the
    // visible range are inside the page anyway (their columns are never stored).
    Stage<DT> st;
    bool st_ok = false;
    uint8_t* const lds_dst0 = &tile[0][kk * kLdsRow + qq * 64];
    uint8_t* const lds_dst1 = &tile[1][kk * kLdsRow + qq * 64];
    // This row's scores go out through a buffer view of its visible columns: lane (m, g) stores
    // the column 32 g + m of each page, one coalesced 256-byte store per wave and page, and the
    // hardware drops the columns past the visible range.
    const __amdgpu_buffer_rsrc_t out_view = buffer_view(out_row, mine ? nv_own : 0);

    // First column of this wave's deferred scores; -64 (no scores yet) puts every lane's store
    // out of the view's range, so the store below needs no condition.
    int32_t pend_s = -kTileKeys;
    float pend_v = 0.0f;
    // Page ids run two pages ahead of the data so that no page-table read is waited on.  Every
    // load below is unconditional (indices clamped to the last page): a conditional load into a
    // loop-carried register would be waited on at once, and with it the page loads before it.
    // (Vector loads: a scalar load would share the LDS completion counter and turn every wait
    // for a B-fragment read into a wait for the page-table read.)
    const int last = n_tiles - 1;
    // The page ids are read through a per-lane index (the same in every lane): a read the
    // compiler knows to be uniform would be moved to a scalar register, and that move waits for
    // the read (and for every load before it) on the spot.
    auto page_id = [&](int tt) {
      int idx = min(tt, last);
      asm volatile("" : "+v"(idx));
      return pt_row[idx];
    };
    int32_t pid_next = page_id(1);
    bool ok_cur = false;
    {
      const int32_t page = pt_row[0];
      st_ok = page >= 0 && page < a.n_pages_pool;
      st.load(a.kcache, st_ok ? page : 0, kk, qq);
      st.commit(lds_dst0, &tscale[0][kk], qq);
    }
    ok_cur = st_ok;
    __syncthreads();
    for (int t = 0; t < n_tiles; ++t) {
      const int buf = t & 1;
      // the next page (the last page again at the end: staged into the idle buffer, never read)
      st_ok = pid_next >= 0 && pid_next < a.n_pages_pool;
      st.load(a.kcache, st_ok ? pid_next : 0, kk, qq);
      pid_next = page_id(t + 2);
      const int32_t s_tile = t * kTileKeys;
      // Scores of the previous page go out first, so that they retire behind this page's work
      // instead of stalling the wait for the next page's loads.
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(pend_v), out_view,
                                            (pend_s + lane) * 4, 0, 0);
      pend_s = -kTileKeys;
      if (mine && s_tile < nv_own) {
        // Both 32-key halves of the page.  Keys past this row's visible count are computed but
        // not stored.
        // Four independent accumulator chains (2 key halves x 2 head tiles), interleaved per
        // k-step so that each chain's next MFMA issues three MFMAs after its previous one.
        floatx16 acc[2][2] = {};
        const u32x4* src0 = reinterpret_cast<const u32x4*>(&tile[buf][m * kLdsRow + 128 * g]);
        const u32x4* src1 =
            reinterpret_cast<const u32x4*>(&tile[buf][(32 + m) * kLdsRow + 128 * g]);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          Frag b0, b1;
          b0.u = src0[jj];
          b1.u = src1[jj];
          acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][jj].v, b0.v, acc[0][0], 0, 0, 0);
          acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][jj].v, b0.v, acc[0][1], 0, 0, 0);
          acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][jj].v, b1.v, acc[1][0], 0, 0, 0);
          acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][jj].v, b1.v, acc[1][1], 0, 0, 0);
        }
        float tot[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          tot[h] = head_sum(acc[h][0], acc[h][1], wv);
          if constexpr (DT != kBf16) tot[h] *= tscale[buf][32 * h + m];
          tot[h] = ok_cur ? tot[h] : -INFINITY;
        }
        // both lane halves hold both halves' sums: lane (m, g) keeps key 32 g + m
        pend_v = g ? tot[1] : tot[0];
        pend_s = s_tile;
      }
      st.commit(buf ? lds_dst0 : lds_dst1, &tscale[buf ^ 1][kk], qq);
      const bool ok_next = st_ok;
      __syncthreads();
      ok_cur = ok_next;
    }
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(pend_v), out_view, (pend_s + lane) * 4,
                                          0, 0);
  }
}

// bf16 keys, prefill-shaped batches: the same work split as score_rows_kernel, but the pages go
// from global memory straight into LDS (gfx950 global_load_lds_dwordx4: each lane's 16 bytes land
// at M0 + 16 * lane), so no registers hold staged data and no VALU or LDS-write work copies it.
// Three page buffers let each page be requested two pages ahead of its use.  Key rows are 256 B
// without padding; the 16-byte chunks of key row kk sit at chunk ^ (kk & 15), which keeps the
// fragment reads of every 16 consecutive lanes (16 consecutive keys) on distinct LDS banks.
// Barriers are bare s_barrier with explicit counter waits: a full __syncthreads() fence would also
// wait for the page requested two pages ahead.
typedef __attribute__((address_space(3))) void lds_void;
constexpr int kPageBytesBf16 = kTileKeys * kHeadDim * 2;   // 16384
constexpr int kBf16RowsPerGroup = 4;    // 4 waves share a page; 3 workgroups per CU

// s_waitcnt with vmcnt <= V and lgkmcnt <= L (expcnt unconstrained); gfx9 field layout: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8.
template <int V, int L>
__device__ __forceinline__ void wait_counts() {
  static_assert(V >= 0 && V < 64 && L >= 0 && L < 16, "counter range");
  __builtin_amdgcn_s_waitcnt((V & 15) | (7 << 4) | (L << 8) | ((V >> 4) << 14));
}

// readfirstlane kept after the preceding barrier (a plain builtin may be hoisted above it, to a
// point where its operand's load has not been waited for yet).
__device__ __forceinline__ int32_t uniform_after_wait(int32_t v) {
  int32_t u;
  asm volatile("v_readfirstlane_b32 %0, %1" : "=s"(u) : "v"(v));
  return u;
}

// s_waitcnt vmcnt(n) for a wave-uniform n in 0..5.
__device__ __forceinline__ void wait_vmcnt_lgkm0(int n) {
  switch (n) {
    case 0: wait_counts<0, 0>(); break;
    case 1: wait_counts<1, 0>(); break;
    case 2: wait_counts<2, 0>(); break;
    case 3: wait_counts<3, 0>(); break;
    case 4: wait_counts<4, 0>(); break;
    default: wait_counts<5, 0>(); break;
  }
}

// W waves (W query rows) per workgroup share every staged page.  A page is 16 requests of 1 KiB
// (4 key rows each); wave w issues requests w, w + W, ... (1 to 4 of them).
template <int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(3, 3)))
void score_rows_bf16_kernel(ScoreArgs a) {
  static_assert(W >= 4 && W <= 16, "4 to 16 waves");
  __shared__ __attribute__((aligned(16))) uint8_t pg0[kPageBytesBf16];
  __shared__ __attribute__((aligned(16))) uint8_t pg1[kPageBytesBf16];
  __shared__ __attribute__((aligned(16))) uint8_t pg2[kPageBytesBf16];
  __shared__ __attribute__((aligned(16))) float wsh[W][kHeads];
  __shared__ int32_t seg_b[W];
  __shared__ int32_t seg_nvis[W];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 31;
  const int g = lane >> 5;
  // Workgroups take their rows in reverse: in a causal chunk the later rows see more keys, and
  // dispatching the longest workgroups first leaves the short ones for the tail.
  const int64_t r = (static_cast<int64_t>(gridDim.x) - 1 - blockIdx.x) * W + wid;
  const bool row_ok = r < a.n_rows;
  const int64_t i = a.q_begin + (row_ok ? r : a.n_rows - 1);

  int32_t b = seq_of_row(a.cu_q, a.n_seq, i);
  int64_t n_vis = 0;
  if (b >= 0) {
    const int64_t q_len = a.cu_q[b + 1] - a.cu_q[b];
    const int64_t t = static_cast<int64_t>(a.seq_lens[b]) - q_len + (i - a.cu_q[b]);
    if (t >= 0) {
      n_vis = (t + 1) / kRatio;
      const int64_t cap = static_cast<int64_t>(a.max_pages) * kPageKeys;
      n_vis = n_vis < cap ? n_vis : cap;
    }
  }
  if (!row_ok) {
    b = -1;
    n_vis = 0;
  }
  const int32_t nv_own = static_cast<int32_t>(min<int64_t>(n_vis, a.n_cols));
  float* out_row = a.out + (row_ok ? r : 0) * a.out_stride;
  if (row_ok) {
    if (a.row_nvis && lane == 0) a.row_nvis[r] = static_cast<int32_t>(n_vis);
    if (a.fill_invisible)
      for (int32_t s = nv_own + lane; s < a.n_cols; s += 64) out_row[s] = -INFINITY;
  }
  if (lane == 0) {
    seg_b[wid] = nv_own > 0 ? b : -1;
    seg_nvis[wid] = nv_own;
  }

  // A operand (this wave's query, both 32-head tiles); the head weights wait in LDS.
  Frag qa[2][8];
  if (nv_own > 0) {
    const uint16_t* qrow = a.q + i * (kHeads * kHeadDim);
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const u32x4* src = reinterpret_cast<const u32x4*>(qrow + (32 * ht + m) * kHeadDim + 64 * g);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) qa[ht][jj].u = src[jj];
    }
    wsh[wid][lane] = a.w[i * kHeads + lane];
  }
  __syncthreads();

  // Page staging: request q (0..15) fills LDS rows 4 q .. 4 q + 3 (1 KiB); lane L of it writes
  // physical chunk L % 16 of row 4 q + L / 16, i.e. logical chunk (L % 16) ^ (row & 15) of that
  // key.  (row & 15 = 4 (q & 3) + L / 16, whose parts have disjoint bits, so the chunk is
  // (L % 16) ^ (L / 16) ^ 4 (q & 3).)
  const int n_req = 16 % W == 0 ? 16 / W : (16 - wid + W - 1) / W;   // this wave's requests
  const int dma_chunk = (lane & 15) ^ (lane >> 4);
  // Fragment reads: key row m (+32 for the second half), logical chunk 8 g + jj.
  const int frag_x = (8 * g) ^ (m & 15);
  const int frag_row = m * (kHeadDim * 2);

  for (int j = 0; j < W; ++j) {
    const int32_t bj = seg_b[j];
    if (bj < 0) continue;
    bool seen = false;
    int32_t nmax = 0;
    for (int jj = 0; jj < W; ++jj) {
      if (jj < j && seg_b[jj] == bj) seen = true;
      if (seg_b[jj] == bj) nmax = max(nmax, seg_nvis[jj]);
    }
    if (seen) continue;
    const bool mine = (b == bj) && nv_own > 0;
    const int32_t bu = __builtin_amdgcn_readfirstlane(bj);
    const int32_t* pt_row = a.page_table + static_cast<int64_t>(bu) * a.max_pages;
    const int n_tiles = (nmax + kTileKeys - 1) / kTileKeys;
    const int last = n_tiles - 1;
    const __amdgpu_buffer_rsrc_t out_view = buffer_view(out_row, mine ? nv_own : 0);

    // Page ids are read through a per-lane index (the same in every lane) so that the compiler
    // does not move them to scalar registers, which would wait for the read on the spot; each is
    // made uniform one page later, after a barrier wait has covered it.
    auto page_id = [&](int tt) {
      int idx = min(tt, last);
      asm volatile("" : "+v"(idx));
      return pt_row[idx];
    };
    auto valid = [&](int32_t pid) { return pid >= 0 && pid < a.n_pages_pool; };
    // Request one page (id pu, wave-uniform, already validated) into buffer dst: this wave's
    // n_req requests.
    auto stage = [&](uint8_t* dst, int32_t pu) {
      const uint8_t* src = a.kcache + static_cast<int64_t>(pu) * kPageBytesBf16;
#pragma unroll
      for (int c = 0; c < (16 + W - 1) / W; ++c) {
        if (c < n_req) {
          const int q = wid + W * c;
          __builtin_amdgcn_global_load_lds(
              src + (4 * q + (lane >> 4)) * (kHeadDim * 2) + 16 * (dma_chunk ^ (4 * (q & 3))),
              (lds_void*)(dst + q * (4 * kHeadDim * 2)), 16, 0, 0);
        }
      }
    };

    int32_t pend_s = -kTileKeys;   // first column of the deferred scores (-64: none)
    float pend_v = 0.0f;
    bool ok0, ok1;                 // validity of the pages of tiles t and t + 1
    int32_t pu2;                   // page id of tile t + 2, wave-uniform
    {
      const int32_t p0 = __builtin_amdgcn_readfirstlane(page_id(0));
      const int32_t p1 = __builtin_amdgcn_readfirstlane(page_id(1));
      ok0 = valid(p0);
      ok1 = valid(p1);
      stage(pg0, ok0 ? p0 : 0);
      const int32_t pid2 = page_id(2);
      stage(pg1, ok1 ? p1 : 0);
      wait_vmcnt_lgkm0(n_req);     // page 0 and pid2 are in; page 1 may still be in flight
      __builtin_amdgcn_s_barrier();
      pu2 = uniform_after_wait(pid2);
    }

    // One tile: scores of page t from buffer cur while page t + 2 streams into buffer nxt2 (last
    // read in tile t - 1, before the barrier that ended it).  The vector-memory operations of a
    // tile are, in order: the page-id read for tile t + 3, the n_req requests of page t + 2 and
    // the previous scores' store, so waiting for all but the last n_req + 1 covers that page id
    // and, issued before it, the page of tile t + 1; the page id is then made uniform (an SGPR value crossing
    // the loop's back edge needs no wait there).  Each page has two tiles to arrive.
    auto tile = [&](int t, const uint8_t* cur, uint8_t* nxt2) {
      const int32_t p2 = pu2;
      const bool ok2 = valid(p2);
      const int32_t pid3 = page_id(t + 3);
      stage(nxt2, ok2 ? p2 : 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(pend_v), out_view,
                                            (pend_s + lane) * 4, 0, 0);
      pend_s = -kTileKeys;
      const int32_t s_tile = t * kTileKeys;
      if (mine && s_tile < nv_own) {
        // an opaque copy: the eight fragment offsets are formed here, per page, instead of being
        // hoisted out of the loop as invariants (which spills them)
        int fx = frag_x;
        asm volatile("" : "+v"(fx));
        floatx16 acc[2][2] = {};
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const uint8_t* src = cur + frag_row + 16 * (fx ^ jj);
          Frag b0, b1;
          b0.u = *reinterpret_cast<const u32x4*>(src);
          b1.u = *reinterpret_cast<const u32x4*>(src + 32 * (kHeadDim * 2));
          acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][jj].v, b0.v, acc[0][0], 0, 0, 0);
          acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][jj].v, b0.v, acc[0][1], 0, 0, 0);
          acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][jj].v, b1.v, acc[1][0], 0, 0, 0);
          acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][jj].v, b1.v, acc[1][1], 0, 0, 0);
        }
        // Weighted ReLU head sum, in the same order as head_sum (bit-identical logits): per key
        // half, four fma chains over head tile 0's rows, then head tile 1's.
        float p[2][4] = {};
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
          float wv[16];
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const float4 w4 = *reinterpret_cast<const float4*>(&wsh[wid][32 * ht + 8 * q4 + 4 * g]);
            wv[4 * q4 + 0] = w4.x;
            wv[4 * q4 + 1] = w4.y;
            wv[4 * q4 + 2] = w4.z;
            wv[4 * q4 + 3] = w4.w;
          }
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr)
              p[h][rr & 3] = fmaf(relu(acc[h][ht][rr]), wv[rr], p[h][rr & 3]);
        }
        float tot[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float part = (p[h][0] + p[h][1]) + (p[h][2] + p[h][3]);
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part),
                                                           __float_as_uint(part), false, false);
          tot[h] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
          tot[h] = ok0 ? tot[h] : -INFINITY;
        }
        pend_v = g ? tot[1] : tot[0];   // lane (m, g) keeps key 32 g + m
        pend_s = s_tile;
      }
      ok0 = ok1;
      ok1 = ok2;
      wait_vmcnt_lgkm0(n_req + 1);   // page t + 1 and pid3 are in; page t + 2 stays in flight
      __builtin_amdgcn_s_barrier();
      pu2 = uniform_after_wait(pid3);
    };

    for (int t = 0; t < n_tiles; t += 3) {
      tile(t, pg0, pg2);
      if (t + 1 >= n_tiles) break;
      tile(t + 1, pg1, pg0);
      if (t + 2 >= n_tiles) break;
      tile(t + 2, pg2, pg1);
    }
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(pend_v), out_view, (pend_s + lane) * 4,
                                          0, 0);
    // the pages requested past the end must land before the buffers are reused or released
    wait_counts<0, 0>();
    __builtin_amdgcn_s_barrier();
  }
  wait_counts<0, 0>();
}

// fp8 x fp8 scoring, prefill-shaped and any other batch: q arrives quantised per (query, head)
// (e4m3 codes plus one fp32 scale) and the key codes go into v_mfma_f32_32x32x64_f8f6f4 as they
// are, at twice the bf16 matrix rate.  The q scale is folded into the head weight and the key
// scale multiplies the head-reduced sum (both are non-negative, so they commute with the ReLU).
// The work split and the page pipeline are those of score_rows_bf16_kernel with W = 4: a page
// buffer holds 64 key rows of 128 code bytes (the 16-byte chunks of row kk at chunk ^ (kk & 7))
// and then the page's 64 scales; a page is 8 requests of 1 KiB (8 rows each) plus 256 B of
// scales, each wave issuing two row requests and one scale request (4 lanes).
//   Operand layout (by probe): in the 32x32x64 fp8 MFMA, lane (m, g) holds row / column m and the
// 32 bytes of K half g, and A byte j of half g meets B byte j of half g.  Lane (m, g) therefore
// holds dims 64 c + 32 g .. 64 c + 32 g + 31 of K chunk c (c = 0, 1) for q and keys alike.
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
constexpr int kFp8PageCodes = kTileKeys * kHeadDim;              // 8192
constexpr int kFp8Buf = kFp8PageCodes + kTileKeys * 4;          // 8448: codes then scales

union Frag8 {
  i32x8 v;
  u32x4 h[2];
};

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
void score_rows_fp8q_kernel(ScoreArgs a) {
  constexpr int W = 4;
  __shared__ __attribute__((aligned(16))) uint8_t pg0[kFp8Buf];
  __shared__ __attribute__((aligned(16))) uint8_t pg1[kFp8Buf];
  __shared__ __attribute__((aligned(16))) uint8_t pg2[kFp8Buf];
  __shared__ __attribute__((aligned(16))) float wsh[W][kHeads];
  __shared__ int32_t seg_b[W];
  __shared__ int32_t seg_nvis[W];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 31;
  const int g = lane >> 5;
  // rows in reverse, longest workgroups first (as in score_rows_bf16_kernel)
  const int64_t r = (static_cast<int64_t>(gridDim.x) - 1 - blockIdx.x) * W + wid;
  const bool row_ok = r < a.n_rows;
  const int64_t i = a.q_begin + (row_ok ? r : a.n_rows - 1);

  int32_t b = seq_of_row(a.cu_q, a.n_seq, i);
  int64_t n_vis = 0;
  if (b >= 0) {
    const int64_t q_len = a.cu_q[b + 1] - a.cu_q[b];
    const int64_t t = static_cast<int64_t>(a.seq_lens[b]) - q_len + (i - a.cu_q[b]);
    if (t >= 0) {
      n_vis = (t + 1) / kRatio;
      const int64_t cap = static_cast<int64_t>(a.max_pages) * kPageKeys;
      n_vis = n_vis < cap ? n_vis : cap;
    }
  }
  if (!row_ok) {
    b = -1;
    n_vis = 0;
  }
  const int32_t nv_own = static_cast<int32_t>(min<int64_t>(n_vis, a.n_cols));
  float* out_row = a.out + (row_ok ? r : 0) * a.out_stride;
  if (row_ok) {
    if (a.row_nvis && lane == 0) a.row_nvis[r] = static_cast<int32_t>(n_vis);
    if (a.fill_invisible)
      for (int32_t s = nv_own + lane; s < a.n_cols; s += 64) out_row[s] = -INFINITY;
  }
  if (lane == 0) {
    seg_b[wid] = nv_own > 0 ? b : -1;
    seg_nvis[wid] = nv_own;
  }

  // A operand: this wave's q codes (both 32-head tiles, both K chunks); the head weights times
  // the q scales wait in LDS.
  Frag8 qa[2][2];
  if (nv_own > 0) {
    const uint8_t* qrow = a.q8 + i * (kHeads * kHeadDim);
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const u32x4* src =
            reinterpret_cast<const u32x4*>(qrow + (32 * ht + m) * kHeadDim + 64 * c + 32 * g);
        qa[ht][c].h[0] = src[0];
        qa[ht][c].h[1] = src[1];
      }
    wsh[wid][lane] = a.w[i * kHeads + lane] * a.q_scale[i * kHeads + lane];
  }
  __syncthreads();

  // Page staging: row request q (0..7) fills LDS rows 8 q .. 8 q + 7; lane L writes physical
  // chunk L % 8 of row 8 q + L / 8, i.e. logical chunk (L % 8) ^ (L / 8) of that key.  The scale
  // request of wave w copies scale bytes 64 w .. 64 w + 63 (lanes 0..3).
  constexpr int n_req = 3;
  const int dma_chunk = (lane & 7) ^ (lane >> 3);

  for (int j = 0; j < W; ++j) {
    const int32_t bj = seg_b[j];
    if (bj < 0) continue;
    bool seen = false;
    int32_t nmax = 0;
    for (int jj = 0; jj < W; ++jj) {
      if (jj < j && seg_b[jj] == bj) seen = true;
      if (seg_b[jj] == bj) nmax = max(nmax, seg_nvis[jj]);
    }
    if (seen) continue;
    const bool mine = (b == bj) && nv_own > 0;
    const int32_t bu = __builtin_amdgcn_readfirstlane(bj);
    const int32_t* pt_row = a.page_table + static_cast<int64_t>(bu) * a.max_pages;
    const int n_tiles = (nmax + kTileKeys - 1) / kTileKeys;
    const int last = n_tiles - 1;
    const __amdgpu_buffer_rsrc_t out_view = buffer_view(out_row, mine ? nv_own : 0);

    auto page_id = [&](int tt) {
      int idx = min(tt, last);
      asm volatile("" : "+v"(idx));
      return pt_row[idx];
    };
    auto valid = [&](int32_t pid) { return pid >= 0 && pid < a.n_pages_pool; };
    auto stage = [&](uint8_t* dst, int32_t pu) {
      if (a.n_pages_pool <= 0) return;   // no page to read (every key scores -inf)
      const uint8_t* src = a.kcache + static_cast<int64_t>(pu) * kFp8PageBytes;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int q = wid + W * c;
        __builtin_amdgcn_global_load_lds(src + (8 * q + (lane >> 3)) * kHeadDim + 16 * dma_chunk,
                                         (lds_void*)(dst + q * 1024), 16, 0, 0);
      }
      if (lane < 4)
        __builtin_amdgcn_global_load_lds(src + kFp8ScaleOffset + 64 * wid + 16 * lane,
                                         (lds_void*)(dst + kFp8PageCodes + 64 * wid), 16, 0, 0);
    };

    int32_t pend_s = -kTileKeys;
    float pend_v = 0.0f;
    bool ok0, ok1;
    int32_t pu2;
    {
      const int32_t p0 = __builtin_amdgcn_readfirstlane(page_id(0));
      const int32_t p1 = __builtin_amdgcn_readfirstlane(page_id(1));
      ok0 = valid(p0);
      ok1 = valid(p1);
      stage(pg0, ok0 ? p0 : 0);
      const int32_t pid2 = page_id(2);
      stage(pg1, ok1 ? p1 : 0);
      wait_vmcnt_lgkm0(n_req);
      __builtin_amdgcn_s_barrier();
      pu2 = uniform_after_wait(pid2);
    }

    auto tile = [&](int t, const uint8_t* cur, uint8_t* nxt2) {
      const int32_t p2 = pu2;
      const bool ok2 = valid(p2);
      const int32_t pid3 = page_id(t + 3);
      stage(nxt2, ok2 ? p2 : 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(pend_v), out_view,
                                            (pend_s + lane) * 4, 0, 0);
      pend_s = -kTileKeys;
      const int32_t s_tile = t * kTileKeys;
      if (mine && s_tile < nv_own) {
        int mx = m & 7;                     // opaque: formed here, per page
        asm volatile("" : "+v"(mx));
        floatx16 acc[2][2] = {};
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          Frag8 kf[2];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const uint8_t* row = cur + (32 * kb + m) * kHeadDim;
            kf[kb].h[0] = *reinterpret_cast<const u32x4*>(row + 16 * ((4 * c + 2 * g) ^ mx));
            kf[kb].h[1] = *reinterpret_cast<const u32x4*>(row + 16 * ((4 * c + 2 * g + 1) ^ mx));
          }
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int ht = 0; ht < 2; ++ht)
              acc[kb][ht] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  qa[ht][c].v, kf[kb].v, acc[kb][ht], 0, 0, 0, 0, 0, 0);
        }
        float p[2][4] = {};
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
          float wv[16];
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const float4 w4 = *reinterpret_cast<const float4*>(&wsh[wid][32 * ht + 8 * q4 + 4 * g]);
            wv[4 * q4 + 0] = w4.x;
            wv[4 * q4 + 1] = w4.y;
            wv[4 * q4 + 2] = w4.z;
            wv[4 * q4 + 3] = w4.w;
          }
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr)
              p[h][rr & 3] = fmaf(relu(acc[h][ht][rr]), wv[rr], p[h][rr & 3]);
        }
        float tot[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float part = (p[h][0] + p[h][1]) + (p[h][2] + p[h][3]);
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part),
                                                           __float_as_uint(part), false, false);
          tot[h] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        }
        // lane (m, g) keeps key 32 g + m, times that key's scale
        const float kscale = *reinterpret_cast<const float*>(cur + kFp8PageCodes + 4 * lane);
        const float v = (g ? tot[1] : tot[0]) * kscale;
        pend_v = ok0 ? v : -INFINITY;
        pend_s = s_tile;
      }
      ok0 = ok1;
      ok1 = ok2;
      wait_vmcnt_lgkm0(n_req + 1);
      __builtin_amdgcn_s_barrier();
      pu2 = uniform_after_wait(pid3);
    };

    for (int t = 0; t < n_tiles; t += 3) {
      tile(t, pg0, pg2);
      if (t + 1 >= n_tiles) break;
      tile(t + 1, pg1, pg0);
      if (t + 2 >= n_tiles) break;
      tile(t + 2, pg2, pg1);
    }
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(pend_v), out_view, (pend_s + lane) * 4,
                                          0, 0);
    wait_counts<0, 0>();
    __builtin_amdgcn_s_barrier();
  }
  wait_counts<0, 0>();
}

}  // namespace

hipError_t launch_score_rows(const ScoreArgs& a, int dtype, hipStream_t stream) {
  if (a.n_rows <= 0) return hipSuccess;
  if (dtype == kBf16) {
    const int64_t groups = (a.n_rows + kBf16RowsPerGroup - 1) / kBf16RowsPerGroup;
    hipLaunchKernelGGL(score_rows_bf16_kernel<kBf16RowsPerGroup>, dim3(static_cast<uint32_t>(groups)),
                       dim3(64 * kBf16RowsPerGroup), 0, stream, a);
    return hipGetLastError();
  }
  const int64_t blocks = (a.n_rows + 3) / 4;
  if (dtype == kFp4)
    hipLaunchKernelGGL(score_rows_kernel<kFp4>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                       stream, a);
  else
    hipLaunchKernelGGL(score_rows_kernel<kFp8>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                       stream, a);
  return hipGetLastError();
}

hipError_t launch_score_fp8q(const ScoreArgs& a, hipStream_t stream) {
  if (a.n_rows <= 0) return hipSuccess;
  const int64_t groups = (a.n_rows + 3) / 4;
  hipLaunchKernelGGL(score_rows_fp8q_kernel, dim3(static_cast<uint32_t>(groups)), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

namespace {

template <int MODE>
void launch_score_mode(const ScoreArgs& a, int dtype, dim3 grid, hipStream_t stream) {
  const dim3 block(256);
  if (dtype == kBf16)
    hipLaunchKernelGGL((score_kernel<kBf16, MODE>), grid, block, 0, stream, a);
  else if (dtype == kFp4)
    hipLaunchKernelGGL((score_kernel<kFp4, MODE>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((score_kernel<kFp8, MODE>), grid, block, 0, stream, a);
}

}  // namespace

hipError_t launch_score(const ScoreArgs& a, int dtype, hipStream_t stream) {
  int64_t blocks;
  const bool bucket = a.wg_hist && a.wg_list;
  if (a.wg_hist) {
    // a histogram workgroup covers 4 chunks of one row; in bucket mode its scores and bucket
    // starts live in LDS arrays of kHistWgKeysMax keys
    if (a.chunk_keys <= 0 || kHistChunks * a.chunk_keys > kHistWgKeysMax ||
        a.wg_per_row <= 0 ||
        static_cast<int64_t>(a.wg_per_row) * kHistChunks * a.chunk_keys < a.n_cols)
      return hipErrorInvalidValue;
    if (bucket ? (!a.wg_off || a.sel_k < 1) : (!a.out || !a.row_ctr)) return hipErrorInvalidValue;
    blocks = a.n_rows * a.wg_per_row;
  } else {
    const int64_t waves = a.n_rows * a.n_chunks;
    blocks = (waves + 3) / 4;
  }
  if (blocks <= 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>(blocks));
  if (bucket)
    launch_score_mode<kModeBucket>(a, dtype, grid, stream);
  else if (a.wg_hist)
    launch_score_mode<kModeHist>(a, dtype, grid, stream);
  else
    launch_score_mode<kModePlain>(a, dtype, grid, stream);
  return hipGetLastError();
}

}  // namespace dsa
