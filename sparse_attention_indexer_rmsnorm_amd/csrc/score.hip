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

union Frag {
  bf16x8 v;
  uint4 u;
  bf16x2 p[4];
};

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

template <int DT>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t r = wave / a.n_chunks;
  const int32_t chunk = static_cast<int32_t>(wave % a.n_chunks);
  if (r >= a.n_rows) return;
  const int64_t i = a.q_begin + r;

  // Query position and visible-key count.
  const int32_t b = seq_of_row(a.cu_q, a.n_seq, i);
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
  if (a.row_nvis && chunk == 0 && lane == 0) a.row_nvis[r] = static_cast<int32_t>(n_vis);

  const int32_t c_begin = chunk * a.chunk_keys;
  const int32_t c_end = min(c_begin + a.chunk_keys, a.n_cols);
  const int32_t s_end = static_cast<int32_t>(min<int64_t>(c_end, n_vis));
  float* out_row = a.out + r * a.out_stride;
  if (a.fill_invisible) {
    for (int32_t s = max(c_begin, s_end) + lane; s < c_end; s += 64) out_row[s] = -INFINITY;
  }
  if (c_begin >= s_end) return;

  const int m = lane & 31;      // MFMA row (A) / column (B, D) index
  const int g = lane >> 5;      // lane group: which 64 dims of head_dim this lane feeds

  // A operand: q[i] for two 32-head tiles, resident for the whole key loop.
  const uint16_t* qrow = a.q + i * (kHeads * kHeadDim);
  Frag qa[2][8];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const uint4* src = reinterpret_cast<const uint4*>(qrow + (32 * ht + m) * kHeadDim + 64 * g);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) qa[ht][jj].u = src[jj];
  }
  // Head weights of the accumulator rows this lane holds: row = 8*(rr/4) + 4*g + rr%4.
  float wv[2][16];
  const float* wrow = a.w + i * kHeads;
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) wv[ht][rr] = wrow[32 * ht + 8 * (rr >> 2) + 4 * g + (rr & 3)];

  const int32_t* pt_row = a.page_table + static_cast<int64_t>(b) * a.max_pages;

  for (int32_t s0 = c_begin; s0 < s_end; s0 += 32) {
    const int32_t s = s0 + m;
    const bool valid = s < s_end;
    int32_t page = valid ? pt_row[s / kPageKeys] : -1;
    const bool ok = valid && page >= 0 && page < a.n_pages_pool;
    const int slot = s % kPageKeys;

    Frag kb[8];
    float kscale = 1.0f;
    if constexpr (DT == kBf16) {
      if (ok) {
        const uint4* src = reinterpret_cast<const uint4*>(
            a.kcache + page * kBf16PageBytes + slot * (kHeadDim * 2) + 128 * g);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) kb[jj].u = src[jj];
      } else {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) kb[jj].u = make_uint4(0, 0, 0, 0);
      }
    } else {
      uint4 raw[4];
      if (ok) {
        const uint8_t* pg = a.kcache + page * kFp8PageBytes;
        const uint4* src = reinterpret_cast<const uint4*>(pg + slot * kHeadDim + 64 * g);
#pragma unroll
        for (int c = 0; c < 4; ++c) raw[c] = src[c];
        kscale = *reinterpret_cast<const float*>(pg + kFp8ScaleOffset + slot * 4);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) raw[c] = make_uint4(0, 0, 0, 0);
      }
      // k-step jj uses code bytes 8jj..8jj+7 of this lane's 64: words 2jj and 2jj+1.
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

    floatx16 acc0 = {}, acc1 = {};
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][jj].v, kb[jj].v, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][jj].v, kb[jj].v, acc1, 0, 0, 0);
    }
    float part = 0.0f;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) part += wv[0][rr] * fmaxf(acc0[rr], 0.0f);
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) part += wv[1][rr] * fmaxf(acc1[rr], 0.0f);
    float tot = part + __shfl_xor(part, 32, 64);
    if constexpr (DT == kFp8) tot *= kscale;
    if (g == 0 && valid) out_row[s] = ok ? tot : -INFINITY;
  }
}

}  // namespace

hipError_t launch_score(const ScoreArgs& a, int dtype, hipStream_t stream) {
  const int64_t waves = a.n_rows * a.n_chunks;
  if (waves <= 0) return hipSuccess;
  const int64_t blocks = (waves + 3) / 4;
  if (dtype == kBf16)
    hipLaunchKernelGGL(score_kernel<kBf16>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                       stream, a);
  else
    hipLaunchKernelGGL(score_kernel<kFp8>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                       stream, a);
  return hipGetLastError();
}

}  // namespace dsa
