// S3: per-row top-k selection (k = 512 or 1024 in the DSA indexer; "The Crash That Changed
// Direction", Context and Pivot).
//
// One workgroup per row.  Scores become order-preserving uint32 keys (-0 folded onto +0), cached in
// LDS when the row fits (up to 32768 keys = 128 KiB of the 160 KiB LDS).  A three-pass radix select
// (11 + 11 + 10 bits, LDS histograms) finds the k-th largest key T and how many keys equal to T
// belong to the answer.  A final pass compacts, in increasing index order, every key > T and the
// lowest-indexed keys == T, with workgroup prefix sums, so the output is unique and deterministic:
// ties go to the lower index, the row comes out sorted by index.
#include "internal.h"

namespace dsa {
namespace {

constexpr int kCacheCap = 32768;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;                          // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the workgroup; *total receives the sum.  Every thread must call it.
template <int BLOCK>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* total, uint32_t* wave_tot) {
  constexpr int kWaves = BLOCK / 64;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wave_tot[wid] = x;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t t = wave_tot[w];
    base += (w < wid) ? t : 0u;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// Number of lanes below this one whose bit is set in `mask` (wave64).
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

template <int BLOCK>
__global__ __launch_bounds__(BLOCK) void topk_kernel(TopkArgs a, int32_t cache_cap) {
  constexpr int kWaves = BLOCK / 64;
  extern __shared__ uint32_t row_cache[];
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t wave_tot[kWaves];
  __shared__ uint32_t wave_cnt[2][kWaves];
  __shared__ uint32_t found[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int64_t r = blockIdx.x;
  int64_t n = a.row_len ? static_cast<int64_t>(a.row_len[r]) : a.row_stride;
  n = n < 0 ? 0 : (n > a.row_stride ? a.row_stride : n);
  const int32_t k = a.k;
  const float* row = a.scores + r * a.row_stride;
  int32_t* oi = a.out_idx + r * k;
  float* ov = a.out_val ? a.out_val + r * k : nullptr;

  if (n <= k) {
    for (int32_t e = tid; e < k; e += BLOCK) {
      oi[e] = e < n ? e : -1;
      if (ov) ov[e] = e < n ? row[e] : -INFINITY;
    }
    return;
  }

  for (int d = tid; d < 2048; d += BLOCK) hist[d] = 0;
  if (tid == 0) {
    found[0] = 0;
    found[1] = 0;
  }
  __syncthreads();

  // Pass 1 fused with the load: order-preserving keys into the LDS cache (when the row fits) and
  // a histogram of their top 11 bits.  Rows whose start is 16 B aligned are read as float4.
  const bool cached = n <= cache_cap;
  const bool vec = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
  const int64_t n4 = vec ? (n >> 2) : 0;
  for (int64_t e4 = tid; e4 < n4; e4 += BLOCK) {
    const float4 v = reinterpret_cast<const float4*>(row)[e4];
    const uint32_t u0 = order_key(v.x), u1 = order_key(v.y), u2 = order_key(v.z),
                   u3 = order_key(v.w);
    if (cached) {   // the dynamic LDS base is only 4 B aligned: plain 32-bit stores
      row_cache[4 * e4] = u0;
      row_cache[4 * e4 + 1] = u1;
      row_cache[4 * e4 + 2] = u2;
      row_cache[4 * e4 + 3] = u3;
    }
    atomicAdd(&hist[u0 >> 21], 1u);
    atomicAdd(&hist[u1 >> 21], 1u);
    atomicAdd(&hist[u2 >> 21], 1u);
    atomicAdd(&hist[u3 >> 21], 1u);
  }
  for (int64_t e = 4 * n4 + tid; e < n; e += BLOCK) {
    const uint32_t u = order_key(row[e]);
    if (cached) row_cache[e] = u;
    atomicAdd(&hist[u >> 21], 1u);
  }
  __syncthreads();

  uint32_t prefix = 0, k_rem = static_cast<uint32_t>(k);
  int prefix_bits = 0;
  for (int pass = 0; pass < 3; ++pass) {
    const int bits = pass < 2 ? 11 : 10;
    const int shift = 32 - prefix_bits - bits;
    const int nb = 1 << bits;
    if (pass > 0) {
      for (int d = tid; d < nb; d += BLOCK) hist[d] = 0;
      __syncthreads();
      for (int64_t e = tid; e < n; e += BLOCK) {
        const uint32_t u = cached ? row_cache[e] : order_key(row[e]);
        if ((u >> (32 - prefix_bits)) == prefix) atomicAdd(&hist[(u >> shift) & (nb - 1)], 1u);
      }
      __syncthreads();
    }
    // Digit of the k_rem-th largest: thread t owns `per` digits, descending from nb-1-t*per.
    const int per = nb / BLOCK > 0 ? nb / BLOCK : 1;
    const int first = tid * per;
    uint32_t local = 0;
    if (first < nb)
      for (int p = 0; p < per; ++p) local += hist[nb - 1 - (first + p)];
    uint32_t total;
    uint32_t run = block_excl_scan<BLOCK>(local, &total, wave_tot);
    if (first < nb) {
      for (int p = 0; p < per; ++p) {
        const int d = nb - 1 - (first + p);
        const uint32_t c = hist[d];
        if (run < k_rem && run + c >= k_rem) {
          found[0] = static_cast<uint32_t>(d);
          found[1] = run;
        }
        run += c;
      }
    }
    __syncthreads();
    prefix = (prefix << bits) | found[0];
    prefix_bits += bits;
    k_rem -= found[1];
    __syncthreads();
  }
  const uint32_t T = prefix;
  const uint32_t n_gt = static_cast<uint32_t>(k) - k_rem;

  // Compaction in index order.  A key > T goes to (#keys > T before it) + (#selected keys == T
  // before it); a key == T is selected while fewer than k_rem equal keys precede it.  Per chunk,
  // wave ballots give the in-wave counts and one LDS exchange the cross-wave ones.
  uint32_t gt_seen = 0, eq_seen = 0;
  int par = 0;
  for (int64_t c0 = 0; c0 < n; c0 += BLOCK) {
    const int64_t e = c0 + tid;
    const uint32_t u = e < n ? (cached ? row_cache[e] : order_key(row[e])) : 0u;
    const bool gt = e < n && u > T;
    const bool eq = e < n && u == T;
    const uint64_t mg = __ballot(gt);
    const uint64_t me = __ballot(eq);
    if (lane == 0)
      wave_cnt[par][wid] = (static_cast<uint32_t>(__popcll(mg)) << 16) |
                           static_cast<uint32_t>(__popcll(me));
    __syncthreads();
    uint32_t bg = 0, be = 0, tg = 0, te = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t v = wave_cnt[par][w];
      if (w < wid) {
        bg += v >> 16;
        be += v & 0xFFFFu;
      }
      tg += v >> 16;
      te += v & 0xFFFFu;
    }
    const uint32_t gpre = gt_seen + bg + lanes_below(mg);
    const uint32_t epre = eq_seen + be + lanes_below(me);
    uint32_t pos = 0xFFFFFFFFu;
    if (gt) pos = gpre + (epre < k_rem ? epre : k_rem);
    else if (eq && epre < k_rem) pos = gpre + epre;
    if (pos < static_cast<uint32_t>(k)) {
      oi[pos] = static_cast<int32_t>(e);
      if (ov) ov[pos] = row[e];
    }
    gt_seen += tg;
    eq_seen += te;
    par ^= 1;
    if (gt_seen >= n_gt && eq_seen >= k_rem) break;
  }
}

template <int BLOCK>
hipError_t launch_topk_block(const TopkArgs& a, int32_t cache_cap, hipStream_t stream) {
  const size_t lds = static_cast<size_t>(cache_cap) * sizeof(uint32_t);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_kernel<BLOCK>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       kCacheCap * static_cast<int>(sizeof(uint32_t)));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(topk_kernel<BLOCK>, dim3(static_cast<uint32_t>(a.n_rows)), dim3(BLOCK), lds,
                     stream, a, cache_cap);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  if (a.n_rows <= 0) return hipSuccess;
  int32_t cache_cap = a.max_row_len < kCacheCap ? a.max_row_len : kCacheCap;
  if (cache_cap < 0) cache_cap = 0;
  if (a.max_row_len >= 16384) return launch_topk_block<1024>(a, cache_cap, stream);
  return launch_topk_block<256>(a, cache_cap, stream);
}

}  // namespace dsa
