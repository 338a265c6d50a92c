// S3: per-row top-k selection (k = 512 or 1024 in the DSA indexer; "The Crash That Changed
// Direction", Context and Pivot).
//
// One wave selects the top-k of one row, or of one segment of a row.  Rows longer than one wave
// can hold (64 lanes x up to 96 keys in registers), and long rows in batches with few rows (decode
// batches, where one wave per row would leave most of the 256 CUs idle), are cut into segments
// whose local top-k are selected in parallel; further passes select among the segments'
// candidates until one segment remains.  A segment's top-k contains every row winner that lies in
// it, so the result is exact, and candidate lists keep index order, so ties still go to the lower
// index.
//
// Within a wave (no workgroup barriers anywhere):
//   1. the segment's scores become order-preserving uint32 keys (-0 folded onto +0) held in
//      registers, lane-strided (element e = 64 j + lane), all loads in flight together;
//   2. a 256-bin histogram (wave-private LDS) of the top 8 key bits -- sign and exponent, one
//      bit-extract and one LDS add per key -- gives the digit D holding the k-th largest key;
//      every key in a higher digit is selected;
//   3. the keys of digit D (a small fraction of the row) are gathered into LDS by ballot
//      compaction, and three more 8-bit passes over them alone yield the k-th largest key T and
//      how many keys equal to T to take (when digit D is too full for LDS, the passes filter the
//      registers instead);
//   4. one pass compacts, in increasing index order, every key > T and the lowest-indexed keys
//      == T, with ballots, writing the winners from registers: the output is unique and
//      deterministic, ties to the lower index, each row sorted by index (values are returned
//      from the keys, so a -0 score comes back as +0).
#include "internal.h"

namespace dsa {
namespace {

constexpr int kWaveCand = 2048;
constexpr int kMaxTopk = 2048;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  u = (u << 1) == 0u ? 0u : u;                         // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Value bits of a padding entry in an intermediate candidate list: a NaN pattern whose order key
// is 0, below every real key (-inf's included).  Scores are never NaN.
constexpr uint32_t kPadBits = 0xFFFFFFFFu;

__device__ __forceinline__ float key_value(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Hide a value from the optimiser (emits nothing): per-key values derived in one pass are then
// recomputed in the next instead of being kept live, which would triple the registers per key.
template <int N>
__device__ __forceinline__ void launder(uint32_t (&v)[N]) {
#pragma unroll
  for (int j = 0; j < N; ++j) asm volatile("" : "+v"(v[j]));
}

// Number of lanes below this one whose bit is set in `mask` (wave64).
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t v, int lane) {
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x - v;
}

// Among nb bins (nb a multiple of 64), the descending digit holding the rank-`want` largest entry
// and the number of entries in higher digits.  Lane l owns digits nb-1-l*per .. nb-per-l*per.
__device__ __forceinline__ void wave_find_digit(const uint32_t* hist, int nb, uint32_t want,
                                                int lane, uint32_t* digit, uint32_t* above) {
  const int per = nb / 64;
  uint32_t local = 0;
  for (int p = 0; p < per; ++p) local += hist[nb - 1 - (lane * per + p)];
  uint32_t run = wave_excl_scan(local, lane);
  uint32_t d_found = 0, a_found = 0;
  bool hit = false;
  for (int p = 0; p < per; ++p) {
    const int d = nb - 1 - (lane * per + p);
    const uint32_t c = hist[d];
    if (!hit && run < want && run + c >= want) {
      hit = true;
      d_found = static_cast<uint32_t>(d);
      a_found = run;
    }
    run += c;
  }
  const uint64_t m = __ballot(hit);
  const int src = m ? __builtin_ctzll(m) : 0;
  *digit = __shfl(d_found, src, 64);
  *above = __shfl(a_found, src, 64);
}

// Exact select within top digit d0: the k_rem-th largest key T among the keys v[0..N) of every
// lane for which take(j) holds (all of them have top byte d0), and how many keys equal to T belong
// to the top k_rem.  Three passes of 8-bit digits.
template <int N, typename Take>
__device__ __forceinline__ void wave_radix_select(const uint32_t (&v)[N], Take take, uint32_t d0,
                                                  uint32_t k_rem, uint32_t* hist, int lane,
                                                  uint32_t* T_out, uint32_t* eq_take) {
  uint32_t prefix = d0;
#pragma unroll 1
  for (int pass = 1; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int d = lane; d < 256; d += 64) hist[d] = 0;
#pragma unroll
    for (int j = 0; j < N; ++j) {
      if (take(j) && (v[j] >> (shift + 8)) == prefix) atomicAdd(&hist[(v[j] >> shift) & 255u], 1u);
    }
    uint32_t d, gt;
    wave_find_digit(hist, 256, k_rem, lane, &d, &gt);
    prefix = (prefix << 8) | d;
    k_rem -= gt;
  }
  *T_out = prefix;
  *eq_take = k_rem;
}

// The same over m candidate keys held in LDS.
__device__ __forceinline__ void wave_radix_select_lds(const uint32_t* cand, uint32_t m, uint32_t d0,
                                                      uint32_t k_rem, uint32_t* hist, int lane,
                                                      uint32_t* T_out, uint32_t* eq_take) {
  uint32_t prefix = d0;
#pragma unroll 1
  for (int pass = 1; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int d = lane; d < 256; d += 64) hist[d] = 0;
    for (uint32_t i = lane; i < m; i += 64) {
      const uint32_t v = cand[i];
      if ((v >> (shift + 8)) == prefix) atomicAdd(&hist[(v >> shift) & 255u], 1u);
    }
    uint32_t d, gt;
    wave_find_digit(hist, 256, k_rem, lane, &d, &gt);
    prefix = (prefix << 8) | d;
    k_rem -= gt;
  }
  *T_out = prefix;
  *eq_take = k_rem;
}

template <int E, bool HAS_IDX>
__global__ __launch_bounds__(256) void topk_wave_kernel(TopkArgs a) {
  __shared__ uint32_t hist_all[4][256];
  __shared__ uint32_t cand_all[4][kWaveCand];
  __shared__ uint16_t sel_all[4][kMaxTopk];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int64_t task = static_cast<int64_t>(blockIdx.x) * 4 + wid;
  if (task >= a.n_rows * a.n_seg) return;
  const int64_t r = task / a.n_seg;
  const int32_t seg = static_cast<int32_t>(task % a.n_seg);
  uint32_t* hist = hist_all[wid];
  uint32_t* cand = cand_all[wid];
  uint16_t* sel = sel_all[wid];

  int64_t len = a.row_len ? static_cast<int64_t>(a.row_len[r]) : a.row_stride;
  len = len < 0 ? 0 : (len > a.row_stride ? a.row_stride : len);
  const int64_t base_e = static_cast<int64_t>(seg) * a.seg_len;
  int64_t n64 = len;
  if (a.n_seg > 1) {
    n64 = len - base_e;
    n64 = n64 < 0 ? 0 : (n64 > a.seg_len ? a.seg_len : n64);
  }
  const int32_t n = static_cast<int32_t>(n64);
  const int32_t k = a.k;
  const float* row = a.scores + r * a.row_stride + base_e;
  const int32_t* ridx = HAS_IDX ? a.src_idx + r * a.row_stride + base_e : nullptr;
  int32_t* oi = a.out_idx + task * k;
  float* ov = a.out_val ? a.out_val + task * k : nullptr;
  const float pad_val = a.pad_bits ? __uint_as_float(kPadBits) : -INFINITY;

  if (n <= k) {
    // Everything is selected.  Loads use an in-range index in every lane and are issued in
    // batches of 8 before the stores, so that they overlap.
    for (int32_t p0 = 0; p0 < k; p0 += 8 * 64) {
      int32_t id[8];
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int32_t e = p0 + i * 64 + lane;
        const int32_t ec = e < n ? e : 0;
        id[i] = HAS_IDX ? (n > 0 ? ridx[ec] : -1) : static_cast<int32_t>(base_e + ec);
        v[i] = n > 0 ? row[ec] : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int32_t e = p0 + i * 64 + lane;
        if (e < k) {
          oi[e] = e < n ? id[i] : -1;
          if (ov) ov[e] = e < n ? v[i] : pad_val;
        }
      }
    }
    return;
  }

  // 1. keys in registers (key 0: past the end or padding, below every real key incl. -inf's).
  //    All loads first, unconditionally (clamped index), so that they are in flight together.
  uint32_t u[E];
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int32_t e = j * 64 + lane;
    u[j] = __float_as_uint(row[e < n ? e : n - 1]);   // n > k >= 1 here
  }
  launder(u);
#pragma unroll
  for (int j = 0; j < E; ++j)
    u[j] = j * 64 + lane < n ? order_key(__uint_as_float(u[j])) : 0u;

  // 2. histogram of the top 8 key bits (sign + 7 exponent bits): the digit D holding the k-th
  //    largest key; everything in higher digits is selected.  Out-of-range slots carry key 0 and
  //    land in digit 0, which the scan only reaches if the row holds fewer than k real keys (it
  //    cannot: n > k).
  for (int d = lane; d < 256; d += 64) hist[d] = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) atomicAdd(&hist[u[j] >> 24], 1u);
  uint32_t dD, above;
  wave_find_digit(hist, 256, static_cast<uint32_t>(k), lane, &dD, &above);
  const uint32_t c_d = hist[dD] - (dD == 0u ? static_cast<uint32_t>(E * 64 - n) : 0u);
  const uint32_t k_rem = static_cast<uint32_t>(k) - above;    // 1 <= k_rem <= c_d

  // 3. exact threshold among the keys of digit D: gathered into LDS (ballot compaction) when they
  //    fit, otherwise filtered in registers; three more 8-bit passes.
  uint32_t T, eq_take;
  if (c_d <= static_cast<uint32_t>(kWaveCand)) {
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const bool ind = (u[j] >> 24) == dD && j * 64 + lane < n;
      const uint64_t m = __ballot(ind);
      if (ind) cand[cnt + lanes_below(m)] = u[j];
      cnt += static_cast<uint32_t>(__popcll(m));
    }
    wave_radix_select_lds(cand, c_d, dD, k_rem, hist, lane, &T, &eq_take);
  } else {
    wave_radix_select(u, [&](int j) { return (u[j] >> 24) == dD && j * 64 + lane < n; }, dD,
                      k_rem, hist, lane, &T, &eq_take);
  }
  const uint32_t n_gt = static_cast<uint32_t>(k) - eq_take;

  // 4. compaction in index order: a key > T goes to (#keys > T before it) + (#selected keys == T
  //    before it); a key == T is selected while fewer than eq_take equal keys precede it.  Values
  //    come from the keys (-0 is returned as +0); candidate lists record positions for step 5.
  launder(u);
  uint32_t gt_seen = 0, eq_seen = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int32_t e = j * 64 + lane;
    const bool gtv = e < n && u[j] > T;
    const bool eqv = e < n && u[j] == T;
    const uint64_t mg = __ballot(gtv);
    const uint64_t me = __ballot(eqv);
    const uint32_t gpre = gt_seen + lanes_below(mg);
    const uint32_t epre = eq_seen + lanes_below(me);
    uint32_t pos = 0xFFFFFFFFu;
    if (gtv) pos = gpre + (epre < eq_take ? epre : eq_take);
    else if (eqv && epre < eq_take) pos = gpre + epre;
    if (pos < static_cast<uint32_t>(k)) {
      if constexpr (HAS_IDX) sel[pos] = static_cast<uint16_t>(e);
      else oi[pos] = static_cast<int32_t>(base_e + e);
      if (ov) ov[pos] = u[j] ? key_value(u[j]) : pad_val;   // key 0: a padding entry
    }
    gt_seen += static_cast<uint32_t>(__popcll(mg));
    eq_seen += static_cast<uint32_t>(__popcll(me));
  }
  // 5. candidate lists: the winners' original indices, gathered 8 per lane at a time
  if constexpr (HAS_IDX) {
    for (int32_t p0 = 0; p0 < k; p0 += 8 * 64) {
      int32_t id[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int32_t p = p0 + i * 64 + lane;
        id[i] = ridx[p < k ? sel[p] : 0];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int32_t p = p0 + i * 64 + lane;
        if (p < k) oi[p] = id[i];
      }
    }
  }
}

template <int E>
hipError_t launch_wave(const TopkArgs& a, hipStream_t stream) {
  const int64_t tasks = a.n_rows * a.n_seg;
  const int64_t blocks = (tasks + 3) / 4;
  if (a.src_idx)
    hipLaunchKernelGGL((topk_wave_kernel<E, true>), dim3(static_cast<uint32_t>(blocks)), dim3(256),
                       0, stream, a);
  else
    hipLaunchKernelGGL((topk_wave_kernel<E, false>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(256), 0, stream, a);
  return hipGetLastError();
}

// One selection pass; every row segment must hold at most kMaxSegment elements.
hipError_t launch_pass(const TopkArgs& a, int32_t seg_elems, hipStream_t stream) {
  if (a.n_rows <= 0) return hipSuccess;
  if (seg_elems <= 16 * 64) return launch_wave<16>(a, stream);
  if (seg_elems <= 32 * 64) return launch_wave<32>(a, stream);
  if (seg_elems <= 64 * 64) return launch_wave<64>(a, stream);
  return launch_wave<96>(a, stream);
}

// Segments per row of pass 1: enough waves for the whole chip (about 1024) when rows are few,
// while one pass over the candidates still fits a single wave when possible; at least as many
// as the wave capacity demands.
int32_t first_pass_segments(int64_t n_rows, int64_t cols, int32_t k) {
  const int64_t need = (cols + kMaxSegment - 1) / kMaxSegment;
  int64_t spread = (1024 + n_rows - 1) / (n_rows > 0 ? n_rows : 1);
  const int64_t fit = kMaxSegment / k;
  const int64_t usable = cols / (2 * static_cast<int64_t>(k));
  int64_t want = spread;
  if (want > fit) want = fit;
  if (want > usable) want = usable;
  int64_t ns = need > want ? need : want;
  if (ns < 1) ns = 1;
  return static_cast<int32_t>(ns);
}

int32_t seg_len_for(int64_t cols, int32_t n_seg) {
  int64_t sl = (cols + n_seg - 1) / n_seg;
  sl = (sl + 63) / 64 * 64;
  return static_cast<int32_t>(sl);
}

}  // namespace

TopkPlan topk_plan(int64_t n_rows, int64_t cols, int32_t k) {
  TopkPlan p{};
  p.passes = 1;
  p.cand_elems = 0;
  int64_t c = cols;
  int32_t ns = first_pass_segments(n_rows, c, k);
  while (ns > 1) {
    const int32_t sl = seg_len_for(c, ns);
    const int32_t real_ns = static_cast<int32_t>((c + sl - 1) / sl);
    const int64_t out = static_cast<int64_t>(real_ns) * k;
    if (out > p.cand_elems) p.cand_elems = out;
    p.passes += 1;
    c = out;
    ns = static_cast<int32_t>((c + kMaxSegment - 1) / kMaxSegment);
  }
  return p;
}

size_t topk_workspace_bytes(int64_t n_rows, int64_t cols, int32_t k) {
  const TopkPlan p = topk_plan(n_rows, cols, k);
  if (p.passes <= 1) return 0;
  // two candidate buffers (index + value each) for ping-pong between passes
  return 2 * (static_cast<size_t>(n_rows) * p.cand_elems * 8 + 256);
}

hipError_t run_topk(const float* scores, int64_t row_stride, const int32_t* row_len,
                    int64_t n_rows, int32_t k, int32_t* out_idx, float* out_val, void* ws,
                    hipStream_t stream) {
  if (n_rows <= 0) return hipSuccess;
  const int64_t cols = row_stride;
  TopkArgs a{};
  a.scores = scores;
  a.row_stride = row_stride;
  a.row_len = row_len;
  a.n_rows = n_rows;
  a.k = k;
  a.src_idx = nullptr;
  a.pad_bits = 0;
  int32_t ns = first_pass_segments(n_rows, cols, k);
  if (ns <= 1) {
    a.n_seg = 1;
    a.seg_len = 0;
    a.out_idx = out_idx;
    a.out_val = out_val;
    return launch_pass(a, static_cast<int32_t>(cols), stream);
  }
  const TopkPlan plan = topk_plan(n_rows, cols, k);
  const size_t half = static_cast<size_t>(n_rows) * plan.cand_elems * 8 + 256;
  char* base = static_cast<char*>(ws);
  int64_t c = cols;
  int which = 0;
  while (true) {
    int32_t sl = seg_len_for(c, ns);
    ns = static_cast<int32_t>((c + sl - 1) / sl);
    const int64_t out_stride = static_cast<int64_t>(ns) * k;
    char* buf = base + which * half;
    int32_t* cidx = reinterpret_cast<int32_t*>(buf);
    float* cval = reinterpret_cast<float*>(buf + ((static_cast<size_t>(n_rows) * plan.cand_elems *
                                                   4 + 255) / 256 * 256));
    a.n_seg = ns;
    a.seg_len = sl;
    a.out_idx = cidx;
    a.out_val = cval;
    a.pad_bits = 1;
    hipError_t e = launch_pass(a, sl, stream);
    if (e != hipSuccess) return e;
    // the candidates, each row a list of ns * k (index, value) pairs in index order
    a.scores = cval;
    a.row_stride = out_stride;
    a.row_len = nullptr;
    a.src_idx = cidx;
    c = out_stride;
    which ^= 1;
    ns = static_cast<int32_t>((c + kMaxSegment - 1) / kMaxSegment);
    if (ns <= 1) {
      a.n_seg = 1;
      a.seg_len = 0;
      a.out_idx = out_idx;
      a.out_val = out_val;
      a.pad_bits = 0;
      return launch_pass(a, static_cast<int32_t>(c), stream);
    }
  }
}

}  // namespace dsa
