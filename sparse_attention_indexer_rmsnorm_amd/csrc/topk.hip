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
//      registers, lane-strided (element e = 64 j + lane), all loads in flight together; a wave
//      reduction gives the smallest and largest key;
//   2. a 4096-bin histogram (wave-private LDS, 16-bit counts packed two to a word) of the keys'
//      offsets above the smallest key, shifted so that the row's key range fills the bins, gives
//      the bin B holding the k-th largest key; every key in a higher bin is selected.  Because the
//      bins follow the row's own range, one wave's LDS adds land on many different addresses;
//   3. the keys of bin B (a small fraction of the row) are gathered into the same LDS area by
//      ballot compaction, and 7-bit radix passes over their remaining low bits yield the k-th
//      largest key T and how many keys equal to T to take (when bin B holds more keys than the
//      area, the passes filter the registers instead);
//   4. one pass compacts, in increasing index order, every key > T and the lowest-indexed keys
//      == T, with ballots, writing the winners from registers: the output is unique and
//      deterministic, ties to the lower index, each row sorted by index (values are returned
//      from the keys, so a -0 score comes back as +0).
#include "internal.h"

namespace dsa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBinBits = 12;
constexpr int kBins = 1 << kBinBits;          // histogram bins of a workgroup
constexpr int kWaveBinBits = 11;
constexpr int kWaveBins = 1 << kWaveBinBits;  // histogram bins of a wave (32-bit counts)
constexpr int kAreaWords = kWaveBins;         // 8 KiB per wave: histogram, then candidates, then slots
constexpr int kWaveCand = kAreaWords;         // candidate keys that fit the area
// Whole-row selection works on blocks of kRowBlk groups of 64 keys without per-lane branches, so
// that the scheduler can overlap the groups of a block.  Its list holds (offset, slot) pairs of
// 8 B; the last 64 pairs of the area take the writes of lanes with nothing to list.
constexpr int kRowBlk = 8;
constexpr int kRowCand = kAreaWords / 2 - 64;
constexpr int kMaxTopk = 2048;
constexpr int kSubBits = 7;                   // refinement digit width
constexpr int kSubBins = 1 << kSubBits;
static_assert(kMaxTopk * 2 <= kAreaWords * 4, "winner slots must fit the area");

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  u = (u << 1) == 0u ? 0u : u;                         // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// order_key of a score that is not a NaN, in four instructions: adding +0 turns -0 into +0 and
// leaves every other value as it is (fp32 denormals are kept), then the sign selects the mask.
__device__ __forceinline__ uint32_t score_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return u ^ (static_cast<uint32_t>(static_cast<int32_t>(u) >> 31) | 0x80000000u);
}

// Value bits of a padding entry in an intermediate candidate list: a NaN pattern whose order key
// is 0, below every real key (-inf's included).  Scores are never NaN.
constexpr uint32_t kPadBits = 0xFFFFFFFFu;

__device__ __forceinline__ float key_value(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Hide a value from the optimiser (emits nothing): per-key values derived in one pass are then
// recomputed in the next instead of being kept live, which would multiply the registers per key.
template <int N>
__device__ __forceinline__ void launder(uint32_t (&v)[N]) {
#pragma unroll
  for (int j = 0; j < N; ++j) asm volatile("" : "+v"(v[j]));
}

// Make v depend on the scalar s (emits nothing).  Chaining each iteration of a ballot loop to the
// previous iteration's count keeps the compiler from evaluating every iteration's ballot up front,
// which would need two SGPRs per key and spill them.
__device__ __forceinline__ uint32_t after(uint32_t v, uint32_t s) {
  asm volatile("" : "+v"(v) : "s"(s));
  return v;
}

// A copy of a wave-uniform value the compiler cannot identify with the original (emits nothing):
// the loops below each test their group index against a fresh copy, so the per-group results of
// one loop are not kept alive for the next.
__device__ __forceinline__ int32_t fresh(int32_t v) {
  v = __builtin_amdgcn_readfirstlane(v);
  asm volatile("" : "+s"(v));
  return v;
}

// Raw buffer view of n floats at p (p wave-uniform): loads whose (vector + immediate) offset lies
// at or past the end return 0 without touching memory, so a wave loads whole 64-slot groups with
// no clamping.  The scalar offset is not range-checked, so it stays 0.  Word 3 of a gfx9-family
// descriptor selects 32-bit elements.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_view(const float* p, int32_t n) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  void* base = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, n * 4, 0x00020000);
}

// Number of lanes below this one whose bit is set in `mask` (wave64), plus `base`.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask, uint32_t base = 0u) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), base));
}

// A wave-uniform constant the compiler cannot see through (emits nothing): per-group values
// formed from it stay where they are used.
__device__ __forceinline__ uint32_t opaque_s(uint32_t v) {
  asm volatile("" : "+s"(v));
  return v;
}

// A per-lane value the compiler cannot see through (emits nothing): a select between it and
// another value stays a select instead of becoming a predicated block that computes it.
__device__ __forceinline__ uint32_t opaque_v(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// s_waitcnt operand: vector memory counter 0, the others left alone (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt in 6:4, lgkmcnt in 11:8)
constexpr int kVmcnt0 = (7 << 4) | (15 << 8);

// Cross-lane steps with DPP (no LDS traffic).  dpp<ctrl, row_mask>(x, id) returns, per lane, x of
// the lane the control selects, or id where there is none (outside the 16-lane row, or in a row
// the mask leaves out).  Controls: row_shr:n = 0x110 + n; row_bcast:15 = 0x142 (lane 15 of each
// row to the next row); row_bcast:31 = 0x143 (lane 31 to rows 2 and 3).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp(uint32_t x, uint32_t id) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(id), static_cast<int>(x),
                                                           CTRL, ROW_MASK, 0xF, false));
}

// Inclusive wave scan with an associative op and its identity.
template <typename Op>
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x, uint32_t id, Op op) {
  x = op(x, dpp<0x111, 0xF>(x, id));
  x = op(x, dpp<0x112, 0xF>(x, id));
  x = op(x, dpp<0x114, 0xF>(x, id));
  x = op(x, dpp<0x118, 0xF>(x, id));
  x = op(x, dpp<0x142, 0xA>(x, id));
  x = op(x, dpp<0x143, 0xC>(x, id));
  return x;
}

__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t v, int /*lane*/) {
  return wave_incl_scan(v, 0u, [](uint32_t p, uint32_t q) { return p + q; }) - v;
}

__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
  v = wave_incl_scan(v, 0xFFFFFFFFu, [](uint32_t p, uint32_t q) { return p < q ? p : q; });
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = wave_incl_scan(v, 0u, [](uint32_t p, uint32_t q) { return p > q ? p : q; });
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

// Value of x in lane src (src wave-uniform).
__device__ __forceinline__ uint32_t lane_value(uint32_t x, int src) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), src));
}

// Descending scan of nb 32-bit bins (nb a multiple of 64): the bin holding the want-th largest
// entry, the count above it and its own count.  Lane l sums bins [nb - per (l+1), nb - per l);
// then the crossing lane's bins are spread over the wave.
template <int NB>
__device__ __forceinline__ void wave_find_bin32(const uint32_t* bins, uint32_t want, int lane,
                                                uint32_t* bin, uint32_t* above, uint32_t* count) {
  constexpr int per = NB / 64;
  static_assert(per % 4 == 0 && per <= 64 && ((per / 4) & (per / 4 - 1)) == 0, "bins per lane");
  const u32x4* blk = reinterpret_cast<const u32x4*>(bins + NB - per * (lane + 1));
  uint32_t local = 0;
  // rotated chunk order: blocks are per * 4 B apart, so reading chunk i in every lane at once
  // would put a whole 16-lane group on the same banks
#pragma unroll
  for (int i = 0; i < per / 4; ++i) {
    const u32x4 v = blk[(i + lane) & (per / 4 - 1)];
    local += (v.x + v.y) + (v.z + v.w);
  }
  const uint32_t run = wave_excl_scan(local, lane);
  const uint64_t hm = __ballot(run < want && run + local >= want);
  const int L = __builtin_amdgcn_readfirstlane(hm ? __builtin_ctzll(hm) : 0);
  const uint32_t run_l = lane_value(run, L);
  const int bi = NB - per * L - 1 - lane;               // lane i < per: the i-th bin from the top
  const uint32_t c = lane < per ? bins[bi] : 0u;
  const uint32_t r2 = run_l + wave_excl_scan(c, lane);
  const uint64_t m = __ballot(lane < per && r2 < want && r2 + c >= want);
  const int src = __builtin_amdgcn_readfirstlane(m ? __builtin_ctzll(m) : 0);
  *bin = static_cast<uint32_t>(NB - per * L - 1 - src);
  *above = lane_value(r2, src);
  *count = lane_value(c, src);
}

// Among kSubBins bins, the descending digit holding the rank-`want` largest entry and the number
// of entries in higher digits.  Lane l owns digits kSubBins-1-2l and kSubBins-2-2l.
__device__ __forceinline__ void wave_find_digit(const uint32_t* hist, uint32_t want, int lane,
                                                uint32_t* digit, uint32_t* above) {
  static_assert(kSubBins == 128, "two digits per lane");
  const uint32_t c0 = hist[kSubBins - 1 - 2 * lane];
  const uint32_t c1 = hist[kSubBins - 2 - 2 * lane];
  const uint32_t run = wave_excl_scan(c0 + c1, lane);
  const bool h0 = run < want && run + c0 >= want;
  const bool h1 = run + c0 < want && run + c0 + c1 >= want;
  const uint64_t m = __ballot(h0 || h1);
  const int src = __builtin_amdgcn_readfirstlane(m ? __builtin_ctzll(m) : 0);
  const uint32_t d = h0 ? static_cast<uint32_t>(kSubBins - 1 - 2 * lane)
                        : static_cast<uint32_t>(kSubBins - 2 - 2 * lane);
  *digit = lane_value(d, src);
  *above = lane_value(h0 ? run : run + c0, src);
}

// Exact select inside fine bin B: the k_rem-th largest offset (key - kmin) among the selected
// keys, whose offsets all share the bits above `bits`, and how many keys equal to it belong to the
// top k_rem.  Radix passes of up to 7 bits, high to low.  `offset_of(i, &d)` yields candidate i's
// offset and whether it is a candidate at all; `count` candidates are visited per lane loop.
template <typename Visit>
__device__ __forceinline__ void refine(Visit visit, uint32_t prefix, int bits, uint32_t k_rem,
                                       uint32_t* sub, int lane, uint32_t* off_out,
                                       uint32_t* eq_take) {
#pragma unroll 1
  while (bits > 0) {
    const int w = bits < kSubBits ? bits : kSubBits;
    const int shift = bits - w;
    sub[lane] = 0u;
    sub[lane + 64] = 0u;
    visit([&](uint32_t off) {
      if ((off >> bits) == prefix) atomicAdd(&sub[(off >> shift) & ((1u << w) - 1u)], 1u);
    });
    uint32_t d, gt;
    wave_find_digit(sub, k_rem, lane, &d, &gt);
    prefix = (prefix << w) | d;
    k_rem -= gt;
    bits = shift;
  }
  *off_out = prefix;
  *eq_take = k_rem;
}

// One wave's selection task: a row, or one segment of a row.
struct WaveTask {
  const float* row;        // the task's scores
  const int32_t* ridx;     // reported indices of the scores (candidate lists) or null
  int32_t* oi;             // k output indices
  float* ov;               // k output values or null
  int64_t base_e;          // index of the task's first score within its row
  int32_t n;               // scores in the task (wave-uniform)
  int32_t k;
  float pad_val;           // value reported for padding
};

__device__ __forceinline__ WaveTask wave_task(const TopkArgs& a, int64_t task) {
  WaveTask t;
  const int64_t r = task / a.n_seg;
  const int32_t seg = static_cast<int32_t>(task % a.n_seg);
  int64_t len = a.row_len ? static_cast<int64_t>(a.row_len[r]) : a.row_stride;
  len = len < 0 ? 0 : (len > a.row_stride ? a.row_stride : len);
  t.base_e = static_cast<int64_t>(seg) * a.seg_len;
  int64_t n64 = len;
  if (a.n_seg > 1) {
    n64 = len - t.base_e;
    n64 = n64 < 0 ? 0 : (n64 > a.seg_len ? a.seg_len : n64);
  }
  t.n = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(n64));
  t.k = a.k;
  t.row = a.scores + r * a.row_stride + t.base_e;
  t.ridx = a.src_idx ? a.src_idx + r * a.row_stride + t.base_e : nullptr;
  t.oi = a.out_idx + task * a.k;
  t.ov = a.out_val ? a.out_val + task * a.k : nullptr;
  t.pad_val = a.pad_bits ? __uint_as_float(kPadBits) : -INFINITY;
  return t;
}

// n <= k: everything is selected, then padding.  Loads use an in-range index in every lane and
// are issued in batches of 8 before the stores, so that they overlap.
template <bool HAS_IDX>
__device__ __forceinline__ void select_all(const WaveTask& t, int lane) {
  for (int32_t p0 = 0; p0 < t.k; p0 += 8 * 64) {
    int32_t id[8];
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int32_t e = p0 + i * 64 + lane;
      const int32_t ec = e < t.n ? e : 0;
      id[i] = HAS_IDX ? (t.n > 0 ? t.ridx[ec] : -1) : static_cast<int32_t>(t.base_e + ec);
      v[i] = t.n > 0 ? t.row[ec] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int32_t e = p0 + i * 64 + lane;
      if (e < t.k) {
        t.oi[e] = e < t.n ? id[i] : -1;
        if (t.ov) t.ov[e] = e < t.n ? v[i] : t.pad_val;
      }
    }
  }
}

// The key range of a task, and the histogram scaling derived from it.
struct KeyRange {
  uint32_t kbase;   // smallest real key - 1: offsets are key - kbase (key 0 -> 0, others >= 1)
  int shift;        // (largest offset >> shift) < kWaveBins
  int32_t groups;   // 64-slot groups holding entries
};

// 1. keys in registers, all loads first (buffer loads, in range or returning 0) so that they are
//    in flight together.  Slots past the end hold key 0 like padding entries.  Key 0 is the lowest
//    key, and equal keys are taken in index order, so a slot past the end is never selected (n > k
//    real entries precede it); whole 64-slot groups past the end are never looked at again (every
//    later loop tests its group index against the wave-uniform group count), and only the group
//    holding the end needs a per-lane test.  Scores hold no padding and take a plain minimum with
//    the lanes past the end left out; candidate lists may hold padding (key 0) anywhere, and there
//    key - 1 wraps key 0 to the top, out of the minimum.
template <int E, bool HAS_IDX>
__device__ __forceinline__ KeyRange load_keys(uint32_t (&u)[E], const WaveTask& t, int lane) {
  {
    const __amdgpu_buffer_rsrc_t view = buffer_view(t.row, t.n);
    // an opaque lane offset: each call's loads form their addresses in place (immediate offsets
    // from few bases) instead of sharing per-load address registers with another call
    const uint32_t lane4 = after(static_cast<uint32_t>(lane) * 4u, 0u);
#pragma unroll
    for (int j = 0; j < E; ++j)
      u[j] = __builtin_amdgcn_raw_buffer_load_b32(view, lane4 + j * 256, 0, 0);
  }
  launder(u);
  KeyRange kr;
  kr.groups = (t.n + 63) >> 6;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  {
    const int32_t ng = fresh(kr.groups);
    const int32_t rem = t.n - 64 * (ng - 1);    // entries in the last group, 1..64
#pragma unroll
    for (int j = 0; j < E; ++j) {
      if (j < ng) {
        uint32_t key = HAS_IDX ? order_key(__uint_as_float(u[j])) : score_key(__uint_as_float(u[j]));
        uint32_t for_min = HAS_IDX ? key - 1u : key;
        if (j == ng - 1) {
          asm volatile("");   // a branch: only the group holding the end tests its lanes
          key = lane < rem ? key : 0u;
          for_min = lane < rem ? for_min : 0xFFFFFFFFu;
        }
        u[j] = key;
        kmin = min(kmin, for_min);
        kmax = max(kmax, key);
      }
    }
  }
  kr.kbase = HAS_IDX ? wave_min(kmin) : wave_min(kmin) - 1u;
  kmax = wave_max(kmax);
  const uint32_t top_off = kmax - kr.kbase;   // kmax is a real key: top_off >= 1
  const int span = 32 - __builtin_clz(top_off);
  kr.shift = span > kWaveBinBits ? span - kWaveBinBits : 0;
  return kr;
}

__device__ __forceinline__ uint32_t key_offset(uint32_t key, uint32_t kbase) {
  return __builtin_elementwise_sub_sat(key, kbase);   // key 0 -> 0
}

// 2. histogram of the offsets (kWaveBins 32-bit bins filling the area), then the bin B holding
//    the k-th largest key, the number of keys in higher bins and B's own count.
template <int E>
__device__ __forceinline__ void bin_of_kth(uint32_t (&u)[E], const KeyRange& kr, int32_t k,
                                           uint32_t* area, int lane, uint32_t* bB,
                                           uint32_t* above, uint32_t* c_b) {
#pragma unroll
  for (int i = 0; i < kAreaWords / 256; ++i)
    reinterpret_cast<u32x4*>(area)[i * 64 + lane] = u32x4{0u, 0u, 0u, 0u};
  launder(u);
  {
    const int32_t ng = fresh(kr.groups);
#pragma unroll
    for (int j = 0; j < E; ++j)   // after(): computed here, not hoisted
      if (j < ng) atomicAdd(&area[key_offset(after(u[j], 0u), kr.kbase) >> kr.shift], 1u);
  }
  wave_find_bin32<kWaveBins>(area, static_cast<uint32_t>(k), lane, bB, above, c_b);
}

// 3-5. selection in index order: the exact threshold T among bin B's offsets (gathered into the
// area by ballot compaction when they fit, otherwise filtered in registers on every radix pass),
// then one compaction pass writing every key > T and the lowest-indexed keys == T, in index
// order, so that each output row is sorted by index (candidate lists rely on this for ties).
template <int E, bool HAS_IDX>
__device__ __forceinline__ void select_ordered(uint32_t (&u)[E], const KeyRange& kr,
                                               const WaveTask& t, uint32_t bB, uint32_t above,
                                               uint32_t c_b, uint32_t* area, uint32_t* sub,
                                               int lane) {
  const uint32_t kbase = kr.kbase;
  const int shift = kr.shift;
  const uint32_t k_rem = static_cast<uint32_t>(t.k) - above;    // 1 <= k_rem <= c_b
  uint32_t t_off, eq_take;
  launder(u);
  if (c_b <= static_cast<uint32_t>(kWaveCand)) {
    uint32_t cnt = 0;
    const int32_t ng = fresh(kr.groups);
#pragma unroll
    for (int j = 0; j < E; ++j) {
      if (j < ng) {
        const uint32_t o = key_offset(after(u[j], cnt), kbase);
        const bool ind = (o >> shift) == bB;
        const uint64_t m = __ballot(ind);
        if (ind) area[cnt + lanes_below(m)] = o;
        cnt += static_cast<uint32_t>(__popcll(m));
      }
    }
    refine([&](auto add) {
             for (uint32_t i = lane; i < c_b; i += 64) add(area[i]);
           },
           bB, shift, k_rem, sub, lane, &t_off, &eq_take);
  } else {
    refine([&](auto add) {
             const int32_t ng = fresh(kr.groups);
#pragma unroll
             for (int j = 0; j < E; ++j) {
               if (j < ng) {
                 const uint32_t o = key_offset(after(u[j], 0u), kbase);   // recomputed every pass
                 if ((o >> shift) == bB) add(o);
               }
             }
           },
           bB, shift, k_rem, sub, lane, &t_off, &eq_take);
  }
  const uint32_t T = t_off ? t_off + kbase : 0u;

  // a key > T goes to (#keys > T before it) + (#selected keys == T before it); a key == T is
  // selected while fewer than eq_take equal keys precede it.  Values come from the keys (-0 is
  // returned as +0); candidate lists record positions for the index gather below.
  uint16_t* sel = reinterpret_cast<uint16_t*>(area);
  launder(u);
  uint32_t gt_seen = 0, eq_seen = 0;
  const int32_t ng = fresh(kr.groups);
#pragma unroll
  for (int j = 0; j < E; ++j) {
    if (j < ng) {
      const int32_t e = j * 64 + lane;
      const uint32_t uj = after(u[j], gt_seen + eq_seen);
      const bool gtv = uj > T;
      const bool eqv = uj == T;
      const uint64_t mg = __ballot(gtv);
      const uint64_t me = __ballot(eqv);
      const uint32_t gpre = gt_seen + lanes_below(mg);
      const uint32_t epre = eq_seen + lanes_below(me);
      uint32_t pos = 0xFFFFFFFFu;
      if (gtv) pos = gpre + (epre < eq_take ? epre : eq_take);
      else if (eqv && epre < eq_take) pos = gpre + epre;
      if (pos < static_cast<uint32_t>(t.k)) {
        if constexpr (HAS_IDX)   // the slot number is formed here rather than kept per key
          sel[pos] = static_cast<uint16_t>(after(static_cast<uint32_t>(lane), 0u) + j * 64);
        else t.oi[pos] = static_cast<int32_t>(t.base_e + e);
        if (t.ov) t.ov[pos] = uj ? key_value(uj) : t.pad_val;   // key 0: a padding entry
      }
      gt_seen += static_cast<uint32_t>(__popcll(mg));
      eq_seen += static_cast<uint32_t>(__popcll(me));
    }
  }
  // candidate lists: the winners' original indices, gathered 8 per lane at a time
  if constexpr (HAS_IDX) {
    for (int32_t p0 = 0; p0 < t.k; p0 += 8 * 64) {
      int32_t id[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int32_t p = p0 + i * 64 + lane;
        id[i] = t.ridx[p < t.k ? sel[p] : 0];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int32_t p = p0 + i * 64 + lane;
        if (p < t.k) t.oi[p] = id[i];
      }
    }
  }
}

// All E loads of a row in flight together (buffer loads: past the end they return 0).
template <int E>
__device__ __forceinline__ void issue_loads(uint32_t (&u)[E], const float* row, int32_t n,
                                            int lane) {
  const __amdgpu_buffer_rsrc_t view = buffer_view(row, n);
#pragma unroll
  for (int j = 0; j < E; ++j)
    u[j] = __builtin_amdgcn_raw_buffer_load_b32(view, static_cast<uint32_t>(lane) * 4u + j * 256,
                                                0, 0);
}

// 1r. keys of a whole row, block by block; only the block holding the row end tests its lanes,
// and there every slot past the end (the rest of the block included) gets key 0 and stays out of
// the minimum.  Blocks past the end are never looked at again.
template <int E>
__device__ __forceinline__ KeyRange row_keys(uint32_t (&u)[E], const WaveTask& t, int lane) {
  static_assert(E % kRowBlk == 0, "whole blocks");
  KeyRange kr;
  kr.groups = (t.n + 63) >> 6;
  const int32_t nb = fresh((kr.groups + kRowBlk - 1) / kRowBlk);
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int b = 0; b < E / kRowBlk; ++b) {
    if (b < nb) {
      if (b == nb - 1) {
        asm volatile("");   // a branch: only this block tests its lanes
        const int32_t rem = t.n - b * kRowBlk * 64 - lane;   // slots of this lane left in the row
#pragma unroll
        for (int i = 0; i < kRowBlk; ++i) {
          const int j = b * kRowBlk + i;
          const bool valid = i * 64 < rem;
          const uint32_t key = score_key(__uint_as_float(u[j]));
          u[j] = valid ? key : 0u;
          kmin = min(kmin, valid ? key : 0xFFFFFFFFu);
          kmax = max(kmax, u[j]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < kRowBlk; ++i) {
          const int j = b * kRowBlk + i;
          u[j] = score_key(__uint_as_float(u[j]));
          kmin = min(kmin, u[j]);
          kmax = max(kmax, u[j]);
        }
      }
    }
  }
  // every load has been used: say so explicitly, or the compiler, unable to prove it on every
  // path, keeps waiting on the memory counter later, where it also counts the output stores
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  kr.kbase = wave_min(kmin) - 1u;
  kmax = wave_max(kmax);
  const uint32_t top_off = kmax - kr.kbase;   // kmax is a real key: top_off >= 1
  const int span = 32 - __builtin_clz(top_off);
  kr.shift = span > kWaveBinBits ? span - kWaveBinBits : 0;
  return kr;
}

// 2r. histogram of a whole row's offsets, block by block (slots past the end count in bin 0),
// then bin B as in bin_of_kth.  The offset base is made opaque per block so that no block's
// arithmetic is moved ahead of the block.
template <int E>
__device__ __forceinline__ void row_bin_of_kth(uint32_t (&u)[E], const KeyRange& kr, int32_t k,
                                               uint32_t* area, int lane, uint32_t* bB,
                                               uint32_t* above, uint32_t* c_b) {
#pragma unroll
  for (int i = 0; i < kAreaWords / 256; ++i)
    reinterpret_cast<u32x4*>(area)[i * 64 + lane] = u32x4{0u, 0u, 0u, 0u};
  const int32_t nb = fresh((kr.groups + kRowBlk - 1) / kRowBlk);
#pragma unroll
  for (int b = 0; b < E / kRowBlk; ++b) {
    if (b < nb) {
      const uint32_t kb = opaque_s(kr.kbase);
#pragma unroll
      for (int i = 0; i < kRowBlk; ++i)
        atomicAdd(&area[key_offset(u[b * kRowBlk + i], kb) >> kr.shift], 1u);
    }
  }
  wave_find_bin32<kWaveBins>(area, static_cast<uint32_t>(k), lane, bB, above, c_b);
}

// 3r-5r. selection of a whole row in any order, when bin B > 0 fits the list: one pass over the
// keys, block by block, writes those in bins above B straight to the output (positions
// 0..above-1, in index order) and lists bin B's offsets with their slots, in index order; the
// radix passes then run over the list alone, and the list's winners (offsets > t_off, then the
// first eq_take offsets == t_off in list order) fill positions above..k-1.  Lanes with nothing
// to store write past the output view (dropped) or to their own spare list entry, so that no
// group branches.  Slots past the row end hold key 0: bin 0 < B, never written.
template <int E, bool VALS>
__device__ __forceinline__ void row_select(uint32_t (&u)[E], const KeyRange& kr,
                                           const WaveTask& t, uint32_t bB, uint32_t above,
                                           uint32_t c_b, uint32_t* area, uint32_t* sub, int lane) {
  const int shift = kr.shift;
  const uint32_t k_rem = static_cast<uint32_t>(t.k) - above;    // 1 <= k_rem <= c_b
  uint2* cand = reinterpret_cast<uint2*>(area);                  // (offset, slot)
  const __amdgpu_buffer_rsrc_t vi = buffer_view(reinterpret_cast<const float*>(t.oi), t.k);
  const __amdgpu_buffer_rsrc_t vv = buffer_view(t.ov, VALS ? t.k : 0);
  // past every output view (k <= 2048 values); the bit pattern of 4.0f, which the hardware takes
  // as an inline constant
  constexpr uint32_t kDrop = 0x40800000u;
  const uint32_t spare = static_cast<uint32_t>(kRowCand + lane);
  uint32_t n_gt = 0, n_in = 0;
  const int32_t nb = fresh((kr.groups + kRowBlk - 1) / kRowBlk);
#pragma unroll
  for (int b = 0; b < E / kRowBlk; ++b) {
    if (b < nb) {
      const uint32_t kb = opaque_s(kr.kbase);
#pragma unroll
      for (int i = 0; i < kRowBlk; ++i) {
        const int j = b * kRowBlk + i;
        const uint32_t o = key_offset(u[j], kb);
        const uint32_t bin = o >> shift;
        const bool gtv = bin > bB;
        const bool inv = bin == bB;
        const uint64_t mg = __ballot(gtv);
        const uint64_t mi = __ballot(inv);
        // the slot number is formed here rather than kept per key (lane < 64: an OR)
        const uint32_t e = static_cast<uint32_t>(lane) | opaque_s(static_cast<uint32_t>(j * 64));
        // both positions are formed in every lane, then selected
        const uint32_t pg = opaque_v(lanes_below(mg, n_gt));
        const uint32_t pi = opaque_v(lanes_below(mi, n_in));
        const uint32_t at = gtv ? 4u * pg : kDrop;
        __builtin_amdgcn_raw_buffer_store_b32(e, vi, at, 0, 0);
        if constexpr (VALS)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(key_value(u[j])), vv, at, 0, 0);
        cand[inv ? pi : spare] = make_uint2(o, e);
        n_gt += static_cast<uint32_t>(__popcll(mg));
        n_in += static_cast<uint32_t>(__popcll(mi));
      }
    }
  }
  uint32_t t_off, eq_take;
  refine([&](auto add) {
           for (uint32_t i = lane; i < c_b; i += 64) add(cand[i].x);
         },
         bB, shift, k_rem, sub, lane, &t_off, &eq_take);
  // t_off >= 1 (n > k real keys), so the 0 taken for a lane past the list is never selected
  uint32_t gt_seen = 0, eq_seen = 0;
  for (uint32_t i0 = 0; i0 < c_b; i0 += 64) {
    const uint32_t i = i0 + static_cast<uint32_t>(lane);
    const uint2 ce = i < c_b ? cand[i] : make_uint2(0u, 0u);
    const uint32_t o = ce.x;
    const bool gtv = o > t_off;
    const bool eqv = o == t_off;
    const uint64_t mg = __ballot(gtv);
    const uint64_t me = __ballot(eqv);
    const uint32_t gpre = gt_seen + lanes_below(mg);
    const uint32_t epre = eq_seen + lanes_below(me);
    uint32_t pos = 0xFFFFFFFFu;
    if (gtv) pos = gpre + (epre < eq_take ? epre : eq_take);
    else if (eqv && epre < eq_take) pos = gpre + epre;
    if (pos < k_rem) {
      const uint32_t at = 4u * (above + pos);
      __builtin_amdgcn_raw_buffer_store_b32(ce.y, vi, at, 0, 0);
      if constexpr (VALS)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(key_value(o + kr.kbase)), vv, at, 0, 0);
    }
    gt_seen += static_cast<uint32_t>(__popcll(mg));
    eq_seen += static_cast<uint32_t>(__popcll(me));
  }
}

// The same selection when bin B does not fit the list (many equal keys): rolled loops that read
// the row again (from cache) instead of the registers, so that this rare case adds little code.
// The radix passes filter the row, then one pass in index order writes the keys above bin B to
// positions 0..above-1 and bin B's winners (offsets > t_off, and the lowest-indexed offsets ==
// t_off) to positions above..k-1.
template <bool VALS>
__device__ __forceinline__ void select_from_memory(const KeyRange& kr, const WaveTask& t, uint32_t bB,
                                                uint32_t above, uint32_t* sub, int lane) {
  const uint32_t kbase = kr.kbase;
  const int shift = kr.shift;
  const uint32_t k_rem = static_cast<uint32_t>(t.k) - above;
  const __amdgpu_buffer_rsrc_t view = buffer_view(t.row, t.n);
  auto key_at = [&](int32_t e) {   // key 0 past the end
    const uint32_t key = score_key(__uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(view, static_cast<uint32_t>(e) * 4u, 0, 0)));
    return e < t.n ? key : 0u;
  };
  uint32_t t_off, eq_take;
  refine([&](auto add) {
#pragma unroll 1
           for (int32_t e = lane; e < t.n; e += 64) {
             const uint32_t o = key_offset(key_at(e), kbase);
             if ((o >> shift) == bB) add(o);
           }
         },
         bB, shift, k_rem, sub, lane, &t_off, &eq_take);
  const __amdgpu_buffer_rsrc_t vi = buffer_view(reinterpret_cast<const float*>(t.oi), t.k);
  const __amdgpu_buffer_rsrc_t vv = buffer_view(t.ov, VALS ? t.k : 0);
  uint32_t n_gt = 0, n_take = 0, eq_seen = 0;
#pragma unroll 1
  for (int32_t e0 = 0; e0 < t.n; e0 += 64) {
    const int32_t e = e0 + lane;
    const uint32_t key = key_at(e);
    const uint32_t o = key_offset(key, kbase);
    const bool gtv = (o >> shift) > bB;
    const bool inv = (o >> shift) == bB;
    const bool eqv = inv && o == t_off;
    const uint64_t mg = __ballot(gtv);
    const uint64_t me = __ballot(eqv);
    const uint32_t epre = eq_seen + lanes_below(me);
    const bool take = (inv && o > t_off) || (eqv && epre < eq_take);
    const uint64_t mt = __ballot(take);
    uint32_t at = 0xFFFFFFFFu;
    if (gtv) at = 4u * (n_gt + lanes_below(mg));
    if (take) at = 4u * (above + n_take + lanes_below(mt));
    if (gtv || take) {
      __builtin_amdgcn_raw_buffer_store_b32(static_cast<uint32_t>(e), vi, at, 0, 0);
      if constexpr (VALS)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(key_value(key)), vv, at, 0, 0);
    }
    n_gt += static_cast<uint32_t>(__popcll(mg));
    n_take += static_cast<uint32_t>(__popcll(mt));
    eq_seen += static_cast<uint32_t>(__popcll(me));
  }
}

// Row segments and candidate lists: output rows sorted by index.
template <int E, bool HAS_IDX>
__global__ __launch_bounds__(256) void topk_wave_kernel(TopkArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t area_all[4][kAreaWords];
  __shared__ uint32_t sub_all[4][kSubBins];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int64_t task = static_cast<int64_t>(blockIdx.x) * 4 + wid;
  if (task >= a.n_rows * a.n_seg) return;
  const WaveTask t = wave_task(a, task);
  if (t.n <= t.k) {
    select_all<HAS_IDX>(t, lane);
    return;
  }
  uint32_t u[E];
  const KeyRange kr = load_keys<E, HAS_IDX>(u, t, lane);
  uint32_t bB, above, c_b;
  bin_of_kth<E>(u, kr, t.k, area_all[wid], lane, &bB, &above, &c_b);
  select_ordered<E, HAS_IDX>(u, kr, t, bB, above, c_b, area_all[wid], sub_all[wid], lane);
}

// Whole rows of scores straight to the caller's output (order within a row unspecified), with
// (VALS) or without their values.
template <int E, bool VALS>
__global__ __launch_bounds__(256) void topk_row_kernel(TopkArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t area_all[4][kAreaWords];
  __shared__ uint32_t sub_all[4][kSubBins];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int64_t task = static_cast<int64_t>(blockIdx.x) * 4 + wid;
  if (task >= a.n_rows) return;
  WaveTask t = wave_task(a, task);
  if constexpr (!VALS) t.ov = nullptr;
  if (t.n <= t.k) {
    select_all<false>(t, lane);
    return;
  }
  uint32_t u[E];
  issue_loads<E>(u, t.row, t.n, lane);
  const KeyRange kr = row_keys<E>(u, t, lane);
  uint32_t bB, above, c_b;
  row_bin_of_kth<E>(u, kr, t.k, area_all[wid], lane, &bB, &above, &c_b);
  if (bB > 0 && c_b <= static_cast<uint32_t>(kRowCand))
    row_select<E, VALS>(u, kr, t, bB, above, c_b, area_all[wid], sub_all[wid], lane);
  else
    select_from_memory<VALS>(kr, t, bB, above, sub_all[wid], lane);
}

// ---------------------------------------------------------------------------------------------
// Batches of few long rows (decode): one workgroup of 16 waves selects one whole row, so that a
// row of up to 16 x 64 x E scores (E <= 32: 32768) is spread over 1024 lanes in a single pass
// instead of a few long-running waves per row.  Wave w holds elements w*64*E + 64 j + lane (contiguous slices, so
// wave order is index order).  The steps are those of the wave kernel, shared through LDS: the
// row's key range (min / max reduced over the waves), one 4096-bin histogram with 32-bit counts,
// the radix refinement of the threshold bin done over the registers of all waves into
// pre-cleared 128-bin histograms (no candidate list, so no capacity limit), and the final
// compaction in index order with per-wave prefix counts of the keys > T and == T.
constexpr int kBlockWaves = 16;
constexpr int kBlockRowsMax = 128;     // batches with at most this many rows use the block kernel
constexpr int kBlockMaxE = 32;        // 1024-lane groups leave 128 VGPRs: up to 32 keys per lane

constexpr int kBlockCand = 4096;       // threshold-bin keys refined from an LDS list

template <int E>
__global__ __launch_bounds__(64 * kBlockWaves) void topk_block_kernel(TopkArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[kBins];
  __shared__ __attribute__((aligned(16))) uint32_t cand[kBlockCand];
  __shared__ __attribute__((aligned(16))) uint32_t sub[3][kSubBins];
  __shared__ uint32_t red[2][kBlockWaves];
  __shared__ uint32_t cnt[2][kBlockWaves];
  __shared__ uint32_t n_cand;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t r = blockIdx.x;
  int64_t len = a.row_len ? static_cast<int64_t>(a.row_len[r]) : a.row_stride;
  len = len < 0 ? 0 : (len > a.row_stride ? a.row_stride : len);
  const int32_t n = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(len));
  const int32_t k = a.k;
  const float* row = a.scores + r * a.row_stride;
  int32_t* oi = a.out_idx + r * k;
  float* ov = a.out_val ? a.out_val + r * k : nullptr;

  if (n <= k) {   // everything is selected, then padding
    for (int32_t e = tid; e < k; e += 64 * kBlockWaves) {
      oi[e] = e < n ? e : -1;
      if (ov) ov[e] = e < n ? key_value(order_key(row[e])) : -INFINITY;
    }
    return;
  }

  // 1. this wave's slice in registers (buffer loads past the row end return 0 -> key 0)
  const int32_t base_w = wid * 64 * E;
  const int32_t groups = min(max((n - base_w + 63) >> 6, 0), E);   // 64-slot groups holding entries
  uint32_t u[E];
  {
    const __amdgpu_buffer_rsrc_t view = buffer_view(row, n);
#pragma unroll
    for (int j = 0; j < E; ++j)
      u[j] = __builtin_amdgcn_raw_buffer_load_b32(view, (base_w + lane) * 4 + j * 256, 0, 0);
  }
  launder(u);
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    u[j] = base_w + j * 64 + lane < n ? order_key(__uint_as_float(u[j])) : 0u;
    kmin = min(kmin, u[j] ? u[j] : 0xFFFFFFFFu);
    kmax = max(kmax, u[j]);
  }
  kmin = wave_min(kmin);
  kmax = wave_max(kmax);
  if (lane == 0) {
    red[0][wid] = kmin;
    red[1][wid] = kmax;
  }
  reinterpret_cast<u32x4*>(hist)[tid] = u32x4{0u, 0u, 0u, 0u};      // 1024 x 16 B = all bins
  if (tid < 3 * kSubBins) (&sub[0][0])[tid] = 0u;
  if (tid == 0) n_cand = 0u;
  __syncthreads();
  kmin = 0xFFFFFFFFu;
  kmax = 0u;
#pragma unroll
  for (int w = 0; w < kBlockWaves; ++w) {
    kmin = min(kmin, red[0][w]);
    kmax = max(kmax, red[1][w]);
  }
  const uint32_t kbase = kmin - 1u;
  const uint32_t top_off = kmax ? kmax - kbase : 0u;
  const int span = top_off ? 32 - __builtin_clz(top_off) : 0;
  const int shift = span > kBinBits ? span - kBinBits : 0;
  auto off_of = [&](uint32_t key) { return key ? key - kbase : 0u; };

  // 2. shared fine histogram
  launder(u);
  {
    const int32_t ng = fresh(groups);
#pragma unroll
    for (int j = 0; j < E; ++j)
      if (j < ng) atomicAdd(&hist[off_of(after(u[j], 0u)) >> shift], 1u);
  }
  __syncthreads();
  uint32_t bB, above, c_b;
  wave_find_bin32<kBins>(hist, static_cast<uint32_t>(k), lane, &bB, &above, &c_b);
  uint32_t k_rem = static_cast<uint32_t>(k) - above;      // 1 <= k_rem <= c_b

  // 3. exact threshold inside bin B: radix passes over its keys, gathered into an LDS list
  //    (one reservation per wave ballot; the list order does not matter) when they fit, else
  //    over every wave's registers
  const bool listed = shift > 0 && c_b <= static_cast<uint32_t>(kBlockCand);
  if (listed) {
    const int32_t ng = fresh(groups);
#pragma unroll
    for (int j = 0; j < E; ++j) {
      if (j < ng) {
        const uint32_t o = off_of(after(u[j], 0u));
        const bool in = (o >> shift) == bB;
        const uint64_t m = __ballot(in);
        if (m) {
          uint32_t at = 0;
          if (lane == 0) at = atomicAdd(&n_cand, static_cast<uint32_t>(__popcll(m)));
          at = lane_value(at, 0);
          if (in) cand[at + lanes_below(m)] = o;
        }
      }
    }
    __syncthreads();
  }
  uint32_t prefix = bB;
  int bits = shift;
#pragma unroll 1
  for (int pass = 0; bits > 0; ++pass) {
    const int w = bits < kSubBits ? bits : kSubBits;
    const int sh = bits - w;
    if (listed) {
      for (uint32_t c = tid; c < c_b; c += 64 * kBlockWaves) {
        const uint32_t o = cand[c];
        if ((o >> bits) == prefix) atomicAdd(&sub[pass][(o >> sh) & ((1u << w) - 1u)], 1u);
      }
    } else {
      const int32_t ng = fresh(groups);
#pragma unroll
      for (int j = 0; j < E; ++j) {
        if (j < ng) {
          const uint32_t o = off_of(after(u[j], 0u));
          if ((o >> bits) == prefix) atomicAdd(&sub[pass][(o >> sh) & ((1u << w) - 1u)], 1u);
        }
      }
    }
    __syncthreads();
    uint32_t d, gt;
    wave_find_digit(sub[pass], k_rem, lane, &d, &gt);
    prefix = (prefix << w) | d;
    k_rem -= gt;
    bits = sh;
  }
  const uint32_t T = prefix ? prefix + kbase : 0u;
  const uint32_t eq_take = k_rem;

  // 4. per-wave counts of keys > T and == T, prefix-summed over the waves
  uint32_t n_gt = 0, n_eq = 0;
  launder(u);
  {
    const int32_t ng = fresh(groups);
#pragma unroll
    for (int j = 0; j < E; ++j) {
      if (j < ng) {
        const uint32_t uj = after(u[j], n_gt + n_eq);
        n_gt += static_cast<uint32_t>(__popcll(__ballot(uj > T)));
        n_eq += static_cast<uint32_t>(__popcll(__ballot(uj == T)));
      }
    }
  }
  if (lane == 0) {
    cnt[0][wid] = n_gt;
    cnt[1][wid] = n_eq;
  }
  __syncthreads();
  uint32_t gt_seen = 0, eq_seen = 0;
  for (int w = 0; w < wid; ++w) {
    gt_seen += cnt[0][w];
    eq_seen += cnt[1][w];
  }

  // 5. compaction in index order (ties: the lowest-indexed keys equal to T)
  launder(u);
  {
    const int32_t ng = fresh(groups);
#pragma unroll
    for (int j = 0; j < E; ++j) {
      if (j < ng) {
        const uint32_t uj = after(u[j], gt_seen + eq_seen);
        const bool gtv = uj > T;
        const bool eqv = uj == T;
        const uint64_t mg = __ballot(gtv);
        const uint64_t me = __ballot(eqv);
        const uint32_t gpre = gt_seen + lanes_below(mg);
        const uint32_t epre = eq_seen + lanes_below(me);
        uint32_t pos = 0xFFFFFFFFu;
        if (gtv) pos = gpre + (epre < eq_take ? epre : eq_take);
        else if (eqv && epre < eq_take) pos = gpre + epre;
        if (pos < static_cast<uint32_t>(k)) {
          oi[pos] = base_w + j * 64 + lane;
          if (ov) ov[pos] = uj ? key_value(uj) : -INFINITY;
        }
        gt_seen += static_cast<uint32_t>(__popcll(mg));
        eq_seen += static_cast<uint32_t>(__popcll(me));
      }
    }
  }
}

namespace seg {

// ---- selection from per-workgroup histograms and scores (decode batches of moderate rows) --------
//
// Workgroup (row r, segment g) of 256 threads, thread t owning scores e0 .. e0 + PER - 1 of the
// segment (e0 = g * seg_len + PER t) and histogram bins 8 t .. 8 t + 7:
//   1. the row's histogram is the sum of its score workgroups' histograms; the bin B holding the
//      k-th largest score, the count `above` of higher bins and B's count c_B follow from a
//      descending scan.  The histograms of the score workgroups before this segment give the
//      numbers of higher-bin and of bin-B keys that precede it in the row;
//   2. every key of a higher bin is a winner and goes straight to its output position (in index
//      order, after the winners of earlier segments); bin B's keys go to the row's candidate list
//      at their position in index order;
//   3. if bin B's keys all win, they go straight to the output instead and nothing more is
//      needed; otherwise the row's last workgroup to finish (one atomic counter per row, zeroed
//      by the score kernel) refines the candidates with two radix passes (11 and 10 bits) to the
//      exact k-th largest key T and how many keys equal to T are taken, then writes the
//      candidates above T and the lowest-indexed ones equal to T after the higher-bin winners.
// The output is deterministic: higher-bin winners in index order, then the threshold bin's.
// Scanning the whole row for bin B in every workgroup instead (no hand-over) was measured slower:
// the scan is bound by issuing per-score work, repeated by every workgroup of the row.
constexpr int kHistWaves = 4;
constexpr int kHistThreads = 64 * kHistWaves;
constexpr int kHistCandLds = 4096;     // candidates refined from LDS; more are read from memory

// Exclusive prefixes over the workgroup (thread order) of N counts, and their totals (one pair
// of barriers for all N).
template <int N>
__device__ __forceinline__ void wg_excl_scan(const uint32_t (&v)[N], uint32_t (*red)[kHistWaves],
                                             int lane, int wid, uint32_t (&pre)[N],
                                             uint32_t (&tot)[N]) {
  uint32_t inc[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    inc[i] = wave_incl_scan(v[i], 0u, [](uint32_t p, uint32_t q) { return p + q; });
    if (lane == 63) red[i][wid] = inc[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    uint32_t o = 0, t = 0;
#pragma unroll
    for (int w = 0; w < kHistWaves; ++w) {
      const uint32_t x = red[i][w];
      o += w < wid ? x : 0u;
      t += x;
    }
    pre[i] = o + inc[i] - v[i];
    tot[i] = t;
  }
  __syncthreads();   // red is reused by the next scan
}

template <int PER>
__global__ __launch_bounds__(kHistThreads) void topk_hist_kernel(HistSelArgs a) {
  __shared__ uint32_t red[4][kHistWaves];
  __shared__ uint32_t info[4];
  __shared__ __attribute__((aligned(16))) uint32_t sub[kHistBins];
  __shared__ __attribute__((aligned(16))) uint64_t lcand[kHistCandLds];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Workgroups go to the 8 XCDs in turn (workgroup b to XCD b % 8): every segment of a row is
  // given to the same XCD, so the row's histograms and scores are read into one L2 and hit there.
  const int64_t slot = blockIdx.x / kXcds;
  const int64_t r = (slot / a.n_seg) * kXcds + blockIdx.x % kXcds;
  const int32_t seg = static_cast<int32_t>(slot % a.n_seg);
  if (r >= a.n_rows) return;
  const int32_t k = a.k;
  const float* row = a.scores + r * a.cols;
  int32_t* oi = a.out_idx + r * k;
  float* ov = a.out_val ? a.out_val + r * k : nullptr;
  const int32_t seg_begin = seg * a.seg_len;
  const int32_t e0 = seg_begin + PER * tid;
  if (tid == 0) {   // defined even if no thread finds the threshold bin below
    info[0] = 0u;
    info[1] = 0u;
    info[2] = 0u;
    info[3] = 0u;
  }
  // The row's visible count, its scores and its histograms are requested together: none of the
  // loads depends on another, so they share one round trip.
  const int32_t len_raw = a.row_nvis[r];

  // scores of this thread (16-byte loads through a view of the row's columns, rounded up to 4,
  // which stays inside the workspace; loads wholly past the view read 0, and slots at or past
  // the visible count are masked below)
  const __amdgpu_buffer_rsrc_t view = buffer_view(row, static_cast<int32_t>((a.cols + 3) & ~3));
  uint32_t key[PER];
#pragma unroll
  for (int j = 0; j < PER; j += 4) {
    const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  view, (e0 + j) * 4, 0, 0));
    key[j] = v.x;
    key[j + 1] = v.y;
    key[j + 2] = v.z;
    key[j + 3] = v.w;
  }

  // 1. the row's histogram (bins 8 t .. 8 t + 7 here), and its part before this segment
  uint32_t tot[8], prev[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) tot[b] = prev[b] = 0u;
  const int32_t w0 = seg * (a.seg_len / a.wg_keys);
  const uint16_t* hrow = a.wg_hist + r * static_cast<int64_t>(a.wg_per_row) * kHistBins + 8 * tid;
  // 16 histograms per round, all requested before the first is summed
  for (int32_t wr = 0; wr < a.wg_per_row; wr += 16) {
    u32x4 h[16];
#pragma unroll
    for (int q = 0; q < 16; ++q)
      h[q] = wr + q < a.wg_per_row
                 ? *reinterpret_cast<const u32x4*>(hrow + static_cast<int64_t>(wr + q) * kHistBins)
                 : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const uint32_t c[8] = {h[q].x & 0xFFFFu, h[q].x >> 16, h[q].y & 0xFFFFu, h[q].y >> 16,
                             h[q].z & 0xFFFFu, h[q].z >> 16, h[q].w & 0xFFFFu, h[q].w >> 16};
      const bool before = wr + q < w0;
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        tot[b] += c[b];
        prev[b] += before ? c[b] : 0u;
      }
    }
  }

  const int64_t len = len_raw < 0 ? 0 : (len_raw > a.cols ? a.cols : len_raw);
  const int32_t n = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(len));
  if (n <= k) {   // every visible key is selected, then padding
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int32_t e = e0 + j;
      if (e < n) {
        oi[e] = e;
        if (ov) ov[e] = key_value(score_order_key(__uint_as_float(key[j])));
      }
    }
    if (seg == 0)
      for (int32_t e = n + tid; e < k; e += kHistThreads) {
        oi[e] = -1;
        if (ov) ov[e] = -INFINITY;
      }
    return;
  }
#pragma unroll
  for (int j = 0; j < PER; ++j)
    key[j] = e0 + j < n ? score_order_key(__uint_as_float(key[j])) : 0u;

  // descending scan: thread t's bins lie above those of every lower thread
  uint32_t mine = 0;
#pragma unroll
  for (int b = 0; b < 8; ++b) mine += tot[b];
  {
    const uint32_t incl = wave_incl_scan(mine, 0u, [](uint32_t p, uint32_t q) { return p + q; });
    if (lane == 63) red[0][wid] = incl;
    __syncthreads();
    uint32_t higher = lane_value(incl, 63) - incl;      // later lanes of this wave
#pragma unroll
    for (int w = 0; w < kHistWaves; ++w)
      if (w > wid) higher += red[0][w];
    if (higher < static_cast<uint32_t>(k) && higher + mine >= static_cast<uint32_t>(k)) {
      uint32_t acc = higher;
#pragma unroll
      for (int b = 7; b >= 0; --b) {
        if (acc < static_cast<uint32_t>(k) && acc + tot[b] >= static_cast<uint32_t>(k)) {
          info[0] = 8 * tid + b;
          info[1] = acc;
          info[2] = tot[b];
        }
        acc += tot[b];
      }
    }
    __syncthreads();
  }
  const uint32_t B = info[0];
  const uint32_t above = min(info[1], static_cast<uint32_t>(k));
  const uint32_t c_b = min(info[2], static_cast<uint32_t>(n));
  const uint32_t k_rem = static_cast<uint32_t>(k) - above;   // 1 <= k_rem <= c_b
  const bool all_win = c_b == k_rem;
  // Every store below is also bounded by its array (k outputs), whatever the counts: they agree
  // with the scores by construction (the scoring kernel counted exactly the values it wrote),
  // and the bounds only keep a broken invariant from writing out of range.

  // 2. higher-bin winners (and, when bin B wins whole, its keys) of this segment
  uint32_t p_hi = 0, p_eq = 0;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const uint32_t bin = 8 * tid + b;
    p_hi += bin > B ? prev[b] : 0u;
    p_eq += bin == B ? prev[b] : 0u;
  }
  uint32_t n_hi = 0, n_eq = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const uint32_t bin = key[j] >> kHistShift;
    n_hi += (e0 + j < n && bin > B) ? 1u : 0u;
    n_eq += (e0 + j < n && bin == B) ? 1u : 0u;
  }
  uint32_t sc_pre[4], sc_tot[4];
  wg_excl_scan<4>({p_hi, p_eq, n_hi, n_eq}, red, lane, wid, sc_pre, sc_tot);
  uint64_t* cand = a.cand + r * a.cols;
  // before this segment (totals of the earlier histograms' counts), then this thread's place
  const uint32_t hi0 = sc_tot[0] + sc_pre[2];
  const uint32_t eq0 = sc_tot[1] + sc_pre[3];
  if (all_win) {
    uint32_t at_hi = hi0, at_eq = eq0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int32_t e = e0 + j;
      const uint32_t bin = key[j] >> kHistShift;
      const bool hi = e < n && bin > B;
      const bool eq = e < n && bin == B;
      if (hi && at_hi < above) {
        oi[at_hi] = e;
        if (ov) ov[at_hi] = key_value(key[j]);
      }
      if (eq && above + at_eq < static_cast<uint32_t>(k)) {
        oi[above + at_eq] = e;
        if (ov) ov[above + at_eq] = key_value(key[j]);
      }
      at_hi += hi ? 1u : 0u;
      at_eq += eq ? 1u : 0u;
    }
    return;
  }

  // A row of one segment is this workgroup's alone: its candidates go to the LDS list, in
  // index order, and the refinement below starts at once (c_b <= seg_len <= kHistCandLds).
  const bool local = a.n_seg == 1;
  if (local) {
    uint32_t at_eq = eq0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int32_t e = e0 + j;
      const bool eq = e < n && (key[j] >> kHistShift) == B;
      if (eq && at_eq < c_b)
        lcand[at_eq] = (static_cast<uint64_t>(key[j]) << 32) | static_cast<uint32_t>(e);
      at_eq += eq ? 1u : 0u;
    }
  }
  // else bin B's keys to the row's candidate list, which the row's last workgroup refines (3.)
  if (!local) {
    uint32_t at_eq = eq0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int32_t e = e0 + j;
      const bool eq = e < n && (key[j] >> kHistShift) == B;
      if (eq && at_eq < c_b) {
        // an agent-scope store writes through to where every XCD's loads of it look
        __hip_atomic_store(cand + at_eq,
                           (static_cast<uint64_t>(key[j]) << 32) | static_cast<uint32_t>(e),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      at_eq += eq ? 1u : 0u;
    }
  }

  // 3. the row's last workgroup refines the threshold bin.  The hand-over needs no cache-wide
  //    write-back or invalidation (an agent-scope fence is both, on every XCD's L2): the
  //    candidates were stored with agent-scope atomic stores, each thread waits until its stores
  //    are acknowledged before the barrier, the counter is an agent-scope atomic, and the last
  //    workgroup reads the candidates with agent-scope atomic loads issued after the counter
  //    returned.  The segment's higher-bin winners are stored after the counter is requested,
  //    as a fixed number of buffer stores (a key that is not one writes past the output view,
  //    which drops the store): the wait for the counter's value then leaves them in flight,
  //    and they hold up neither the hand-over nor the workgroups that are not last.
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  __syncthreads();
  int32_t ticket = a.n_seg - 1;   // a local row's workgroup is its last
  if (tid == 0 && !local)
    ticket = __hip_atomic_fetch_add(a.row_ctr + r, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  {
    const __amdgpu_buffer_rsrc_t vi = buffer_view(reinterpret_cast<const float*>(oi), k);
    const __amdgpu_buffer_rsrc_t vv = buffer_view(ov, ov ? k : 0);
    constexpr uint32_t kDrop = 0x40800000u;   // past every output view (k <= 2048 values)
    uint32_t at_hi = hi0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int32_t e = e0 + j;
      const bool hi = e < n && (key[j] >> kHistShift) > B;
      const uint32_t at = (hi && at_hi < above) ? 4u * at_hi : kDrop;
      __builtin_amdgcn_raw_buffer_store_b32(static_cast<uint32_t>(e), vi, at, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(key_value(key[j])), vv, at, 0, 0);
      at_hi += hi ? 1u : 0u;
    }
  }
  if (tid == 0) info[3] = static_cast<uint32_t>(ticket);
  // LDS-only barrier: the winner stores stay in flight
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt not waited for
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if (info[3] != static_cast<uint32_t>(a.n_seg - 1)) return;

  auto load_cand = [&](uint32_t c) {
    return __hip_atomic_load(cand + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  const bool listed = c_b <= static_cast<uint32_t>(kHistCandLds);
  if (listed && !local) {
    for (uint32_t c = tid; c < c_b; c += kHistThreads) lcand[c] = load_cand(c);
    __syncthreads();
  }
  auto cand_at = [&](uint32_t c) { return listed ? lcand[c] : load_cand(c); };
  // pass 1: bits 20..10 of the keys of bin B; pass 2: bits 9..0 of those in the chosen digit
  uint32_t want = k_rem;
  uint32_t prefix = B;
  uint32_t T = 0u, eq_take = 0u;
  bool resolved = false;
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 10 : 0;
    const int width = pass == 0 ? 11 : 10;
    const int nb = 1 << width;
    for (int c = tid; c < nb; c += kHistThreads) sub[c] = 0u;
    __syncthreads();
    for (uint32_t c = tid; c < c_b; c += kHistThreads) {
      const uint32_t kk = static_cast<uint32_t>(cand_at(c) >> 32);
      if ((kk >> (shift + width)) == prefix) atomicAdd(&sub[(kk >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    uint32_t d, gt, cnt;
    if (pass == 0)
      wave_find_bin32<2048>(sub, want, lane, &d, &gt, &cnt);
    else
      wave_find_bin32<1024>(sub, want, lane, &d, &gt, &cnt);
    prefix = (prefix << width) | d;
    want -= gt;
    __syncthreads();   // sub is cleared again by the next pass
    // Every key of the chosen digit is taken (the usual case: bin B's few hundred keys spread
    // over 2048 digits): the winners are the keys whose top 21 bits are at least `prefix`, i.e.
    // the keys above T = (prefix << 10) - 1 with no tie taken, and the second pass is not needed.
    // (cnt and want come from the same LDS counts in every wave, so the exit is uniform; a zero
    // prefix, only reachable by NaN keys, keeps the second pass.)
    if (pass == 0 && cnt == want && prefix != 0u) {
      T = (prefix << 10) - 1u;
      eq_take = 0u;
      resolved = true;
      break;
    }
  }
  if (!resolved) {
    T = prefix;
    eq_take = want;
  }

  // candidates above T, then the lowest-indexed ones equal to T, after the higher-bin winners:
  // thread t visits a contiguous slice of the (index-ordered) list
  const uint32_t per_t = (c_b + kHistThreads - 1) / kHistThreads;
  const uint32_t c_lo = min(c_b, per_t * tid), c_hi = min(c_b, c_lo + per_t);
  uint32_t m_gt = 0, m_eq = 0;
  for (uint32_t c = c_lo; c < c_hi; ++c) {
    const uint32_t kk = static_cast<uint32_t>(cand_at(c) >> 32);
    m_gt += kk > T ? 1u : 0u;
    m_eq += kk == T ? 1u : 0u;
  }
  uint32_t o_pre[2], o_tot[2];
  wg_excl_scan<2>({m_gt, m_eq}, red, lane, wid, o_pre, o_tot);
  uint32_t g_before = o_pre[0], e_before = o_pre[1];
  for (uint32_t c = c_lo; c < c_hi; ++c) {
    const uint64_t ce = cand_at(c);
    const uint32_t kk = static_cast<uint32_t>(ce >> 32);
    uint32_t pos = 0xFFFFFFFFu;
    if (kk > T) pos = g_before + min(e_before, eq_take);
    else if (kk == T && e_before < eq_take) pos = g_before + e_before;
    if (pos < k_rem) {
      oi[above + pos] = static_cast<int32_t>(static_cast<uint32_t>(ce));
      if (ov) ov[above + pos] = key_value(kk);
    }
    g_before += kk > T ? 1u : 0u;
    e_before += kk == T ? 1u : 0u;
  }
}

}  // namespace seg

namespace lst {

// ---- selection from bucketed lists (decode batches of long rows) --------------------------------
//
// One workgroup of 1024 threads per row.  The scoring kernel left, for each of its workgroups j
// of the row, a histogram of the order keys' top 11 bits, the start of every bin's bucket, and
// the keys bucketed by bin, highest bin first (see ScoreArgs).  Thread t owns bins 2 t, 2 t + 1:
//   1. the row's histogram is the sum of its workgroups'; a descending scan gives the bin B that
//      holds the k-th largest key, the count `above` of higher bins and B's count c_B;
//   2. list j holds hi_j keys of higher bins at its front and bin B's eq_j keys behind them
//      (two 16-bit loads per list); prefix sums over the lists place them: the `above` winners
//      and bin B's keys are loaded into registers;
//   3. unless bin B's keys all win, two radix passes over them (bits 20..10, then 9..0) give the
//      exact k-th largest key T and how many keys equal to T win; when they are only some of
//      the keys equal to T, a bitmap of those keys' indices gives the index of the last one
//      taken (ties go to the lower index);
//   4. a bitmap of the winners' indices and its running popcount give every winner its output
//      position: each row comes out sorted by index, and the result is deterministic although
//      the buckets are filled in no set order.
// The scoring kernel writes no bucket below its workgroup's own k-th largest key; every read
// here is of a bucket at or above B, which lies at or above each of those.
constexpr int kHistWaves = 16;         // 1024 threads: 4 waves per SIMD on the row's CU
constexpr int kHistThreads = 64 * kHistWaves;
constexpr int kBinsPer = kHistBins / kHistThreads;   // histogram bins per thread
constexpr int kListCandLds = 4096;     // bin B's keys held in registers; more are read from the lists
constexpr int kSpec = 6;               // list positions each thread reads before the threshold is known
constexpr int kBitWords = kHistMaxCols / 32;
constexpr int kWordsPerThread = kBitWords / kHistThreads;
static_assert(kWordsPerThread * kHistThreads == kBitWords && kWordsPerThread % 4 == 0,
              "bitmap words per thread");
static_assert(kBitWords * 2 <= kHistBins * 4, "16-bit word ranks fit the digit counts' area");

// Exclusive prefixes over the workgroup (thread order) of N counts, and their totals (one pair
// of barriers for all N).
template <int N>
__device__ __forceinline__ void wg_excl_scan(const uint32_t (&v)[N], uint32_t (*red)[kHistWaves],
                                             int lane, int wid, uint32_t (&pre)[N],
                                             uint32_t (&tot)[N]) {
  uint32_t inc[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    inc[i] = wave_incl_scan(v[i], 0u, [](uint32_t p, uint32_t q) { return p + q; });
    if (lane == 63) red[i][wid] = inc[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    uint32_t o = 0, t = 0;
#pragma unroll
    for (int w = 0; w < kHistWaves; ++w) {
      const uint32_t x = red[i][w];
      o += w < wid ? x : 0u;
      t += x;
    }
    pre[i] = o + inc[i] - v[i];
    tot[i] = t;
  }
  __syncthreads();   // red is reused by the next scan
}

// The lists holding entries f[0..N) of a run laid out list after list: for each, the largest
// j < n with off[j] <= f (off non-decreasing from off[0] = 0, so empty lists are passed over).
// A branch-free search of fixed depth (n <= kMaxHistWgPerRow), so that the N searches' LDS reads
// are in flight together.
template <int N>
__device__ __forceinline__ void lists_of(const uint32_t* off, int n, const uint32_t (&f)[N],
                                         int (&j)[N]) {
  static_assert(kMaxHistWgPerRow == 64, "six halving steps");
#pragma unroll
  for (int u = 0; u < N; ++u) j[u] = 0;
#pragma unroll
  for (int step = 32; step >= 1; step >>= 1) {
#pragma unroll
    for (int u = 0; u < N; ++u) {
      const int mid = min(j[u] + step, n - 1);
      j[u] = off[mid] <= f[u] ? mid : j[u];
    }
  }
}

__global__ __launch_bounds__(kHistThreads) void topk_list_kernel(ListSelArgs a) {
  __shared__ uint32_t red[4][kHistWaves];
  __shared__ uint32_t info[8];
  __shared__ __attribute__((aligned(16))) uint32_t hist_l[kHistBins];   // the row's histogram
  __shared__ __attribute__((aligned(16))) uint32_t sub[kHistBins];      // digit counts, then ranks
  __shared__ __attribute__((aligned(16))) uint32_t bits[kBitWords];
  __shared__ uint32_t lhoff[kMaxHistWgPerRow], leoff[kMaxHistWgPerRow], lhi[kMaxHistWgPerRow];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t r = blockIdx.x;
  if (r >= a.n_rows) return;
  static_assert(kHistBins == 2 * kHistThreads, "two digit counters per thread");
  const int32_t k = a.k;
  const int32_t wpr = a.wg_per_row;
  const int32_t wk = a.wg_keys;
  const uint64_t* lrow = a.wg_list + r * wpr * static_cast<int64_t>(wk);
  int32_t* oi = a.out_idx + r * k;
  float* ov = a.out_val ? a.out_val + r * k : nullptr;
  if (tid < 8) info[tid] = 0u;
  reinterpret_cast<u32x4*>(bits)[tid] = u32x4{0u, 0u, 0u, 0u};
  reinterpret_cast<uint2*>(sub)[tid] = uint2{0u, 0u};
  reinterpret_cast<uint2*>(hist_l)[tid] = uint2{0u, 0u};
  // The front of every list, read before anything about the row is known: thread t reads
  // positions q + tpl u (u < kSpec) of list t / tpl, tpl = 1024 / wg_per_row threads per list,
  // within the first min(kSpec tpl, k) positions.  A list's keys of bin B and above lie at its
  // front; they are usually all inside this window, which is then all that is read.
  // (info: [5] keys in the window, [7] one above the highest bin at which the window cuts a list.)
  const int tpl = kHistThreads / wpr;
  const int sj = tid / tpl, sq = tid % tpl;
  const int32_t swin = min(min(kSpec * tpl, k), wk);
  uint64_t spec[kSpec];
#pragma unroll
  for (int u = 0; u < kSpec; ++u) {
    const int32_t p = sq + tpl * u;
    spec[u] = sj < wpr && p < swin ? lrow[static_cast<int64_t>(sj) * wk + p] : 0ull;
  }
  const int32_t len_raw = a.row_nvis[r];
  const int64_t len = len_raw < 0 ? 0 : (len_raw > a.cols ? a.cols : len_raw);
  const int32_t n = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(len));
  if (n <= k) {
    // Every visible key is selected.  No workgroup of the row holds more than k keys, so every
    // list is written in full, and the lists' n entries lie at the front of the row's area.
    // All of a thread's entries are requested before any is stored.
    constexpr int kPer = kMaxTopk / kHistThreads;
    uint64_t e[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int32_t f = tid + kHistThreads * u;
      e[u] = f < n ? lrow[f] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const uint32_t idx = static_cast<uint32_t>(e[u]);
      if (tid + kHistThreads * u < n && idx < static_cast<uint32_t>(k)) {
        oi[idx] = static_cast<int32_t>(idx);
        if (ov) ov[idx] = key_value(static_cast<uint32_t>(e[u] >> 32));
      }
    }
    for (int32_t f = n + tid; f < k; f += kHistThreads) {
      oi[f] = -1;
      if (ov) ov[f] = -INFINITY;
    }
    return;
  }

  // 1. The bin B holding the k-th largest key, from an LDS histogram of the window.  A position
  //    below min(the workgroup's key count, k) always holds one of its keys (the scoring kernel
  //    leaves out only keys below its own k-th largest), and a list is bucketed from its highest
  //    bin down, so the window holds all of a list's keys of every bin above the bin of its last
  //    window entry.  When the bin where the window's count from the top reaches k lies above
  //    every such cut, it is the row's B, and the window holds every key of B and above.
  //    Otherwise the workgroups' histograms give B and the lists are read in full (below).
  __syncthreads();   // the LDS counters cleared above are zero before any thread adds to them
  const int64_t cnt_l =
      sj < wpr ? min<int64_t>(max<int64_t>(n - static_cast<int64_t>(sj) * wk, 0), wk) : 0;
  const int32_t lim = static_cast<int32_t>(min<int64_t>(cnt_l, swin));
  {
    // The lanes of a wave hold consecutive positions of a list (for each u), and a list's
    // buckets are runs of positions, so equal bins sit in runs of lanes: the first lane of each
    // run adds the run's length (one LDS add per bin instead of one per key; the window's keys
    // crowd into a few bins).
    uint32_t nv = 0;
#pragma unroll
    for (int u = 0; u < kSpec; ++u) {
      const int32_t p = sq + tpl * u;
      const bool in = p < lim;
      const uint32_t bin = in ? static_cast<uint32_t>(spec[u] >> 32) >> kHistShift : 0xFFFFFFFFu;
      // the previous lane's bin (DPP wave_shr:1); lane 0 has none
      const uint32_t prev = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
          static_cast<int>(0xFFFFFFFEu), static_cast<int>(bin), 0x138, 0xF, 0xF, false));
      const bool head = in && (sq == 0 || prev != bin);
      const uint64_t ends = __ballot(head) | __ballot(!in);   // a run stops before these lanes
      if (head) {
        const uint64_t later = lane == 63 ? 0ull : ends >> (lane + 1);
        const uint32_t run = later ? static_cast<uint32_t>(__builtin_ctzll(later)) + 1u
                                   : static_cast<uint32_t>(64 - lane);
        atomicAdd(&hist_l[bin], run);
      }
      nv += in ? 1u : 0u;
      if (in && p == lim - 1 && lim < cnt_l) atomicMax(&info[7], bin + 1u);   // the list is cut here
    }
    nv = wave_incl_scan(nv, 0u, [](uint32_t p, uint32_t q) { return p + q; });
    if (lane == 63) atomicAdd(&info[5], nv);
  }
  __syncthreads();
  uint32_t B, above_raw, count_b;
  wave_find_bin32<kHistBins>(hist_l, static_cast<uint32_t>(k), lane, &B, &above_raw, &count_b);
  // Every bin above B lies above every cut when B is at or above the highest cut bin: then B
  // and the count above it are the row's.  Bin B itself is whole in the window only when B lies
  // above every cut.
  const bool b_ok = info[5] >= static_cast<uint32_t>(k) && B + 1u >= info[7];
  const bool fast = b_ok && B >= info[7];
  if (!b_ok) {
    // the row's histogram: the sum of its workgroups' (thread t: bins 2 t, 2 t + 1)
    static_assert(kBinsPer == 2, "two 16-bit counts per thread and list");
    uint32_t tot[kBinsPer] = {0u, 0u};
    const uint32_t* hrow = reinterpret_cast<const uint32_t*>(
        a.wg_hist + r * static_cast<int64_t>(wpr) * kHistBins + kBinsPer * tid);
    for (int32_t wr = 0; wr < wpr; wr += 16) {   // 16 histograms requested before any is summed
      uint32_t h[16];
#pragma unroll
      for (int q = 0; q < 16; ++q)
        h[q] = wr + q < wpr ? hrow[static_cast<int64_t>(wr + q) * (kHistBins / 2)] : 0u;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        tot[0] += h[q] & 0xFFFFu;
        tot[1] += h[q] >> 16;
      }
    }
    __syncthreads();   // every wave has read the window's histogram
    reinterpret_cast<uint2*>(hist_l)[tid] = uint2{tot[0], tot[1]};
    __syncthreads();
    wave_find_bin32<kHistBins>(hist_l, static_cast<uint32_t>(k), lane, &B, &above_raw, &count_b);
  }
  if (!fast) {
    // list j holds hi_j keys of higher bins at its front and bin B's eq_j keys behind them (two
    // 16-bit loads per list); prefix sums over the lists place them, and their total of bin B
    // is B's count
    uint32_t hj = 0, ej = 0;
    if (tid < wpr) {
      const int64_t L = (r * wpr + tid) * static_cast<int64_t>(kHistBins) + B;
      hj = a.wg_off[L];
      ej = a.wg_hist[L];
    }
    uint32_t pre[2], sums[2];
    wg_excl_scan<2>({hj, ej}, red, lane, wid, pre, sums);
    if (tid < wpr) {
      lhoff[tid] = pre[0];
      leoff[tid] = pre[1];
      lhi[tid] = hj;
    }
    count_b = sums[1];
    __syncthreads();
  }
  const uint32_t above = min(above_raw, static_cast<uint32_t>(k));
  const uint32_t c_b = min(count_b, static_cast<uint32_t>(n));
  const uint32_t k_rem = static_cast<uint32_t>(k) - above;   // 1 <= k_rem <= c_b
  const bool all_win = c_b == k_rem;
  // Every access below is also bounded by its array, whatever the counts: they agree with the
  // lists by construction (the scoring kernel counted exactly the keys it bucketed), and the
  // bounds only keep a broken invariant from reading or writing out of range.

  // 2. The window's keys of higher bins (winners) and of bin B (candidates), and the
  //    candidates' first radix digits (bits 20..10).
  uint32_t hm = 0u, em = 0u;   // bit u: spec[u] is a higher-bin key / a bin-B key
  if (fast) {
#pragma unroll
    for (int u = 0; u < kSpec; ++u) {
      const uint32_t kk = static_cast<uint32_t>(spec[u] >> 32);
      const uint32_t bin = kk >> kHistShift;
      const bool in = sq + tpl * u < lim;
      const bool h = in && bin > B, e = in && bin == B;
      hm |= h ? 1u << u : 0u;
      em |= e ? 1u << u : 0u;
      if (e && !all_win) atomicAdd(&sub[(kk >> 10) & (kHistBins - 1)], 1u);
    }
    __syncthreads();
  }
  // Otherwise every list's keys of bin B and above are read in full, from the places found
  // above: kMaxTopk / 1024 winners and kListCandLds / 1024 candidates per thread (candidates
  // beyond that are read from the lists where needed).
  constexpr int kHiPer = kMaxTopk / kHistThreads;
  constexpr int kEqPer = kListCandLds / kHistThreads;
  static_assert(kHiPer + kEqPer <= kSpec, "the searched path reuses the window's registers");
  const bool listed = fast || c_b <= static_cast<uint32_t>(kListCandLds);
  auto entry = [&](int j, uint32_t p) -> uint64_t {
    return p < static_cast<uint32_t>(wk) ? lrow[static_cast<int64_t>(j) * wk + p] : 0ull;
  };
  auto cand_mem = [&](uint32_t f) -> uint64_t {
    uint32_t ff[1] = {f};
    int j[1];
    lists_of<1>(leoff, wpr, ff, j);
    return entry(j[0], lhi[j[0]] + f - leoff[j[0]]);
  };
  // fn(e) for every key of bin B
  auto for_cand = [&](auto fn) {
    if (listed) {
#pragma unroll
      for (int u = 0; u < kSpec; ++u)
        if (em & (1u << u)) fn(spec[u]);
    } else {
      for (uint32_t c = tid; c < c_b; c += kHistThreads) fn(cand_mem(c));
    }
  };
  if (!fast) {
    hm = 0u;
    em = 0u;
    uint32_t fh[kHiPer], fe[kEqPer];
    int jh[kHiPer], je[kEqPer];
#pragma unroll
    for (int u = 0; u < kHiPer; ++u) fh[u] = tid + kHistThreads * u;
#pragma unroll
    for (int u = 0; u < kEqPer; ++u) fe[u] = tid + kHistThreads * u;
    lists_of<kHiPer>(lhoff, wpr, fh, jh);
    lists_of<kEqPer>(leoff, wpr, fe, je);
#pragma unroll
    for (int u = 0; u < kHiPer; ++u) {
      const bool h = fh[u] < above;
      spec[u] = h ? entry(jh[u], fh[u] - lhoff[jh[u]]) : 0ull;
      hm |= h ? 1u << u : 0u;
    }
#pragma unroll
    for (int u = 0; u < kEqPer; ++u) {
      const bool e = listed && fe[u] < c_b;
      spec[kHiPer + u] = e ? entry(je[u], lhi[je[u]] + fe[u] - leoff[je[u]]) : 0ull;
      em |= e ? 1u << (kHiPer + u) : 0u;
    }
    if (!all_win) {   // the first digits again, over every candidate
      for (int c = tid; c < kHistBins; c += kHistThreads) sub[c] = 0u;
      __syncthreads();
      for_cand([&](uint64_t e) {
        atomicAdd(&sub[(static_cast<uint32_t>(e >> 32) >> 10) & (kHistBins - 1)], 1u);
      });
      __syncthreads();
    }
  }

  // 3. the exact threshold T among bin B's keys, and which keys equal to T win.  Every key of
  //    the chosen first digit usually wins (bin B's few hundred keys spread over 2048 digits):
  //    then the winners are the keys above T = (prefix << 10) - 1, no tie taken, and the second
  //    digit (bits 9..0) is not needed.  (The digit counts are the same LDS values in every
  //    wave, so every branch here is uniform; a zero prefix, only reachable by NaN keys, takes
  //    the second digit.)
  uint32_t T = 0u, eq_take = 0u;
  bool ties_all = true;   // every key equal to T that is a candidate wins
  if (!all_win) {
    uint32_t d, gt, cnt;
    wave_find_bin32<kHistBins>(sub, k_rem, lane, &d, &gt, &cnt);
    const uint32_t prefix = (B << 11) | d;
    uint32_t want = k_rem - gt;
    if (cnt == want && prefix != 0u) {
      T = (prefix << 10) - 1u;
    } else {
      __syncthreads();   // every wave has read the first digits' counts
      for (int c = tid; c < 1024; c += kHistThreads) sub[c] = 0u;
      __syncthreads();
      for_cand([&](uint64_t e) {
        const uint32_t kk = static_cast<uint32_t>(e >> 32);
        if ((kk >> 10) == prefix) atomicAdd(&sub[kk & 1023u], 1u);
      });
      __syncthreads();
      uint32_t d2, gt2, cnt2;
      wave_find_bin32<1024>(sub, want, lane, &d2, &gt2, &cnt2);
      want -= gt2;
      T = (prefix << 10) | d2;
      eq_take = want;
      ties_all = cnt2 == want;
    }
  }
  auto wins = [&](uint32_t kk, uint32_t idx, uint32_t cut) {
    return all_win || kk > T || (kk == T && eq_take > 0u && (ties_all || idx <= cut));
  };
  auto set_bit = [&](uint32_t idx) {
    if (idx < static_cast<uint32_t>(kHistMaxCols)) atomicOr(&bits[idx >> 5], 1u << (idx & 31));
  };
  // Thread t owns bitmap words 4 t .. 4 t + 3: the set bits before each of them (after the
  // barrier the caller provides once every bit is set), using partial-sum slot `slot` of red.
  auto word_ranks = [&](int slot, uint32_t (&pre)[4]) {
    static_assert(kWordsPerThread == 4, "one 16-byte word group per thread");
    const u32x4 x = reinterpret_cast<const u32x4*>(bits)[tid];
    pre[0] = 0u;
    pre[1] = __popc(x.x);
    pre[2] = pre[1] + __popc(x.y);
    pre[3] = pre[2] + __popc(x.z);
    const uint32_t mine = pre[3] + __popc(x.w);
    const uint32_t incl = wave_incl_scan(mine, 0u, [](uint32_t p, uint32_t q) { return p + q; });
    if (lane == 63) red[slot][wid] = incl;
    __syncthreads();
    uint32_t base = incl - mine;
#pragma unroll
    for (int w = 0; w < kHistWaves; ++w) base += w < wid ? red[slot][w] : 0u;
#pragma unroll
    for (int c = 0; c < 4; ++c) pre[c] += base;
  };
  uint32_t cut = 0xFFFFFFFFu;
  if (!ties_all) {
    // some of the keys equal to T win: the eq_take lowest-indexed ones, up to index `cut`
    for_cand([&](uint64_t e) {
      if (static_cast<uint32_t>(e >> 32) == T) set_bit(static_cast<uint32_t>(e));
    });
    __syncthreads();
    uint32_t pre[4];
    word_ranks(2, pre);
    const u32x4 x = reinterpret_cast<const u32x4*>(bits)[tid];
    const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t cnt = __popc(w4[c]);
      if (pre[c] < eq_take && pre[c] + cnt >= eq_take) {
        uint32_t y = w4[c];
        for (uint32_t i = pre[c] + 1; i < eq_take; ++i) y &= y - 1u;   // drop the lower bits taken
        info[4] = 32u * (4 * tid + c) + static_cast<uint32_t>(__builtin_ctz(y));
      }
    }
    __syncthreads();
    reinterpret_cast<u32x4*>(bits)[tid] = u32x4{0u, 0u, 0u, 0u};
    cut = info[4];
    __syncthreads();
  }

  // 4. output positions from the bitmap of the winners' indices
  uint32_t wm = hm;   // bit u: spec[u] wins
#pragma unroll
  for (int u = 0; u < kSpec; ++u)
    if ((em & (1u << u)) &&
        wins(static_cast<uint32_t>(spec[u] >> 32), static_cast<uint32_t>(spec[u]), cut))
      wm |= 1u << u;
#pragma unroll
  for (int u = 0; u < kSpec; ++u)
    if (wm & (1u << u)) set_bit(static_cast<uint32_t>(spec[u]));
  if (!listed) {
    for (uint32_t c = tid; c < c_b; c += kHistThreads) {
      const uint64_t e = cand_mem(c);
      if (wins(static_cast<uint32_t>(e >> 32), static_cast<uint32_t>(e), cut))
        set_bit(static_cast<uint32_t>(e));
    }
  }
  __syncthreads();
  uint16_t* rank16 = reinterpret_cast<uint16_t*>(sub);   // output position of each word's first
  {
    uint32_t pre[4];
    word_ranks(3, pre);
#pragma unroll
    for (int c = 0; c < 4; ++c) rank16[4 * tid + c] = static_cast<uint16_t>(pre[c]);
  }
  __syncthreads();
  auto pos_of = [&](uint32_t idx, uint32_t rank_w, uint32_t word) {
    return rank_w + __popc(word & ((1u << (idx & 31)) - 1u));
  };
  auto put = [&](uint64_t e, uint32_t pos) {
    if (pos < static_cast<uint32_t>(k)) {
      oi[pos] = static_cast<int32_t>(static_cast<uint32_t>(e));
      if (ov) ov[pos] = key_value(static_cast<uint32_t>(e >> 32));
    }
  };
  {
    // every word read first, then the stores
    uint32_t rw[kSpec], bw[kSpec];
#pragma unroll
    for (int u = 0; u < kSpec; ++u) {
      const uint32_t idx = static_cast<uint32_t>(spec[u]);
      const uint32_t w =
          (wm & (1u << u)) && idx < static_cast<uint32_t>(kHistMaxCols) ? idx >> 5 : 0u;
      rw[u] = rank16[w];
      bw[u] = bits[w];
    }
#pragma unroll
    for (int u = 0; u < kSpec; ++u)
      if ((wm & (1u << u)) && static_cast<uint32_t>(spec[u]) < static_cast<uint32_t>(kHistMaxCols))
        put(spec[u], pos_of(static_cast<uint32_t>(spec[u]), rw[u], bw[u]));
  }
  if (!listed) {
    for (uint32_t c = tid; c < c_b; c += kHistThreads) {
      const uint64_t e = cand_mem(c);
      const uint32_t idx = static_cast<uint32_t>(e);
      if (wins(static_cast<uint32_t>(e >> 32), idx, cut) && idx < static_cast<uint32_t>(kHistMaxCols))
        put(e, pos_of(idx, rank16[idx >> 5], bits[idx >> 5]));
    }
  }
}

}  // namespace lst

bool use_block(int64_t n_rows, int64_t cols) {
  return n_rows <= kBlockRowsMax && cols <= static_cast<int64_t>(kBlockWaves) * 64 * kBlockMaxE;
}

hipError_t launch_block(const TopkArgs& a, int64_t cols, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(a.n_rows)), block(64 * kBlockWaves);
  if (cols <= kBlockWaves * 64 * 8)
    hipLaunchKernelGGL(topk_block_kernel<8>, grid, block, 0, stream, a);
  else if (cols <= kBlockWaves * 64 * 16)
    hipLaunchKernelGGL(topk_block_kernel<16>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(topk_block_kernel<kBlockMaxE>, grid, block, 0, stream, a);
  return hipGetLastError();
}

template <int E>
hipError_t launch_wave(const TopkArgs& a, hipStream_t stream) {
  const int64_t tasks = a.n_rows * a.n_seg;
  const int64_t blocks = (tasks + 3) / 4;
  if (a.n_seg == 1 && !a.src_idx && !a.pad_bits && a.out_val)
    hipLaunchKernelGGL((topk_row_kernel<E, true>), dim3(static_cast<uint32_t>(blocks)), dim3(256),
                       0, stream, a);
  else if (a.n_seg == 1 && !a.src_idx && !a.pad_bits)
    hipLaunchKernelGGL((topk_row_kernel<E, false>), dim3(static_cast<uint32_t>(blocks)), dim3(256),
                       0, stream, a);
  else if (a.src_idx)
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

hipError_t launch_topk_hist(const HistSelArgs& a, hipStream_t stream) {
  if (a.n_rows <= 0) return hipSuccess;
  // rows rounded up to a multiple of the XCD count (see the row mapping in the kernel)
  const int64_t rows8 = (a.n_rows + kXcds - 1) / kXcds * kXcds;
  const dim3 grid(static_cast<uint32_t>(rows8 * a.n_seg)), block(64 * seg::kHistWaves);
  if (a.seg_len == 16 * seg::kHistThreads)
    hipLaunchKernelGGL(seg::topk_hist_kernel<16>, grid, block, 0, stream, a);
  else if (a.seg_len == 8 * seg::kHistThreads)
    hipLaunchKernelGGL(seg::topk_hist_kernel<8>, grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_topk_list(const ListSelArgs& a, hipStream_t stream) {
  if (a.n_rows <= 0) return hipSuccess;
  if (a.k < 1 || a.k > kMaxTopk || a.cols > kHistMaxCols || a.wg_per_row < 1 ||
      a.wg_per_row > kMaxHistWgPerRow || a.wg_keys < 1 || a.wg_keys > kHistWgKeysMax ||
      static_cast<int64_t>(a.wg_per_row) * a.wg_keys < a.cols)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(lst::topk_list_kernel, dim3(static_cast<uint32_t>(a.n_rows)), dim3(lst::kHistThreads), 0,
                     stream, a);
  return hipGetLastError();
}

TopkPlan topk_plan(int64_t n_rows, int64_t cols, int32_t k) {
  TopkPlan p{};
  p.passes = 1;
  p.cand_elems = 0;
  if (use_block(n_rows, cols)) return p;
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

int64_t topk_cand_bound(int64_t cols, int32_t k) {
  // The first pass cuts a row into at most max(need, min(fit, usable)) segments (the wave
  // spread only lowers the count as rows grow); each later pass's candidate row is no wider,
  // because ceil(ns * k / kMaxSegment) <= ns for k <= kMaxSegment.
  const int64_t need = (cols + kMaxSegment - 1) / kMaxSegment;
  int64_t want = kMaxSegment / k;
  const int64_t usable = cols / (2 * static_cast<int64_t>(k));
  if (want > usable) want = usable;
  int64_t ns = need > want ? need : want;
  if (ns <= 1) return 0;
  return ns * k;
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
  if (use_block(n_rows, cols)) {
    a.n_seg = 1;
    a.seg_len = 0;
    a.out_idx = out_idx;
    a.out_val = out_val;
    return launch_block(a, cols, stream);
  }
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
