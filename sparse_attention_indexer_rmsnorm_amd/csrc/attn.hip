// Sparse attention over the keys the indexer selects: for query row i and head h, a softmax over
// the listed entries of q[i][h] . v_j (scaled), and the weighted sum of the 512-dim latents v_j,
// which serve as key and value of every head ("When the Fused Kernel Isn't Enough", Input
// Knowledge: the sparse attention reads the top-K entries, the main KV cache is bf16 with
// head_dim 512; "The Fused Kernel Decision", Message: that cache is unpaged, one slot per entry).
//
// Work items are (query row, split of the list, block of HW = min(H, 64) heads); a workgroup of
// HW / 16 waves, one per CU (its LDS fills the CU), takes items blockIdx.x, blockIdx.x + G, ...
// (G workgroups), and loads the next item's list entries, latent rows and q while it works on the
// current one, so only the first item waits for them.  Wave w owns 32 heads of the block,
// 32 (w / 2) .., and one half of the 512 output dims, 256 (w % 2) ...  Per 32 listed keys:
//   1. the keys' latents go from global memory straight into LDS (global_load_lds_dwordx4: one
//      instruction per 1 KB latent row, each lane's 16 bytes landing at its own slot), up to three
//      chunks ahead of their use in four buffers, so no registers or VALU work stage them; the
//      16-byte chunks of row r are XOR-swizzled by sw(r) = 2 (r % 4) + (r / 4) % 2;
//   2. S^T = K Q^T on bf16 MFMA 32x32x16 with the latents as A operand (ds_read_b128): each wave
//      of a pair sums over its own 256 dims, and the pair swaps partial sums through LDS (fp32
//      addition commutes, so both hold the same S);
//   3. online softmax in base 2: each lane owns one head and 16 of the 32 keys, the maximum is
//      shared with the lane holding the other 16, a reference maximum moves only when exceeded
//      by more than 2^8, and the weights are rounded to bf16 (the weight sum adds the rounded
//      values, so the weights used sum to the divisor);
//   4. O^T += K^T P^T on the same MFMA: the accumulator of S^T, rounded, is already the B operand
//      of this product (lane = head, 8 keys), and the A operand, latents transposed to (dim,
//      4 keys) per lane, comes from the same row-major buffer through gfx950's transposing LDS
//      read ds_read_b64_tr_b16 (in each 16-lane group, lane j's element f is element j % 4 of
//      lane 4 f + j / 4's 8-byte read).
// Chunks are software-pipelined: S of chunk c + 1 is issued before the softmax of chunk c, so
// its MFMAs run while the VALU computes the weights.
// Batches of few rows split each list over several workgroups; a second kernel merges their
// partial outputs by their maxima and weight sums.

#include <math.h>

#include "attn.h"

namespace dsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

union AFrag {
  bf16x8 v;
  u32x4 u;
};

constexpr int kRowBytes = kLatentDim * 2;                  // 1024: one latent
constexpr int kChunkBytes = kAttnChunk * kRowBytes;         // 32 KB
constexpr int kAttnBufs = 4;                                // chunk buffers in LDS

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Sequence b with cu_q[b] <= i < cu_q[b + 1], or -1.  i is workgroup-uniform and the table
// read-only, so it is read through the constant address space: scalar loads, which leave the
// vector memory counter (and the transfers it tracks) alone.
__device__ __forceinline__ int32_t seq_of_row(const int32_t* cu_q_ptr, int32_t n_seq, int64_t i) {
  typedef __attribute__((address_space(4))) const int32_t const_i32;
  const_i32* cu_q = (const_i32*)cu_q_ptr;
  if (n_seq <= 0 || i < cu_q[0] || i >= cu_q[n_seq]) return -1;
  int32_t lo = 0, hi = n_seq;
  while (hi - lo > 1) {
    const int32_t mid = (lo + hi) >> 1;
    if (cu_q[mid] <= i) lo = mid;
    else hi = mid;
  }
  return lo;
}

// 16-byte chunk c of latent row r (r < 32) sits at chunk c ^ sw(r) of the buffer row.  Eight
// consecutive rows (one operand read of 8 lanes) get eight distinct values, and the rows 4u..4u+3
// of one transposing read get four distinct values of bits 1-2, i.e. four distinct 32-byte
// groups of banks.
__device__ __forceinline__ int sw(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, not for its
// global loads, so the next chunk's latents stay in flight across it (a __syncthreads() fence
// would wait for them too).  The empty asm statements keep the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // gfx9: lgkmcnt 0, vmcnt 63 and expcnt 7 (no wait)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One 16-byte global-to-LDS transfer per lane (global_load_lds_dwordx4): lane L's 16 bytes land
// at LDS byte lds + 16 L, lds being wave-uniform.  Written as inline assembly so that the
// compiler does not see an LDS write: it cannot tell the four chunk buffers apart and would
// otherwise wait for every transfer in flight before each LDS read.  The kernel orders the
// buffers itself, with counter waits and barriers.  (M0 takes the LDS address; one wait state
// separates its write from the transfer.)
__device__ __forceinline__ void dma_row16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds)
               : "memory", "m0");
}

template <int HW>
__global__ __launch_bounds__(HW * 4) void sparse_attn_kernel(AttnArgs a) {
  constexpr int NW = HW / 16;                  // waves
  constexpr int NT = 64 * NW;
  constexpr int kRowsPerWave = kAttnChunk / NW;
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[kAttnBufs][kChunkBytes];   // latents
  __shared__ __attribute__((aligned(16))) float ex[NW * 16 * 64];         // S^T partial sums
  __shared__ __attribute__((aligned(16))) int32_t sl[kMaxAttnList];   // latent row per entry, -1 none
  __shared__ int32_t last_w[NW];              // per wave: one past its last valid entry

  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int hg = wid >> 1, dh = wid & 1;
  const int m = lane & 31, g = lane >> 5;
  const int H = a.n_heads;
  const int n_hb = H / HW;
  const int64_t n_items = a.n_q * a.n_split * n_hb;

  // Item it = (i * n_split + sp) * n_hb + hb: row i, split sp, head block hb; b is its sequence.
  struct Item {
    int64_t i;
    int32_t b;
    int sp, hb, n_list;
  };
  auto item_of = [&](int64_t it) {
    Item t;
    const int64_t rs = it / n_hb;
    t.hb = static_cast<int>(it - rs * n_hb);
    t.i = rs / a.n_split;
    t.sp = static_cast<int>(rs - t.i * a.n_split);
    t.b = seq_of_row(a.cu_q, a.n_seq, t.i);
    const int j0 = t.sp * a.split_keys;
    t.n_list = t.b >= 0 ? max(0, min(a.k, j0 + a.split_keys) - j0) : 0;
    return t;
  };
  constexpr int kPer = attn_max_list(HW) / NT;   // list entries per thread
  static_assert(kPer == 8, "eight list entries per thread");
  int32_t ent[kPer];
  AFrag qf[16], qn[16];
  // list entries of an item (-1 = none), then their latent rows (-1 = none)
  auto load_entries = [&](const Item& t, int32_t (&ent)[kPer]) {
    const int32_t* src = a.idx + t.i * a.k + t.sp * a.split_keys;
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int e = threadIdx.x + p * NT;
      ent[p] = e < t.n_list ? src[e] : -1;
    }
  };
  // (every load is issued before any result is tested, so they overlap: an entry out of range
  // reads column 0 of the row, and a row outside the sequences row 0, and the result is dropped)
  auto resolve_rows = [&](const Item& t, int32_t (&ent)[kPer]) {
    const int32_t* srow = a.kv_slot + static_cast<int64_t>(max(t.b, 0)) * a.max_keys;
    int32_t v[kPer];
#pragma unroll
    for (int p = 0; p < kPer; ++p) v[p] = srow[(ent[p] >= 0 && ent[p] < a.max_keys) ? ent[p] : 0];
#pragma unroll
    for (int p = 0; p < kPer; ++p)
      ent[p] = (ent[p] >= 0 && ent[p] < a.max_keys && v[p] >= 0 && v[p] < a.n_slots) ? v[p] : -1;
  };
  // q as the B operand of S^T = K Q^T: lane (m, g) holds head h, dims 256 dh + 16 ks + 8 g ..
  auto load_q = [&](const Item& t, AFrag (&qd)[16]) {
    const int h = HW * t.hb + 32 * hg + m;
    const uint16_t* qrow = a.q + (t.i * H + h) * kLatentDim + 256 * dh + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qd[ks].u = *reinterpret_cast<const u32x4*>(qrow + 16 * ks);
  };
  // The item's latent rows into the slot table; returns its number of 32-entry chunks, up to the
  // last valid entry.  The caller has made sure no wave still reads the table.
  // (the wave's maximum of one past its last valid entry is taken first, on its own, so that the
  // lookups are waited for where nothing else is in flight)
  auto wave_last = [&](const Item& t, const int32_t (&ent)[kPer]) {
    int last = 0;
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int e = threadIdx.x + p * NT;
      if (e < t.n_list && ent[p] >= 0) last = e + 1;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o, 64));
    return last;
  };
  auto install = [&](const Item& t, const int32_t (&ent)[kPer], int last) {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int e = threadIdx.x + p * NT;
      if (e < ((t.n_list + kAttnChunk - 1) & ~(kAttnChunk - 1))) sl[e] = e < t.n_list ? ent[p] : -1;
    }
    if (lane == 0) last_w[wid] = last;
    lds_barrier();
    int n_used = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) n_used = max(n_used, last_w[w]);
    return (n_used + kAttnChunk - 1) / kAttnChunk;
  };

  // 1. Wave w requests rows w * kRowsPerWave .. of chunk c into buffer c % 4: lane L fetches the
  //    logical chunk L ^ sw(r) of its row, which then lands at physical chunk L.  An entry with
  //    no latent reads row 0 (some row is valid when a chunk is requested); its score is masked,
  //    and its weight 0 times finite latents adds nothing.
  //    The wave's row entries are read from the slot table together (16-byte reads), so the
  //    transfers do not each wait for an LDS round trip.
  const uint32_t kbuf_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) uint8_t*)&kbuf[0][0]));
  auto request = [&](int c) {
    int32_t slot[kRowsPerWave];
#pragma unroll
    for (int q4 = 0; q4 < kRowsPerWave / 4; ++q4) {
      const u32x4 v =
          *reinterpret_cast<const u32x4*>(&sl[c * kAttnChunk + wid * kRowsPerWave + 4 * q4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) slot[4 * q4 + e] = static_cast<int32_t>(v[e]);
    }
    const uint32_t buf = kbuf_lds + static_cast<uint32_t>(c % kAttnBufs) * kChunkBytes;
#pragma unroll
    for (int rr = 0; rr < kRowsPerWave; ++rr) {
      const int r = wid * kRowsPerWave + rr;
      dma_row16(a.kv + static_cast<int64_t>(max(slot[rr], 0)) * kLatentDim + 8 * (lane ^ sw(r)),
                __builtin_amdgcn_readfirstlane(buf + r * kRowBytes));
    }
  };

  // First item: its entries and q are loaded together, then its latent rows; q reaches the
  // operand registers through the same copy as every later item's (so no load into them is
  // outstanding where the products read them).  The next item's entries and q are issued before
  // the first chunks are requested: all requests then complete in order behind them, so the
  // chunk waits below stay exact.
  int64_t it = blockIdx.x;
  if (it >= n_items) return;
  Item cur = item_of(it);
  load_entries(cur, ent);
  load_q(cur, qn);
  resolve_rows(cur, ent);
  int n_chunks = install(cur, ent, wave_last(cur, ent));
  __builtin_amdgcn_s_waitcnt(0x0070);
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) qf[ks] = qn[ks];
  int64_t it_next = it + gridDim.x;
  Item nxt = item_of(it_next < n_items ? it_next : it);
  if (it_next < n_items) load_entries(nxt, ent);
#pragma unroll
  for (int c = 0; c < kAttnBufs - 1; ++c)
    if (c < n_chunks) request(c);

  // Operand addresses inside a buffer (bytes):
  //  - S^T, A = latents: lane (m, g) reads row m, chunk 32 dh + 2 ks + g; the swizzle reaches
  //    the low 3 bits only, so four offsets (ks % 4) plus 128 B per 4 steps cover it;
  //  - O^T, A = transposed latents, k-step kk, half e / 4 = hf, tile t: the lane's 8-byte read
  //    is row 16 kk + 8 hf + 4 g' + f of group G = lane / 16 (g' = G / 2, f = (lane % 16) / 4),
  //    dims 256 dh + 32 t + 16 (G % 2) + 4 q (q = lane % 4); the swizzle moves bits 0-2 of the
  //    chunk, where t contributes bit 2, so t % 2 picks one of two offsets and t / 2 adds 128 B.
  int s_off[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) s_off[c] = m * kRowBytes + 512 * dh + (((2 * c + g) ^ sw(m)) << 4);
  int t_off[2][2][2];
  {
    const int G = lane >> 4, f = (lane >> 2) & 3, q = lane & 3, gg = G >> 1;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {
          const int r = 16 * kk + 8 * hf + 4 * gg + f;
          const int ch = (4 * tp + 2 * (G & 1) + (q >> 1)) ^ sw(r);
          t_off[kk][hf][tp] = r * kRowBytes + 512 * dh + (ch << 4) + 8 * (q & 1);
        }
  }

  // gfx9 s_waitcnt immediates: vmcnt in bits 3:0 and 15:14, expcnt 6:4 (7: no wait), lgkmcnt
  // 11:8.  Requests complete in order, so "at most n chunks outstanding" means every older one
  // has landed.
  static_assert(3 * kRowsPerWave < 64, "vmcnt range");
  auto wait_chunks_left = [&](int n) {        // n = 0..2, uniform
    if (n >= 2)
      __builtin_amdgcn_s_waitcnt(((2 * kRowsPerWave) & 15) | 0x0070 |
                                 (((2 * kRowsPerWave) >> 4) << 14));
    else if (n == 1)
      __builtin_amdgcn_s_waitcnt((kRowsPerWave & 15) | 0x0070 | ((kRowsPerWave >> 4) << 14));
    else
      __builtin_amdgcn_s_waitcnt(0x0070);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // 2. partial S^T of chunk c over this wave's 256 dims (operands read four steps ahead of their
  //    MFMA; two accumulators, even and odd steps, so that consecutive MFMAs do not wait for each
  //    other's result), and the sum with the partner wave's partial through LDS
  auto s_partial = [&](int c) {
    const uint8_t* buf = kbuf[c % kAttnBufs];
    floatx16 sacc2[2] = {floatx16{}, floatx16{}};
    AFrag ka[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      ka[ks].u = *reinterpret_cast<const u32x4*>(buf + s_off[ks]);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      sacc2[ks & 1] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks & 3].v, qf[ks].v, sacc2[ks & 1], 0, 0, 0);
      if (ks + 4 < 16)
        ka[ks & 3].u = *reinterpret_cast<const u32x4*>(buf + s_off[ks & 3] + 128 * ((ks + 4) >> 2));
    }
    return sacc2[0] + sacc2[1];
  };
  auto s_exchange = [&](floatx16 part) {
#pragma unroll
    for (int r = 0; r < 16; ++r) ex[(wid * 16 + r) * 64 + lane] = part[r];
    lds_barrier();
    float other[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) other[r] = ex[((wid ^ 1) * 16 + r) * 64 + lane];
#pragma unroll
    for (int r = 0; r < 16; ++r) part[r] += other[r];
    return part;
  };

  for (;;) {
  const bool has_next_item = it_next < n_items;
  const int h = HW * cur.hb + 32 * hg + m;
  const int64_t i = cur.i;
  // q kept in accumulation registers: the MFMA reads its B operand from there, and the arch
  // registers stay free for the outputs and for several operand reads in flight
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) asm volatile("" : "+a"(qf[ks].u));
  floatx16 oacc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) oacc[t] = floatx16{};
  float m_run = -INFINITY, l_run = 0.0f;

  // S of the chunk being finished, and its validity mask
  floatx16 s_cur = floatx16{};
  uint32_t vmask_cur = 0;
  if (n_chunks > 0) {
    wait_chunks_left(min(n_chunks - 1, kAttnBufs - 2));
    s_cur = s_exchange(s_partial(0));
    vmask_cur = static_cast<uint32_t>(__ballot(sl[m] >= 0));
  }

  // One step per chunk c: S of chunk c + 1 is computed while the softmax of chunk c runs (its
  // MFMAs execute in the matrix pipe while the VALU works), then P.V of chunk c.
  for (int c = 0; c < n_chunks; ++c) {
    const bool has_next = c + 1 < n_chunks;
    // chunk c + 1 has landed in every wave's rows; every wave is done with chunk c - 1, whose
    // buffer chunk c + kAttnBufs - 1 now overwrites
    wait_chunks_left(min(n_chunks - c - 2, kAttnBufs - 3));
    // the next item's q, at the second step rather than at the item boundary, where every
    // workgroup (all run the same steps at about the same time) would load it at once; issued
    // before this step's request, so the counted waits still find the chunks in order
    if (has_next_item && c == 1) load_q(nxt, qn);
    if (c + kAttnBufs - 1 < n_chunks) request(c + kAttnBufs - 1);
    // last chunk: every request has landed, so the next item's latent rows are looked up now,
    // behind this chunk's softmax and P.V
    if (c == n_chunks - 1 && has_next_item) resolve_rows(nxt, ent);
    floatx16 s_next = floatx16{};
    if (has_next) s_next = s_partial(c + 1);

    // 3. online softmax of chunk c in base 2: lane (m, g) holds head h and keys
    //    8 (r / 4) + 4 g + r % 4.  The reference maximum moves only when a chunk's maximum
    //    exceeds it by more than 2^8, so the outputs are rescaled rarely; weights stay below 2^8.
    floatx16 sv = s_cur;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * g + (r & 3);
      sv[r] = ((vmask_cur >> key) & 1u) ? sv[r] : -INFINITY;
    }
    float smax = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
#pragma unroll
    for (int r = 4; r < 16; r += 4)
      smax = fmaxf(smax, fmaxf(fmaxf(sv[r], sv[r + 1]), fmaxf(sv[r + 2], sv[r + 3])));
    smax = fmaxf(smax, __shfl_xor(smax, 32, 64));
    const float mloc = smax * a.scale_log2;    // the scale is positive
    const bool move = mloc > m_run + 8.0f;     // -inf m_run: the first listed key moves it
    const float m_new = move ? mloc : m_run;
    const bool rescale = move && m_run != -INFINITY;
    const float alpha = rescale ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
    m_run = m_new;
    const float neg_m = m_run == -INFINITY ? 0.0f : -m_run;   // nothing listed yet: weights 0
    union {
      bf16x8 v;
      uint32_t w[4];
    } pf[2];
    float psum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r], a.scale_log2, neg_m));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r + 1], a.scale_log2, neg_m));
      const bf16x2 pb = {static_cast<__bf16>(p0), static_cast<__bf16>(p1)};   // RNE
      const uint32_t u = __builtin_bit_cast(uint32_t, pb);
      psum += __uint_as_float(u << 16) + __uint_as_float(u & 0xFFFF0000u);
      pf[r >> 3].w[(r & 7) >> 1] = u;
    }
    l_run = l_run * alpha + psum;
    if (__ballot(rescale)) {
#pragma unroll
      for (int t = 0; t < 8; ++t) oacc[t] *= alpha;
    }

    // 4. O^T += K^T P^T of chunk c over this wave's dims: A = latents transposed by the LDS
    //    read (operands read four MFMAs ahead)
    const uint8_t* buf = kbuf[c % kAttnBufs];
    auto tr_frag = [&](int n) {                // n = t + 8 kk: a tile's two steps 8 apart
      const int t = n & 7, kk = n >> 3;
      const int add = 128 * (t >> 1);
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4i16*)(buf + t_off[kk][0][t & 1] + add));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4i16*)(buf + t_off[kk][1][t & 1] + add));
      AFrag f;
      f.u = u32x4{__builtin_bit_cast(u32x2, lo).x, __builtin_bit_cast(u32x2, lo).y,
                  __builtin_bit_cast(u32x2, hi).x, __builtin_bit_cast(u32x2, hi).y};
      return f;
    };
    AFrag kt[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) kt[n] = tr_frag(n);
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      oacc[n & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt[n & 3].v, pf[n >> 3].v,
                                                           oacc[n & 7], 0, 0, 0);
      if (n + 4 < 16) kt[n & 3] = tr_frag(n + 4);
    }

    if (has_next) {
      s_cur = s_exchange(s_next);
      vmask_cur = static_cast<uint32_t>(__ballot(sl[(c + 1) * kAttnChunk + m] >= 0));
    }
  }
  // no request is left in flight: the last chunk requests nothing
  if (n_chunks == 0 && has_next_item) resolve_rows(nxt, ent);
  // the item after the next one
  const int64_t it_nn = it_next + gridDim.x;
  const Item nn = item_of(it_nn < n_items ? it_nn : it);
  // the next item's q into the operand registers (this item's last S is done).  Every load is
  // waited for here, where only the latent-row lookups are still in flight, so that no load
  // into those registers is pending when the next item's products read them.
  if (has_next_item) {
    if (n_chunks < 2) load_q(nxt, qn);                   // the steps did not reach it
    __builtin_amdgcn_s_waitcnt(0x0070);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qf[ks] = qn[ks];
  }
  const int nx_last = has_next_item ? wave_last(nxt, ent) : 0;

  // lanes (m, 0) and (m, 1) summed different keys of head h under the same maximum
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (a.n_split == 1) {
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if constexpr (HW == 64) {
      // The wave's [32 heads x 256 dims] bf16 output goes through LDS so that every store writes
      // whole 512-byte row segments: from the accumulators, lane (m, g) holds 8-byte units
      // u = 8 t + 2 j + g (dims 4 u ..) of head m, and a direct store would touch 32 rows per
      // instruction.  The tile sits in one half of a chunk buffer the last step no longer uses
      // (chunks n - 2 and n - 3 are done once the last step's barrier is passed, and nothing is
      // requested after chunk n - 1), head m's row at 512 m, unit u at 8 (u ^ m), so the 32 heads
      // of one write land in distinct banks.  Each wave reads back only its own tile.  (Two-wave
      // workgroups, for 32 heads, store directly: their registers have no room for the staging.)
      uint8_t* stg = kbuf[(n_chunks + 1 + (wid >> 1)) % kAttnBufs] + (wid & 1) * (kChunkBytes / 2);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x2 v;
          v.x = bf16_rne_bits(oacc[t][4 * j] * inv) |
                (bf16_rne_bits(oacc[t][4 * j + 1] * inv) << 16);
          v.y = bf16_rne_bits(oacc[t][4 * j + 2] * inv) |
                (bf16_rne_bits(oacc[t][4 * j + 3] * inv) << 16);
          const int u = 8 * t + 2 * j + g;
          *reinterpret_cast<u32x2*>(stg + 512 * m + 8 * (u ^ m)) = v;
        }
      }
      // read back: lane L takes head 2 s + L / 32 and its 16-byte piece p = L % 32 (units 2 p and
      // 2 p + 1, found at chunk p ^ (head / 2), in swapped order when the head is odd)
      uint16_t* obase = a.out + (i * H + HW * cur.hb + 32 * hg) * kLatentDim + 256 * dh;
#pragma unroll 4
      for (int st = 0; st < 16; ++st) {
        const int hh = 2 * st + g, pc = m;
        u32x4 v = *reinterpret_cast<const u32x4*>(stg + 512 * hh + 16 * (pc ^ (hh >> 1)));
        if (hh & 1) v = u32x4{v.z, v.w, v.x, v.y};
        *reinterpret_cast<u32x4*>(obase + hh * kLatentDim + 8 * pc) = v;
      }
    } else {
      uint16_t* orow = a.out + (i * H + h) * kLatentDim + 256 * dh + 4 * g;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x2 v;
          v.x = bf16_rne_bits(oacc[t][4 * j] * inv) |
                (bf16_rne_bits(oacc[t][4 * j + 1] * inv) << 16);
          v.y = bf16_rne_bits(oacc[t][4 * j + 2] * inv) |
                (bf16_rne_bits(oacc[t][4 * j + 3] * inv) << 16);
          *reinterpret_cast<u32x2*>(orow + 32 * t + 8 * j) = v;
        }
      }
    }
    if (a.lse && dh == 0 && g == 0)
      a.lse[i * H + h] = l_tot > 0.0f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  } else {
    const int64_t part = (i * a.n_split + cur.sp) * H + h;
    if constexpr (HW == 64) {
      // Staged like the bf16 output, so each store writes a whole 1 KB row: once every wave is
      // past its last chunk all four buffers are free, and wave w's [32 heads x 256 dims] fp32
      // tile goes into buffer w, head m's row at 1024 m and its 16-byte unit u (dims 4 u ..) at
      // 16 (u ^ m) (16 consecutive heads of one write on distinct banks).
      lds_barrier();
      uint8_t* stg = kbuf[wid];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const floatx4 v = {oacc[t][4 * j], oacc[t][4 * j + 1], oacc[t][4 * j + 2],
                             oacc[t][4 * j + 3]};
          const int u = 8 * t + 2 * j + g;
          *reinterpret_cast<floatx4*>(stg + 1024 * m + 16 * (u ^ m)) = v;
        }
      }
      float* pbase = a.part_o +
                     ((i * a.n_split + cur.sp) * H + HW * cur.hb + 32 * hg) * kLatentDim + 256 * dh;
#pragma unroll 4
      for (int hh = 0; hh < 32; ++hh) {
        const floatx4 v = *reinterpret_cast<const floatx4*>(stg + 1024 * hh + 16 * (lane ^ hh));
        *reinterpret_cast<floatx4*>(pbase + hh * kLatentDim + 4 * lane) = v;
      }
    } else {
      float* po = a.part_o + part * kLatentDim + 256 * dh + 4 * g;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const floatx4 v = {oacc[t][4 * j], oacc[t][4 * j + 1], oacc[t][4 * j + 2],
                             oacc[t][4 * j + 3]};
          *reinterpret_cast<floatx4*>(po + 32 * t + 8 * j) = v;
        }
      }
    }
    if (dh == 0 && g == 0) {
      a.part_ml[2 * part] = l_tot > 0.0f ? m_run : -INFINITY;
      a.part_ml[2 * part + 1] = l_tot;
    }
  }
  if (!has_next_item) break;

  // Next item: once every wave is done with this item's slot table and buffers, its latent rows
  // go into the table, the item after it has its entries and q issued, and its first chunks are
  // requested.
  lds_barrier();
  n_chunks = install(nxt, ent, nx_last);
  cur = nxt;
  it = it_next;
  it_next = it_nn;
  nxt = nn;
  if (it_next < n_items) load_entries(nxt, ent);
#pragma unroll
  for (int c = 0; c < kAttnBufs - 1; ++c)
    if (c < n_chunks) request(c);
  }
}

// Merge of the splits of one (row, head) per wave: weights 2^(m_sp - M), M the largest maximum.
__global__ __launch_bounds__(256) void sparse_attn_merge_kernel(AttnArgs a) {
  const int H = a.n_heads;
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);   // i * H + h
  if (row >= a.n_q * H) return;
  const int64_t i = row / H;
  const int h = static_cast<int>(row - i * H);
  // one pass with a running maximum (rescaling when it moves), so the loads of several splits
  // are in flight together
  float mx = -INFINITY;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float l = 0.0f;
#pragma unroll 4
  for (int sp = 0; sp < a.n_split; ++sp) {
    const int64_t part = (i * a.n_split + sp) * H + h;
    const float ms = a.part_ml[2 * part];
    const float ls = a.part_ml[2 * part + 1];
    const floatx4* po = reinterpret_cast<const floatx4*>(a.part_o + part * kLatentDim + 8 * lane);
    const floatx4 v0 = po[0], v1 = po[1];
    if (ms == -INFINITY) continue;
    if (ms > mx) {
      const float r = exp2f(mx - ms);     // 0 for the first split with keys
      l *= r;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= r;
      mx = ms;
    }
    const float wgt = exp2f(ms - mx);
    l += wgt * ls;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] += wgt * v0[e];
      acc[4 + e] += wgt * v1[e];
    }
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    o[e] = bf16_rne_bits(acc[2 * e] * inv) | (bf16_rne_bits(acc[2 * e + 1] * inv) << 16);
  *reinterpret_cast<u32x4*>(a.out + row * kLatentDim + 8 * lane) = o;
  if (a.lse && lane == 0)
    a.lse[row] = l > 0.0f ? (mx + log2f(l)) * 0.69314718055994531f : -INFINITY;
}

// Compute units of the current device (one workgroup of the attention kernel fits per CU).
int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < 64 && cached[dev] > 0) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev >= 0 && dev < 64) cached[dev] = n;
  return n;
}

template <int HW>
hipError_t launch_h(const AttnArgs& a, hipStream_t stream) {
  const int64_t items = a.n_q * a.n_split * (a.n_heads / HW);
  const int64_t blocks = items < cu_count() ? items : cu_count();
  hipLaunchKernelGGL(sparse_attn_kernel<HW>, dim3(static_cast<uint32_t>(blocks)), dim3(HW * 4), 0,
                     stream, a);
  if (a.n_split > 1) {
    const int64_t mblocks = (a.n_q * a.n_heads + 3) / 4;
    hipLaunchKernelGGL(sparse_attn_merge_kernel, dim3(static_cast<uint32_t>(mblocks)), dim3(256),
                       0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

// Rows are split when the batch has too few of them to fill the chip, and when a list is longer
// than one workgroup's slot table.  More splits shorten each workgroup's run of 32-key steps
// (about 1.8 us each), but every split adds an item start and a partial output to write and
// merge.  Measured on 32 decode rows x 64 heads x 1024 keys: 2 splits 41 us, 4 splits 31 us,
// 5 splits 30.8 us, 8 splits 33 us.  The count is near sqrt(1765 * chunks / (n_q * H)), a fit
// of those timings, without exceeding the CUs' worth of items or going below two steps per split.
void attn_plan(int64_t n_q, int32_t n_heads, int32_t k, int32_t* n_split, int32_t* split_keys) {
  const int32_t chunks = (k + kAttnChunk - 1) / kAttnChunk;
  int32_t s = 1;
  if (n_q > 0 && n_q < 256) {
    const int64_t n_hb = n_heads > 64 ? n_heads / 64 : 1;
    const int64_t fill = (256 + n_q * n_hb - 1) / (n_q * n_hb);
    const int64_t cost = static_cast<int64_t>(
        sqrt(1765.0 * chunks / (static_cast<double>(n_q) * (n_heads > 0 ? n_heads : 64))) + 0.5);
    int64_t t = fill < cost ? fill : cost;
    t = t < chunks / 2 ? t : chunks / 2;
    s = t < 1 ? 1 : static_cast<int32_t>(t);
  }
  const int32_t max_list = attn_max_list(n_heads);
  const int32_t min_s = (chunks * kAttnChunk + max_list - 1) / max_list;
  if (s < min_s) s = min_s;
  const int32_t per = (chunks + s - 1) / s;
  *n_split = (chunks + per - 1) / per;
  *split_keys = per * kAttnChunk;
}

size_t attn_workspace_bytes(int64_t n_q, int32_t n_heads, int32_t k) {
  int32_t s = 1, per = 0;
  attn_plan(n_q, n_heads, k, &s, &per);
  if (s <= 1) return 0;
  const size_t parts = static_cast<size_t>(n_q) * s * n_heads;
  return parts * kLatentDim * 4 + parts * 2 * 4;
}

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t stream) {
  if (a.n_q <= 0) return hipSuccess;
  switch (a.n_heads) {
    case 32: return launch_h<32>(a, stream);
    case 64:
    case 128: return launch_h<64>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsa
