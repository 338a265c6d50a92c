// Sparse attention over the keys the indexer selects: for query row i and head h, a softmax over
// the listed entries of q[i][h] . v_j (scaled), and the weighted sum of the 512-dim latents v_j,
// which serve as key and value of every head ("When the Fused Kernel Isn't Enough", Input
// Knowledge: the sparse attention reads the top-K entries, the main KV cache is bf16 with
// head_dim 512; "The Fused Kernel Decision", Message: that cache is unpaged, one slot per entry).
//
// One workgroup per (query row, split of the list, block of HW = min(H, 64) heads), HW / 16
// waves.  Wave w owns 32 heads of the block, 32 (w / 2) .., and one half of the 512 output dims,
// 256 (w % 2) ...  Per 32 listed keys:
//   1. the keys' latents are gathered into LDS twice: row-major (16-byte chunks XOR-swizzled by
//      row) and transposed [dim][key] (chunks swizzled by dim), the key order inside each 16-key
//      step permuted so that the transposed operand matches the accumulator layout below;
//   2. S^T = K Q^T on bf16 MFMA 32x32x16: each wave of a pair sums over its own 256 dims, and the
//      pair swaps partial sums through LDS (fp32 addition commutes, so both hold the same S);
//   3. online softmax in base 2: each lane owns one head and 16 of the 32 keys, the maximum is
//      shared with the lane holding the other 16, a reference maximum moves only when exceeded
//      by more than 2^8, and the weights are rounded to bf16 (the weight sum adds the rounded
//      values, so the weights used sum to the divisor);
//   4. O^T += K^T P^T on the same MFMA: the accumulator of S^T, rounded, is already the B operand
//      of this product (lane = head, 8 keys), and the transposed latents are its A operand.
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
constexpr int kRowMajorBytes = kAttnChunk * kRowBytes;      // 32 KB
constexpr int kTransBytes = kLatentDim * kAttnChunk * 2;    // 32 KB: [512 dims][32 keys]

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Sequence b with cu_q[b] <= i < cu_q[b + 1], or -1.
__device__ __forceinline__ int32_t seq_of_row(const int32_t* cu_q, int32_t n_seq, int64_t i) {
  if (n_seq <= 0 || i < cu_q[0] || i >= cu_q[n_seq]) return -1;
  int32_t lo = 0, hi = n_seq;
  while (hi - lo > 1) {
    const int32_t mid = (lo + hi) >> 1;
    if (cu_q[mid] <= i) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Row-major copy: 16-byte chunk c of key row r sits at chunk c ^ row_swizzle(r).  Eight
// consecutive rows (an MFMA operand read) and the rows 4q + e of eight key quads q (one staging
// write) both land on eight distinct 16-byte bank groups.
__device__ __forceinline__ int row_swizzle(int r) { return (r ^ (r >> 2)) & 7; }

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

// Position of key kappa (0..31) in a transposed row: inside each 16-key step, bits 2 and 3 of
// the key swap, so that positions 16 kk + 8 g + e hold keys 16 kk + 8 (e / 4) + 4 g + e % 4.
__device__ __forceinline__ int trans_pos(int kappa) {
  return (kappa & ~12) | ((kappa & 4) << 1) | ((kappa & 8) >> 1);
}

template <int HW>
__global__ __launch_bounds__(HW * 4) void sparse_attn_kernel(AttnArgs a) {
  constexpr int NT = HW * 4;                   // HW / 16 waves
  constexpr int kItems = kAttnChunk / 4 * (kLatentDim / 8) / NT;   // (4 keys x 8 dims) per thread
  static_assert(kItems >= 1 && kItems * NT == 512, "staging items");
  __shared__ __attribute__((aligned(16))) uint8_t kr[kRowMajorBytes];   // also the S exchange
  __shared__ __attribute__((aligned(16))) uint8_t kt[kTransBytes];
  __shared__ int32_t sl[kMaxAttnList];        // latent row of each list entry, -1 = none
  __shared__ int32_t n_used;
  static_assert(HW / 16 * 16 * 64 * 4 <= kRowMajorBytes, "exchange fits the row-major buffer");

  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int hg = wid >> 1, dh = wid & 1;
  const int m = lane & 31, g = lane >> 5;
  const int H = a.n_heads;
  const int n_hb = H / HW;
  const int64_t rs = blockIdx.x / n_hb;                 // i * n_split + sp
  const int hb = blockIdx.x - static_cast<int>(rs * n_hb);
  const int64_t i = rs / a.n_split;
  const int sp = static_cast<int>(rs - i * a.n_split);
  const int32_t b = seq_of_row(a.cu_q, a.n_seq, i);
  const int h = HW * hb + 32 * hg + m;

  // q as the B operand of S^T = K Q^T: lane (m, g) holds head h, dims 256 dh + 16 ks + 8 g ..
  AFrag qf[16];
  {
    const uint16_t* qrow = a.q + (i * H + h) * kLatentDim + 256 * dh + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qf[ks].u = *reinterpret_cast<const u32x4*>(qrow + 16 * ks);
  }

  floatx16 oacc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) oacc[t] = floatx16{};
  float m_run = -INFINITY, l_run = 0.0f;

  const uint8_t* s_base[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    s_base[c] = kr + m * kRowBytes + 512 * dh + (((2 * c + g) ^ row_swizzle(m)) << 4);
  const uint8_t* t_base[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
    t_base[kk] = kt + (256 * dh + m) * (kAttnChunk * 2) + (((2 * kk + g) ^ ((m >> 1) & 3)) << 4);

  // The workgroup's list entries, resolved to latent rows once: slot or -1.
  const int j0 = sp * a.split_keys;
  const int n_list = max(0, min(a.k, j0 + a.split_keys) - j0);
  if (threadIdx.x == 0) n_used = 0;
  __syncthreads();
  int last = 0;
  for (int e = threadIdx.x; e < n_list; e += NT) {
    int32_t slot = -1;
    if (b >= 0) {
      const int32_t s = a.idx[i * a.k + j0 + e];
      if (s >= 0 && s < a.max_keys) {
        const int32_t v = a.kv_slot[static_cast<int64_t>(b) * a.max_keys + s];
        if (v >= 0 && v < a.n_slots) slot = v;
      }
    }
    sl[e] = slot;
    if (slot >= 0) last = e + 1;
  }
  for (int e = n_list + threadIdx.x; e < ((n_list + kAttnChunk - 1) & ~(kAttnChunk - 1)); e += NT)
    sl[e] = -1;
  if (last) atomicMax(&n_used, last);
  __syncthreads();
  const int n_chunks = (n_used + kAttnChunk - 1) / kAttnChunk;   // up to the last valid entry

  // 1. gather: thread item = 4 keys x 8 dims (4 rows x 16 B).  The next chunk's rows are loaded
  //    into registers before the current chunk is computed, so their latency overlaps the MFMAs.
  u32x4 rows[kItems][4];
  // Item of a thread: key quad q4 = item % 8 (fastest, so that the eight lanes writing one
  // transposed row are neighbours), dim octet oct = item / 8.
  auto load_chunk = [&](int c) {
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
      const int item = threadIdx.x + it * NT;
      const int q4 = item & 7, oct = item >> 3;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int32_t slot = sl[c * kAttnChunk + 4 * q4 + e];
        rows[it][e] = slot >= 0 ? *reinterpret_cast<const u32x4*>(
                                      a.kv + static_cast<int64_t>(slot) * kLatentDim + 8 * oct)
                                : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  if (n_chunks > 0) load_chunk(0);

  for (int c = 0; c < n_chunks; ++c) {
    lds_barrier();                             // the previous chunk's LDS readers are done
    const uint32_t vmask = static_cast<uint32_t>(__ballot(sl[c * kAttnChunk + m] >= 0));
    // row-major and transposed copies of the chunk
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
      const int item = threadIdx.x + it * NT;
      const int q4 = item & 7, oct = item >> 3;
      const u32x4* r = rows[it];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = 4 * q4 + e;
        *reinterpret_cast<u32x4*>(kr + key * kRowBytes + ((oct ^ row_swizzle(key)) << 4)) = r[e];
      }
      // transposed: the 8 quads of a dim fill its 64-byte row (8 distinct (chunk, half) slots);
      // lanes with odd oct take the dims of the other parity first, so that the 16 lanes of one
      // write cover both halves of the banks
      const int pos = trans_pos(4 * q4);
      const int flip = oct & 1;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int hh = k2 ^ flip;
          const uint32_t sel = hh ? 0x07060302u : 0x05040100u;
          const int d = 8 * oct + 2 * w + hh;
          u32x2 v;
          v.x = __builtin_amdgcn_perm(r[1][w], r[0][w], sel);   // keys 0, 1 of the quad at dim d
          v.y = __builtin_amdgcn_perm(r[3][w], r[2][w], sel);   // keys 2, 3
          const int phys = (((pos >> 3) ^ ((d >> 1) & 3)) << 4) | (((pos >> 2) & 1) << 3);
          *reinterpret_cast<u32x2*>(kt + d * (kAttnChunk * 2) + phys) = v;
        }
      }
    }
    if (c + 1 < n_chunks) load_chunk(c + 1);
    lds_barrier();

    // 2. S^T partial over this wave's 256 dims: A = latents (key m, 8 dims), B = q
    //    chunk 32 dh + 2 ks + g of row m sits at chunk ^ row_swizzle(m): the swizzle reaches only
    //    the low 3 bits, so four bases (ks % 4) and immediate offsets of 128 B per 4 steps cover it
    floatx16 sacc = floatx16{};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      AFrag ka;
      ka.u = *reinterpret_cast<const u32x4*>(s_base[ks & 3] + 128 * (ks >> 2));
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka.v, qf[ks].v, sacc, 0, 0, 0);
    }
    lds_barrier();                             // every wave is done with the row-major latents
    float* ex = reinterpret_cast<float*>(kr);
#pragma unroll
    for (int r = 0; r < 16; ++r) ex[(wid * 16 + r) * 64 + lane] = sacc[r];
    lds_barrier();
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] += ex[((wid ^ 1) * 16 + r) * 64 + lane];

    // 3. online softmax in base 2: lane (m, g) holds head h and keys 8 (r / 4) + 4 g + r % 4.
    //    The reference maximum moves only when a chunk's maximum exceeds it by more than 2^8, so
    //    the outputs are rescaled rarely; weights stay below 2^8, exact in range for bf16 / fp32.
    if (vmask != 0xFFFFFFFFu) {                // the same for every lane of the wave
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * g + (r & 3);
        sacc[r] = ((vmask >> key) & 1u) ? sacc[r] : -INFINITY;
      }
    }
    float smax = fmaxf(fmaxf(sacc[0], sacc[1]), fmaxf(sacc[2], sacc[3]));
#pragma unroll
    for (int r = 4; r < 16; r += 4)
      smax = fmaxf(smax, fmaxf(fmaxf(sacc[r], sacc[r + 1]), fmaxf(sacc[r + 2], sacc[r + 3])));
    smax = fmaxf(smax, __shfl_xor(smax, 32, 64));
    const float mloc = smax * a.scale_log2;    // the scale is positive
    const bool move = mloc > m_run + 8.0f;     // -inf m_run: the first listed key moves it
    const float m_new = move ? mloc : m_run;
    if (__ballot(move && m_run != -INFINITY)) {
      const float alpha = (move && m_run != -INFINITY) ? __builtin_amdgcn_exp2f(m_run - m_new)
                                                       : 1.0f;
#pragma unroll
      for (int t = 0; t < 8; ++t) oacc[t] *= alpha;
      l_run *= alpha;
    }
    m_run = m_new;
    const float neg_m = m_run == -INFINITY ? 0.0f : -m_run;   // nothing listed yet: weights 0
    union {
      bf16x8 v;
      uint32_t w[4];
    } pf[2];
    float psum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], a.scale_log2, neg_m));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r + 1], a.scale_log2, neg_m));
      const bf16x2 pb = {static_cast<__bf16>(p0), static_cast<__bf16>(p1)};   // RNE
      const uint32_t u = __builtin_bit_cast(uint32_t, pb);
      psum += __uint_as_float(u << 16) + __uint_as_float(u & 0xFFFF0000u);
      pf[r >> 3].w[(r & 7) >> 1] = u;
    }
    l_run += psum;

    // 4. O^T += K^T P^T over this wave's dims: A = transposed latents (dim m, 8 keys)
    //    dim d = 256 dh + 32 t + m, chunk (2 kk + g) ^ ((d / 2) % 4) = (2 kk + g) ^ ((m / 2) % 4):
    //    two bases and immediate offsets of 2 KB per tile
#pragma unroll
    for (int t = 0; t < 8; ++t) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        AFrag ka;
        ka.u = *reinterpret_cast<const u32x4*>(t_base[kk] + 32 * (kAttnChunk * 2) * t);
        oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka.v, pf[kk].v, oacc[t], 0, 0, 0);
      }
    }
  }

  // lanes (m, 0) and (m, 1) summed different keys of head h under the same maximum
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (a.n_split == 1) {
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    uint16_t* orow = a.out + (i * H + h) * kLatentDim + 256 * dh + 4 * g;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 v;
        v.x = bf16_rne_bits(oacc[t][4 * j] * inv) | (bf16_rne_bits(oacc[t][4 * j + 1] * inv) << 16);
        v.y = bf16_rne_bits(oacc[t][4 * j + 2] * inv) |
              (bf16_rne_bits(oacc[t][4 * j + 3] * inv) << 16);
        *reinterpret_cast<u32x2*>(orow + 32 * t + 8 * j) = v;
      }
    }
    if (a.lse && dh == 0 && g == 0)
      a.lse[i * H + h] = l_tot > 0.0f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  } else {
    const int64_t part = (i * a.n_split + sp) * H + h;
    float* po = a.part_o + part * kLatentDim + 256 * dh + 4 * g;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        floatx4 v = {oacc[t][4 * j], oacc[t][4 * j + 1], oacc[t][4 * j + 2], oacc[t][4 * j + 3]};
        *reinterpret_cast<floatx4*>(po + 32 * t + 8 * j) = v;
      }
    }
    if (dh == 0 && g == 0) {
      a.part_ml[2 * part] = l_tot > 0.0f ? m_run : -INFINITY;
      a.part_ml[2 * part + 1] = l_tot;
    }
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
  float mx = -INFINITY;
  for (int sp = 0; sp < a.n_split; ++sp)
    mx = fmaxf(mx, a.part_ml[2 * ((i * a.n_split + sp) * H + h)]);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float l = 0.0f;
  if (mx != -INFINITY) {
    for (int sp = 0; sp < a.n_split; ++sp) {
      const int64_t part = (i * a.n_split + sp) * H + h;
      const float ms = a.part_ml[2 * part];
      if (ms == -INFINITY) continue;
      const float wgt = exp2f(ms - mx);
      l += wgt * a.part_ml[2 * part + 1];
      const floatx4* po = reinterpret_cast<const floatx4*>(a.part_o + part * kLatentDim + 8 * lane);
      const floatx4 v0 = po[0], v1 = po[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] += wgt * v0[e];
        acc[4 + e] += wgt * v1[e];
      }
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

template <int HW>
hipError_t launch_h(const AttnArgs& a, hipStream_t stream) {
  const int64_t blocks = a.n_q * a.n_split * (a.n_heads / HW);
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

// Rows are split when the batch has too few of them to fill the chip (each split keeping at
// least two 32-key steps) and when a list is longer than one workgroup's slot table.
void attn_plan(int64_t n_q, int32_t k, int32_t* n_split, int32_t* split_keys) {
  const int32_t chunks = (k + kAttnChunk - 1) / kAttnChunk;
  int32_t s = 1;
  if (n_q > 0 && n_q < 256) {
    s = static_cast<int32_t>((256 + n_q - 1) / n_q);
    s = s < chunks / 2 ? s : chunks / 2;
    if (s < 1) s = 1;
  }
  const int32_t min_s = (chunks * kAttnChunk + kMaxAttnList - 1) / kMaxAttnList;
  if (s < min_s) s = min_s;
  const int32_t per = (chunks + s - 1) / s;
  *n_split = (chunks + per - 1) / per;
  *split_keys = per * kAttnChunk;
}

size_t attn_workspace_bytes(int64_t n_q, int32_t n_heads, int32_t k) {
  int32_t s = 1, per = 0;
  attn_plan(n_q, k, &s, &per);
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
