// S1: fused RMSNorm + RoPE + quantise + paged store of compressed index keys.
//
// The fused store of the DSA indexer ("The Moment of Validation", Input Knowledge Required: one
// kernel normalises, rotates and writes the cache; "The Fused Kernel Decision", Message: the cache
// is [npages, 64*128] and a key goes to (page, offset)).  fp8 keys are e4m3 codes plus one fp32
// scale per key, 132 B/token; bf16 keys are 256 B/token ("When the Fused Kernel Isn't Enough",
// Input Knowledge Required).
//
// The rotated store ("When the Fused Kernel Isn't Enough", the fused vs. non-fused paths: one
// kernel normalises, applies RoPE and the Hadamard transform, and stores; "The Fused Kernel
// Decision", Assumptions: q and k share the transform's output order) multiplies the key by the
// normalised 128-point Walsh-Hadamard matrix after RoPE, before the rounding; q goes through the
// same map (rotate_q_kernel), so q.k is kept.
//
// Work mapping: four lanes (a quad) per key.  The key's 128 dims are 8 chunks of 16; lane l owns
// dims 16 i + 4 l .. 16 i + 4 l + 3 of every chunk i, so each load and store instruction covers a
// contiguous 64-byte (activations) or 16-, 32- or 8-byte (codes) span per key, and the per-key
// work (the norm's square root and division, the fp8 scale and its reciprocal) is repeated by 4
// lanes instead of 32.  Chunks 4..7 are the rotated half: lane l holds the RoPE pairs 8 (i - 4) +
// 2 l and 8 (i - 4) + 2 l + 1.  The arithmetic before the format rounding is fp64 so that the
// stored bytes are a function of the inputs alone, not of the reduction order: a result only
// depends on the order when it sits within ~2^-50 of a rounding boundary.
#include "internal.h"

namespace dsa {
namespace {

// fma(a, b, c) for a constant c, taken from scalar registers in the three-operand form.  Left to
// itself the compiler copies each 64-bit constant into a vector register pair (two VALU moves) to
// use the two-address form, which in the polynomials below costs two moves per step.
__device__ __forceinline__ double fma_const(double a, double b, double c) {
  double d;
  asm("v_fma_f64 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "s"(c));
  return d;
}

// cos and sin of a RoPE angle th = 4 s f_j, exact in fp64 (0 <= th < 2^26 rad for s < 2^24):
// Cody-Waite reduction by pi/2 (th - n pi/2 with pi/2 split into two 27-bit parts, whose
// products with n < 2^26 are exact, and a 53-bit third), then polynomials in z = r^2 on
// [-pi/4, pi/4] and the quadrant n mod 4.  The polynomials interpolate (sin r - r) / r^3 and
// (cos r - 1) / z at Chebyshev nodes on [0, (pi/4)^2], solved in 80-digit arithmetic
// (rope_poly.py): near-minimax, their error is below 2^-56 of r and 2^-62 respectively.  The
// result is within about 2 ulp of the exact cosine and sine.
__device__ __forceinline__ void rope_sincos(double th, double* sn, double* cs) {
  const double n = __builtin_rint(th * 0x1.45f306dc9c883p-1);   // th * 2/pi
  double r = fma(-n, 0x1.921fb54000000p+0, th);
  r = fma(-n, 0x1.10b4610000000p-30, r);
  r = fma(-n, 0x1.a62633145c06ep-58, r);
  const double z = r * r;
  // sin r = r + r^3 P(z)
  double ps = 0x1.5e0b19f8b1451p-33;
  ps = fma_const(ps, z, -0x1.ae600b02b6262p-26);
  ps = fma_const(ps, z, 0x1.71de37968a100p-19);
  ps = fma_const(ps, z, -0x1.a01a019e83aaep-13);
  ps = fma_const(ps, z, 0x1.1111111110bb2p-7);
  ps = fma_const(ps, z, -0x1.5555555555555p-3);
  const double sr = fma(r * z, ps, r);
  // cos r = 1 + z Q(z)
  double pc = -0x1.8ff9d439a204ap-37;
  pc = fma_const(pc, z, 0x1.1eea7f259b344p-29);
  pc = fma_const(pc, z, -0x1.27e4f8e4a2e74p-22);
  pc = fma_const(pc, z, 0x1.a01a019de131fp-16);
  pc = fma_const(pc, z, -0x1.6c16c16c15d79p-10);
  pc = fma_const(pc, z, 0x1.5555555555551p-5);
  pc = fma_const(pc, z, -0x1.0000000000000p-1);
  const double cr = fma(z, pc, 1.0);
  // th = n pi/2 + r: (sin, cos) th = (s, c), (c, -s), (-s, -c), (-c, s) for n = 0, 1, 2, 3 mod 4
  const int q = static_cast<int>(n) & 3;
  const double s1 = (q & 1) ? cr : sr;
  const double c1 = (q & 1) ? sr : cr;
  *sn = (q & 2) ? -s1 : s1;
  *cs = ((q + 1) & 2) ? -c1 : c1;
}

// Round a finite fp32 to bf16, nearest-even, returned in the low 16 bits.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// The nearest double to 2^-3.5 (sqrt(2) / 16): the normalisation of the 128-point transform.
constexpr double kHadamardScale = 0x1.6a09e667f3bcdp-4;

// Value of lane (lane ^ M) of the same quad, M = 1 or 2 (DPP quad permutation; no LDS).
template <int M>
__device__ __forceinline__ double quad_xor(double v) {
  constexpr int kCtrl = M == 1 ? 0xB1 : 0x4E;   // quad_perm [1,0,3,2] / [2,3,0,1]
  const uint64_t u = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(u), kCtrl, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(u >> 32), kCtrl, 0xF, 0xF,
                                             false);
  return __longlong_as_double((static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                              static_cast<uint32_t>(lo));
}

// q of the rotated store: each 128-dim bf16 vector to fp64, the same transform as the keys, then
// rounded to fp32 and to bf16 (nearest-even).  Four lanes (a quad) per vector, lane l holding
// dims 32l..32l+31: butterfly spans 1..16 pair values inside a lane, spans 32 and 64 pair lane l
// with lanes l ^ 1 and l ^ 2 (the lower taking the sum, the upper the difference), in the order
// of hadamard128, so the fp64 result is the same.  Each quad reads its whole vector before it
// writes, so in and out may be the same buffer.
__global__ __launch_bounds__(256) void rotate_q_kernel(const uint16_t* in, uint16_t* out,
                                                       int64_t n_vec) {
#pragma clang fp contract(off)
  const int64_t v = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 2;
  const int l = threadIdx.x & 3;
  if (v >= n_vec) return;   // whole quads leave together: the exchanges stay in a quad
  const uint4* src = reinterpret_cast<const uint4*>(in + v * kHeadDim + 32 * l);
  uint4 w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = src[i];
  double x[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t word[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[8 * i + 2 * k] = __uint_as_float(word[k] << 16);
      x[8 * i + 2 * k + 1] = __uint_as_float(word[k] & 0xFFFF0000u);
    }
  }
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (i & h) continue;
      const double a = x[i], b = x[i + h];
      x[i] = a + b;
      x[i + h] = a - b;
    }
  }
  const bool up1 = (l & 1) != 0, up2 = (l & 2) != 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const double p = quad_xor<1>(x[i]);
    x[i] = up1 ? p - x[i] : x[i] + p;
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const double p = quad_xor<2>(x[i]);
    x[i] = up2 ? p - x[i] : x[i] + p;
  }
  uint4* dst = reinterpret_cast<uint4*>(out + v * kHeadDim + 32 * l);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t word[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      word[k] = bf16_rne(static_cast<float>(x[8 * i + 2 * k] * kHadamardScale)) |
                (bf16_rne(static_cast<float>(x[8 * i + 2 * k + 1] * kHadamardScale)) << 16);
    dst[i] = make_uint4(word[0], word[1], word[2], word[3]);
  }
}

typedef float float2_v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Round a finite fp32 of magnitude <= 2^15 to OCP e4m3fn (bias 7, max 448, no inf), nearest-even,
// saturating to 448.  Normal range [2^-6, 448): keep 3 mantissa bits of the fp32 significand with
// round-half-even, a carry out of the mantissa moving to the next binade by plain addition of the
// code.  Subnormal range [0, 2^-6): the code is the integer round-half-even of |v| * 2^9 (8 =
// 2^-6).  Both codes are formed and one is selected, so lanes of different magnitudes do not split
// the wave.
__device__ __forceinline__ uint32_t e4m3_rne_sat_nb(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  const uint32_t sub = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
  const uint32_t ua = __float_as_uint(a);
  const uint32_t m = ua & 0x7FFFFFu;
  const uint32_t r = (m + 0x7FFFFu + ((m >> 20) & 1u)) >> 20;
  const uint32_t nrm = min((((ua >> 23) - 120u) << 3) + r, 0x7Eu);
  return (a < 0.015625f ? sub : nrm) | sign;
}

// q for fp8 x fp8 scoring, quantised like an fp8 key: four lanes (a quad) per 128-dim vector,
// lane l holding dims 32l..32l+31; scale = fp32(absmax / 448) and codes = e4m3 RNE of
// RN32(q_i / scale) (computed as RN32(q_i * RN64(1 / scale)), equal as for the keys: q_i is a
// bf16 value, and |q_i / scale| <= 448 (1 + 2^-23) stays in e4m3_rne_sat_nb's range).
__global__ __launch_bounds__(256) void quantize_q_kernel(const uint16_t* q, uint8_t* codes,
                                                         float* scales, int64_t n_vec) {
  const int64_t v = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 2;
  const int l = threadIdx.x & 3;
  if (v >= n_vec) return;   // whole quads leave together
  const uint4* src = reinterpret_cast<const uint4*>(q + v * kHeadDim + 32 * l);
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 x = src[i];
    w[4 * i] = x.x;
    w[4 * i + 1] = x.y;
    w[4 * i + 2] = x.z;
    w[4 * i + 3] = x.w;
  }
  // |q| as bit patterns: the max of non-negative floats is the max of their patterns
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    amax = max(amax, max((w[i] << 16) & 0x7FFF0000u, w[i] & 0x7FFF0000u));
  amax = max(amax, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
                       0, static_cast<int>(amax), 0xB1, 0xF, 0xF, false)));   // quad xor 1
  amax = max(amax, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
                       0, static_cast<int>(amax), 0x4E, 0xF, 0xF, false)));   // quad xor 2
  const float scale = static_cast<float>(static_cast<double>(__uint_as_float(amax)) / 448.0);
  const double inv = scale > 0.0f ? 1.0 / static_cast<double>(scale) : 0.0;
  uint32_t c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t bits = w[2 * i + k / 2];
      const float f = __uint_as_float(k & 1 ? bits & 0xFFFF0000u : bits << 16);
      word |= e4m3_rne_sat_nb(static_cast<float>(static_cast<double>(f) * inv)) << (8 * k);
    }
    c[i] = word;   // scale 0: every quotient is 0 (or -0 -> 0x80), replaced below
  }
  uint4* dst = reinterpret_cast<uint4*>(codes + v * kHeadDim + 32 * l);
  const bool zero = !(scale > 0.0f);
  dst[0] = zero ? make_uint4(0, 0, 0, 0) : make_uint4(c[0], c[1], c[2], c[3]);
  dst[1] = zero ? make_uint4(0, 0, 0, 0) : make_uint4(c[4], c[5], c[6], c[7]);
  if (l == 0) scales[v] = scale;
}

// Value of quad lane (lane ^ M), fp32 bits.
template <int M>
__device__ __forceinline__ uint32_t quad_xor_u32(uint32_t v) {
  constexpr int kCtrl = M == 1 ? 0xB1 : 0x4E;
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), kCtrl, 0xF, 0xF, false));
}

// One butterfly stage of span 4 (M = 1) or 8 (M = 2) across the quad: lane l pairs with l ^ M,
// the lower lane taking x_i + x_{i+h} and the upper one x_i - x_{i+h}.
template <int M>
__device__ __forceinline__ void quad_butterfly(double (&v)[8][4], int l) {
#pragma clang fp contract(off)
  const bool upper = (l & M) != 0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const double p = quad_xor<M>(v[i][c]);
      v[i][c] = upper ? p - v[i][c] : v[i][c] + p;
    }
}

// Normalised 128-point Walsh-Hadamard transform (Sylvester order) of the key a quad holds, lane l
// holding dim 16 i + 4 l + c in v[i][c].  Stages of span h = 1, 2, ..., 64 map (x_d, x_{d+h}) to
// (x_d + x_{d+h}, x_d - x_{d+h}) for the d whose bit h is clear: spans 1 and 2 are bits of c,
// spans 4 and 8 bits of l, spans 16, 32 and 64 bits of i.  Every output is the same single
// addition or subtraction of the same two values as in the definition, in stage order, so the
// fp64 result does not depend on the lane mapping.  Then one multiplication by 2^-3.5.
__device__ __forceinline__ void hadamard128_quad(double (&v)[8][4], int l) {
#pragma clang fp contract(off)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    double a = v[i][0], b = v[i][1];
    v[i][0] = a + b;
    v[i][1] = a - b;
    a = v[i][2];
    b = v[i][3];
    v[i][2] = a + b;
    v[i][3] = a - b;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    double a = v[i][0], b = v[i][2];
    v[i][0] = a + b;
    v[i][2] = a - b;
    a = v[i][1];
    b = v[i][3];
    v[i][1] = a + b;
    v[i][3] = a - b;
  }
  quad_butterfly<1>(v, l);
  quad_butterfly<2>(v, l);
#pragma unroll
  for (int h = 1; h <= 4; h <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i & h) continue;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const double a = v[i][c], b = v[i + h][c];
        v[i][c] = a + b;
        v[i + h][c] = a - b;
      }
    }
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) v[i][c] *= kHadamardScale;
}

// Quad q of the grid stores key q.  Quads past the end leave (whole quads together, so the quad
// exchanges stay inside live quads); keys with a bad sequence, index or page are computed and not
// stored.  (Two keys per quad, each wave overlapping its loads of the second key with the
// arithmetic of the first, measured no faster and needed 230-256 registers.)
template <int DT, bool HAD>
__global__ __launch_bounds__(256) void store_keys_kernel(StoreArgs a) {
#pragma clang fp contract(off)
  const int64_t n = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 2;
  const int l = threadIdx.x & 3;
  if (n >= a.n_keys) return;
  const int32_t b = a.key_seq ? a.key_seq[n] : 0;
  const int32_t s = a.key_idx[n];
  float4 xv[8];
  const float* xr = a.x + n * kHeadDim + 4 * l;
#pragma unroll
  for (int i = 0; i < 8; ++i) xv[i] = *reinterpret_cast<const float4*>(xr + 16 * i);
  bool ok = b >= 0 && b < a.n_seq && s >= 0 &&
            static_cast<int64_t>(s) < static_cast<int64_t>(a.max_pages) * kPageKeys;
  const int32_t page = ok ? a.page_table[static_cast<int64_t>(b) * a.max_pages + s / kPageKeys]
                          : -1;
  ok = ok && page >= 0 && page < a.n_pages_pool;
  // gamma: the lane's slices, read up front for the plain store and where each chunk needs them
  // for the rotated one (see below)
  const float* gl = a.gamma + 4 * l;
  float4 gv[8];
  if constexpr (!HAD) {
#pragma unroll
    for (int i = 0; i < 8; ++i) gv[i] = *reinterpret_cast<const float4*>(gl + 16 * i);
  }
  // The frequencies of the lane's pairs p = 8 (t / 2) + 2 l + t % 2, all read here, ahead of the
  // arithmetic: read inside the RoPE, each would be a load that its sincos waits for.
  float fr[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int p0 = 8 * (t / 2) + (t % 2);   // the pair of lane 0
    fr[t] = l < 2 ? (l == 0 ? a.rope.f[p0] : a.rope.f[p0 + 2])
                  : (l == 2 ? a.rope.f[p0 + 4] : a.rope.f[p0 + 6]);
  }

  // RMSNorm in fp64: the squares of fp32 values are exact, summed in the lane, then the quad.
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double x0 = xv[i].x, x1 = xv[i].y, x2 = xv[i].z, x3 = xv[i].w;
    ss = ss + x0 * x0;
    ss = ss + x1 * x1;
    ss = ss + x2 * x2;
    ss = ss + x3 * x3;
  }
  ss = ss + quad_xor<1>(ss);
  ss = ss + quad_xor<2>(ss);
  const double r = 1.0 / sqrt(ss / 128.0 + static_cast<double>(a.eps));

  // RoPE on the pairs (64 + 2p, 65 + 2p) at position 4s, p = 8 (i - 4) + 2 l + c / 2.
  const double pos = static_cast<double>(kRatio) * static_cast<double>(s < 0 ? 0 : s);
  // The rotated store holds the whole key in fp64 for the transform; there each chunk converts
  // its x again (the empty asm hides the reuse), since keeping the norm sum's 32 fp64 values live
  // across the RoPE would cost a wave per SIMD: 150 registers and 3 waves instead of 182 and 2,
  // 5-8% faster.  The plain store is faster with the reuse.
  auto chunk = [&](int i, double (&y)[4]) {
    float4 gi, xi = xv[i];
    if constexpr (HAD) {
      gi = *reinterpret_cast<const float4*>(gl + 16 * i);
      asm volatile("" : "+v"(xi.x), "+v"(xi.y), "+v"(xi.z), "+v"(xi.w));
    } else {
      gi = gv[i];
    }
    y[0] = static_cast<double>(xi.x) * r * static_cast<double>(gi.x);
    y[1] = static_cast<double>(xi.y) * r * static_cast<double>(gi.y);
    y[2] = static_cast<double>(xi.z) * r * static_cast<double>(gi.z);
    y[3] = static_cast<double>(xi.w) * r * static_cast<double>(gi.w);
    if (i < 4) return;
#pragma unroll
    for (int c = 0; c < 4; c += 2) {
      double sn, cs;
      const double th = pos * static_cast<double>(fr[2 * (i - 4) + c / 2]);
      if (s < (1 << 24))
        rope_sincos(th, &sn, &cs);
      else
        sincos(th, &sn, &cs);
      const double ye = y[c], yo = y[c + 1];
      y[c] = ye * cs - yo * sn;
      y[c + 1] = ye * sn + yo * cs;
    }
  };
  float k[8][4];
  if constexpr (HAD) {
    // the rotated store: the Hadamard transform of the whole key, still in fp64
    double v[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) chunk(i, v[i]);
    hadamard128_quad(v, l);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) k[i][c] = static_cast<float>(v[i][c]);
  } else if constexpr (DT == kBf16) {
    // bf16 needs no key-wide maximum: each chunk is rounded and stored as soon as it is computed,
    // one chunk at a time, so that few values are live: 127 registers and 4 waves per SIMD
    // instead of 182 and 2
    if (!ok) return;
    uint8_t* dst = a.kcache + page * kBf16PageBytes + (s % kPageKeys) * (kHeadDim * 2) + 8 * l;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      double y[4];
      chunk(i, y);
      const bf16x2 lo = __builtin_convertvector(
          float2_v{static_cast<float>(y[0]), static_cast<float>(y[1])}, bf16x2);
      const bf16x2 hi = __builtin_convertvector(
          float2_v{static_cast<float>(y[2]), static_cast<float>(y[3])}, bf16x2);
      *reinterpret_cast<uint2*>(dst + 32 * i) =
          make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
      __builtin_amdgcn_sched_barrier(0);
    }
    return;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      double y[4];
      chunk(i, y);
#pragma unroll
      for (int c = 0; c < 4; ++c) k[i][c] = static_cast<float>(y[c]);
    }
  }

  const int slot = s % kPageKeys;
  // The format conversions are the hardware's (v_cvt_pk_bf16_f32, v_cvt_pk_fp8_f32,
  // v_cvt_scalef32_pk_fp4_f32 with scale 1): each rounds to nearest even, gives subnormal codes
  // and keeps the sign of zero, and agrees with the integer round-half-even encoders (bf16_rne
  // and e4m3_rne_sat_nb above, and the same construction with one mantissa bit for e2m1) on every
  // fp32 input of the ranges used here (checked exhaustively on gfx950).  Quotients stay within 448 (1 + 2^-23) (fp8) or
  // 6 (1 + 2^-23) (fp4), which round to the largest finite code, so no saturation is needed.
  if constexpr (DT == kBf16) {
    if (!ok) return;
    uint8_t* dst = a.kcache + page * kBf16PageBytes + slot * (kHeadDim * 2) + 8 * l;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bf16x2 lo = __builtin_convertvector(float2_v{k[i][0], k[i][1]}, bf16x2);
      const bf16x2 hi = __builtin_convertvector(float2_v{k[i][2], k[i][3]}, bf16x2);
      *reinterpret_cast<uint2*>(dst + 32 * i) =
          make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
    }
  } else {
    // |k| as bit patterns: the max of non-negative floats is the max of their patterns
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) am = max(am, __float_as_uint(k[i][c]) & 0x7FFFFFFFu);
    am = max(am, quad_xor_u32<1>(am));
    am = max(am, quad_xor_u32<2>(am));
    if (!ok) return;
    const float amax = __uint_as_float(am);
    if constexpr (DT == kFp4) {
      // as for fp8 below, with the largest e2m1 value 6 for 448
      const float scale = amax / 6.0f;
      const double inv = scale > 0.0f ? 1.0 / static_cast<double>(scale) : 0.0;
      uint8_t* pg = a.kcache + page * kFp4PageBytes;
      uint8_t* dst = pg + slot * (kHeadDim / 2) + 2 * l;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = static_cast<float>(static_cast<double>(k[i][c]) * inv);
        // dims 2m, 2m + 1 are the low and high nibbles of byte m
        uint32_t c4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[0], v[1], 1.0f, 0);
        c4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c4, v[2], v[3], 1.0f, 1);
        *reinterpret_cast<uint16_t*>(dst + 8 * i) = static_cast<uint16_t>(scale > 0.0f ? c4 : 0u);
      }
      if (l == 0) *reinterpret_cast<float*>(pg + kFp4ScaleOffset + slot * 4) = scale;
    } else {
      // The correctly rounded fp32 quotient (HIP's fp32 division is correctly rounded unless
      // fast-math is asked for), which is also the fp64 quotient rounded once to fp32: 53 >= 2 x
      // 24 + 2 bits make that double rounding harmless.
      const float scale = amax / 448.0f;
      // RN32(k * RN64(1/scale)) equals RN32(k / scale): the fp64 product is within 2^-52
      // (relative) of the exact quotient, while a quotient of two fp32 numbers is never closer
      // than ~2^-49 (relative) to an fp32 rounding midpoint.
      const double inv = scale > 0.0f ? 1.0 / static_cast<double>(scale) : 0.0;
      uint8_t* pg = a.kcache + page * kFp8PageBytes;
      uint8_t* dst = pg + slot * kHeadDim + 4 * l;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = static_cast<float>(static_cast<double>(k[i][c]) * inv);
        int c4 = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
        c4 = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], c4, true);
        *reinterpret_cast<uint32_t*>(dst + 16 * i) = scale > 0.0f ? static_cast<uint32_t>(c4) : 0u;
      }
      if (l == 0) *reinterpret_cast<float*>(pg + kFp8ScaleOffset + slot * 4) = scale;
    }
  }
}

}  // namespace

hipError_t launch_quantize_q(const uint16_t* q, uint8_t* codes, float* scales, int64_t n_vec,
                             hipStream_t stream) {
  if (n_vec <= 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>((n_vec + 63) / 64));
  hipLaunchKernelGGL(quantize_q_kernel, grid, dim3(256), 0, stream, q, codes, scales, n_vec);
  return hipGetLastError();
}

hipError_t launch_store(const StoreArgs& a, int dtype, bool hadamard, hipStream_t stream) {
  if (a.n_keys <= 0) return hipSuccess;
  const int64_t keys_per_block = 256 / 4;
  const dim3 grid(static_cast<uint32_t>((a.n_keys + keys_per_block - 1) / keys_per_block));
  if (dtype == kBf16 && hadamard)
    hipLaunchKernelGGL((store_keys_kernel<kBf16, true>), grid, dim3(256), 0, stream, a);
  else if (dtype == kBf16)
    hipLaunchKernelGGL((store_keys_kernel<kBf16, false>), grid, dim3(256), 0, stream, a);
  else if (dtype == kFp4 && hadamard)
    hipLaunchKernelGGL((store_keys_kernel<kFp4, true>), grid, dim3(256), 0, stream, a);
  else if (dtype == kFp4)
    hipLaunchKernelGGL((store_keys_kernel<kFp4, false>), grid, dim3(256), 0, stream, a);
  else if (hadamard)
    hipLaunchKernelGGL((store_keys_kernel<kFp8, true>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((store_keys_kernel<kFp8, false>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_rotate_q(const uint16_t* in, uint16_t* out, int64_t n_vec, hipStream_t stream) {
  if (n_vec <= 0) return hipSuccess;
  const int64_t vec_per_block = 256 / 4;
  const dim3 grid(static_cast<uint32_t>((n_vec + vec_per_block - 1) / vec_per_block));
  hipLaunchKernelGGL(rotate_q_kernel, grid, dim3(256), 0, stream, in, out, n_vec);
  return hipGetLastError();
}

}  // namespace dsa
