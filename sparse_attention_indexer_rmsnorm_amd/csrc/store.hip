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
// Work mapping: one half-wave (32 lanes) per key.  Lane j owns the unrotated dims 2j, 2j+1 and the
// rotated pair (64+2j, 65+2j), so every lane evaluates exactly one sincos.  The arithmetic before
// the format rounding is fp64 so that the stored bytes are a function of the inputs alone, not of
// the reduction order: a result only depends on the order when it sits within ~2^-50 of a
// rounding boundary.  The work is HBM-bound (512 B read and 132/256 B written per key).
#include "internal.h"

namespace dsa {
namespace {

// Round a finite fp32 to bf16, nearest-even, returned in the low 16 bits.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Round a finite fp32 to OCP e4m3fn (bias 7, max 448, no inf), nearest-even, saturating to 448.
// Normal range [2^-6, 448): keep 3 mantissa bits of the fp32 significand with round-half-even;
// a carry out of the mantissa moves to the next binade by plain addition of the code.
// Subnormal range [0, 2^-6): the code is the integer round-half-even of |v| * 2^9 (8 = 2^-6).
__device__ __forceinline__ uint32_t e4m3_rne_sat(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t code;
  if (a >= 448.0f) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {
    code = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
  } else {
    const uint32_t ua = __float_as_uint(a);
    const uint32_t e = (ua >> 23) - 120u;
    const uint32_t m = ua & 0x7FFFFFu;
    const uint32_t r = (m + 0x7FFFFu + ((m >> 20) & 1u)) >> 20;
    code = (e << 3) + r;
    code = code > 0x7Eu ? 0x7Eu : code;
  }
  return code | sign;
}

// Round a finite fp32 to OCP e2m1 (sign, 2 exponent bits with bias 1, 1 mantissa bit; largest
// 6), nearest-even, saturating to 6.  |v| >= 1: keep 1 mantissa bit with round-half-even, a carry
// moving to the next binade by plain addition of the code; |v| < 1: the code is the integer
// round-half-even of |v| * 2 (0, 0.5 or 1.0).  Without branches.
__device__ __forceinline__ uint32_t e2m1_rne_sat(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 28) & 0x8u;
  const float a = fabsf(v);
  const uint32_t sub = static_cast<uint32_t>(__builtin_rintf(a * 2.0f));
  const uint32_t ua = __float_as_uint(a);
  const uint32_t m = ua & 0x7FFFFFu;
  const uint32_t r = (m + 0x1FFFFFu + ((m >> 22) & 1u)) >> 22;
  const uint32_t nrm = min((((ua >> 23) - 126u) << 1) + r, 7u);
  return (a < 1.0f ? sub : nrm) | sign;
}

template <typename T>
__device__ __forceinline__ T half_wave_sum(T v) {
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float half_wave_max(float v) {
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// The nearest double to 2^-3.5 (sqrt(2) / 16): the normalisation of the 128-point transform.
constexpr double kHadamardScale = 0x1.6a09e667f3bcdp-4;

// Normalised 128-point Walsh-Hadamard transform (Sylvester order) of the vector a half-wave holds,
// lane j (0..31) owning dims 2j, 2j+1 (v0, v1) and 64+2j, 65+2j (v2, v3).  Butterfly stages of
// span h = 1, 2, ..., 64 map (x_i, x_{i+h}) to (x_i + x_{i+h}, x_i - x_{i+h}) for the i whose bit
// h is clear; spans 1 and 64 pair values inside a lane, spans 2..32 pair lane j with lane
// j ^ (h/2), the lower lane taking the sum and the upper one the difference.  The operations are
// those of the definition, in a fixed order, so the fp64 result does not depend on the lane
// mapping.  Then one multiplication by 2^-3.5.
__device__ __forceinline__ void hadamard128(double& v0, double& v1, double& v2, double& v3,
                                            int j) {
#pragma clang fp contract(off)
  double a = v0, b = v1;
  v0 = a + b;
  v1 = a - b;
  a = v2;
  b = v3;
  v2 = a + b;
  v3 = a - b;
#pragma unroll
  for (int m = 1; m <= 16; m <<= 1) {
    const bool upper = (j & m) != 0;
    const double p0 = __shfl_xor(v0, m, 64), p1 = __shfl_xor(v1, m, 64);
    const double p2 = __shfl_xor(v2, m, 64), p3 = __shfl_xor(v3, m, 64);
    v0 = upper ? p0 - v0 : v0 + p0;
    v1 = upper ? p1 - v1 : v1 + p1;
    v2 = upper ? p2 - v2 : v2 + p2;
    v3 = upper ? p3 - v3 : v3 + p3;
  }
  a = v0;
  b = v2;
  v0 = a + b;
  v2 = a - b;
  a = v1;
  b = v3;
  v1 = a + b;
  v3 = a - b;
  v0 *= kHadamardScale;
  v1 *= kHadamardScale;
  v2 *= kHadamardScale;
  v3 *= kHadamardScale;
}

// Keys per half-wave: all of them are requested (indices, activations, then page ids) before any
// is computed, so a wave has several rows of activations in flight.
constexpr int kStoreKeysPerHalfWave = 4;

// One key (row n, sequence b, index s, activations xa/xb, destination page), computed and stored
// by the 32 lanes of a half-wave; lane j owns dims 2j, 2j+1 and the rotated pair 64+2j, 65+2j.
template <int DT, bool HAD>
__device__ __forceinline__ void store_one(const StoreArgs& a, int j, bool ok, int32_t page,
                                          int32_t s, float2 xa, float2 xb, float2 ga, float2 gb) {
#pragma clang fp contract(off)
  // RMSNorm in fp64.
  const double x0 = xa.x, x1 = xa.y, x2 = xb.x, x3 = xb.y;
  double ss = x0 * x0 + x1 * x1 + x2 * x2 + x3 * x3;
  ss = half_wave_sum(ss);
  const double r = 1.0 / sqrt(ss / 128.0 + static_cast<double>(a.eps));
  double y0 = x0 * r * static_cast<double>(ga.x);
  double y1 = x1 * r * static_cast<double>(ga.y);
  double y2 = x2 * r * static_cast<double>(gb.x);
  double y3 = x3 * r * static_cast<double>(gb.y);

  // RoPE on the pair (64+2j, 65+2j) at position 4s.
  const double phi = static_cast<double>(kRatio) * static_cast<double>(s < 0 ? 0 : s) *
                     static_cast<double>(a.rope.f[j]);
  double sn, cs;
  sincos(phi, &sn, &cs);
  double r2 = y2 * cs - y3 * sn;
  double r3 = y2 * sn + y3 * cs;
  // the rotated store: the Hadamard transform of the whole key, still in fp64
  if constexpr (HAD) hadamard128(y0, y1, r2, r3, j);

  const float k0 = static_cast<float>(y0), k1 = static_cast<float>(y1);
  const float k2 = static_cast<float>(r2), k3 = static_cast<float>(r3);

  if constexpr (DT == kBf16) {
    if (!ok) return;
    uint8_t* dst = a.kcache + page * kBf16PageBytes + (s % kPageKeys) * (kHeadDim * 2);
    *reinterpret_cast<uint32_t*>(dst + 4 * j) = bf16_rne(k0) | (bf16_rne(k1) << 16);
    *reinterpret_cast<uint32_t*>(dst + 128 + 4 * j) = bf16_rne(k2) | (bf16_rne(k3) << 16);
  } else if constexpr (DT == kFp4) {
    float amax = fmaxf(fmaxf(fabsf(k0), fabsf(k1)), fmaxf(fabsf(k2), fabsf(k3)));
    amax = half_wave_max(amax);
    if (!ok) return;
    // as for fp8 below, with the largest e2m1 value 6 for 448
    const float scale = amax / 6.0f;
    uint32_t c01 = 0, c23 = 0;
    if (scale > 0.0f) {
      const double inv = 1.0 / static_cast<double>(scale);
      c01 = e2m1_rne_sat(static_cast<float>(static_cast<double>(k0) * inv)) |
            (e2m1_rne_sat(static_cast<float>(static_cast<double>(k1) * inv)) << 4);
      c23 = e2m1_rne_sat(static_cast<float>(static_cast<double>(k2) * inv)) |
            (e2m1_rne_sat(static_cast<float>(static_cast<double>(k3) * inv)) << 4);
    }
    uint8_t* pg = a.kcache + page * kFp4PageBytes;
    uint8_t* dst = pg + (s % kPageKeys) * (kHeadDim / 2);
    dst[j] = static_cast<uint8_t>(c01);         // dims 2j, 2j+1: low, high nibble of byte j
    dst[32 + j] = static_cast<uint8_t>(c23);    // dims 64+2j, 65+2j
    if (j == 0) *reinterpret_cast<float*>(pg + kFp4ScaleOffset + (s % kPageKeys) * 4) = scale;
  } else {
    float amax = fmaxf(fmaxf(fabsf(k0), fabsf(k1)), fmaxf(fabsf(k2), fabsf(k3)));
    amax = half_wave_max(amax);
    if (!ok) return;
    // The correctly rounded fp32 quotient (HIP's fp32 division is correctly rounded unless
    // fast-math is asked for), which is also the fp64 quotient rounded once to fp32: 53 >= 2 x 24
    // + 2 bits make that double rounding harmless.
    const float scale = amax / 448.0f;
    uint32_t c01 = 0, c23 = 0;
    if (scale > 0.0f) {
      // RN32(k * RN64(1/scale)) equals RN32(k / scale): the fp64 product is within 2^-52
      // (relative) of the exact quotient, while a quotient of two fp32 numbers is never closer
      // than ~2^-49 (relative) to an fp32 rounding midpoint.
      const double inv = 1.0 / static_cast<double>(scale);
      const float v0 = static_cast<float>(static_cast<double>(k0) * inv);
      const float v1 = static_cast<float>(static_cast<double>(k1) * inv);
      const float v2 = static_cast<float>(static_cast<double>(k2) * inv);
      const float v3 = static_cast<float>(static_cast<double>(k3) * inv);
      c01 = e4m3_rne_sat(v0) | (e4m3_rne_sat(v1) << 8);
      c23 = e4m3_rne_sat(v2) | (e4m3_rne_sat(v3) << 8);
    }
    uint8_t* pg = a.kcache + page * kFp8PageBytes;
    uint8_t* dst = pg + (s % kPageKeys) * kHeadDim;
    *reinterpret_cast<uint16_t*>(dst + 2 * j) = static_cast<uint16_t>(c01);
    *reinterpret_cast<uint16_t*>(dst + 64 + 2 * j) = static_cast<uint16_t>(c23);
    if (j == 0) *reinterpret_cast<float*>(pg + kFp8ScaleOffset + (s % kPageKeys) * 4) = scale;
  }
}

// Half-wave h of the grid stores keys h U .. h U + U - 1 (U = kStoreKeysPerHalfWave).  Half-waves
// past the end recompute the last key without storing it, so every lane takes part in the
// half-wave reductions.
template <int DT, bool HAD>
__global__ __launch_bounds__(256) void store_keys_kernel(StoreArgs a) {
  constexpr int U = kStoreKeysPerHalfWave;
  const int64_t hw = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 5;
  const int j = threadIdx.x & 31;
  int32_t bq[U], sq[U], page[U];
  bool ok[U];
  float2 xa[U], xb[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t n_raw = hw * U + u;
    ok[u] = n_raw < a.n_keys;
    const int64_t n = ok[u] ? n_raw : a.n_keys - 1;
    bq[u] = a.key_seq ? a.key_seq[n] : 0;
    sq[u] = a.key_idx[n];
    const float* xr = a.x + n * kHeadDim;
    xa[u] = *reinterpret_cast<const float2*>(xr + 2 * j);
    xb[u] = *reinterpret_cast<const float2*>(xr + 64 + 2 * j);
  }
  const float2 ga = *reinterpret_cast<const float2*>(a.gamma + 2 * j);
  const float2 gb = *reinterpret_cast<const float2*>(a.gamma + 64 + 2 * j);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int32_t b = bq[u], s = sq[u];
    ok[u] = ok[u] && b >= 0 && b < a.n_seq && s >= 0 &&
            static_cast<int64_t>(s) < static_cast<int64_t>(a.max_pages) * kPageKeys;
    page[u] = ok[u] ? a.page_table[static_cast<int64_t>(b) * a.max_pages + s / kPageKeys] : -1;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const bool okp = ok[u] && page[u] >= 0 && page[u] < a.n_pages_pool;
    store_one<DT, HAD>(a, j, okp, page[u], sq[u], xa[u], xb[u], ga, gb);
  }
}

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

// e4m3_rne_sat without branches (the same code for every finite input of magnitude <= 2^15):
// the normal-range and subnormal-range codes are both formed and one is selected, so lanes of
// different magnitudes do not split the wave.
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
  const int64_t keys_per_block = 256 / 32 * kStoreKeysPerHalfWave;
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
