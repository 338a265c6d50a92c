// S1: fused RMSNorm + RoPE + quantise + paged store of compressed index keys.
//
// The fused store of the DSA indexer ("The Moment of Validation", Input Knowledge Required: one
// kernel normalises, rotates and writes the cache; "The Fused Kernel Decision", Message: the cache
// is [npages, 64*128] and a key goes to (page, offset)).  fp8 keys are e4m3 codes plus one fp32
// scale per key, 132 B/token; bf16 keys are 256 B/token ("When the Fused Kernel Isn't Enough",
// Input Knowledge Required).
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

template <int DT>
__global__ __launch_bounds__(256) void store_keys_kernel(StoreArgs a) {
#pragma clang fp contract(off)
  const int64_t n_raw = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 5;
  const int j = threadIdx.x & 31;
  const bool in_range = n_raw < a.n_keys;
  const int64_t n = in_range ? n_raw : a.n_keys - 1;   // idle half-waves recompute the last key

  const int32_t b = a.key_seq ? a.key_seq[n] : 0;
  const int32_t s = a.key_idx[n];
  bool ok = in_range && b >= 0 && b < a.n_seq && s >= 0 &&
            static_cast<int64_t>(s) < static_cast<int64_t>(a.max_pages) * kPageKeys;
  int32_t page = -1;
  if (ok) {
    page = a.page_table[static_cast<int64_t>(b) * a.max_pages + s / kPageKeys];
    ok = page >= 0 && page < a.n_pages_pool;
  }

  const float* xr = a.x + n * kHeadDim;
  const float2 xa = *reinterpret_cast<const float2*>(xr + 2 * j);
  const float2 xb = *reinterpret_cast<const float2*>(xr + 64 + 2 * j);
  const float2 ga = *reinterpret_cast<const float2*>(a.gamma + 2 * j);
  const float2 gb = *reinterpret_cast<const float2*>(a.gamma + 64 + 2 * j);

  // RMSNorm in fp64.
  const double x0 = xa.x, x1 = xa.y, x2 = xb.x, x3 = xb.y;
  double ss = x0 * x0 + x1 * x1 + x2 * x2 + x3 * x3;
  ss = half_wave_sum(ss);
  const double r = 1.0 / sqrt(ss / 128.0 + static_cast<double>(a.eps));
  const double y0 = x0 * r * static_cast<double>(ga.x);
  const double y1 = x1 * r * static_cast<double>(ga.y);
  double y2 = x2 * r * static_cast<double>(gb.x);
  double y3 = x3 * r * static_cast<double>(gb.y);

  // RoPE on the pair (64+2j, 65+2j) at position 4s.
  const double phi = static_cast<double>(kRatio) * static_cast<double>(s < 0 ? 0 : s) *
                     static_cast<double>(a.rope.f[j]);
  double sn, cs;
  sincos(phi, &sn, &cs);
  const double r2 = y2 * cs - y3 * sn;
  const double r3 = y2 * sn + y3 * cs;

  const float k0 = static_cast<float>(y0), k1 = static_cast<float>(y1);
  const float k2 = static_cast<float>(r2), k3 = static_cast<float>(r3);

  if constexpr (DT == kBf16) {
    if (!ok) return;
    uint8_t* dst = a.kcache + page * kBf16PageBytes + (s % kPageKeys) * (kHeadDim * 2);
    *reinterpret_cast<uint32_t*>(dst + 4 * j) = bf16_rne(k0) | (bf16_rne(k1) << 16);
    *reinterpret_cast<uint32_t*>(dst + 128 + 4 * j) = bf16_rne(k2) | (bf16_rne(k3) << 16);
  } else {
    float amax = fmaxf(fmaxf(fabsf(k0), fabsf(k1)), fmaxf(fabsf(k2), fabsf(k3)));
    amax = half_wave_max(amax);
    if (!ok) return;
    // fp64 quotient of fp32 operands rounded once = the correctly rounded fp32 quotient.
    const float scale = static_cast<float>(static_cast<double>(amax) / 448.0);
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

}  // namespace

hipError_t launch_store(const StoreArgs& a, int dtype, hipStream_t stream) {
  if (a.n_keys <= 0) return hipSuccess;
  const int64_t keys_per_block = 256 / 32;
  const int64_t blocks = (a.n_keys + keys_per_block - 1) / keys_per_block;
  if (dtype == kBf16)
    hipLaunchKernelGGL(store_keys_kernel<kBf16>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                       stream, a);
  else
    hipLaunchKernelGGL(store_keys_kernel<kFp8>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                       stream, a);
  return hipGetLastError();
}

}  // namespace dsa
