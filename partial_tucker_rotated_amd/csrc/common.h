// Device-side helpers shared by the JoLT kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

#define JOLT_KMAX 32      // largest truncated rank on the grid {4, 8, 16, 32, full}
#define JOLT_NCHAIN 6     // 5 feature ranks (token rank nested) + the full-token chain
#define JOLT_PSUB 64      // columns of the exact-mode token subspace iteration
#define JOLT_GRAM_PARTS 32  // most row-chunk partials of an orthonormalisation Gram

struct TablePtrs {
  const void* p[64];
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp64 -> bf16 with round-to-nearest-even on the bit pattern (finite, bf16-normal range)
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  const uint64_t u = __double_as_longlong(x);
  const uint64_t sign = u >> 63;
  const uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
  if (a == 0) return (uint16_t)(sign << 15);
  const int64_t e8 = (int64_t)(a >> 52) - 1023 + 127;
  if (e8 < 1) return (uint16_t)(sign << 15);            // below the bf16 normal range
  if (e8 > 254) return (uint16_t)((sign << 15) | 0x7F80u);
  uint64_t mag = ((uint64_t)e8 << 7) | ((a >> 45) & 0x7Fu);
  const uint64_t rem = a & ((1ull << 45) - 1), half = 1ull << 44;
  if (rem > half || (rem == half && (mag & 1))) mag += 1;
  return (uint16_t)((sign << 15) | mag);
}

// The same rounding through fp32: fp64 -> fp32 rounded to odd (the nearest fp32, moved one
// ulp toward zero and given an odd last bit when inexact), then fp32 -> bf16 to nearest even.
// Rounding to odd with at least two more bits than the target makes the second rounding
// equal to the direct one (Boldo and Melquiond, "Emulation of FMA and correctly rounded
// sums: proved algorithms using rounding to odd", 2008); same range handling as above.
__device__ __forceinline__ uint16_t f64_to_bf16_rto(double x) {
  const uint16_t sign = (uint16_t)((__double_as_longlong(x) >> 48) & 0x8000);
  const double ax = fabs(x);
  if (!(ax < 0x1p128)) return (uint16_t)(sign | 0x7F80u);
  if (ax < 0x1p-126) return sign;
  const float f = (float)x;
  uint32_t u = __float_as_uint(f);
  if ((double)f != x) {
    if (fabs((double)f) > ax) u -= 1u;
    u |= 1u;
  }
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp64 -> fp16 with round-to-nearest-even on the bit pattern (no double rounding)
__device__ __forceinline__ _Float16 f64_to_f16(double x) {
  const uint64_t u = __double_as_longlong(x);
  const uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
  const uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
  if (a == 0) return __builtin_bit_cast(_Float16, sign);
  const int e = (int)(a >> 52) - 1023;
  if (e > 15) return __builtin_bit_cast(_Float16, (uint16_t)(sign | 0x7C00u));  // overflow -> inf
  uint64_t mant = (a & ((1ull << 52) - 1)) | (1ull << 52);  // 53-bit significand
  int shift;  // bits to drop from the 53-bit significand
  uint16_t expbits;
  if (e >= -14) {
    shift = 52 - 10;
    expbits = (uint16_t)((e + 15) << 10);
  } else {
    shift = 52 - 10 + (-14 - e);  // subnormal: value = m * 2^-24
    expbits = 0;
    if (shift > 63) return __builtin_bit_cast(_Float16, sign);
  }
  uint64_t q = mant >> shift;
  const uint64_t rem = mant & ((1ull << shift) - 1), half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) q += 1;
  uint16_t bits;
  if (expbits) {
    bits = (uint16_t)(expbits + (uint16_t)(q - (1u << 10)));  // carry moves into the exponent
    if (q >> 11) bits = (uint16_t)(expbits + (1u << 10));      // significand overflowed to 2.0
  } else {
    bits = (uint16_t)q;  // may become the smallest normal through carry
  }
  if ((bits & 0x7C00u) == 0x7C00u) bits = 0x7C00u;
  return __builtin_bit_cast(_Float16, (uint16_t)(sign | bits));
}

__device__ __forceinline__ float4_t mfma16(half4_t a, half4_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4_t mfma16bf(short4_t a, short4_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// scale 2^(14 - ceil(log2(x))) that maps a Gram bounded by x (> 0) below 2^14
__device__ __forceinline__ float gram_scale_from_norm(double x) {
  if (!(x > 0.0)) return 1.0f;
  int e;
  frexp(x, &e);  // x = f * 2^e, f in [0.5, 1)
  return ldexpf(1.0f, 14 - e);
}

// cross-lane moves within 16-lane rows (DPP; all lanes of the wave must be active)
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const long long u = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_mov_dpp((int)u, CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp((int)(u >> 32), CTRL, 0xF, 0xF, true);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
// sum over each group of 16 lanes, returned to every lane of the group
// (quad xor 1, quad xor 2, half-row mirror, row mirror)
__device__ __forceinline__ double row16_sum_f64(double v) {
  v += dpp_f64<0xB1>(v);
  v += dpp_f64<0x4E>(v);
  v += dpp_f64<0x141>(v);
  v += dpp_f64<0x140>(v);
  return v;
}
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const long long u = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)u, lane);
  const int hi = __builtin_amdgcn_readlane((int)(u >> 32), lane);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
// sum over the 64 lanes of a wave, uniform result (all lanes must be active)
__device__ __forceinline__ double wave_sum_f64(double v) {
  v = row16_sum_f64(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}
__device__ __forceinline__ float wave_max_f32(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
