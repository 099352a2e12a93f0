// Device helpers for the pkv kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

template <class To, class From>
__device__ __forceinline__ To bitcast(const From& x) {
  static_assert(sizeof(To) == sizeof(From), "size mismatch");
  To r;
  __builtin_memcpy(&r, &x, sizeof(To));
  return r;
}

// ---------------------------------------------------------------- formats
// All encoders below round to nearest, ties to even, on the exact fp32
// input, using integer arithmetic on the bit pattern so that the result
// does not depend on the hardware rounding or denormal modes.

// fp32 -> binary16 bits (overflow to +-inf, NaN to a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  const uint32_t x = __float_as_uint(f);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const uint32_t ax = x & 0x7FFFFFFFu;
  if (ax > 0x7F800000u) return sign | 0x7E00u;
  if (ax >= 0x477FF000u) return sign | 0x7C00u;  // >= 65520 rounds past 65504
  if (ax >= 0x38800000u) {                        // >= 2^-14: normal result
    uint32_t r = ((ax >> 23) - 112u) << 10 | ((ax >> 13) & 0x3FFu);
    const uint32_t rem = ax & 0x1FFFu;
    r += (rem > 0x1000u) | ((rem == 0x1000u) & (r & 1u));
    return sign | r;
  }
  // subnormal result: quantum 2^-24; |f| * 2^24 < 1024 is exact in fp32
  const float a = __uint_as_float(ax) * 16777216.0f;
  return sign | (uint32_t)__builtin_rintf(a);
}

// fp32 -> bfloat16 bits.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t x = __float_as_uint(f);
  if ((x & 0x7FFFFFFFu) > 0x7F800000u) return ((x >> 16) & 0x8000u) | 0x7FC0u;
  const uint32_t r = x + 0x7FFFu + ((x >> 16) & 1u);
  return r >> 16;
}

// binary16 bits -> fp32 (exact, subnormals included).
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  const uint32_t sign = (h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1Fu, m = h & 0x3FFu;
  if (e == 0) {
    const float v = (float)m * 5.9604644775390625e-8f;  // m * 2^-24, exact
    return __uint_as_float(__float_as_uint(v) | sign);
  }
  if (e == 31) return __uint_as_float(sign | 0x7F800000u | (m << 13));
  return __uint_as_float(sign | ((e + 112u) << 23) | (m << 13));
}

// fp32 -> OCP E4M3 code, saturating at +-448 (largest finite magnitude).
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  const uint32_t x = __float_as_uint(y);
  const uint32_t sign = (x >> 24) & 0x80u;
  const uint32_t ax = x & 0x7FFFFFFFu;
  if (ax > 0x7F800000u) return sign | 0x7Fu;
  if (ax >= 0x43E80000u) return sign | 0x7Eu;  // >= 464: past 448 (464 itself ties to 448)
  if (ax >= 0x3C800000u) {                     // >= 2^-6: normal code
    uint32_t r = ((ax >> 23) - 120u) << 3 | ((ax >> 20) & 0x7u);
    const uint32_t rem = ax & 0xFFFFFu;
    r += (rem > 0x80000u) | ((rem == 0x80000u) & (r & 1u));
    return sign | r;
  }
  const float a = __uint_as_float(ax) * 512.0f;  // subnormal quantum 2^-9
  return sign | (uint32_t)__builtin_rintf(a);
}

// OCP E4M3 code -> fp32 (exact; NaN for the two NaN codes).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xFu, f = c & 0x7u;
  float v;
  if (e == 15u && f == 7u)
    v = __builtin_nanf("");
  else if (e == 0u)
    v = (float)f * 0.001953125f;  // f * 2^-9
  else
    v = __uint_as_float(((e + 120u) << 23) | (f << 20));
  return (c & 0x80u) ? -v : v;
}

// fp32 -> OCP E5M2 code, saturating at +-57344 (largest finite magnitude).
__device__ __forceinline__ uint32_t f32_to_e5m2(float y) {
  const uint32_t x = __float_as_uint(y);
  const uint32_t sign = (x >> 24) & 0x80u;
  const uint32_t ax = x & 0x7FFFFFFFu;
  if (ax > 0x7F800000u) return sign | 0x7Fu;
  if (ax >= 0x47600000u) return sign | 0x7Bu;  // >= 57344 (infinities included)
  if (ax >= 0x38800000u) {                     // >= 2^-14: normal code
    uint32_t r = ((ax >> 23) - 112u) << 2 | ((ax >> 21) & 0x3u);
    const uint32_t rem = ax & 0x1FFFFFu;
    r += (rem > 0x100000u) | ((rem == 0x100000u) & (r & 1u));
    return sign | r;
  }
  const float a = __uint_as_float(ax) * 65536.0f;  // subnormal quantum 2^-16
  return sign | (uint32_t)__builtin_rintf(a);
}

// ------------------------------------------------------------ wave reduce

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

template <int WIDTH>
__device__ __forceinline__ float group_min(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}

template <int WIDTH>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace pkv
