// dkv_device.h - device helpers shared by the gfx950 kernel files: bf16
// conversions with one rounding, vector types, and the cache slot of an
// appended token.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "dkv_internal.h"

namespace dkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// double -> bf16 bits with one rounding (nearest, ties to even).
__device__ __forceinline__ uint32_t f64_to_bf16(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t sign = (uint32_t)(u >> 63) << 15;
  const int e = (int)((u >> 52) & 0x7ff);
  if (e == 0x7ff) return sign | ((u << 12) ? 0x7fc0u : 0x7f80u);
  const double ax = fabs(x);
  if (ax < 0x1p-126) {
    // subnormal bf16 grid: quantum 2^-133
    const double q = rint(ax * 0x1p133);  // 0 .. 128 (128 = smallest normal)
    return sign | (uint32_t)q;
  }
  const uint64_t mant = u & ((1ull << 52) - 1);
  uint64_t keep = mant >> 45;
  const uint64_t rest = mant & ((1ull << 45) - 1);
  const uint64_t half = 1ull << 44;
  uint32_t em = (uint32_t)((e - 1023 + 127) << 7) | (uint32_t)keep;
  if (rest > half || (rest == half && (keep & 1))) em += 1;  // may carry into the exponent
  if (em >= 0x7f80u) em = 0x7f80u;                           // overflow -> inf
  return sign | em;
}

}  // namespace dkv
