// dkv_device.h - device helpers shared by the gfx950 kernel files: bf16
// conversions with one rounding, vector types, and buffer accesses coherent
// across XCDs.
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

// Buffer accesses that are coherent across XCDs: cache policy sc1 makes a
// store write through to the device-coherent level and a load read from it,
// so no L2 write-back or invalidate is needed around them.
constexpr int kCoherent = 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}

__device__ __forceinline__ void coherent_store4(__amdgpu_buffer_rsrc_t r, int byte_off, floatx4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, byte_off, 0, kCoherent);
}
__device__ __forceinline__ void coherent_store1(__amdgpu_buffer_rsrc_t r, int byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, byte_off, 0, kCoherent);
}
__device__ __forceinline__ floatx4 coherent_load4(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kCoherent));
}
__device__ __forceinline__ float coherent_load1(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, kCoherent));
}

// Waits until this thread's stores are acknowledged (written at the coherent
// level for the sc1 stores above).
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace dkv
