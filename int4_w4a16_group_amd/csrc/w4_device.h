// Device-side helpers for the gfx950 kernels: fp16 vectors, MFMA operand
// types, and the int4 -> fp16 operand conversion of the repacked bank.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
// IEEE round to nearest even (v_cvt_f16_f32 in the default rounding mode).
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

__device__ __forceinline__ f4 mfma16x16x32(const h8& a, const h8& b, const f4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// One repacked dword (8 offset-binary codes, see Mat in w4_internal.h) to the
// 8 fp16 codes of k = k0 .. k0+7 in order.  (1024 + u) - 1032 = u - 8 = code,
// exact in fp16.
__device__ __forceinline__ h8 dq8(uint32_t w) {
  const h2 bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const h2 p0 = __builtin_bit_cast(h2, (w & 0x000F000Fu) | 0x64006400u) + bias;
  const h2 p1 = __builtin_bit_cast(h2, ((w >> 4) & 0x000F000Fu) | 0x64006400u) + bias;
  const h2 p2 = __builtin_bit_cast(h2, ((w >> 8) & 0x000F000Fu) | 0x64006400u) + bias;
  const h2 p3 = __builtin_bit_cast(h2, ((w >> 12) & 0x000F000Fu) | 0x64006400u) + bias;
  return h8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

__device__ __forceinline__ h8 ld_h8(const uint16_t* p) { return *reinterpret_cast<const h8*>(p); }

}  // namespace w4
