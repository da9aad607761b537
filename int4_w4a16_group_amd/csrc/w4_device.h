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

// One repacked dword (8 offset-binary codes u = code + 8, see Mat in
// w4_internal.h: nibble j holds element 2j, nibble j+4 holds element 2j+1) to
// the 8 fp16 codes of k = k0 .. k0+7 in order, 9 VALU operations:
//   pair (2j, 2j+1) for j = 0, 2: (w' & 0x000F000F) | 0x6400 6400 is the fp16
//     pair (1024 + u, 1024 + u'), minus 1032 gives the codes;
//   pair for j = 1, 3: (w' & 0x00F000F0) | 0x6400 6400 is (1024 + 16u, ...),
//     times 1/16 minus 72 (one fma) gives the codes;
// with w' = w for j = 0, 1 and w >> 8 for j = 2, 3.  Every step is exact in
// fp16 (integers below 2048, a power-of-two scale, one rounding of an exact
// integer result).  The masks sit in VGPRs so each and-or is one v_and_or_b32
// (two literal operands would not encode in one VOP3 instruction).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t vmask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(vmask), "s"(magic));
  return r;
}

struct DqConst {
  uint32_t m_lo, m_hi;  // 0x000F000F, 0x00F000F0 held in VGPRs
  __device__ __forceinline__ DqConst() {
    asm("v_mov_b32 %0, 0x000F000F" : "=v"(m_lo));
    asm("v_mov_b32 %0, 0x00F000F0" : "=v"(m_hi));
  }
};

__device__ __forceinline__ h8 dq8(uint32_t w, const DqConst& k) {
  const h2 bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const h2 bias16 = {(_Float16)-72.0f, (_Float16)-72.0f};
  const uint32_t ws = w >> 8;
  const h2 p0 = __builtin_bit_cast(h2, and_or(w, k.m_lo, 0x64006400u)) + bias;
  const h2 p1 = __builtin_elementwise_fma(__builtin_bit_cast(h2, and_or(w, k.m_hi, 0x64006400u)), sixteenth, bias16);
  const h2 p2 = __builtin_bit_cast(h2, and_or(ws, k.m_lo, 0x64006400u)) + bias;
  const h2 p3 = __builtin_elementwise_fma(__builtin_bit_cast(h2, and_or(ws, k.m_hi, 0x64006400u)), sixteenth, bias16);
  return h8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

__device__ __forceinline__ h8 ld_h8(const uint16_t* p) { return *reinterpret_cast<const h8*>(p); }

// Non-temporal loads (the nt bit) for data a step reads once: the weight
// tiles and the KV chunks.  Measured on MI355X, one pass over 4 GiB with
// 16-byte loads streams at 6.3-6.75 TB/s non-temporal against 5.4-6.0 TB/s
// plain.
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ h8 ld_h8_nt(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const h8*>(p));
}
__device__ __forceinline__ uint32_t ld_u32_nt(const uint32_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ uint16_t ld_u16_nt(const uint16_t* p) { return __builtin_nontemporal_load(p); }

}  // namespace w4
