// Device helpers shared by the gfx950 kernels of the quantizer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tqd {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// 32x32x16 fp16 MFMA (fp32 accumulate).  Operand layout (gfx950): lane l
// supplies row/column l % 32 and the 8 consecutive K values of group l / 32;
// output element (row 8*(r/4) + 4*(l/32) + r%4, column l%32) sits in
// register r of lane l.
__device__ __forceinline__ f32x16 mfma32(half8 a, half8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// 16x16x64 int8 MFMA (int32 accumulate).  Lane l supplies row/column l % 16
// and 16 K values of group l / 16; output (row 4*(l/16) + i, column l%16) is
// register i of lane l.
__device__ __forceinline__ i32x4 mfma_i8(i32x4 a, i32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  _Float16 h;
  __builtin_memcpy(&h, &b, 2);
  return (float)h;
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
  _Float16 h = (_Float16)v;  // round to nearest even
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFF) ? 0x40 : 0));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Correctly rounded (nearest even) fp64 -> fp16 bits, including subnormal
// results and overflow to infinity.  Avoids the double rounding of
// fp64 -> fp32 -> fp16.
__device__ __forceinline__ uint16_t f64_to_f16_bits(double v) {
  uint64_t b = (uint64_t)__double_as_longlong(v);
  uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  b &= 0x7FFFFFFFFFFFFFFFull;
  if (b >= 0x7FF0000000000000ull) {  // inf or nan
    return sign | (b > 0x7FF0000000000000ull ? 0x7E00u : 0x7C00u);
  }
  int e = (int)(b >> 52) - 1023;
  uint64_t mant = (b & 0x000FFFFFFFFFFFFFull) | 0x0010000000000000ull;
  if ((b >> 52) == 0) return sign;  // fp64 subnormal -> 0 in fp16
  if (e > 15) return sign | 0x7C00u;
  int shift;
  uint32_t base;
  if (e >= -14) {
    shift = 42;  // keep 11 significant bits
    base = (uint32_t)(e + 15) << 10;
  } else {
    shift = 42 + (-14 - e);  // subnormal: units of 2^-24
    base = 0;
    if (shift > 63) return sign;
  }
  uint64_t q = mant >> shift;
  uint64_t rem = mant & ((1ull << shift) - 1);
  uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) q += 1;
  uint32_t res;
  if (e >= -14)
    res = base + (uint32_t)(q - 1024);  // carry into the exponent is correct
  else
    res = (uint32_t)q;                  // may round up into the smallest normal
  if (res >= 0x7C00u) res = 0x7C00u;
  return sign | (uint16_t)res;
}

// Write a wave-uniform 32-bit value into one lane of a VGPR (v_writelane_b32).
// Clang has no builtin for it, so the LLVM intrinsic is declared directly;
// going through the compiler (not inline asm) lets its hazard recognizer put
// the required wait states between a v_cmp that writes the mask SGPRs and the
// v_writelane that reads them.  `lane` must be a constant 0..63.
__device__ int tq_llvm_writelane(int val, int lane, int old) __asm("llvm.amdgcn.writelane.i32");

__device__ __forceinline__ uint32_t write_lane(uint32_t old, uint32_t val, int lane) {
  return (uint32_t)tq_llvm_writelane((int)val, lane, (int)old);
}

template <typename T>
__device__ __forceinline__ T wave_xor(T v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

}  // namespace tqd
