// Device helpers shared by the gfx950 kernels of the quantizer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tqd {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));
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

// fp32 -> bf16, round to nearest even (gfx950's v_cvt_pk_bf16_f32; NaN stays
// NaN).  The pair form converts two values with one instruction: a in the low
// half, b in the high half.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_bits(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// Correctly rounded (nearest even) fp64 -> fp16 bits.  The value is first
// rounded to fp32 with round-to-odd (round to nearest, step back toward zero
// if that went up, then set the last bit when anything was dropped) and then
// converted to fp16 by the hardware in nearest-even mode.  Rounding to odd at
// a precision at least two bits finer than the target makes the second
// rounding equal to a direct one (Boldo and Melquiond, "Emulation of FMA and
// correctly rounded sums: proved algorithms using rounding to odd", IEEE
// Trans. Computers 57(4), 2008); fp32 keeps 24 bits against fp16's 11.
// Branch-free; overflow gives infinity, NaN stays NaN.
__device__ __forceinline__ uint16_t f64_to_f16_bits(double v) {
  const double av = fabs(v);
  const float f = (float)av;
  const double back = (double)f;
  uint32_t u = __float_as_uint(f);
  u -= back > av ? 1u : 0u;
  u |= back != av ? 1u : 0u;
  const uint16_t sign = (uint16_t)((__double_as_longlong(v) >> 48) & 0x8000);
  return sign | f32_to_f16_bits(__uint_as_float(u));
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

// Raw buffer access (MUBUF): a 128-bit resource (base, byte range, format
// word) in SGPRs plus a 32-bit per-lane byte offset.  Loads past `bytes`
// return 0 and stores past it are dropped by the hardware range check.  The
// format word 0x00020000 selects 32-bit raw data on gfx9-family parts.
typedef int i32x3 __attribute__((ext_vector_type(3)));
__device__ int tq_llvm_buf_ld_b32(i32x4 rsrc, int voff, int soff, int aux) __asm("llvm.amdgcn.raw.buffer.load.i32");
__device__ i32x3 tq_llvm_buf_ld_b96(i32x4 rsrc, int voff, int soff, int aux) __asm("llvm.amdgcn.raw.buffer.load.v3i32");
__device__ i32x4 tq_llvm_buf_ld_b128(i32x4 rsrc, int voff, int soff, int aux) __asm("llvm.amdgcn.raw.buffer.load.v4i32");
__device__ short tq_llvm_buf_ld_b16(i32x4 rsrc, int voff, int soff, int aux) __asm("llvm.amdgcn.raw.buffer.load.i16");
__device__ void tq_llvm_buf_st_f32(float v, i32x4 rsrc, int voff, int soff, int aux) __asm("llvm.amdgcn.raw.buffer.store.f32");
__device__ void tq_llvm_buf_st_v4f32(f32x4 v, i32x4 rsrc, int voff, int soff, int aux) __asm("llvm.amdgcn.raw.buffer.store.v4f32");
__device__ void tq_llvm_buf_st_b32(int v, i32x4 rsrc, int voff, int soff, int aux) __asm("llvm.amdgcn.raw.buffer.store.i32");
__device__ void tq_llvm_buf_st_b16(short v, i32x4 rsrc, int voff, int soff, int aux) __asm("llvm.amdgcn.raw.buffer.store.i16");
// Scalar buffer load (s_buffer_load_dword): a wave-uniform word through the
// scalar data cache, counted apart from the vector loads in flight.
__device__ int tq_llvm_s_buf_ld_b32(i32x4 rsrc, int off, int aux) __asm("llvm.amdgcn.s.buffer.load.i32");

// A byte offset that every resource built here treats as out of range (the
// ranges are kept below 2^31), so a lane can drop its store without a branch.
constexpr uint32_t kNoStore = 0x80000000u;

__device__ __forceinline__ i32x4 make_rsrc(const void *base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)((uint32_t)(a >> 32) & 0xFFFFu);  // stride 0
  r[2] = (int)bytes;
  r[3] = 0x00020000;
  return r;
}

// Cache-policy bits of the buffer instructions.  Streams that are read or
// written exactly once use the non-temporal policy (bit 1), which keeps them
// from displacing reused data in L2 and lifts streaming bandwidth.
constexpr int kStream = 2;

template <int N, int AUX = kStream>
__device__ __forceinline__ void buf_load_words(i32x4 rsrc, uint32_t off, uint32_t (&out)[N]) {
  if constexpr (N == 1) {
    out[0] = (uint32_t)tq_llvm_buf_ld_b32(rsrc, (int)off, 0, AUX);
  } else if constexpr (N == 2) {
    out[0] = (uint32_t)tq_llvm_buf_ld_b32(rsrc, (int)off, 0, AUX);
    out[1] = (uint32_t)tq_llvm_buf_ld_b32(rsrc, (int)(off + 4), 0, AUX);
  } else if constexpr (N == 3) {
    const i32x3 v = tq_llvm_buf_ld_b96(rsrc, (int)off, 0, AUX);
    out[0] = (uint32_t)v[0]; out[1] = (uint32_t)v[1]; out[2] = (uint32_t)v[2];
  } else if constexpr (N == 4) {
    const i32x4 v = tq_llvm_buf_ld_b128(rsrc, (int)off, 0, AUX);
    out[0] = (uint32_t)v[0]; out[1] = (uint32_t)v[1]; out[2] = (uint32_t)v[2]; out[3] = (uint32_t)v[3];
  } else {
    static_assert(N > 4 && N <= 8, "1..8 words");
    uint32_t lo[4], hi[N - 4];
    buf_load_words<4, AUX>(rsrc, off, lo);
    buf_load_words<N - 4, AUX>(rsrc, off + 16, hi);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = lo[i];
#pragma unroll
    for (int i = 0; i < N - 4; ++i) out[4 + i] = hi[i];
  }
}

template <int AUX = kStream>
__device__ __forceinline__ uint16_t buf_load_u16(i32x4 rsrc, uint32_t off) {
  return (uint16_t)tq_llvm_buf_ld_b16(rsrc, (int)off, 0, AUX);
}

template <int AUX = kStream>
__device__ __forceinline__ void buf_store_f32(i32x4 rsrc, uint32_t off, float v) {
  tq_llvm_buf_st_f32(v, rsrc, (int)off, 0, AUX);
}

template <int AUX = kStream>
__device__ __forceinline__ void buf_store_f32x4(i32x4 rsrc, uint32_t off, f32x4 v) {
  tq_llvm_buf_st_v4f32(v, rsrc, (int)off, 0, AUX);
}

template <int AUX = kStream>
__device__ __forceinline__ void buf_store_u32(i32x4 rsrc, uint32_t off, uint32_t v) {
  tq_llvm_buf_st_b32((int)v, rsrc, (int)off, 0, AUX);
}

template <int AUX = kStream>
__device__ __forceinline__ void buf_store_u16(i32x4 rsrc, uint32_t off, uint16_t v) {
  tq_llvm_buf_st_b16((short)v, rsrc, (int)off, 0, AUX);
}

}  // namespace tqd
