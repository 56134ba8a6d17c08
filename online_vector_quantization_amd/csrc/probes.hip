// Ceiling probes: the best this GPU does on a plain read stream, a plain
// write stream and a loop of matrix-core instructions with no memory
// traffic.  The rooflines of the hot-path kernels are reported as fractions
// of these measured ceilings next to the published peaks (an HBM read
// stream, not the vendor's 8 TB/s, is what a streaming kernel can reach).
#include "tq_device.h"
#include "tq_internal.h"

namespace {

using namespace tqd;

constexpr int kProbeThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Every thread reads 16-byte pieces 4 at a time (non-temporal), grid-strided
// over the buffer, and folds them into one word so no load is dead; the
// block's fold goes to sink[block].
__global__ __launch_bounds__(kProbeThreads) void read_stream_kernel(const u32x4 *__restrict__ buf, int64_t n16,
                                                                   uint32_t *__restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(buf + i);
    const u32x4 b = __builtin_nontemporal_load(buf + i + stride);
    const u32x4 c = __builtin_nontemporal_load(buf + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(buf + i + 3 * stride);
    acc ^= (a ^ b) ^ (c ^ d);
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(buf + i);
  uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v ^= (uint32_t)__shfl_xor((int)v, off, 64);
  __shared__ uint32_t part[kProbeThreads / 64];
  if (lane_id() == 0) part[threadIdx.x / 64] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
    for (int w = 0; w < kProbeThreads / 64; ++w) s ^= part[w];
    sink[blockIdx.x] = s;
  }
}

// Every thread writes 16-byte pieces (non-temporal), grid-strided.
__global__ __launch_bounds__(kProbeThreads) void write_stream_kernel(u32x4 *__restrict__ buf, int64_t n16,
                                                                    uint32_t value) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  const u32x4 v = {value, value, value, value};
  for (int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x; i < n16; i += stride)
    __builtin_nontemporal_store(v, buf + i);
}

// Four independent chains of 32x32x16 fp16 MFMAs per wave, `iters` steps
// each, on register operands; the lanes' sums go to sink[wave].
__global__ __launch_bounds__(kProbeThreads) void mfma_f16_loop_kernel(int iters, uint32_t *__restrict__ sink) {
  half8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(0.001f * (float)(threadIdx.x + i));
    b[i] = (_Float16)(0.002f * (float)(threadIdx.x - i));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int k = 0; k < iters; ++k) {
    c0 = mfma32(a, b, c0);
    c1 = mfma32(a, b, c1);
    c2 = mfma32(a, b, c2);
    c3 = mfma32(a, b, c3);
  }
  float s = 0.0f;
  for (int r = 0; r < 16; ++r) s += (c0[r] + c1[r]) + (c2[r] + c3[r]);
  if (s == 12345.0f) sink[blockIdx.x * (kProbeThreads / 64) + threadIdx.x / 64] = 1u;   // keeps the chains live
}

// The same with 16x16x64 int8 MFMAs (the logit kernel's instruction).
__global__ __launch_bounds__(kProbeThreads) void mfma_i8_loop_kernel(int iters, uint32_t *__restrict__ sink) {
  const i32x4 a = {(int)threadIdx.x, 3, 5, 7}, b = {11, (int)threadIdx.x, 13, 17};
  i32x4 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int k = 0; k < iters; ++k) {
    c0 = mfma_i8(a, b, c0);
    c1 = mfma_i8(a, b, c1);
    c2 = mfma_i8(a, b, c2);
    c3 = mfma_i8(a, b, c3);
  }
  const int s = (c0[0] + c1[1]) + (c2[2] + c3[3]);
  if (s == 12345) sink[blockIdx.x * (kProbeThreads / 64) + threadIdx.x / 64] = 1u;
}

}  // namespace

namespace tqi {

int probe_blocks() { return device_cu_count() * 8; }

hipError_t launch_probe(int kind, void *buf, int64_t bytes, int iters, uint32_t *sink, hipStream_t s) {
  const int blocks = probe_blocks();
  switch (kind) {
    case 0:
      hipLaunchKernelGGL(read_stream_kernel, dim3(blocks), dim3(kProbeThreads), 0, s, (const u32x4 *)buf,
                         bytes / 16, sink);
      break;
    case 1:
      hipLaunchKernelGGL(write_stream_kernel, dim3(blocks), dim3(kProbeThreads), 0, s, (u32x4 *)buf, bytes / 16,
                         0u);
      break;
    case 2:
      hipLaunchKernelGGL(mfma_f16_loop_kernel, dim3(blocks), dim3(kProbeThreads), 0, s, iters, sink);
      break;
    case 3:
      hipLaunchKernelGGL(mfma_i8_loop_kernel, dim3(blocks), dim3(kProbeThreads), 0, s, iters, sink);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tqi
