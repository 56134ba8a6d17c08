// Reconstruction of packed vectors:
//   x_hat = n * (Pi^T c[idx] + sqrt(pi/2)/d * gamma * S^T s).
// Page "TurboQuant 설명", section "2단계: QJL 잔차 보정" (reconstructed
// vectors) and section "1단계" (the codebook and rotation being inverted).
//
// Layout mirrors the quantiser: D/32 waves, wave w owns output columns
// [32w, 32w+32) and keeps its columns of Pi (and S) in VGPRs as fp16 hi + lo
// (scaled by 2^8).  Each 32-vector tile is decoded once into LDS: the
// centroid of every coordinate as fp16 hi + lo (scaled by 2^10) and, in
// inner-product mode, the sign as an exact fp16 +-1.  Products run on the
// 32x32x16 fp16 MFMA with fp32 accumulation; the output tile has one column
// per lane, so each register row is a coalesced 128-byte store.
#include "tq_device.h"
#include "tq_internal.h"

namespace {

using namespace tqd;

constexpr float kMatScale = 256.0f;
constexpr float kCenScale = 1024.0f;

template <int D>
struct DLayout {
  static constexpr int NW = D / 32;
  static constexpr int NT = NW * kWave;
  static constexpr int KS = D / 16;
  static constexpr int PITCH = D + 8;
  static constexpr int TPV = D / 16;
};

// B fragments of columns [32w, 32w+32) of a d x d matrix (B[k][n] = mat[k][32w+n]).
template <int D>
__device__ void load_columns(const float *__restrict__ mat, int w, half8 (&hi)[D / 16],
                             half8 (&lo)[D / 16]) {
  const int l = lane_id();
  const int col = 32 * w + (l & 31);
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = 16 * s + 8 * (l >> 5) + i;
      const float sv = mat[(size_t)k * D + col] * kMatScale;
      const _Float16 h = (_Float16)sv;
      hi[s][i] = h;
      lo[s][i] = (_Float16)(sv - (float)h);
    }
  }
}

template <int D, int LB, bool PROD, bool OUT_F32>
__global__ __launch_bounds__(DLayout<D>::NT) void dequant_kernel(tqi::DequantArgs a) {
  using L = DLayout<D>;
  constexpr int K = 1 << LB;
  constexpr int PB = D / 8;
  constexpr int NPL = LB + (PROD ? 1 : 0);  // planes per record (sign on top)
  constexpr int RB = NPL * PB;
  __shared__ __attribute__((aligned(16))) _Float16 ch[32 * L::PITCH];
  __shared__ __attribute__((aligned(16))) _Float16 cl[32 * L::PITCH];
  __shared__ __attribute__((aligned(16))) _Float16 sg[PROD ? 32 * L::PITCH : 8];
  __shared__ __attribute__((aligned(16))) float vfac[2][32];
  __shared__ uint32_t ctab[K];

  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int l = lane_id();
  const int m = l & 31;
  const int h = l >> 5;

  half8 ph[L::KS], pl[L::KS];
  load_columns<D>(a.pi, w, ph, pl);
  half8 sh[PROD ? L::KS : 1], sl[PROD ? L::KS : 1];
  if constexpr (PROD) load_columns<D>(a.s_mat, w, sh, sl);
  if (tid < K) {
    const float cv = a.centroids[tid] * kCenScale;
    const _Float16 hv = (_Float16)cv;
    const _Float16 lv = (_Float16)(cv - (float)hv);
    uint16_t hb, lb;
    __builtin_memcpy(&hb, &hv, 2);
    __builtin_memcpy(&lb, &lv, 2);
    ctab[tid] = (uint32_t)hb | ((uint32_t)lb << 16);
  }
  const float kappa = (float)(1.2533141373155003 / D);  // sqrt(pi/2) / d
  __syncthreads();

  const int64_t n_tiles = (a.n_vec + 31) / 32;
  for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int64_t base = tile * 32;
    {  // decode 16 coordinates of one vector per thread
      const int v = tid / L::TPV;
      const int c = tid % L::TPV;
      const int64_t gv = base + v;
      const bool valid = gv < a.n_vec;
      uint32_t pw[LB];
#pragma unroll
      for (int p = 0; p < LB; ++p)
        pw[p] = valid ? *(const uint16_t *)(a.codes + gv * RB + 4 * ((c >> 1) * NPL + p) + 2 * (c & 1)) : 0u;
      uint32_t sw = 0;
      if constexpr (PROD)
        sw = valid ? *(const uint16_t *)(a.codes + gv * RB + 4 * ((c >> 1) * NPL + LB) + 2 * (c & 1)) : 0u;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        uint32_t idx = 0;
#pragma unroll
        for (int p = 0; p < LB; ++p) idx |= ((pw[p] >> i) & 1u) << p;
        const uint32_t e = ctab[idx];
        uint16_t hb = (uint16_t)(e & 0xFFFF), lb = (uint16_t)(e >> 16);
        __builtin_memcpy(&ch[v * L::PITCH + 16 * c + i], &hb, 2);
        __builtin_memcpy(&cl[v * L::PITCH + 16 * c + i], &lb, 2);
        if constexpr (PROD) sg[v * L::PITCH + 16 * c + i] = ((sw >> i) & 1u) ? (_Float16)1.0f : (_Float16)-1.0f;
      }
      if (c == 0) {
        const float nrm = valid ? f16_bits_to_f32(a.norm[gv]) : 0.0f;
        vfac[0][v] = nrm * (1.0f / (kCenScale * kMatScale));
        vfac[1][v] = PROD && valid ? nrm * kappa * f16_bits_to_f32(a.rnorm[gv]) * (1.0f / kMatScale) : 0.0f;
      }
    }
    __syncthreads();
    f32x16 acc = {};
    f32x16 acc2 = {};
#pragma unroll
    for (int s = 0; s < L::KS; ++s) {
      const half8 ah = *(const half8 *)&ch[m * L::PITCH + 16 * s + 8 * h];
      const half8 al = *(const half8 *)&cl[m * L::PITCH + 16 * s + 8 * h];
      acc = mfma32(al, ph[s], acc);
      acc = mfma32(ah, pl[s], acc);
      acc = mfma32(ah, ph[s], acc);
      if constexpr (PROD) {
        const half8 as = *(const half8 *)&sg[m * L::PITCH + 16 * s + 8 * h];
        acc2 = mfma32(as, sl[s], acc2);
        acc2 = mfma32(as, sh[s], acc2);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int v = 8 * (r >> 2) + 4 * h + (r & 3);
      const int64_t gv = base + v;
      float val = acc[r] * vfac[0][v];
      if constexpr (PROD) val += acc2[r] * vfac[1][v];
      if (gv < a.n_vec) {
        if constexpr (OUT_F32)
          ((float *)a.out)[gv * D + 32 * w + m] = val;
        else
          ((uint16_t *)a.out)[gv * D + 32 * w + m] = f32_to_bf16_bits(val);
      }
    }
    __syncthreads();
  }
}

template <int D, int LB, bool PROD, bool OUT_F32>
hipError_t launch_t(const tqi::DequantArgs &a, hipStream_t s) {
  using L = DLayout<D>;
  const int64_t n_tiles = (a.n_vec + 31) / 32;
  int blocks_per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &blocks_per_cu, dequant_kernel<D, LB, PROD, OUT_F32>, L::NT, 0);
  if (e != hipSuccess) return e;
  if (blocks_per_cu < 1) blocks_per_cu = 1;
  int64_t grid = (int64_t)tqi::device_cu_count() * blocks_per_cu;
  if (grid > n_tiles) grid = n_tiles;
  hipLaunchKernelGGL((dequant_kernel<D, LB, PROD, OUT_F32>), dim3((unsigned)grid), dim3(L::NT), 0,
                     s, a);
  return hipGetLastError();
}

template <int D, int LB, bool PROD>
hipError_t launch_o(const tqi::DequantArgs &a, hipStream_t s) {
  return a.out_f32 ? launch_t<D, LB, PROD, true>(a, s) : launch_t<D, LB, PROD, false>(a, s);
}

template <int D, bool PROD>
hipError_t launch_lb(int lb, const tqi::DequantArgs &a, hipStream_t s, bool *ok) {
  *ok = true;
  switch (lb) {
    case 1: return launch_o<D, 1, PROD>(a, s);
    case 2: return launch_o<D, 2, PROD>(a, s);
    case 3: return launch_o<D, 3, PROD>(a, s);
    case 4: return launch_o<D, 4, PROD>(a, s);
  }
  *ok = false;
  return hipSuccess;
}

}  // namespace

namespace tqi {

hipError_t launch_dequant(int d, int lbits, bool prod, const DequantArgs &a, hipStream_t s,
                          bool *supported) {
  *supported = false;
  if (d == 64) return prod ? launch_lb<64, true>(lbits, a, s, supported)
                           : launch_lb<64, false>(lbits, a, s, supported);
  if (d == 128) return prod ? launch_lb<128, true>(lbits, a, s, supported)
                            : launch_lb<128, false>(lbits, a, s, supported);
  if (d == 256 && !prod) return launch_lb<256, false>(lbits, a, s, supported);
  return hipSuccess;
}

}  // namespace tqi
