// Fused online quantiser: norm -> rotation -> nearest Lloyd-Max centroid ->
// bit-plane packing -> (inner-product mode) residual -> QJL projection ->
// sign packing, for tiles of 32 vectors.
//
// Page "TurboQuant 설명: 무엇인지와 LLM 메모리 6배 절약 구현 방법":
//   "1단계: 무작위 회전 + PolarQuant 압축" - normalise, rotate with Pi, map each
//   rotated coordinate to its Lloyd-Max cell;
//   "2단계: QJL 잔차 보정" - one sign bit of S r per coordinate, r the stage-1
//   residual of the unit vector; on the device S r = M (Pi u - c_hat) with
//   M = S Pi^T.
//
// Design (gfx950):
// * One workgroup = D/32 waves; wave w owns the output coordinates
//   [32w, 32w+32).  Its slice of Pi (and of M) stays in VGPRs as fp16
//   hi + lo pairs (22 significant bits) for the whole launch: the rotation is
//   "weight stationary" and the inputs stream through.
// * Inputs are staged once per tile in LDS as fp16, scaled per vector by a
//   power of two so the largest element sits in [2^14, 2^15); bf16 inputs
//   are then exact, fp32 inputs are split into hi + lo.  The norm is
//   accumulated in fp64 from the exact inputs and rounded once to fp16.
// * y = X Pi^T runs on 32x32x16 fp16 MFMA (fp32 accumulate); the output tile
//   has one coordinate per lane, so each boundary comparison is a single
//   v_cmp whose 64-bit lane mask is a piece of the thermometer code; the
//   bit planes of the indices are XORs of those masks on the scalar unit
//   (plane p = XOR of the masks for boundaries (k*2^p - 1)).
// * Inner-product mode: the rotated residual y/n - c_hat is written to LDS
//   as fp16 hi + lo, then z = (y/n - c_hat) M^T runs on MFMA against the
//   stationary M slice; sign masks are ballots of z >= 0 and become the top
//   bit plane of each coordinate's record.
#include "tq_device.h"
#include "tq_internal.h"

namespace {

using namespace tqd;

constexpr float kPiScale = 256.0f;   // Pi and M are scaled by 2^8 before the fp16 split
constexpr float kResScale = 1024.0f; // residual scale before its fp16 split

template <int D>
struct QLayout {
  static constexpr int NW = D / 32;          // waves per workgroup
  static constexpr int NT = NW * kWave;      // threads
  static constexpr int KS = D / 16;          // K steps of the 32x32x16 MFMA
  static constexpr int PITCH = D + 8;        // halves per LDS row (16 B pad)
  static constexpr int TPV = D / 16;         // staging threads per vector
};

// Load this lane's B fragments (hi, lo) of rows [32w, 32w+32) of a d x d
// fp32 matrix scaled by 2^8: lane l holds row 32w + l%32, columns
// 16s + 8(l/32) + 0..7 for K step s.
template <int D>
__device__ void load_stationary(const float *__restrict__ mat, int w, half8 (&hi)[D / 16],
                                half8 (&lo)[D / 16]) {
  const int l = lane_id();
  const float *row = mat + (size_t)(32 * w + (l & 31)) * D + 8 * (l >> 5);
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    f32x4 v0 = *(const f32x4 *)(row + 16 * s);
    f32x4 v1 = *(const f32x4 *)(row + 16 * s + 4);
    float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float sv = v[i] * kPiScale;
      _Float16 h = (_Float16)sv;
      hi[s][i] = h;
      lo[s][i] = (_Float16)(sv - (float)h);
    }
  }
}

template <int D, int LB, bool PROD, bool IN_F32>
__global__ __launch_bounds__(QLayout<D>::NT) void quantize_kernel(tqi::QuantizeArgs a) {
  using L = QLayout<D>;
  constexpr int K = 1 << LB;                  // centroids
  constexpr int PB = D / 8;                   // bytes per plane
  constexpr int NPL = LB + (PROD ? 1 : 0);    // planes per record (sign on top)
  constexpr int RB = NPL * PB;                // bytes per packed row
  __shared__ __attribute__((aligned(16))) _Float16 xh[32 * L::PITCH];
  __shared__ __attribute__((aligned(16))) _Float16 xl[IN_F32 ? 32 * L::PITCH : 1];
  __shared__ __attribute__((aligned(16))) _Float16 rh[PROD ? 32 * L::PITCH : 1];
  __shared__ __attribute__((aligned(16))) _Float16 rl[PROD ? 32 * L::PITCH : 1];
  __shared__ __attribute__((aligned(16))) float vinv[32];

  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int l = lane_id();
  const int m = l & 31;          // MFMA row (A) / column (B, C) of this lane
  const int h = l >> 5;          // K group / row group

  half8 pih[L::KS], pil[L::KS];
  load_stationary<D>(a.pi, w, pih, pil);
  half8 mh[PROD ? L::KS : 1], ml[PROD ? L::KS : 1];
  if constexpr (PROD) load_stationary<D>(a.m, w, mh, ml);

  float bnd[K - 1];
#pragma unroll
  for (int k = 0; k < K - 1; ++k) bnd[k] = a.boundaries[k];
  float cen[K];
#pragma unroll
  for (int k = 0; k < K; ++k) cen[k] = PROD ? a.centroids[k] : 0.0f;

  const int64_t n_tiles = (a.n_vec + 31) / 32;
  for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int64_t base = tile * 32;
    // ---------------------------------------------------------------- stage
    {
      const int v = tid / L::TPV;
      const int c = tid % L::TPV;
      const int64_t gv = base + v;
      const bool valid = gv < a.n_vec;
      float xv[16];
      if (valid) {
        if constexpr (IN_F32) {
          const f32x4 *p = (const f32x4 *)((const float *)a.x + gv * a.x_stride + 16 * c);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f32x4 t = p[q];
            xv[4 * q] = t[0]; xv[4 * q + 1] = t[1]; xv[4 * q + 2] = t[2]; xv[4 * q + 3] = t[3];
          }
        } else {
          const i32x4 *p = (const i32x4 *)((const uint16_t *)a.x + gv * a.x_stride + 16 * c);
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            i32x4 t = p[q];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              uint32_t u = (uint32_t)t[e];
              xv[8 * q + 2 * e] = __uint_as_float(u << 16);
              xv[8 * q + 2 * e + 1] = __uint_as_float(u & 0xFFFF0000u);
            }
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) xv[i] = 0.0f;
      }
      double ss = 0.0;
      float mx = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        ss += (double)xv[i] * (double)xv[i];
        mx = fmaxf(mx, fabsf(xv[i]));
      }
#pragma unroll
      for (int off = 1; off < L::TPV; off <<= 1) {
        ss += wave_xor(ss, off);
        mx = fmaxf(mx, wave_xor(mx, off));
      }
      int e = 0;
      if (mx > 0.0f) {
        e = ilogbf(mx);
        e = e < -140 ? -140 : (e > 127 ? 127 : e);
      }
      const float sc = ldexpf(1.0f, 14 - e);
      const double nrm = sqrt(ss);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float sv = xv[i] * sc;
        _Float16 hv = (_Float16)sv;
        xh[v * L::PITCH + 16 * c + i] = hv;
        if constexpr (IN_F32) xl[v * L::PITCH + 16 * c + i] = (_Float16)(sv - (float)hv);
      }
      if (c == 0) {
        vinv[v] = nrm > 0.0 ? (float)(1.0 / ((double)sc * (double)kPiScale * nrm)) : 0.0f;
        if (valid) a.norm[a.out_offset + gv] = f64_to_f16_bits(nrm);
      }
    }
    __syncthreads();
    // ---------------------------------------------------------- y = X Pi^T
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < L::KS; ++s) {
      half8 ah = *(const half8 *)&xh[m * L::PITCH + 16 * s + 8 * h];
      if constexpr (IN_F32) {
        half8 al = *(const half8 *)&xl[m * L::PITCH + 16 * s + 8 * h];
        acc = mfma32(al, pih[s], acc);
      }
      acc = mfma32(ah, pil[s], acc);
      acc = mfma32(ah, pih[s], acc);
    }
    // ------------------------------------------ codes: compares + bit planes
    float inv[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 t = *(const f32x4 *)&vinv[8 * g + 4 * h];
      inv[4 * g] = t[0]; inv[4 * g + 1] = t[1]; inv[4 * g + 2] = t[2]; inv[4 * g + 3] = t[3];
    }
    uint32_t outw[2] = {0u, 0u};   // up to 128 plane words per wave
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float u = acc[r] * inv[r];
      uint64_t planes[LB];
#pragma unroll
      for (int p = 0; p < LB; ++p) planes[p] = 0;
      float chat = cen[0];
#pragma unroll
      for (int k = 0; k < K - 1; ++k) {
        const bool ge = u >= bnd[k];
        const uint64_t mk = __ballot(ge);
        if constexpr (PROD) chat = ge ? cen[k + 1] : chat;
#pragma unroll
        for (int p = 0; p < LB; ++p)
          if (((k + 1) & ((1 << p) - 1)) == 0) planes[p] ^= mk;
      }
#pragma unroll
      for (int p = 0; p < LB; ++p) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int slot = (r * LB + p) * 2 + hh;
          const uint32_t word = (uint32_t)(planes[p] >> (32 * hh));
          outw[slot >> 6] = write_lane(outw[slot >> 6], word, slot & 63);
        }
      }
      if constexpr (PROD) {
        const int v = 8 * (r >> 2) + 4 * h + (r & 3);
        const float rs = (u - chat) * kResScale;
        const _Float16 hv = (_Float16)rs;
        rh[v * L::PITCH + 32 * w + m] = hv;
        rl[v * L::PITCH + 32 * w + m] = (_Float16)(rs - (float)hv);
      }
    }
    // store plane words: slot = (r*LB + p)*2 + hh -> vector 8(r/4)+4hh+r%4
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int slot = 64 * g + l;
      if (slot < 32 * LB) {
        const int hh = slot & 1;
        const int p = (slot >> 1) % LB;
        const int r = (slot >> 1) / LB;
        const int v = 8 * (r >> 2) + 4 * hh + (r & 3);
        const int64_t gv = base + v;
        if (gv < a.n_vec) {
          uint32_t *dst = (uint32_t *)(a.codes + (a.out_offset + gv) * RB + 4 * (w * NPL + p));
          *dst = outw[g];
        }
      }
    }
    if constexpr (PROD) {
      __syncthreads();
      // ------------------------------------ z = (y/n - c_hat) M^T, sign bits
      f32x16 acc2 = {};
#pragma unroll
      for (int s = 0; s < L::KS; ++s) {
        half8 ah = *(const half8 *)&rh[m * L::PITCH + 16 * s + 8 * h];
        half8 al = *(const half8 *)&rl[m * L::PITCH + 16 * s + 8 * h];
        acc2 = mfma32(al, mh[s], acc2);
        acc2 = mfma32(ah, ml[s], acc2);
        acc2 = mfma32(ah, mh[s], acc2);
      }
      uint32_t sw = 0u;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint64_t mk = __ballot(acc2[r] >= 0.0f || inv[r] == 0.0f);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          sw = write_lane(sw, (uint32_t)(mk >> (32 * hh)), 2 * r + hh);
      }
      if (l < 32) {
        const int r = l >> 1, hh = l & 1;
        const int v = 8 * (r >> 2) + 4 * hh + (r & 3);
        const int64_t gv = base + v;
        if (gv < a.n_vec) *(uint32_t *)(a.codes + (a.out_offset + gv) * RB + 4 * (w * NPL + LB)) = sw;
      }
      // residual norm of the unit vector from the staged residual tile
      {
        const int v = tid / L::TPV;
        const int c = tid % L::TPV;
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float r = (float)rh[v * L::PITCH + 16 * c + i] + (float)rl[v * L::PITCH + 16 * c + i];
          ss += r * r;
        }
#pragma unroll
        for (int off = 1; off < L::TPV; off <<= 1) ss += wave_xor(ss, off);
        const int64_t gv = base + v;
        if (c == 0 && gv < a.n_vec) {
          const float gam = vinv[v] == 0.0f ? 0.0f : sqrtf(ss) * (1.0f / kResScale);
          a.rnorm[a.out_offset + gv] = f32_to_f16_bits(gam);
        }
      }
    }
    __syncthreads();
  }
}

template <int D, int LB, bool PROD, bool IN_F32>
hipError_t launch_t(const tqi::QuantizeArgs &a, hipStream_t s) {
  using L = QLayout<D>;
  const int64_t n_tiles = (a.n_vec + 31) / 32;
  int blocks_per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &blocks_per_cu, quantize_kernel<D, LB, PROD, IN_F32>, L::NT, 0);
  if (e != hipSuccess) return e;
  if (blocks_per_cu < 1) blocks_per_cu = 1;
  int64_t grid = (int64_t)tqi::device_cu_count() * blocks_per_cu;
  if (grid > n_tiles) grid = n_tiles;
  hipLaunchKernelGGL((quantize_kernel<D, LB, PROD, IN_F32>), dim3((unsigned)grid), dim3(L::NT),
                     0, s, a);
  return hipGetLastError();
}

template <int D, int LB, bool PROD>
hipError_t launch_dt(bool in_f32, const tqi::QuantizeArgs &a, hipStream_t s) {
  return in_f32 ? launch_t<D, LB, PROD, true>(a, s) : launch_t<D, LB, PROD, false>(a, s);
}

template <int D, bool PROD>
hipError_t launch_lb(int lb, bool in_f32, const tqi::QuantizeArgs &a, hipStream_t s,
                     bool *ok) {
  *ok = true;
  switch (lb) {
    case 1: return launch_dt<D, 1, PROD>(in_f32, a, s);
    case 2: return launch_dt<D, 2, PROD>(in_f32, a, s);
    case 3: return launch_dt<D, 3, PROD>(in_f32, a, s);
    case 4: return launch_dt<D, 4, PROD>(in_f32, a, s);
  }
  *ok = false;
  return hipSuccess;
}

}  // namespace

namespace tqi {

hipError_t launch_quantize(int d, int lbits, bool prod, bool in_f32, const QuantizeArgs &a,
                           hipStream_t s, bool *supported) {
  *supported = false;
  if (d == 64) return prod ? launch_lb<64, true>(lbits, in_f32, a, s, supported)
                           : launch_lb<64, false>(lbits, in_f32, a, s, supported);
  if (d == 128) return prod ? launch_lb<128, true>(lbits, in_f32, a, s, supported)
                            : launch_lb<128, false>(lbits, in_f32, a, s, supported);
  if (d == 256 && !prod) return launch_lb<256, false>(lbits, in_f32, a, s, supported);
  return hipSuccess;
}

}  // namespace tqi
