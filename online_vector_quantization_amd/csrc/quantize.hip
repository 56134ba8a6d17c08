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

// Codes, norms and signs leave as scattered 2- and 4-byte pieces of rows:
// stored with the default (write-back) policy so that L2 merges them into
// whole lines; with the streaming policy each piece reaches HBM on its own.
constexpr int kWriteBack = 0;

// Raw input of one staging thread: 16 consecutive elements of one vector.
template <bool IN_F32>
struct RawInput {
  i32x4 q[IN_F32 ? 4 : 2];
};

template <int D, int LB, bool PROD, bool IN_F32>
__global__ __launch_bounds__(QLayout<D>::NT) void quantize_kernel(tqi::QuantizeArgs a) {
  using L = QLayout<D>;
  constexpr int K = 1 << LB;                  // centroids
  constexpr int PB = D / 8;                   // bytes per plane
  constexpr int NPL = LB + (PROD ? 1 : 0);    // planes per record (sign on top)
  constexpr int RB = NPL * PB;                // bytes per packed row
  constexpr int TILE = 32 * L::PITCH;
  // Two LDS buffers, alternated per tile: a tile's staging never overwrites
  // data that the previous tile may still read, so one barrier per stage
  // suffices.
  __shared__ __attribute__((aligned(16))) _Float16 xh[2][TILE];
  __shared__ __attribute__((aligned(16))) _Float16 xl[IN_F32 ? 2 : 1][IN_F32 ? TILE : 8];
  __shared__ __attribute__((aligned(16))) _Float16 rh[PROD ? 2 : 1][PROD ? TILE : 8];
  __shared__ __attribute__((aligned(16))) _Float16 rl[PROD ? 2 : 1][PROD ? TILE : 8];
  __shared__ __attribute__((aligned(16))) float vinv[2][32];

  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int l = lane_id();
  const int m = l & 31;          // MFMA row (A) / column (B, C) of this lane
  const int h = l >> 5;          // K group / row group
  const int sv_v = tid / L::TPV; // staging: vector within the tile
  const int sv_c = tid % L::TPV; //          16-element chunk of it

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

  // Buffer resources over this call's rows.  The host keeps every range below
  // 2^31 bytes (large calls are split), so rows past n_vec and kNoStore fall
  // outside: such loads return 0 and such stores are dropped by the hardware.
  // No load or store sits behind a branch, which lets the compiler wait for
  // the next tile's loads without also waiting for this tile's stores.
  constexpr int ESZ = IN_F32 ? 4 : 2;
  const i32x4 rx = make_rsrc(a.x, (uint32_t)(((a.n_vec - 1) * a.x_stride + D) * ESZ));
  const i32x4 rc = make_rsrc(a.codes + a.out_offset * RB, (uint32_t)(a.n_vec * RB));
  const i32x4 rn = make_rsrc(a.norm + a.out_offset, (uint32_t)(a.n_vec * 2));
  const i32x4 rr = make_rsrc(PROD ? a.rnorm + a.out_offset : a.norm, PROD ? (uint32_t)(a.n_vec * 2) : 0u);

  // Non-temporal loads of a tile's inputs (16 elements per staging thread).
  auto load_raw = [&](int64_t tile, RawInput<IN_F32> &r) {
    const int64_t gv = tile * 32 + sv_v;
    const uint32_t off = gv < a.n_vec ? (uint32_t)((gv * a.x_stride + 16 * sv_c) * ESZ) : kNoStore;
#pragma unroll
    for (int q = 0; q < (IN_F32 ? 4 : 2); ++q) r.q[q] = tq_llvm_buf_ld_b128(rx, (int)(off + 16 * q), 0, kStream);
  };

  // Stages a tile into LDS buffer `buf`; returns this thread's fp16 norm
  // bits, stored by the caller once the next tile's loads are in flight.
  auto stage = [&](int64_t tile, const RawInput<IN_F32> &r, int buf) -> uint16_t {
    {
      float xv[16];
      if constexpr (IN_F32) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) xv[4 * q + e] = __int_as_float(r.q[q][e]);
      } else {
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t u = (uint32_t)r.q[q][e];
            xv[8 * q + 2 * e] = __uint_as_float(u << 16);
            xv[8 * q + 2 * e + 1] = __uint_as_float(u & 0xFFFF0000u);
          }
      }
      double ss = 0.0;
      float mx = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        ss = fma((double)xv[i], (double)xv[i], ss);
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
      half8 hv[2], lv[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float sv = xv[i] * sc;
        const _Float16 hh = (_Float16)sv;
        hv[i >> 3][i & 7] = hh;
        if constexpr (IN_F32) lv[i >> 3][i & 7] = (_Float16)(sv - (float)hh);
      }
      half8 *dh = (half8 *)&xh[buf][sv_v * L::PITCH + 16 * sv_c];
      dh[0] = hv[0];
      dh[1] = hv[1];
      if constexpr (IN_F32) {
        half8 *dl = (half8 *)&xl[buf][sv_v * L::PITCH + 16 * sv_c];
        dl[0] = lv[0];
        dl[1] = lv[1];
      }
      // 1 / (sc * 2^8 * |x|): the scaled sum of squares lies in [2^28, 2^37),
      // so fp32 holds it; v_rsq_f32 is good to about one ulp.
      const float ss_sc = (float)(ss * ((double)sc * (double)sc));
      const float inv_n = ss > 0.0 ? __builtin_amdgcn_rsqf(ss_sc) * (1.0f / kPiScale) : 0.0f;
      if (sv_c == 0) vinv[buf][sv_v] = inv_n;
      return f64_to_f16_bits(sqrt(ss));
    }
  };

  auto compute = [&](int64_t tile, int buf) {
    const int64_t base = tile * 32;
    // ---------------------------------------------------------- y = X Pi^T
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < L::KS; ++s) {
      half8 ah = *(const half8 *)&xh[buf][m * L::PITCH + 16 * s + 8 * h];
      if constexpr (IN_F32) {
        half8 al = *(const half8 *)&xl[buf][m * L::PITCH + 16 * s + 8 * h];
        acc = mfma32(al, pih[s], acc);
      }
      acc = mfma32(ah, pil[s], acc);
      acc = mfma32(ah, pih[s], acc);
    }
    // ------------------------------------------ codes: compares + bit planes
    float inv[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 t = *(const f32x4 *)&vinv[buf][8 * g + 4 * h];
      inv[4 * g] = t[0]; inv[4 * g + 1] = t[1]; inv[4 * g + 2] = t[2]; inv[4 * g + 3] = t[3];
    }
    uint32_t outw[2] = {0u, 0u};   // up to 128 plane words per wave
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float u = acc[r] * inv[r];
      uint64_t planes[LB];
#pragma unroll
      for (int p = 0; p < LB; ++p) planes[p] = 0;
      uint64_t ge[K - 1];   // thermometer masks: bit l = (u >= t_k) in lane l
#pragma unroll
      for (int k = 0; k < K - 1; ++k) {
        ge[k] = __ballot(u >= bnd[k]);
#pragma unroll
        for (int p = 0; p < LB; ++p)
          if (((k + 1) & ((1 << p) - 1)) == 0) planes[p] ^= ge[k];
      }
      // Centroid of the chosen cell from the thermometer masks, using the
      // codebook's antisymmetry c[K/2-1-j] = -c[K/2+j]: pick the magnitude
      // level j (|idx - K/2 + 1/2| - 1/2 >= j  <=>  idx >= K/2+j or
      // idx <= K/2-1-j), then the sign (idx >= K/2  <=>  u >= t[K/2-1]).
      float chat = 0.0f;
      if constexpr (PROD) {
        constexpr int MID = K / 2;
        float mag = cen[MID];
#pragma unroll
        for (int j = 1; j < MID; ++j)   // mask logic stays on the scalar unit
          mag = __builtin_amdgcn_inverse_ballot_w64(ge[MID - 1 + j] | ~ge[MID - 1 - j]) ? cen[MID + j] : mag;
        chat = __builtin_amdgcn_inverse_ballot_w64(ge[MID - 1]) ? mag : -mag;
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
        rh[buf][v * L::PITCH + 32 * w + m] = hv;
        rl[buf][v * L::PITCH + 32 * w + m] = (_Float16)(rs - (float)hv);
      }
    }
    // store plane words: slot = (r*LB + p)*2 + hh -> vector 8(r/4)+4hh+r%4
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      if (64 * g < 32 * LB) {
        const int slot = 64 * g + l;
        const int hh = slot & 1;
        const int p = (slot >> 1) % LB;
        const int r = (slot >> 1) / LB;
        const int v = 8 * (r >> 2) + 4 * hh + (r & 3);
        const int64_t gv = base + v;
        const uint32_t off =
            (slot < 32 * LB && gv < a.n_vec) ? (uint32_t)(gv * RB + 4 * (w * NPL + p)) : kNoStore;
        buf_store_u32<kWriteBack>(rc, off, outw[g]);
      }
    }
    if constexpr (PROD) {
      __syncthreads();
      // ------------------------------------ z = (y/n - c_hat) M^T, sign bits
      f32x16 acc2 = {};
#pragma unroll
      for (int s = 0; s < L::KS; ++s) {
        half8 ah = *(const half8 *)&rh[buf][m * L::PITCH + 16 * s + 8 * h];
        half8 al = *(const half8 *)&rl[buf][m * L::PITCH + 16 * s + 8 * h];
        acc2 = mfma32(al, mh[s], acc2);
        acc2 = mfma32(ah, ml[s], acc2);
        acc2 = mfma32(ah, mh[s], acc2);
      }
      uint32_t sw = 0u;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint64_t mk = __ballot(acc2[r] >= 0.0f);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) sw = write_lane(sw, (uint32_t)(mk >> (32 * hh)), 2 * r + hh);
      }
      {
        const int r = (l >> 1) & 15, hh = l & 1;
        const int v = 8 * (r >> 2) + 4 * hh + (r & 3);
        const int64_t gv = base + v;
        if (vinv[buf][v] == 0.0f) sw = 0xFFFFFFFFu;   // zero vector: all signs +1
        const uint32_t off = (l < 32 && gv < a.n_vec) ? (uint32_t)(gv * RB + 4 * (w * NPL + LB)) : kNoStore;
        buf_store_u32<kWriteBack>(rc, off, sw);
      }
      // residual norm of the unit vector from the staged residual tile
      {
        // sum of (hi + lo)^2 = hi.hi + 2 hi.lo + lo.lo, each term a
        // two-wide fp16 dot product accumulated in fp32 (v_dot2_f32_f16)
        float s_hh = 0.0f, s_hl = 0.0f, s_ll = 0.0f;
        const half8 *ph = (const half8 *)&rh[buf][sv_v * L::PITCH + 16 * sv_c];
        const half8 *pl = (const half8 *)&rl[buf][sv_v * L::PITCH + 16 * sv_c];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const half8 hq = ph[q], lq = pl[q];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const half2 h2 = {hq[2 * i], hq[2 * i + 1]}, l2 = {lq[2 * i], lq[2 * i + 1]};
            s_hh = __builtin_amdgcn_fdot2(h2, h2, s_hh, false);
            s_hl = __builtin_amdgcn_fdot2(h2, l2, s_hl, false);
            s_ll = __builtin_amdgcn_fdot2(l2, l2, s_ll, false);
          }
        }
        float ss = s_hh + (2.0f * s_hl + s_ll);
#pragma unroll
        for (int off = 1; off < L::TPV; off <<= 1) ss += wave_xor(ss, off);
        const int64_t gv = base + sv_v;
        const float gam = vinv[buf][sv_v] == 0.0f ? 0.0f : sqrtf(ss) * (1.0f / kResScale);
        buf_store_u16<kWriteBack>(rr, (sv_c == 0 && gv < a.n_vec) ? (uint32_t)(2 * gv) : kNoStore, f32_to_f16_bits(gam));
      }
    }
  };

  // One register set of raw input: the next tile's loads are issued as soon
  // as the current tile has been staged, so they fly during its GEMMs and
  // coding.
  const int64_t step = gridDim.x;
  int64_t tile = blockIdx.x;
  RawInput<IN_F32> raw;
  load_raw(tile, raw);
  // Range-dropped stores: with them, on entry as on every later iteration,
  // stores follow the pending input loads, so the compiler can wait for
  // those loads alone (it merges the counts of both paths into the loop).
#pragma unroll
  for (int i = 0; i < 5; ++i) buf_store_u32<kWriteBack>(rn, kNoStore + 4 * i, 0u);
  int buf = 0;
  for (; tile < n_tiles; tile += step, buf ^= 1) {
    const uint16_t n16 = stage(tile, raw, buf);
    load_raw(tile + step, raw);
    __builtin_amdgcn_sched_barrier(0);
    const int64_t gv = tile * 32 + sv_v;
    buf_store_u16<kWriteBack>(rn, (sv_c == 0 && gv < a.n_vec) ? (uint32_t)(2 * gv) : kNoStore, n16);
    __syncthreads();
    compute(tile, buf);
  }
}

template <int D, int LB, bool PROD, bool IN_F32>
hipError_t launch_t(const tqi::QuantizeArgs &a, hipStream_t s) {
  using L = QLayout<D>;
  constexpr int64_t ESZ = IN_F32 ? 4 : 2;
  constexpr int64_t RB = (LB + (PROD ? 1 : 0)) * D / 8;
  constexpr int64_t kRange = (int64_t{1} << 31) - 1;   // kernel byte ranges stay below 2^31
  if (a.x_stride * ESZ > kRange) return hipErrorInvalidValue;
  // Rows per launch so that the input, code and norm ranges fit.
  int64_t rows = kRange / (a.x_stride * ESZ);
  if (rows > kRange / RB) rows = kRange / RB;
  if (rows >= 32) rows &= ~int64_t{31};
  int blocks_per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &blocks_per_cu, quantize_kernel<D, LB, PROD, IN_F32>, L::NT, 0);
  if (e != hipSuccess) return e;
  if (blocks_per_cu < 1) blocks_per_cu = 1;
  for (int64_t start = 0; start < a.n_vec; start += rows) {
    tqi::QuantizeArgs c = a;
    c.x = (const char *)a.x + start * a.x_stride * ESZ;
    c.n_vec = a.n_vec - start < rows ? a.n_vec - start : rows;
    c.out_offset = a.out_offset + start;
    const int64_t n_tiles = (c.n_vec + 31) / 32;
    int64_t grid = (int64_t)tqi::device_cu_count() * blocks_per_cu;
    if (grid > n_tiles) grid = n_tiles;
    hipLaunchKernelGGL((quantize_kernel<D, LB, PROD, IN_F32>), dim3((unsigned)grid), dim3(L::NT),
                       0, s, c);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
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
