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
// * A wave owns 32 output coordinates and keeps its 32-row slice of Pi (or
//   of M) in VGPRs as fp16 hi + lo pairs (22 significant bits) for the whole
//   launch: the matrices are "weight stationary", the inputs stream through
//   a persistent grid.
// * Inputs are staged once per tile in LDS as fp16, scaled per vector by a
//   power of two so the largest element sits in [2^14, 2^15); bf16 inputs
//   are then exact, fp32 inputs are split into hi + lo.  The fp16 norm is
//   the nearest-even rounding of the exact norm: fp64 sums of the exact
//   squares, or (bf16 inputs in the one-kind kernels) fp32 sums of the
//   staged squares with the exact fp64 sum taken only where the fp32 result
//   cannot decide the rounding.
// * y = X Pi^T runs on 32x32x16 fp16 MFMA (fp32 accumulate); the output tile
//   has one coordinate per lane, so each boundary comparison is a single
//   v_cmp whose 64-bit lane mask is a piece of the thermometer code; the
//   bit planes of the indices are XORs of those masks on the scalar unit
//   (plane p = XOR of the masks for boundaries (k*2^p - 1)).
// * Inner-product mode: the rotated residual y/n - c_hat is written to LDS
//   as fp16 hi + lo, then z = (y/n - c_hat) M^T runs on MFMA against the
//   stationary M slice; sign masks are ballots of z >= 0 and become the top
//   bit plane of each coordinate's record.
// * Two kernels share those steps.  quantize_kernel (MSE mode, and d = 256):
//   D/32 waves, each tile staged, rotated and coded by the same waves (at
//   d = 256 in inner-product mode the M slice does not fit beside Pi's, so
//   its fragments are read from L2 and split per tile).
//   quantize_pc_kernel (inner-product mode, d <= 128): D/32 "producer" waves
//   hold Pi and rotate + code tile k, D/32 "sketch" waves hold M and run the
//   QJL projection of tile k-1, D/32 "stage" waves stage tile k+1 and take
//   the residual norms; one barrier per tile.  No wave carries both
//   matrices, and with three waves per SIMD each one's latencies are covered
//   by the others.  (Measured on gfx950: an MFMA of one wave does not run
//   alongside VALU work of another wave on the same SIMD, so the tile time is
//   close to the sum of the SIMD's MFMA and VALU time.)
#include "tq_device.h"
#include "tq_internal.h"

namespace {

using namespace tqd;

constexpr float kPiScale = 256.0f;   // Pi and M are scaled by 2^8 before the fp16 split
constexpr float kResScale = 1024.0f; // residual scale before its fp16 split

// Codes, norms and signs leave as scattered 2- and 4-byte pieces of rows:
// stored with the default (write-back) policy so that L2 merges them into
// whole lines; with the streaming policy each piece reaches HBM on its own.
constexpr int kWriteBack = 0;

template <int D>
struct QLayout {
  static constexpr int NW = D / 32;          // waves per 32-coordinate split
  static constexpr int NT = NW * kWave;      // threads of the fused kernel
  static constexpr int KS = D / 16;          // K steps of the 32x32x16 MFMA
  static constexpr int PITCH = D + 8;        // halves per LDS row (16 B pad)
  static constexpr int TPV = D / 16;         // staging threads per vector
  static constexpr int TILE = 32 * PITCH;    // halves per LDS tile
};

template <int D, int LB, bool PROD>
struct QFormat {
  static constexpr int K = 1 << LB;                  // centroids
  static constexpr int NPL = LB + (PROD ? 1 : 0);    // planes per record (sign on top)
  static constexpr int RB = NPL * D / 8;             // bytes per packed row
};

// This lane's B fragment (hi, lo) for K step s of rows [32w, 32w+32) of a
// d x d fp32 matrix scaled by 2^8: lane l holds row 32w + l%32, columns
// 16s + 8(l/32) + 0..7.
template <int D>
__device__ __forceinline__ const float *fragment_row(const float *__restrict__ mat, int w) {
  const int l = lane_id();
  return mat + (size_t)(32 * w + (l & 31)) * D + 8 * (l >> 5);
}

__device__ __forceinline__ void split_fragment(const float *row, int s, half8 &hi, half8 &lo) {
  const f32x4 v0 = *(const f32x4 *)(row + 16 * s);
  const f32x4 v1 = *(const f32x4 *)(row + 16 * s + 4);
  const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float sv = v[i] * kPiScale;
    const _Float16 h = (_Float16)sv;
    hi[i] = h;
    lo[i] = (_Float16)(sv - (float)h);
  }
}

// All K steps' fragments, held in VGPRs for the whole launch.
template <int D>
__device__ void load_stationary(const float *__restrict__ mat, int w, half8 (&hi)[D / 16],
                                half8 (&lo)[D / 16]) {
  const float *row = fragment_row<D>(mat, w);
#pragma unroll
  for (int s = 0; s < D / 16; ++s) split_fragment(row, s, hi[s], lo[s]);
}

// Reductions over the N = 4, 8 or 16 consecutive lanes that share a vector,
// all in DPP (no LDS permute): two quad permutes, then the half-row mirror
// (lane i <-> 7 - i within 8) and the row mirror (lane i <-> 15 - i within
// 16).  Every lane ends with the same value (each step adds a lane's value
// to its partner's, so both orders give the same sum).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint64_t r = (uint64_t)dpp_u32<CTRL>((uint32_t)b) | ((uint64_t)dpp_u32<CTRL>((uint32_t)(b >> 32)) << 32);
  return __builtin_bit_cast(double, r);
}

template <int N>
__device__ __forceinline__ double lanes_sum(double v) {
  static_assert(N == 4 || N == 8 || N == 16, "4, 8 or 16 lanes");
  v += dpp_f64<0xB1>(v);
  v += dpp_f64<0x4E>(v);
  if constexpr (N >= 8) v += dpp_f64<0x141>(v);
  if constexpr (N >= 16) v += dpp_f64<0x140>(v);
  return v;
}

template <int N>
__device__ __forceinline__ float lanes_sum(float v) {
  static_assert(N == 4 || N == 8 || N == 16, "4, 8 or 16 lanes");
  v += __uint_as_float(dpp_u32<0xB1>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x4E>(__float_as_uint(v)));
  if constexpr (N >= 8) v += __uint_as_float(dpp_u32<0x141>(__float_as_uint(v)));
  if constexpr (N >= 16) v += __uint_as_float(dpp_u32<0x140>(__float_as_uint(v)));
  return v;
}

// Maximum of non-negative values (magnitudes): on their bit patterns the
// unsigned integer order is the float order, and 0 (the DPP fill value) is
// the identity, so each step is a single v_max_u32 with a DPP operand.
template <int N>
__device__ __forceinline__ float lanes_max(float v) {
  static_assert(N == 4 || N == 8 || N == 16, "4, 8 or 16 lanes");
  uint32_t u = __float_as_uint(v);
  u = max(u, dpp_u32<0xB1>(u));
  u = max(u, dpp_u32<0x4E>(u));
  if constexpr (N >= 8) u = max(u, dpp_u32<0x141>(u));
  if constexpr (N >= 16) u = max(u, dpp_u32<0x140>(u));
  return __uint_as_float(u);
}

// OR over the N consecutive lanes of a vector (same DPP steps as lanes_sum).
template <int N>
__device__ __forceinline__ uint32_t lanes_or(uint32_t v) {
  static_assert(N == 4 || N == 8 || N == 16, "4, 8 or 16 lanes");
  v |= dpp_u32<0xB1>(v);
  v |= dpp_u32<0x4E>(v);
  if constexpr (N >= 8) v |= dpp_u32<0x141>(v);
  if constexpr (N >= 16) v |= dpp_u32<0x140>(v);
  return v;
}

// Value of a lane in the other half of this lane's aligned group of
// 2 * SPAN lanes (SPAN = 1, 2, 4, 8): the pair neighbour, the other pair of
// the quad, the mirrored lane of the 8 (7 - i) or of the 16 (15 - i).  Where
// the values are uniform over aligned groups of SPAN lanes, this is the
// value of the group's partner group.
template <int SPAN>
__device__ __forceinline__ float partner_half(float v) {
  static_assert(SPAN == 1 || SPAN == 2 || SPAN == 4 || SPAN == 8, "span");
  constexpr int CTRL = SPAN == 1 ? 0xB1 : SPAN == 2 ? 0x4E : SPAN == 4 ? 0x141 : 0x140;
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}

// Raw input of one staging thread: 16 consecutive elements of one vector.
template <bool IN_F32>
struct RawInput {
  i32x4 q[IN_F32 ? 4 : 2];
};

// Non-temporal loads of a staging thread's inputs of `tile`; rows past n_vec
// (and tiles past the end) read zeros through the range check.
template <bool IN_F32>
__device__ __forceinline__ void load_raw(const i32x4 &rx, int64_t n_vec, int64_t x_stride, int64_t tile,
                                         int sv_v, int sv_c, RawInput<IN_F32> &r) {
  constexpr int ESZ = IN_F32 ? 4 : 2;
  const int64_t gv = tile * 32 + sv_v;
  const uint32_t off = gv < n_vec ? (uint32_t)((gv * x_stride + 16 * sv_c) * ESZ) : kNoStore;
#pragma unroll
  for (int q = 0; q < (IN_F32 ? 4 : 2); ++q) r.q[q] = tq_llvm_buf_ld_b128(rx, (int)(off + 16 * q), 0, kStream);
}

// Stages 16 elements of vector sv_v into an LDS tile (fp16, and fp16 lo for
// fp32 inputs) after the per-vector power-of-two scale; every thread of
// a vector writes 1 / (scale * 2^8 * |x|) to vinv.  Returns the fp16 norm,
// the nearest-even rounding of the exact |x|.  FP32_SUMS (bf16 inputs):
// sums of squares in fp32 with an exact fp64 fallback near fp16 midpoints,
// else fp64 throughout.
template <int D, bool IN_F32, bool FP32_SUMS = true>
__device__ __forceinline__ uint16_t stage_vector(const RawInput<IN_F32> &r, _Float16 *xh, _Float16 *xl,
                                                 float *vinv, int sv_v, int sv_c) {
  using L = QLayout<D>;
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
  // fp32 inputs: the squares are not exact in fp32, so the sum of squares
  // runs in fp64 from the start
  constexpr bool F64 = IN_F32 || !FP32_SUMS;
  double ss = 0.0;
  float mx = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if constexpr (F64) ss = fma((double)xv[i], (double)xv[i], ss);
    mx = fmaxf(mx, fabsf(xv[i]));
  }
  if constexpr (F64) ss = lanes_sum<L::TPV>(ss);
  mx = lanes_max<L::TPV>(mx);
  // exponent of the largest element (frexp's is one above ilogb's; a zero
  // vector gets -1 and stays zero).  The scale 2^se can exceed the fp32
  // range for tiny vectors (se up to 163), so it is applied with v_ldexp_f32,
  // which is exact without forming 2^se.
  int e = __builtin_amdgcn_frexp_expf(mx) - 1;
  e = e < -149 ? -149 : (e > 127 ? 127 : e);
  const int se = 14 - e;
  half8 hv[2], lv[2];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float sv = ldexpf(xv[i], se);
    const _Float16 hh = (_Float16)sv;
    hv[i >> 3][i & 7] = hh;
    if constexpr (IN_F32) lv[i >> 3][i & 7] = (_Float16)(sv - (float)hh);
  }
  half8 *dh = (half8 *)&xh[sv_v * L::PITCH + 16 * sv_c];
  dh[0] = hv[0];
  dh[1] = hv[1];
  if constexpr (IN_F32) {
    half8 *dl = (half8 *)&xl[sv_v * L::PITCH + 16 * sv_c];
    dl[0] = lv[0];
    dl[1] = lv[1];
  }
  if constexpr (F64) {
    // 1 / (sc * 2^8 * |x|), correctly rounded to fp32: the scaled sum of
    // squares lies in [2^28, 2^37); v_rsq_f32 (about one ulp) is refined by
    // one Newton step in fp64 (error ~2^-45) before the single rounding.
    const double ss_sc = ldexp(ss, 2 * se);
    const double r0 = (double)__builtin_amdgcn_rsqf((float)ss_sc);
    const double r1 = fma(r0, fma(-0.5 * ss_sc, r0 * r0, 0.5), r0);
    vinv[sv_v] = ss > 0.0 ? (float)r1 * (1.0f / kPiScale) : 0.0f;   // the vector's threads all hold it
    return f64_to_f16_bits(sqrt(ss));
  } else {
    // bf16 inputs: the staged fp16 values are the scaled inputs exactly
    // (8 significant bits; only elements below 2^-28 of the largest, in the
    // fp16 subnormal range, round), so their squares are exact in fp32 and
    // the scaled sum of squares s2 in [2^28, 2^37) is formed with two-wide
    // fp16 dot products in fp32: at most 19 roundings of partial sums no
    // larger than s2, i.e. a relative error below 19 * 2^-24.
    float s2 = 0.0f;
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const half2 h2 = {hv[q][2 * i], hv[q][2 * i + 1]};
        s2 = __builtin_amdgcn_fdot2(h2, h2, s2, false);
      }
    s2 = lanes_sum<L::TPV>(s2);
    // 1 / (sc * 2^8 * |x|): v_rsq_f32 and one Newton step in fp32 (a common
    // factor of the vector's unit coordinates; its error, about 2^-23
    // relative, enters the residual norm gamma one to one)
    const float r0 = __builtin_amdgcn_rsqf(s2);
    const float r1 = fmaf(r0, fmaf(-0.5f * s2, r0 * r0, 0.5f), r0);
    vinv[sv_v] = s2 > 0.0f ? r1 * (1.0f / kPiScale) : 0.0f;
    // The scaled norm n32 = sqrt(s2) (v_sqrt_f32, one ulp) is within about
    // 12.5 * 2^-24 of the exact one, so the exact norm lies between
    // n32 (1 - 2^-19) and n32 (1 + 2^-19).  Where both ends round to the
    // same fp16 (nearest even is monotone) that is the answer; otherwise
    // (about 0.5% of vectors: the norm is near an fp16 midpoint) the wave
    // forms the exact sum of squares in fp64 and rounds it once.
    const float n32 = __builtin_amdgcn_sqrtf(s2);
    const uint16_t lo16 = f32_to_f16_bits(ldexpf(n32 * (1.0f - 0x1p-19f), -se));
    const uint16_t hi16 = f32_to_f16_bits(ldexpf(n32 * (1.0f + 0x1p-19f), -se));
    uint16_t n16 = lo16;
    if (__builtin_expect(__ballot(lo16 != hi16) != 0, 0)) {   // wave-uniform branch
#pragma unroll
      for (int i = 0; i < 16; ++i) ss = fma((double)xv[i], (double)xv[i], ss);
      ss = lanes_sum<L::TPV>(ss);
      const uint16_t exact = f64_to_f16_bits(sqrt(ss));
      n16 = lo16 == hi16 ? lo16 : exact;
    }
    return n16;
  }
}

// y = X Pi^T for the wave's 32 columns of a staged tile (A fragments read
// from LDS up front).  With NACC = 2 the K steps alternate between two
// accumulators, so consecutive MFMAs do not wait on each other; that pays
// where the wave has nothing else to issue meanwhile (the MSE kernel) and
// costs 16 adds where other waves fill the SIMD (the split kernel).
template <int D, bool IN_F32, int NACC = 2>
__device__ __forceinline__ f32x16 rotate_tile(const _Float16 *xh, const _Float16 *xl,
                                              const half8 (&pih)[D / 16], const half8 (&pil)[D / 16], int m,
                                              int h) {
  using L = QLayout<D>;
  static_assert(NACC == 1 || NACC == 2, "one or two accumulators");
  f32x16 acc[2] = {{}, {}};
  half8 ah[L::KS];
#pragma unroll
  for (int s = 0; s < L::KS; ++s) ah[s] = *(const half8 *)&xh[m * L::PITCH + 16 * s + 8 * h];
#pragma unroll
  for (int s = 0; s < L::KS; ++s) {
    const half8 a0 = ah[s];
    const int c = s % NACC;
    if constexpr (IN_F32) {
      half8 al = *(const half8 *)&xl[m * L::PITCH + 16 * s + 8 * h];
      acc[c] = mfma32(al, pih[s], acc[c]);
    }
    acc[c] = mfma32(a0, pil[s], acc[c]);
    acc[c] = mfma32(a0, pih[s], acc[c]);
  }
  if constexpr (NACC == 2) return acc[0] + acc[1];
  return acc[0];
}

// Codes of the wave's 32 x 32 block: plane words go to outw (lane slot
// (r*LB + p)*2 + hh holds plane p of vector 8(r/4)+4hh+r%4); in
// inner-product mode the residual y/n - c_hat (scaled 2^10, fp16 hi + lo) is
// written to column 32w + m of rh/rl.
template <int D, int LB, bool PROD>
__device__ __forceinline__ void code_block(const f32x16 &acc, const float *vinv, const float *bnd,
                                           const float *cen, _Float16 *rh, _Float16 *rl, int w, int m, int h,
                                           uint32_t (&outw)[2]) {
  using L = QLayout<D>;
  constexpr int K = 1 << LB;
  float inv[16];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    f32x4 t = *(const f32x4 *)&vinv[8 * g + 4 * h];
    inv[4 * g] = t[0]; inv[4 * g + 1] = t[1]; inv[4 * g + 2] = t[2]; inv[4 * g + 3] = t[3];
  }
  outw[0] = 0u;
  outw[1] = 0u;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float u = acc[r] * inv[r];
    // The codebook is antisymmetric (boundary K/2-1 is 0, boundary K/2-1-j
    // is minus boundary K/2-1+j), so the cell is the sign s = (u >= 0) and
    // the magnitude level lvl = #{j >= 1 : |u| >= t[K/2-1+j]}: idx = K/2 + lvl
    // for s, K/2-1-lvl otherwise, i.e. the low LB-1 bits are lvl, inverted
    // when u < 0 (u exactly on a negative boundary falls one cell higher
    // than with the full thermometer; such values are within any rounding
    // of the boundary).  K/2 compares instead of K-1.
    constexpr int MID = K / 2;
    const uint64_t sgn = __ballot(u >= 0.0f);
    uint64_t g[MID > 1 ? MID - 1 : 1];   // g[j-1]: |u| >= t[MID-1+j]
#pragma unroll
    for (int j = 1; j < MID; ++j) g[j - 1] = __ballot(fabsf(u) >= bnd[MID - 1 + j]);
    uint64_t planes[LB];
    planes[LB - 1] = sgn;
#pragma unroll
    for (int p = 0; p < LB - 1; ++p) {
      uint64_t lp = 0;                  // bit p of the thermometer count
#pragma unroll
      for (int j = 1; j < MID; ++j)
        if ((j & ((1 << p) - 1)) == 0) lp ^= g[j - 1];   // multiples of 2^p
      planes[p] = lp ^ ~sgn;
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
      // centroid of the chosen cell: magnitude cen[MID + lvl], sign of u
      float mag = cen[MID];
#pragma unroll
      for (int j = 1; j < MID; ++j) mag = __builtin_amdgcn_inverse_ballot_w64(g[j - 1]) ? cen[MID + j] : mag;
      const float chat = __builtin_amdgcn_inverse_ballot_w64(sgn) ? mag : -mag;
      const int v = 8 * (r >> 2) + 4 * h + (r & 3);
      const float rs = (u - chat) * kResScale;
      const _Float16 hv = (_Float16)rs;
      rh[v * L::PITCH + 32 * w + m] = hv;
      rl[v * L::PITCH + 32 * w + m] = (_Float16)(rs - (float)hv);
    }
  }
}


// Plane words of the block into their rows (rows past n_vec or a `live`
// of false are dropped).
template <int D, int LB, bool PROD>
__device__ __forceinline__ void store_planes(const i32x4 &rc, const uint32_t (&outw)[2], int64_t base,
                                             int64_t n_vec, bool live, int w, int l) {
  using F = QFormat<D, LB, PROD>;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    if (64 * g < 32 * LB) {
      const int slot = 64 * g + l;
      const int hh = slot & 1;
      const int p = (slot >> 1) % LB;
      const int r = (slot >> 1) / LB;
      const int v = 8 * (r >> 2) + 4 * hh + (r & 3);
      const int64_t gv = base + v;
      const uint32_t off = (live && slot < 32 * LB && gv < n_vec)
                               ? (uint32_t)(gv * F::RB + 4 * (w * F::NPL + p)) : kNoStore;
      buf_store_u32<kWriteBack>(rc, off, outw[g]);
    }
  }
}

// z = R M^T for rows [32wq, 32wq+32) of M from a staged residual tile.
template <int D>
__device__ __forceinline__ f32x16 sketch_tile(const _Float16 *rh, const _Float16 *rl, const half8 (&mh)[D / 16],
                                              const half8 (&ml)[D / 16], int m, int h) {
  using L = QLayout<D>;
  f32x16 acc = {};
#pragma unroll
  for (int s = 0; s < L::KS; ++s) {
    half8 ah = *(const half8 *)&rh[m * L::PITCH + 16 * s + 8 * h];
    half8 al = *(const half8 *)&rl[m * L::PITCH + 16 * s + 8 * h];
    acc = mfma32(al, mh[s], acc);
    acc = mfma32(ah, ml[s], acc);
    acc = mfma32(ah, mh[s], acc);
  }
  return acc;
}

// Sign words of a 32 x 32 block of z: lane 2r + hh holds the word of vector
// 8(r/4)+4hh+r%4.
__device__ __forceinline__ uint32_t sign_bits(const f32x16 &z) {
  uint32_t sw = 0u;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const uint64_t mk = __ballot(z[r] >= 0.0f);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) sw = write_lane(sw, (uint32_t)(mk >> (32 * hh)), 2 * r + hh);
  }
  return sw;
}

template <int D>
__device__ __forceinline__ uint32_t sign_words(const _Float16 *rh, const _Float16 *rl,
                                               const half8 (&mh)[D / 16], const half8 (&ml)[D / 16], int m,
                                               int h) {
  return sign_bits(sketch_tile<D>(rh, rl, mh, ml, m, h));
}

// The same product with M's fragments read (from L2) and split per tile
// instead of held: for d = 256, where the Pi and M slices together would
// take every VGPR of a wave.
template <int D>
__device__ __forceinline__ uint32_t sign_words_streamed(const _Float16 *rh, const _Float16 *rl,
                                                        const float *__restrict__ mat, int w, int m, int h) {
  using L = QLayout<D>;
  const float *row = fragment_row<D>(mat, w);
  f32x16 acc = {};
#pragma unroll 2
  for (int s = 0; s < L::KS; ++s) {
    half8 bh, bl;
    split_fragment(row, s, bh, bl);
    const half8 ah = *(const half8 *)&rh[m * L::PITCH + 16 * s + 8 * h];
    const half8 al = *(const half8 *)&rl[m * L::PITCH + 16 * s + 8 * h];
    acc = mfma32(al, bh, acc);
    acc = mfma32(ah, bl, acc);
    acc = mfma32(ah, bh, acc);
  }
  return sign_bits(acc);
}

// Sign words into the top plane of group wq (lanes 0..31; zero vectors get
// all signs +1).
template <int D, int LB>
__device__ __forceinline__ void store_signs(const i32x4 &rc, uint32_t sw, const float *vinv, int64_t base,
                                            int64_t n_vec, bool live, int wq, int l) {
  using F = QFormat<D, LB, true>;
  const int r = (l >> 1) & 15, hh = l & 1;
  const int v = 8 * (r >> 2) + 4 * hh + (r & 3);
  const int64_t gv = base + v;
  if (vinv[v] == 0.0f) sw = 0xFFFFFFFFu;
  const uint32_t off = (live && l < 32 && gv < n_vec) ? (uint32_t)(gv * F::RB + 4 * (wq * F::NPL + LB)) : kNoStore;
  buf_store_u32<kWriteBack>(rc, off, sw);
}

// gamma = |residual| of the unit vector sv_v from its staged residual row:
// sum of (hi + lo)^2 = hi.hi + 2 hi.lo + lo.lo, each a two-wide fp16 dot
// product accumulated in fp32 (v_dot2_f32_f16), reduced over the vector's
// TPV threads.
template <int D>
__device__ __forceinline__ float residual_norm(const _Float16 *rh, const _Float16 *rl, const float *vinv,
                                               int sv_v, int sv_c) {
  using L = QLayout<D>;
  float s_hh = 0.0f, s_hl = 0.0f, s_ll = 0.0f;
  const half8 *ph = (const half8 *)&rh[sv_v * L::PITCH + 16 * sv_c];
  const half8 *pl = (const half8 *)&rl[sv_v * L::PITCH + 16 * sv_c];
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
  ss = lanes_sum<L::TPV>(ss);
  return vinv[sv_v] == 0.0f ? 0.0f : sqrtf(ss) * (1.0f / kResScale);
}

// Buffer resources over one call's rows.  The host keeps every range below
// 2^31 bytes (large calls are split), so rows past n_vec and kNoStore fall
// outside: such loads return 0 and such stores are dropped by the hardware.
// No load or store sits behind a branch, which lets the compiler wait for
// the next tile's loads without also waiting for this tile's stores.
template <int D, int LB, bool PROD, bool IN_F32>
struct QResources {
  i32x4 rx, rc, rn, rr;
  __device__ __forceinline__ explicit QResources(const tqi::QuantizeArgs &a) {
    using F = QFormat<D, LB, PROD>;
    constexpr int ESZ = IN_F32 ? 4 : 2;
    rx = make_rsrc(a.x, (uint32_t)(((a.n_vec - 1) * a.x_stride + D) * ESZ));
    rc = make_rsrc(a.codes + a.out_offset * F::RB, (uint32_t)(a.n_vec * F::RB));
    rn = make_rsrc(a.norm + a.out_offset, (uint32_t)(a.n_vec * 2));
    rr = make_rsrc(PROD ? a.rnorm + a.out_offset : a.norm, PROD ? (uint32_t)(a.n_vec * 2) : 0u);
  }
};

template <int D, int LB, bool PROD, bool IN_F32>
__global__ __launch_bounds__(QLayout<D>::NT) void quantize_kernel(tqi::QuantizeArgs a) {
  using L = QLayout<D>;
  constexpr int K = 1 << LB;
  constexpr int TILE = L::TILE;
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
  // inner-product mode: M's slice stationary too, except at d = 256 (read
  // per tile, see sign_words_streamed)
  constexpr bool HOLD_M = PROD && D <= 128;
  half8 mh[HOLD_M ? L::KS : 1], ml[HOLD_M ? L::KS : 1];
  if constexpr (HOLD_M) load_stationary<D>(a.m, w, mh, ml);

  float bnd[K - 1];
#pragma unroll
  for (int k = 0; k < K - 1; ++k) bnd[k] = a.boundaries[k];
  float cen[K];
#pragma unroll
  for (int k = 0; k < K; ++k) cen[k] = PROD ? a.centroids[k] : 0.0f;

  const int64_t n_tiles = (a.n_vec + 31) / 32;
  const QResources<D, LB, PROD, IN_F32> res(a);

  // One register set of raw input: the next tile's loads are issued as soon
  // as the current tile has been staged, so they fly during its GEMMs and
  // coding.
  const int64_t step = gridDim.x;
  int64_t tile = blockIdx.x;
  RawInput<IN_F32> raw;
  load_raw<IN_F32>(res.rx, a.n_vec, a.x_stride, tile, sv_v, sv_c, raw);
  // Range-dropped stores: with them, on entry as on every later iteration,
  // stores follow the pending input loads, so the compiler can wait for
  // those loads alone (it merges the counts of both paths into the loop).
#pragma unroll
  for (int i = 0; i < 5; ++i) buf_store_u32<kWriteBack>(res.rn, kNoStore + 4 * i, 0u);
  int buf = 0;
  for (; tile < n_tiles; tile += step, buf ^= 1) {
    const uint16_t n16 = stage_vector<D, IN_F32>(raw, xh[buf], xl[IN_F32 ? buf : 0], vinv[buf], sv_v, sv_c);
    load_raw<IN_F32>(res.rx, a.n_vec, a.x_stride, tile + step, sv_v, sv_c, raw);
    __builtin_amdgcn_sched_barrier(0);
    const int64_t base = tile * 32;
    buf_store_u16<kWriteBack>(res.rn, (sv_c == 0 && base + sv_v < a.n_vec) ? (uint32_t)(2 * (base + sv_v)) : kNoStore,
                              n16);
    __syncthreads();
    const f32x16 acc = rotate_tile<D, IN_F32>(xh[buf], xl[IN_F32 ? buf : 0], pih, pil, m, h);
    uint32_t outw[2];
    code_block<D, LB, PROD>(acc, vinv[buf], bnd, cen, rh[PROD ? buf : 0], rl[PROD ? buf : 0], w, m, h, outw);
    store_planes<D, LB, PROD>(res.rc, outw, base, a.n_vec, true, w, l);
    if constexpr (PROD) {
      __syncthreads();
      uint32_t sw;
      if constexpr (HOLD_M)
        sw = sign_words<D>(rh[buf], rl[buf], mh, ml, m, h);
      else
        sw = sign_words_streamed<D>(rh[buf], rl[buf], a.m, w, m, h);
      store_signs<D, LB>(res.rc, sw, vinv[buf], base, a.n_vec, true, w, l);
      const float gam = residual_norm<D>(rh[buf], rl[buf], vinv[buf], sv_v, sv_c);
      buf_store_u16<kWriteBack>(res.rr, (sv_c == 0 && base + sv_v < a.n_vec) ? (uint32_t)(2 * (base + sv_v)) : kNoStore,
                                f32_to_f16_bits(gam));
    }
  }
}

// Inner-product mode, three kinds of wave.  Waves [0, D/32) produce: rotate
// and code tile k from xh[k%2] (staged in the previous iteration) and write
// its residual to rh/rl[k%2].  Waves [D/32, D/16) sketch: the QJL projection
// and sign words of tile k-1 from rh/rl[(k+1)%2].  Waves [D/16, 3D/32) stage:
// tile k+1 into xh[(k+1)%2] from the prefetched input, then the residual norm
// of tile k-1.  Every buffer a kind writes in iteration k is read by another
// kind in a later iteration (vinv is a ring of four), so one barrier per
// iteration orders everything.  The loop runs one iteration past the last
// tile to drain the sketch; work on a missing tile is done on stale data and
// its stores are dropped, which keeps the loop free of branches.  Only
// producers and sketchers hold a stationary matrix, which keeps the kernel
// within the 168 VGPRs that three waves per SIMD allow.
template <int D, int LB, bool IN_F32>
__global__ __launch_bounds__(3 * QLayout<D>::NT) void quantize_pc_kernel(tqi::QuantizeArgs a) {
  using L = QLayout<D>;
  constexpr int K = 1 << LB;
  constexpr int TILE = L::TILE;
  constexpr int NWP = L::NW;        // waves of each kind
  __shared__ __attribute__((aligned(16))) _Float16 xh[2][TILE];
  __shared__ __attribute__((aligned(16))) _Float16 xl[IN_F32 ? 2 : 1][IN_F32 ? TILE : 8];
  __shared__ __attribute__((aligned(16))) _Float16 rh[2][TILE];
  __shared__ __attribute__((aligned(16))) _Float16 rl[2][TILE];
  __shared__ __attribute__((aligned(16))) float vinv[4][32];   // this workgroup's k-th tile in slot k % 4

  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int l = lane_id();
  const int m = l & 31;
  const int h = l >> 5;
  const int kind = w / NWP;                     // 0 produce, 1 sketch, 2 stage (wave-uniform)
  const int wq = w % NWP;                       // 32-row slice of Pi (producer) or M (sketcher)
  const int ct = tid - 2 * NWP * kWave;         // stager thread: staging / residual-norm mapping
  const int sv_v = ct / L::TPV;
  const int sv_c = ct % L::TPV;

  half8 sh[L::KS], sl[L::KS];
  if (kind < 2) load_stationary<D>(kind == 0 ? a.pi : a.m, wq, sh, sl);
  float bnd[K - 1];
#pragma unroll
  for (int k = 0; k < K - 1; ++k) bnd[k] = a.boundaries[k];
  float cen[K];
#pragma unroll
  for (int k = 0; k < K; ++k) cen[k] = a.centroids[k];

  const int64_t n_tiles = (a.n_vec + 31) / 32;
  const QResources<D, LB, true, IN_F32> res(a);
  const int64_t step = gridDim.x;
  const int64_t t0 = blockIdx.x;

  RawInput<IN_F32> raw;
  // The stage waves keep the fp64 sums of squares: with fp32 sums and the
  // midpoint fallback this kernel measured 0.5 us slower (its stage waves
  // are not what bounds it), the one-kind kernels about 2 us faster.
  if (kind == 2) {
    load_raw<IN_F32>(res.rx, a.n_vec, a.x_stride, t0, sv_v, sv_c, raw);
    const uint16_t n16 = stage_vector<D, IN_F32, false>(raw, xh[0], xl[0], vinv[0], sv_v, sv_c);
    buf_store_u16<kWriteBack>(res.rn, (sv_c == 0 && t0 * 32 + sv_v < a.n_vec) ? (uint32_t)(2 * (t0 * 32 + sv_v)) : kNoStore,
                              n16);
    load_raw<IN_F32>(res.rx, a.n_vec, a.x_stride, t0 + step, sv_v, sv_c, raw);
  }
  __syncthreads();
  for (int k = 0;; ++k) {
    const int64_t tp = t0 + k * step;               // the producers' tile
    if (tp >= n_tiles + step) break;                // the sketch has drained
    const int kb = k & 1;
    const int64_t tc = tp - step;                   // the sketch's tile
    const bool live = k > 0;
    if (kind == 0) {
      const f32x16 acc = rotate_tile<D, IN_F32, 1>(xh[kb], xl[IN_F32 ? kb : 0], sh, sl, m, h);
      uint32_t outw[2];
      code_block<D, LB, true>(acc, vinv[k & 3], bnd, cen, rh[kb], rl[kb], wq, m, h, outw);
      store_planes<D, LB, true>(res.rc, outw, tp * 32, a.n_vec, tp < n_tiles, wq, l);
    } else if (kind == 1) {
      const uint32_t sw = sign_words<D>(rh[kb ^ 1], rl[kb ^ 1], sh, sl, m, h);
      store_signs<D, LB>(res.rc, sw, vinv[(k + 3) & 3], tc * 32, a.n_vec, live, wq, l);
    } else {
      // stage tile tp + step (zeros past the end), prefetch the one after
      const int64_t ts = tp + step;
      const uint16_t n16 = stage_vector<D, IN_F32, false>(raw, xh[kb ^ 1], xl[IN_F32 ? kb ^ 1 : 0], vinv[(k + 1) & 3], sv_v, sv_c);
      load_raw<IN_F32>(res.rx, a.n_vec, a.x_stride, ts + step, sv_v, sv_c, raw);
      __builtin_amdgcn_sched_barrier(0);
      buf_store_u16<kWriteBack>(res.rn, (sv_c == 0 && ts * 32 + sv_v < a.n_vec) ? (uint32_t)(2 * (ts * 32 + sv_v)) : kNoStore,
                                n16);
      const float gam = residual_norm<D>(rh[kb ^ 1], rl[kb ^ 1], vinv[(k + 3) & 3], sv_v, sv_c);
      buf_store_u16<kWriteBack>(res.rr, (live && sv_c == 0 && tc * 32 + sv_v < a.n_vec) ? (uint32_t)(2 * (tc * 32 + sv_v)) : kNoStore,
                                f32_to_f16_bits(gam));
    }
    __syncthreads();
  }
}

// PolarQuant variant of stage 1 (page section "1단계": the unit vector is
// paired recursively into polar form; radii carry magnitude, angles
// direction).  The tile is staged and rotated as above; the rotated unit
// coordinates go to LDS and the D/16 staging threads of a vector take 16
// coordinates each.  No angle is ever evaluated: phi >= beta and psi >= beta
// are decided on squared radii, which only needs sums of squares --
//   level 1: the quadrant of (y_2i, y_2i+1) from signs, then within it the
//     local angle against pi/8, pi/4, 3pi/8 as b^2 >= tan^2(beta) a^2;
//   level l >= 2: psi >= beta  <=>  R_b >= tan^2(beta) R_a, R the squared
//     radii of the two halves (an angle of a zero block, R_b = 0, is 0).
// Levels 2..4 stay inside a thread, the rest pair threads by DPP steps.
// Codes: 4 level-1 planes (word 4g + p), then 2 planes of the higher levels
// in level order (word D/16 + 2g + p); bits are gathered with or-reductions
// over the vector's threads (DPP steps as well).
template <int D>
struct PolarLayout {
  static constexpr int LV = D == 64 ? 6 : (D == 128 ? 7 : 8);   // levels
  static constexpr int TPV = D / 16;        // threads per vector
  static constexpr int NG1 = D / 64;        // level-1 groups of 32 slots
  static constexpr int NGU = D / 64;        // upper-level groups
  static constexpr int RB = 3 * D / 8;      // bytes per row
  static_assert((1 << LV) == D && TPV >= 4, "polar layout");
};

// First slot of level l >= 2 among the higher-level slots.
template <int D>
__host__ __device__ constexpr int polar_level_slot(int level) {
  return D / 2 - (D >> (level - 1));
}

template <int D, bool IN_F32>
__global__ __launch_bounds__(QLayout<D>::NT) void quantize_polar_kernel(tqi::QuantizeArgs a) {
  using L = QLayout<D>;
  using P = PolarLayout<D>;
  constexpr int TILE = L::TILE;
  constexpr float kT1 = 0.17157287525381f;    // tan^2(pi/8)  = 3 - 2 sqrt 2
  constexpr float kT3 = 5.82842712474619f;    // tan^2(3pi/8) = 3 + 2 sqrt 2
  __shared__ __attribute__((aligned(16))) _Float16 xh[2][TILE];
  __shared__ __attribute__((aligned(16))) _Float16 xl[IN_F32 ? 2 : 1][IN_F32 ? TILE : 8];
  __shared__ __attribute__((aligned(16))) float vinv[2][32];
  __shared__ __attribute__((aligned(16))) float us[32][D + 4];
  __shared__ float tq2[P::LV - 1][3];

  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int l = lane_id();
  const int m = l & 31;
  const int h = l >> 5;
  const int sv_v = tid / L::TPV;
  const int sv_c = tid % L::TPV;

  half8 pih[L::KS], pil[L::KS];
  load_stationary<D>(a.pi, w, pih, pil);
  if (tid < 3 * (P::LV - 1)) {
    const double t = tan((double)a.boundaries[tid]);
    tq2[tid / 3][tid % 3] = (float)(t * t);
  }
  const int64_t n_tiles = (a.n_vec + 31) / 32;
  const i32x4 rx = make_rsrc(a.x, (uint32_t)(((a.n_vec - 1) * a.x_stride + D) * (IN_F32 ? 4 : 2)));
  const i32x4 rc = make_rsrc(a.codes + a.out_offset * P::RB, (uint32_t)(a.n_vec * P::RB));
  const i32x4 rn = make_rsrc(a.norm + a.out_offset, (uint32_t)(a.n_vec * 2));

  const int64_t step = gridDim.x;
  int64_t tile = blockIdx.x;
  RawInput<IN_F32> raw;
  load_raw<IN_F32>(rx, a.n_vec, a.x_stride, tile, sv_v, sv_c, raw);
#pragma unroll
  for (int i = 0; i < 3; ++i) buf_store_u32<kWriteBack>(rn, kNoStore + 4 * i, 0u);
  int buf = 0;
  for (; tile < n_tiles; tile += step, buf ^= 1) {
    const uint16_t n16 = stage_vector<D, IN_F32>(raw, xh[buf], xl[IN_F32 ? buf : 0], vinv[buf], sv_v, sv_c);
    load_raw<IN_F32>(rx, a.n_vec, a.x_stride, tile + step, sv_v, sv_c, raw);
    __builtin_amdgcn_sched_barrier(0);
    const int64_t base = tile * 32;
    const bool row_ok = base + sv_v < a.n_vec;
    buf_store_u16<kWriteBack>(rn, (sv_c == 0 && row_ok) ? (uint32_t)(2 * (base + sv_v)) : kNoStore, n16);
    __syncthreads();
    const f32x16 acc = rotate_tile<D, IN_F32>(xh[buf], xl[IN_F32 ? buf : 0], pih, pil, m, h);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int v = 8 * (r >> 2) + 4 * h + (r & 3);
      us[v][32 * w + m] = acc[r] * vinv[buf][v];
    }
    __syncthreads();

    // ---- coding of vector sv_v, coordinates [16 sv_c, 16 sv_c + 16)
    const bool zero = vinv[buf][sv_v] == 0.0f;
    float y[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 t = *(const f32x4 *)&us[sv_v][16 * sv_c + 4 * q];
      y[4 * q] = t[0]; y[4 * q + 1] = t[1]; y[4 * q + 2] = t[2]; y[4 * q + 3] = t[3];
    }
    float r1[8];
    uint32_t b1[4] = {0u, 0u, 0u, 0u};      // level-1 bits of this thread, plane p
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float ye = y[2 * i], yo = y[2 * i + 1];
      const float e2 = ye * ye, o2 = yo * yo;
      r1[i] = e2 + o2;
      const bool q0 = ye > 0.0f && yo >= 0.0f, q1 = ye <= 0.0f && yo > 0.0f;
      const bool q2 = ye < 0.0f && yo <= 0.0f, q3 = ye >= 0.0f && yo < 0.0f;
      const float A = (q1 || q3) ? o2 : e2;   // squared local x
      const float B = (q1 || q3) ? e2 : o2;   // squared local y
      const int sub = (B >= kT1 * A ? 1 : 0) + (B >= A ? 1 : 0) + (B >= kT3 * A ? 1 : 0);
      int idx = (q1 ? 4 : 0) + (q2 ? 8 : 0) + (q3 ? 12 : 0) + sub;
      idx = (q0 || q1 || q2 || q3) && !zero ? idx : 0;
#pragma unroll
      for (int p = 0; p < 4; ++p) b1[p] |= (uint32_t)((idx >> p) & 1) << i;
    }
    // higher levels: bits into the upper-group words of this thread
    uint32_t bu[P::NGU][2];
#pragma unroll
    for (int g = 0; g < P::NGU; ++g) bu[g][0] = bu[g][1] = 0u;
    auto put = [&](int level, int node, int idx) __attribute__((always_inline)) {
      const int slot = polar_level_slot<D>(level) + node;
      idx = zero ? 0 : idx;
#pragma unroll
      for (int g = 0; g < P::NGU; ++g)
#pragma unroll
        for (int p = 0; p < 2; ++p)
          if (slot / 32 == g) bu[g][p] |= (uint32_t)((idx >> p) & 1) << (slot % 32);
    };
    auto angle = [&](float ra, float rb, int level) __attribute__((always_inline)) -> int {
      const float *t = tq2[level - 2];
      const int c = (rb >= t[0] * ra ? 1 : 0) + (rb >= t[1] * ra ? 1 : 0) + (rb >= t[2] * ra ? 1 : 0);
      return rb > 0.0f ? c : 0;
    };
    float r2[4], r3[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      put(2, 4 * sv_c + i, angle(r1[2 * i], r1[2 * i + 1], 2));
      r2[i] = r1[2 * i] + r1[2 * i + 1];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      put(3, 2 * sv_c + i, angle(r2[2 * i], r2[2 * i + 1], 3));
      r3[i] = r2[2 * i] + r2[2 * i + 1];
    }
    put(4, sv_c, angle(r3[0], r3[1], 4));
    // levels 5..LV across threads: rr is uniform over each aligned group of
    // `span` threads, so any lane of the partner group supplies its radius
    float rr = r3[0] + r3[1];
    auto level_step = [&](auto span_c, int level) __attribute__((always_inline)) {
      constexpr int span = decltype(span_c)::value;   // threads per half at this level
      const float other = partner_half<span>(rr);
      if ((sv_c & (2 * span - 1)) == 0) put(level, sv_c >> (level - 4), angle(rr, other, level));
      rr += other;
    };
    level_step(std::integral_constant<int, 1>(), 5);
    if constexpr (P::LV >= 6) level_step(std::integral_constant<int, 2>(), 6);
    if constexpr (P::LV >= 7) level_step(std::integral_constant<int, 4>(), 7);
    if constexpr (P::LV >= 8) level_step(std::integral_constant<int, 8>(), 8);
    // level-1 plane words: 8 bits per thread, 4 threads per 32-slot group
    uint32_t wl[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) wl[p] = lanes_or<4>(b1[p] << (8 * (sv_c & 3)));
#pragma unroll
    for (int g = 0; g < P::NGU; ++g)
#pragma unroll
      for (int p = 0; p < 2; ++p) bu[g][p] = lanes_or<L::TPV>(bu[g][p]);
    const uint32_t row = (uint32_t)((base + sv_v) * P::RB);
    uint32_t wv1 = wl[0];
#pragma unroll
    for (int p = 1; p < 4; ++p) wv1 = (sv_c & 3) == p ? wl[p] : wv1;
    buf_store_u32<kWriteBack>(rc, row_ok ? row + 4 * (4 * (sv_c >> 2) + (sv_c & 3)) : kNoStore, wv1);
    uint32_t wvu = bu[0][0];
#pragma unroll
    for (int g = 0; g < P::NGU; ++g)
#pragma unroll
      for (int p = 0; p < 2; ++p) wvu = sv_c == 2 * g + p ? bu[g][p] : wvu;
    buf_store_u32<kWriteBack>(rc, (row_ok && sv_c < 2 * P::NGU) ? row + 4 * (D / 16 + sv_c) : kNoStore, wvu);
  }
}

// Rows per launch so that the input, code and norm byte ranges stay below
// 2^31; 0 if one row's input is already too wide.
template <int D, int LB, bool PROD, bool IN_F32>
int64_t rows_per_launch(int64_t x_stride) {
  constexpr int64_t ESZ = IN_F32 ? 4 : 2;
  constexpr int64_t kRange = (int64_t{1} << 31) - 1;
  if (x_stride * ESZ > kRange) return 0;
  int64_t rows = kRange / (x_stride * ESZ);
  if (rows > kRange / QFormat<D, LB, PROD>::RB) rows = kRange / QFormat<D, LB, PROD>::RB;
  if (rows >= 32) rows &= ~int64_t{31};
  return rows;
}

template <typename Kernel>
hipError_t launch_chunks(Kernel kernel, int threads, int64_t rows, int64_t esz, const tqi::QuantizeArgs &a,
                         hipStream_t s) {
  if (rows <= 0) return hipErrorInvalidValue;
  int blocks_per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks_per_cu, kernel, threads, 0);
  if (e != hipSuccess) return e;
  if (blocks_per_cu < 1) blocks_per_cu = 1;
  for (int64_t start = 0; start < a.n_vec; start += rows) {
    tqi::QuantizeArgs c = a;
    c.x = (const char *)a.x + start * a.x_stride * esz;
    c.n_vec = a.n_vec - start < rows ? a.n_vec - start : rows;
    c.out_offset = a.out_offset + start;
    const int64_t n_tiles = (c.n_vec + 31) / 32;
    int64_t grid = (int64_t)tqi::device_cu_count() * blocks_per_cu;
    if (grid > n_tiles) grid = n_tiles;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(threads), 0, s, c);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int D, int LB, bool PROD, bool IN_F32>
hipError_t launch_t(const tqi::QuantizeArgs &a, hipStream_t s) {
  using L = QLayout<D>;
  const int64_t rows = rows_per_launch<D, LB, PROD, IN_F32>(a.x_stride);
  const int64_t esz = IN_F32 ? 4 : 2;
  if constexpr (PROD && D <= 128)
    return launch_chunks(quantize_pc_kernel<D, LB, IN_F32>, 3 * L::NT, rows, esz, a, s);
  else
    return launch_chunks(quantize_kernel<D, LB, PROD, IN_F32>, L::NT, rows, esz, a, s);
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

template <int D, bool IN_F32>
hipError_t launch_polar_t(const tqi::QuantizeArgs &a, hipStream_t s) {
  constexpr int64_t ESZ = IN_F32 ? 4 : 2;
  constexpr int64_t kRange = (int64_t{1} << 31) - 1;
  if (a.x_stride * ESZ > kRange) return hipErrorInvalidValue;
  int64_t rows = kRange / (a.x_stride * ESZ);
  if (rows > kRange / PolarLayout<D>::RB) rows = kRange / PolarLayout<D>::RB;
  if (rows >= 32) rows &= ~int64_t{31};
  return launch_chunks(quantize_polar_kernel<D, IN_F32>, QLayout<D>::NT, rows, ESZ, a, s);
}

}  // namespace

namespace tqi {

hipError_t launch_quantize_polar(int d, bool in_f32, const QuantizeArgs &a, hipStream_t s, bool *supported) {
  *supported = d == 64 || d == 128 || d == 256;
  if (d == 64) return in_f32 ? launch_polar_t<64, true>(a, s) : launch_polar_t<64, false>(a, s);
  if (d == 128) return in_f32 ? launch_polar_t<128, true>(a, s) : launch_polar_t<128, false>(a, s);
  if (d == 256) return in_f32 ? launch_polar_t<256, true>(a, s) : launch_polar_t<256, false>(a, s);
  return hipSuccess;
}

hipError_t launch_quantize(int d, int lbits, bool prod, bool in_f32, const QuantizeArgs &a,
                           hipStream_t s, bool *supported) {
  *supported = false;
  if (d == 64) return prod ? launch_lb<64, true>(lbits, in_f32, a, s, supported)
                           : launch_lb<64, false>(lbits, in_f32, a, s, supported);
  if (d == 128) return prod ? launch_lb<128, true>(lbits, in_f32, a, s, supported)
                            : launch_lb<128, false>(lbits, in_f32, a, s, supported);
  if (d == 256) return prod ? launch_lb<256, true>(lbits, in_f32, a, s, supported)
                            : launch_lb<256, false>(lbits, in_f32, a, s, supported);
  return hipSuccess;
}

}  // namespace tqi
