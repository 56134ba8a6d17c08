// Reconstruction of packed vectors:
//   x_hat = n * (Pi^T c[idx] + sqrt(pi/2)/d * gamma * S^T s).
// Page "TurboQuant 설명", section "2단계: QJL 잔차 보정" (reconstructed
// vectors) and section "1단계" (the codebook and rotation being inverted).
//
// Layout mirrors the quantiser: D/32 waves, wave w owns output columns
// [32w, 32w+32) and keeps its columns of Pi (and S) in VGPRs as fp16 hi + lo
// (scaled by 2^8).  Each 32-vector tile is decoded once into LDS: the
// centroid of every coordinate as fp16 hi + lo (scaled by 2^10), two
// coordinates per read of a K^2-entry pair table, and, in inner-product
// mode, the sign as an exact fp16 +-1.  Products run on the 32x32x16 fp16
// MFMA with fp32 accumulation, with the matrix as the A operand, so that a
// lane's accumulators are 16 coordinates (four runs of four) of one vector:
// the per-vector factor is one value per lane, and each run goes to the
// LDS output tile as one 8-byte (bf16) or 16-byte (fp32) write, from which
// whole rows leave as 16-byte stores.  For bf16 output one fp16 product
// (hi x hi, about 2^-11 relative per element) meets the output precision, so
// the lo halves are skipped.
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

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The 16 low bits of x (one plane of 16 coordinates) with bit pair k
// (coordinates 2k and 2k + 1) moved to bits 4k and 4k + 1.
__device__ __forceinline__ uint32_t spread_pairs(uint32_t x) {
  x &= 0xFFFFu;
  x = (x | (x << 8)) & 0x00FF00FFu;
  x = (x | (x << 4)) & 0x0F0F0F0Fu;
  x = (x | (x << 2)) & 0x33333333u;
  return x;
}

// B fragment for K step s of columns [32w, 32w+32) of a d x d matrix
// (B[k][n] = mat[k][32w+n]), as fp16 hi + lo of the entries scaled by 2^8.
template <int D>
__device__ __forceinline__ void column_fragment(const float *__restrict__ mat, int w, int s, half8 &hi,
                                                half8 &lo) {
  const int l = lane_id();
  const int col = 32 * w + (l & 31);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int k = 16 * s + 8 * (l >> 5) + i;
    const float sv = mat[(size_t)k * D + col] * kMatScale;
    const _Float16 h = (_Float16)sv;
    hi[i] = h;
    lo[i] = (_Float16)(sv - (float)h);
  }
}

template <int D>
__device__ void load_columns(const float *__restrict__ mat, int w, half8 (&hi)[D / 16],
                             half8 (&lo)[D / 16]) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s) column_fragment<D>(mat, w, s, hi[s], lo[s]);
}

// Raw inputs of one decoding thread (16 coordinates of one vector): the
// 16-bit halves of its plane words (polar format: its level-1 group's four
// plane words and the higher-level plane words), and for the first thread of
// a vector the fp16 norm and residual norm.
template <int NPL>
struct DecodeRaw {
  uint32_t pw[NPL];
  uint32_t nrm, gam;
};

// Polar format (PolarQuant variant of stage 1, page section "1단계"):
// levels, upper-level groups and the first slot of each higher level.
template <int D>
struct DPolar {
  static constexpr int LV = D == 64 ? 6 : (D == 128 ? 7 : 8);
  static constexpr int NGU = D / 64;
  static constexpr int RB = 3 * D / 8;
  static constexpr int NW = 4 + 2 * NGU;   // words a decoding thread reads
  __host__ __device__ static constexpr int slot(int level) { return D / 2 - (D >> (level - 1)); }
};

template <int D, int LB, bool PROD, bool OUT_F32, bool POLAR = false>
__global__ __launch_bounds__(DLayout<D>::NT) void dequant_kernel(tqi::DequantArgs a) {
  using L = DLayout<D>;
  using PF = DPolar<D>;
  constexpr int K = 1 << LB;
  constexpr int PB = D / 8;
  constexpr int NPL = POLAR ? PF::NW : LB + (PROD ? 1 : 0);  // words read per thread
  constexpr int RB = POLAR ? PF::RB : NPL * PB;
  constexpr int TILE = 32 * L::PITCH;
  constexpr int OSZ = OUT_F32 ? 4 : 2;      // bytes per output element
  constexpr int OCH = 32 * D * OSZ / 16;    // 16-byte output chunks per tile
  constexpr int OPITCH = D * OSZ + 16;      // bytes per output tile row (the pad spreads a run's banks)
  constexpr int KK = K * K;
  // Two barriers per tile: decoded tile -> products, output tile -> stores.
  // The second also orders this tile's products before the next decoding,
  // so one decode buffer suffices.  The output tile is written back as full
  // 16-byte pieces of rows.
  __shared__ __attribute__((aligned(16))) _Float16 ch[TILE];
  // bf16 output needs 8 bits: one fp16 product (about 2^-11 per element)
  // suffices and the lo halves are not formed; fp32 output uses three.
  constexpr bool SPLIT = OUT_F32;
  __shared__ __attribute__((aligned(16))) _Float16 cl[SPLIT ? TILE : 8];
  __shared__ __attribute__((aligned(16))) _Float16 sg[PROD ? TILE : 8];
  __shared__ __attribute__((aligned(16))) float vfac[2][32];
  __shared__ __attribute__((aligned(16))) uint8_t otile[32 * OPITCH];
  // pair table: entry e holds the (even, odd) coordinates' centroids as two
  // fp16 (hi halves, then at KK + e the lo halves); bits 2p and 2p + 1 of e
  // are plane p of the even and of the odd coordinate
  __shared__ uint32_t ptab[POLAR ? 1 : (SPLIT ? 2 : 1) * KK];
  // polar: cos and sin of the level-1 sector midpoints and of the centroid
  // angles of levels 2..LV
  __shared__ float pc1[POLAR ? 16 : 1], ps1[POLAR ? 16 : 1];
  __shared__ float pcu[POLAR ? PF::LV - 1 : 1][4], psu[POLAR ? PF::LV - 1 : 1][4];

  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int l = lane_id();
  const int m = l & 31;
  const int h = l >> 5;
  const int dv = tid / L::TPV;   // decoding: vector of the tile
  const int dc = tid % L::TPV;   //           16-coordinate chunk

  half8 ph[L::KS], pl[L::KS];
  load_columns<D>(a.pi, w, ph, pl);
  // inner-product mode: S's columns stationary too, except at d = 256, where
  // they do not fit beside Pi's and are read (from L2) per tile
  constexpr bool HOLD_S = PROD && D <= 128;
  half8 sh[HOLD_S ? L::KS : 1], sl[HOLD_S ? L::KS : 1];
  if constexpr (HOLD_S) load_columns<D>(a.s_mat, w, sh, sl);
  if constexpr (POLAR) {
    if (tid < 16) {
      const double ph = 2.0 * M_PI * (tid + 0.5) / 16.0;
      pc1[tid] = (float)cos(ph);
      ps1[tid] = (float)sin(ph);
    } else if (tid < 16 + 4 * (PF::LV - 1)) {
      const int i = tid - 16;
      const double ps = (double)a.centroids[i];
      pcu[i / 4][i % 4] = (float)cos(ps);
      psu[i / 4][i % 4] = (float)sin(ps);
    }
  } else {
    for (int e = tid; e < KK; e += L::NT) {
      int i0 = 0, i1 = 0;
#pragma unroll
      for (int p = 0; p < LB; ++p) {
        i0 |= ((e >> (2 * p)) & 1) << p;
        i1 |= ((e >> (2 * p + 1)) & 1) << p;
      }
      const float c0 = a.centroids[i0] * kCenScale, c1 = a.centroids[i1] * kCenScale;
      const _Float16 h0 = (_Float16)c0, h1 = (_Float16)c1;
      ptab[e] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
      if constexpr (SPLIT) {
        const _Float16 l0 = (_Float16)(c0 - (float)h0), l1 = (_Float16)(c1 - (float)h1);
        ptab[KK + e] =
            (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
      }
    }
  }
  const float kappa = (float)(1.2533141373155003 / D);  // sqrt(pi/2) / d

  // Buffer resources over this call's rows (the host keeps each range below
  // 2^31 bytes): reads past n_vec return 0, stores there are dropped, so no
  // memory access sits behind a branch.
  const i32x4 rc = make_rsrc(a.codes, (uint32_t)(a.n_vec * RB));
  const i32x4 rn = make_rsrc(a.norm, (uint32_t)(a.n_vec * 2));
  const i32x4 rg = make_rsrc(PROD ? a.rnorm : a.norm, PROD ? (uint32_t)(a.n_vec * 2) : 0u);
  const i32x4 ro = make_rsrc(a.out, (uint32_t)(a.n_vec * D * OSZ));
  const int64_t n_tiles = (a.n_vec + 31) / 32;

  auto load_raw = [&](int64_t tile, DecodeRaw<NPL> &r) {
    const int64_t gv = tile * 32 + dv;
    const uint32_t row = gv < a.n_vec ? (uint32_t)(gv * RB) : kNoStore;
    if constexpr (POLAR) {
      // the four level-1 plane words of group dc / 4, then the upper words
      uint32_t w1[4], wu[2 * PF::NGU];
      buf_load_words<4>(rc, row == kNoStore ? kNoStore : row + 16 * (dc >> 2), w1);
      buf_load_words<2 * PF::NGU>(rc, row == kNoStore ? kNoStore : row + 4 * (D / 16), wu);
#pragma unroll
      for (int p = 0; p < 4; ++p) r.pw[p] = w1[p];
#pragma unroll
      for (int i = 0; i < 2 * PF::NGU; ++i) r.pw[4 + i] = wu[i];
    } else {
#pragma unroll
      for (int p = 0; p < NPL; ++p)
        r.pw[p] = buf_load_u16(rc, row + 4 * ((dc >> 1) * NPL + p) + 2 * (dc & 1));
    }
    const uint32_t sc = (gv < a.n_vec && dc == 0) ? (uint32_t)(2 * gv) : kNoStore;
    r.nrm = buf_load_u16(rn, sc);
    r.gam = PROD ? buf_load_u16(rg, sc) : 0u;
  };

  // 16 coordinates of one vector into LDS: centroid halves (scaled by
  // 2^10), signs as exact fp16 +-1, and the per-vector factors.
  auto decode = [&](const DecodeRaw<NPL> &r) {
    half8 hv[2], lv[2], sv[2];
    if constexpr (POLAR) {
      // y_hat of coordinates [16 dc, 16 dc + 16): the product of the
      // factors on the path from the root (radius 1) down to each pair
      auto upper = [&](int level, int node) -> int {
        const int sl = PF::slot(level) + node;
        const int g = sl >> 5, b = sl & 31;
        uint32_t w0 = r.pw[4], w1 = r.pw[5];
#pragma unroll
        for (int gg = 1; gg < PF::NGU; ++gg) {
          w0 = g == gg ? r.pw[4 + 2 * gg] : w0;
          w1 = g == gg ? r.pw[5 + 2 * gg] : w1;
        }
        return (int)(((w0 >> b) & 1u) | (((w1 >> b) & 1u) << 1));
      };
      float pf = 1.0f;
#pragma unroll
      for (int level = PF::LV; level >= 5; --level) {
        const int node = dc >> (level - 4);            // node holding this thread
        const int c = upper(level, node);
        pf *= ((dc >> (level - 5)) & 1) ? psu[level - 2][c] : pcu[level - 2][c];
      }
      float r3[2], r2[4], r1[8];
      {
        const int c = upper(4, dc);
        r3[0] = pf * pcu[2][c];
        r3[1] = pf * psu[2][c];
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int c = upper(3, 2 * dc + e);
        r2[2 * e] = r3[e] * pcu[1][c];
        r2[2 * e + 1] = r3[e] * psu[1][c];
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c = upper(2, 4 * dc + k);
        r1[2 * k] = r2[k] * pcu[0][c];
        r1[2 * k + 1] = r2[k] * psu[0][c];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int b = 8 * (dc & 3) + i;
        int c = 0;
#pragma unroll
        for (int p = 0; p < 4; ++p) c |= (int)((r.pw[p] >> b) & 1u) << p;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float yv = r1[i] * (e ? ps1[c] : pc1[c]) * kCenScale;
          const _Float16 hf = (_Float16)yv;
          hv[(2 * i + e) >> 3][(2 * i + e) & 7] = hf;
          lv[(2 * i + e) >> 3][(2 * i + e) & 7] = (_Float16)(yv - (float)hf);
        }
      }
    } else {
      // pair indices of the 8 pairs: the planes' bit pairs spread to a
      // 4-bit pitch (planes 0-1 in z01, 2-3 in z23), one nibble per pair
      uint32_t z01 = spread_pairs(r.pw[0]);
      if constexpr (LB >= 2) z01 |= spread_pairs(r.pw[1]) << 2;
      uint32_t z23 = 0;
      if constexpr (LB >= 3) z23 = spread_pairs(r.pw[2]);
      if constexpr (LB >= 4) z23 |= spread_pairs(r.pw[3]) << 2;
      uint32_t hw[8], lw[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        uint32_t pidx = (z01 >> (4 * k)) & 15u;
        if constexpr (LB >= 3) pidx |= ((z23 >> (4 * k)) & 15u) << 4;
        hw[k] = ptab[pidx];
        if constexpr (SPLIT) lw[k] = ptab[KK + pidx];
      }
      const u32x4 h0 = {hw[0], hw[1], hw[2], hw[3]}, h1 = {hw[4], hw[5], hw[6], hw[7]};
      hv[0] = __builtin_bit_cast(half8, h0);
      hv[1] = __builtin_bit_cast(half8, h1);
      if constexpr (SPLIT) {
        const u32x4 l0 = {lw[0], lw[1], lw[2], lw[3]}, l1 = {lw[4], lw[5], lw[6], lw[7]};
        lv[0] = __builtin_bit_cast(half8, l0);
        lv[1] = __builtin_bit_cast(half8, l1);
      }
      if constexpr (PROD) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          sv[i >> 3][i & 7] = ((r.pw[LB] >> i) & 1u) ? (_Float16)1.0f : (_Float16)-1.0f;
      }
    }
    const int o = dv * L::PITCH + 16 * dc;
    *(half8 *)&ch[o] = hv[0];
    *(half8 *)&ch[o + 8] = hv[1];
    if constexpr (SPLIT) {
      *(half8 *)&cl[o] = lv[0];
      *(half8 *)&cl[o + 8] = lv[1];
    }
    if constexpr (PROD) {
      *(half8 *)&sg[o] = sv[0];
      *(half8 *)&sg[o + 8] = sv[1];
    }
    if (dc == 0) {
      const float nrm = f16_bits_to_f32((uint16_t)r.nrm);
      vfac[0][dv] = nrm * (1.0f / (kCenScale * kMatScale));
      vfac[1][dv] = PROD ? nrm * kappa * f16_bits_to_f32((uint16_t)r.gam) * (1.0f / kMatScale) : 0.0f;
    }
  };

  const int64_t step = gridDim.x;
  int64_t tile = blockIdx.x;
  DecodeRaw<NPL> raw;
  load_raw(tile, raw);
  __syncthreads();   // tables
  // Range-dropped stores: on entry, as on every later iteration, stores
  // follow the pending loads (see the loop), so the compiler waits for the
  // loads alone.
#pragma unroll
  for (int i = 0; i < OCH / DLayout<D>::NT; ++i) buf_store_f32x4(ro, kNoStore + 16 * i, f32x4{0.f, 0.f, 0.f, 0.f});
  for (; tile < n_tiles; tile += step) {
    decode(raw);
    load_raw(tile + step, raw);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    // fragments read up front; K steps alternate between two accumulators
    // so that consecutive MFMAs are independent
    f32x16 accp[2] = {{}, {}};
    f32x16 acc2 = {};
    half8 ahs[L::KS];
#pragma unroll
    for (int s = 0; s < L::KS; ++s) ahs[s] = *(const half8 *)&ch[m * L::PITCH + 16 * s + 8 * h];
#pragma unroll
    for (int s = 0; s < L::KS; ++s) {
      const half8 ah = ahs[s];
      if constexpr (SPLIT) {
        const half8 al = *(const half8 *)&cl[m * L::PITCH + 16 * s + 8 * h];
        accp[s & 1] = mfma32(ph[s], al, accp[s & 1]);
        accp[s & 1] = mfma32(pl[s], ah, accp[s & 1]);
      }
      accp[s & 1] = mfma32(ph[s], ah, accp[s & 1]);
      if constexpr (HOLD_S) {
        const half8 as = *(const half8 *)&sg[m * L::PITCH + 16 * s + 8 * h];
        if constexpr (SPLIT) acc2 = mfma32(sl[s], as, acc2);
        acc2 = mfma32(sh[s], as, acc2);
      }
    }
    if constexpr (PROD && !HOLD_S) {
      // a few K steps' fragments in flight at a time
#pragma unroll 2
      for (int s = 0; s < L::KS; ++s) {
        half8 bh, bl;
        column_fragment<D>(a.s_mat, w, s, bh, bl);
        const half8 as = *(const half8 *)&sg[m * L::PITCH + 16 * s + 8 * h];
        if constexpr (SPLIT) acc2 = mfma32(bl, as, acc2);
        acc2 = mfma32(bh, as, acc2);
      }
    }
    const f32x16 acc = accp[0] + accp[1];
    // this lane's vector m: registers 4q .. 4q + 3 are its coordinates
    // 32w + 8q + 4h + 0..3
    const float f0 = vfac[0][m];
    const float f1 = PROD ? vfac[1][m] : 0.0f;
    uint8_t *orow = otile + m * OPITCH;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float val[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        val[e] = acc[4 * q + e] * f0;
        if constexpr (PROD) val[e] = fmaf(acc2[4 * q + e], f1, val[e]);
      }
      const int col = 32 * w + 8 * q + 4 * h;
      if constexpr (OUT_F32) {
        *(f32x4 *)(orow + 4 * col) = f32x4{val[0], val[1], val[2], val[3]};
      } else {
        *(uint2 *)(orow + 2 * col) = make_uint2(f32x2_to_bf16x2_bits(val[0], val[1]),
                                                f32x2_to_bf16x2_bits(val[2], val[3]));
      }
    }
    __syncthreads();
    // 16-byte pieces of whole output rows; rows past n_vec are dropped
    const int64_t base = tile * 32;
#pragma unroll
    for (int i = 0; i < OCH / DLayout<D>::NT; ++i) {
      const int ck = tid + DLayout<D>::NT * i;
      const int v = ck / (D * OSZ / 16);
      const int64_t gv = base + v;
      const f32x4 val = *(const f32x4 *)&otile[v * OPITCH + 16 * (ck % (D * OSZ / 16))];
      buf_store_f32x4(ro, gv < a.n_vec ? (uint32_t)(base * D * OSZ + 16 * ck) : kNoStore, val);
    }
  }
}

template <int D, int LB, bool PROD, bool OUT_F32, bool POLAR = false>
hipError_t launch_t(const tqi::DequantArgs &a, hipStream_t s) {
  using L = DLayout<D>;
  constexpr int64_t RB = POLAR ? DPolar<D>::RB : (LB + (PROD ? 1 : 0)) * D / 8;
  constexpr int64_t OSZ = OUT_F32 ? 4 : 2;
  constexpr int64_t kRange = (int64_t{1} << 31) - 1;   // kernel byte ranges stay below 2^31
  int64_t rows = kRange / (D * OSZ);                    // the output range is the largest
  if (rows > kRange / RB) rows = kRange / RB;
  rows &= ~int64_t{31};
  int blocks_per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &blocks_per_cu, dequant_kernel<D, LB, PROD, OUT_F32, POLAR>, L::NT, 0);
  if (e != hipSuccess) return e;
  if (blocks_per_cu < 1) blocks_per_cu = 1;
  for (int64_t start = 0; start < a.n_vec; start += rows) {
    tqi::DequantArgs c = a;
    c.codes = a.codes + start * RB;
    c.norm = a.norm + start;
    c.rnorm = PROD ? a.rnorm + start : a.rnorm;
    c.out = (char *)a.out + start * D * OSZ;
    c.n_vec = a.n_vec - start < rows ? a.n_vec - start : rows;
    const int64_t n_tiles = (c.n_vec + 31) / 32;
    int64_t grid = (int64_t)tqi::device_cu_count() * blocks_per_cu;
    if (grid > n_tiles) grid = n_tiles;
    hipLaunchKernelGGL((dequant_kernel<D, LB, PROD, OUT_F32, POLAR>), dim3((unsigned)grid), dim3(L::NT), 0,
                       s, c);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
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

hipError_t launch_dequant_polar(int d, const DequantArgs &a, hipStream_t s, bool *supported) {
  *supported = d == 64 || d == 128 || d == 256;
  if (d == 64) return a.out_f32 ? launch_t<64, 1, false, true, true>(a, s) : launch_t<64, 1, false, false, true>(a, s);
  if (d == 128) return a.out_f32 ? launch_t<128, 1, false, true, true>(a, s) : launch_t<128, 1, false, false, true>(a, s);
  if (d == 256) return a.out_f32 ? launch_t<256, 1, false, true, true>(a, s) : launch_t<256, 1, false, false, true>(a, s);
  return hipSuccess;
}

hipError_t launch_dequant(int d, int lbits, bool prod, const DequantArgs &a, hipStream_t s,
                          bool *supported) {
  *supported = false;
  if (d == 64) return prod ? launch_lb<64, true>(lbits, a, s, supported)
                           : launch_lb<64, false>(lbits, a, s, supported);
  if (d == 128) return prod ? launch_lb<128, true>(lbits, a, s, supported)
                            : launch_lb<128, false>(lbits, a, s, supported);
  if (d == 256) return prod ? launch_lb<256, true>(lbits, a, s, supported)
                            : launch_lb<256, false>(lbits, a, s, supported);
  return hipSuccess;
}

}  // namespace tqi
