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

// Raw inputs of one decoding thread (16 coordinates of one vector): the
// 16-bit halves of its plane words, and for the first thread of a vector the
// fp16 norm and residual norm.
template <int NPL>
struct DecodeRaw {
  uint32_t pw[NPL];
  uint32_t nrm, gam;
};

template <int D, int LB, bool PROD, bool OUT_F32>
__global__ __launch_bounds__(DLayout<D>::NT) void dequant_kernel(tqi::DequantArgs a) {
  using L = DLayout<D>;
  constexpr int K = 1 << LB;
  constexpr int PB = D / 8;
  constexpr int NPL = LB + (PROD ? 1 : 0);  // planes per record (sign on top)
  constexpr int RB = NPL * PB;
  constexpr int TILE = 32 * L::PITCH;
  constexpr int OSZ = OUT_F32 ? 4 : 2;      // bytes per output element
  constexpr int OCH = 32 * D * OSZ / 16;    // 16-byte output chunks per tile
  // Two barriers per tile: decoded tile -> products, output tile -> stores.
  // The second also orders this tile's products before the next decoding,
  // so one decode buffer suffices.  The output tile is written back as full
  // 16-byte pieces of rows.
  __shared__ __attribute__((aligned(16))) _Float16 ch[TILE];
  __shared__ __attribute__((aligned(16))) _Float16 cl[TILE];
  __shared__ __attribute__((aligned(16))) _Float16 sg[PROD ? TILE : 8];
  __shared__ __attribute__((aligned(16))) float vfac[2][32];
  __shared__ __attribute__((aligned(16))) uint8_t otile[32 * D * OSZ];
  __shared__ uint32_t ctab[K];

  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int l = lane_id();
  const int m = l & 31;
  const int h = l >> 5;
  const int dv = tid / L::TPV;   // decoding: vector of the tile
  const int dc = tid % L::TPV;   //           16-coordinate chunk

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
#pragma unroll
    for (int p = 0; p < NPL; ++p)
      r.pw[p] = buf_load_u16(rc, row + 4 * ((dc >> 1) * NPL + p) + 2 * (dc & 1));
    const uint32_t sc = (gv < a.n_vec && dc == 0) ? (uint32_t)(2 * gv) : kNoStore;
    r.nrm = buf_load_u16(rn, sc);
    r.gam = PROD ? buf_load_u16(rg, sc) : 0u;
  };

  // 16 coordinates of one vector into LDS: centroid halves (scaled by
  // 2^10), signs as exact fp16 +-1, and the per-vector factors.
  auto decode = [&](const DecodeRaw<NPL> &r) {
    half8 hv[2], lv[2], sv[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint32_t idx = 0;
#pragma unroll
      for (int p = 0; p < LB; ++p) idx |= ((r.pw[p] >> i) & 1u) << p;
      const uint32_t e = ctab[idx];
      const uint16_t hb = (uint16_t)(e & 0xFFFF), lb = (uint16_t)(e >> 16);
      _Float16 hf, lf;
      __builtin_memcpy(&hf, &hb, 2);
      __builtin_memcpy(&lf, &lb, 2);
      hv[i >> 3][i & 7] = hf;
      lv[i >> 3][i & 7] = lf;
      if constexpr (PROD) sv[i >> 3][i & 7] = ((r.pw[LB] >> i) & 1u) ? (_Float16)1.0f : (_Float16)-1.0f;
    }
    const int o = dv * L::PITCH + 16 * dc;
    *(half8 *)&ch[o] = hv[0];
    *(half8 *)&ch[o + 8] = hv[1];
    *(half8 *)&cl[o] = lv[0];
    *(half8 *)&cl[o + 8] = lv[1];
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
  __syncthreads();   // ctab
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
      float val = acc[r] * vfac[0][v];
      if constexpr (PROD) val += acc2[r] * vfac[1][v];
      const int e = v * D + 32 * w + m;
      if constexpr (OUT_F32)
        ((float *)otile)[e] = val;
      else
        ((uint16_t *)otile)[e] = f32_to_bf16_bits(val);
    }
    __syncthreads();
    // 16-byte pieces of whole output rows; rows past n_vec are dropped
    const int64_t base = tile * 32;
#pragma unroll
    for (int i = 0; i < OCH / DLayout<D>::NT; ++i) {
      const int ck = tid + DLayout<D>::NT * i;
      const int v = ck / (D * OSZ / 16);
      const int64_t gv = base + v;
      const f32x4 val = *(const f32x4 *)&otile[16 * ck];
      buf_store_f32x4(ro, gv < a.n_vec ? (uint32_t)(base * D * OSZ + 16 * ck) : kNoStore, val);
    }
  }
}

template <int D, int LB, bool PROD, bool OUT_F32>
hipError_t launch_t(const tqi::DequantArgs &a, hipStream_t s) {
  using L = DLayout<D>;
  constexpr int64_t RB = (LB + (PROD ? 1 : 0)) * D / 8;
  constexpr int64_t OSZ = OUT_F32 ? 4 : 2;
  constexpr int64_t kRange = (int64_t{1} << 31) - 1;   // kernel byte ranges stay below 2^31
  int64_t rows = kRange / (D * OSZ);                    // the output range is the largest
  if (rows > kRange / RB) rows = kRange / RB;
  rows &= ~int64_t{31};
  int blocks_per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &blocks_per_cu, dequant_kernel<D, LB, PROD, OUT_F32>, L::NT, 0);
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
    hipLaunchKernelGGL((dequant_kernel<D, LB, PROD, OUT_F32>), dim3((unsigned)grid), dim3(L::NT), 0,
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
