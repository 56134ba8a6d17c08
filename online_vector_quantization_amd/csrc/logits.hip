// Attention logits straight from bit-packed keys.
//
// Page "TurboQuant 설명: 무엇인지와 LLM 메모리 6배 절약 구현 방법", closing
// paragraphs of "2단계: QJL 잔차 보정" and "TurboQuant 구현 방법": the query is
// rotated once and the logits are formed from the compressed indices, never
// reconstructing the keys:
//   logit = scale * n * ( <Pi q, c[idx]> + sqrt(pi/2)/d * gamma * <S q, s> ).
//
// Reformulation used here (exact in real arithmetic, DESIGN.md "Logit
// kernel"):
// * The Lloyd-Max codebook is antisymmetric (c[K-1-i] = -c[i]), so on the
//   index bits b_0..b_{B-1} it is a sum of odd Walsh functions:
//   c[idx] = sum_S beta_S (2 P_S - 1), S over the subsets of bit positions of
//   odd size, P_S the XOR of the bits in S, beta_S = 2^-B sum_i c[i] sigma_S(i).
//   Hence <q', c[idx]> = 2 sum_S beta_S <q', P_S> - (sum_S beta_S)(sum_j q'_j),
//   and likewise <q'', s> = 2 <q'', bits> - sum_i q''_i.
// * Every term is then a 0/1 plane of the key times a per-query weight.  The
//   weights are turned into 32-bit fixed point (4 signed byte pieces) once per
//   query, and the planes are fed, byte-expanded, to the int8 MFMA
//   (16x16x64, int32 accumulate): integer sums are exact, so the only error
//   is the rounding of the weights (< 2^-24 of the largest weight).
// * One MFMA row block holds 4 queries x 4 byte pieces; the K dimension
//   enumerates (plane, coordinate).  A plane dword w of 32 coordinates gives
//   the 16 bytes of one lane as w & (0x01010101 << s), s = 0..3 or 4..7: the
//   byte equals 2^s * bit, and the matching weight is quantised with
//   resolution 2^(s-F) (negated for s = 7, where the byte reads -128).
//
// Query prep (one small kernel per call) writes the A operands and four
// constants per query to a workspace; the streaming kernel keeps them in
// VGPRs and reads each key once: 16-byte code/sign planes, two fp16 scalars.
#include "tq_device.h"
#include "tq_internal.h"

namespace {

using namespace tqd;

struct PrepArgs {
  const void *q;
  bool q_f32;
  int n_q_heads, n_kv_heads, group, row_tiles;
  const float *pi;
  const float *s_mat;
  const float *centroids;
  int8_t *table;   // [stream][row_tile][chunk][64 lanes][16 bytes]
  float *consts;   // [stream][group][4]
};

template <int LB>
struct Walsh {
  static constexpr int K = 1 << LB;
  static constexpr int P = 1 << (LB - 1);   // subsets of odd size
  __host__ __device__ static constexpr int subset(int r) {
    int found = -1;
    for (int s = 1; s < K; ++s) {
      if (__builtin_popcount(s) & 1) {
        if (++found == r) return s;
      }
    }
    return 0;
  }
};

template <int D, int LB, bool PROD>
struct LLayout {
  static constexpr int P = Walsh<LB>::P;
  static constexpr int CPP = D / 64;                    // MFMA chunks per plane
  static constexpr int NCH = (P + (PROD ? 1 : 0)) * CPP;
  static constexpr int PB = D / 8;
};

template <int D, int LB, bool PROD>
__global__ __launch_bounds__(256) void logit_prep_kernel(PrepArgs a) {
  using L = LLayout<D, LB, PROD>;
  constexpr int K = 1 << LB;
  constexpr int P = L::P;
  __shared__ float qin[4][D];
  __shared__ double qr[4][D];
  __shared__ double qs[PROD ? 4 : 1][D];
  __shared__ double beta[P];
  __shared__ int fexp[4][2];

  const int stream = blockIdx.x;
  const int rt = blockIdx.y;
  const int b = stream / a.n_kv_heads;
  const int kvh = stream % a.n_kv_heads;
  const int tid = threadIdx.x;

  for (int i = tid; i < 4 * D; i += blockDim.x) {
    const int g = i / D, k = i % D;
    const int gg = 4 * rt + g;
    float v = 0.0f;
    if (gg < a.group) {
      const int64_t off = ((int64_t)b * a.n_q_heads + (int64_t)kvh * a.group + gg) * D + k;
      v = a.q_f32 ? ((const float *)a.q)[off] : bf16_to_f32(((const uint16_t *)a.q)[off]);
    }
    qin[g][k] = v;
  }
  if (tid < P) {
    const int sub = Walsh<LB>::subset(tid);
    double acc = 0.0;
    for (int i = 0; i < K; ++i) {
      const int sg = (__builtin_popcount(i & sub) + __builtin_popcount(sub)) & 1;
      // sigma_S(i) = prod_{p in S} (2 b_p - 1) = (-1)^(|S| - popcount(i & S))
      acc += sg ? -(double)a.centroids[i] : (double)a.centroids[i];
    }
    beta[tid] = acc / K;
  }
  __syncthreads();
  for (int i = tid; i < 4 * D; i += blockDim.x) {
    const int g = i / D, j = i % D;
    const float *row = a.pi + (size_t)j * D;
    double acc = 0.0;
    for (int k = 0; k < D; ++k) acc += (double)row[k] * (double)qin[g][k];
    qr[g][j] = acc;
    if constexpr (PROD) {
      const float *srow = a.s_mat + (size_t)j * D;
      double acc2 = 0.0;
      for (int k = 0; k < D; ++k) acc2 += (double)srow[k] * (double)qin[g][k];
      qs[g][j] = acc2;
    }
  }
  __syncthreads();
  if (tid < 4) {
    const int g = tid;
    double mq = 0.0, sq = 0.0, mqs = 0.0, sqs = 0.0, mb = 0.0, sb = 0.0;
    for (int j = 0; j < D; ++j) {
      mq = fmax(mq, fabs(qr[g][j]));
      sq += qr[g][j];
      if constexpr (PROD) {
        mqs = fmax(mqs, fabs(qs[g][j]));
        sqs += qs[g][j];
      }
    }
    for (int r = 0; r < P; ++r) {
      mb = fmax(mb, fabs(beta[r]));
      sb += beta[r];
    }
    int e1 = 0, e2 = 0;
    if (mq * mb > 0.0) frexp(mq * mb, &e1);
    if (mqs > 0.0) frexp(mqs, &e2);
    const int f1 = 30 - e1, f2 = 30 - e2;
    fexp[g][0] = f1;
    fexp[g][1] = f2;
    const int gg = 4 * rt + g;
    if (gg < a.group) {
      const double kappa = sqrt(M_PI / 2.0) / D;
      float *cst = a.consts + ((int64_t)stream * a.group + gg) * 4;
      cst[0] = (float)ldexp(2.0, -f1);
      cst[1] = (float)(sb * sq);
      cst[2] = PROD ? (float)(ldexp(2.0, -f2) * kappa) : 0.0f;
      cst[3] = PROD ? (float)(kappa * sqs) : 0.0f;
    }
  }
  __syncthreads();
  int8_t *tab = a.table + ((int64_t)stream * a.row_tiles + rt) * (L::NCH * 64 * 16);
  for (int i = tid; i < L::NCH * 64; i += blockDim.x) {
    const int cidx = i / 64, l = i % 64;
    const int row = l & 15, kg = l >> 4;
    const int g = row >> 2, piece = row & 3;
    const int r = cidx / L::CPP, c = cidx % L::CPP;
    const int q = c >> 1, hh = c & 1;
    int8_t out[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int t = e >> 2, ib = e & 3;
      const int j = 32 * (kg + 4 * q) + 8 * ib + 4 * hh + t;
      const int s = 4 * hh + t;
      const bool sign_plane = r >= P;
      const double av = sign_plane ? qs[PROD ? g : 0][j] : beta[r < P ? r : 0] * qr[g][j];
      const int f = fexp[g][sign_plane ? 1 : 0];
      long long n = llrint(ldexp(av, f - s));
      if (s == 7) n = -n;
      long long rem = n;
      int digit = 0;
#pragma unroll
      for (int pc = 0; pc < 4; ++pc) {
        const int dgt = (int)(int8_t)(rem & 0xFF);
        if (pc == piece) digit = dgt;
        rem = (rem - dgt) >> 8;
      }
      out[e] = (4 * rt + g < a.group) ? (int8_t)digit : (int8_t)0;
    }
    int8_t *dst = tab + ((int64_t)cidx * 64 + l) * 16;
#pragma unroll
    for (int e = 0; e < 16; ++e) dst[e] = out[e];
  }
}

struct StreamArgs {
  const int8_t *table;
  const float *consts;
  const uint8_t *codes;
  const uint8_t *signs;
  const uint16_t *norm;
  const uint16_t *rnorm;
  int64_t row_tokens, seq_len, tokens_per_block;
  int n_splits, n_kv_heads, n_q_heads, group, row_tiles;
  float scale;
  float *logits;
};

template <int D, int LB, bool PROD, int RT>
__global__ __launch_bounds__(256) void logit_kernel(StreamArgs a) {
  using L = LLayout<D, LB, PROD>;
  constexpr int P = L::P;
  constexpr int CPP = L::CPP;
  constexpr int NCH = L::NCH;
  constexpr int PB = L::PB;
  constexpr int NQ = D / 128;  // plane dwords per lane group

  int bid = blockIdx.x;
  if ((gridDim.x & 7) == 0) {  // keep a stream's blocks on one XCD (L2)
    const int per = gridDim.x >> 3;
    bid = (bid & 7) * per + (bid >> 3);
  }
  const int stream = bid / a.n_splits;
  const int split = bid % a.n_splits;
  const int b = stream / a.n_kv_heads;
  const int kvh = stream % a.n_kv_heads;
  const int64_t t_begin = (int64_t)split * a.tokens_per_block;
  int64_t t_end = t_begin + a.tokens_per_block;
  if (t_end > a.seq_len) t_end = a.seq_len;
  if (t_begin >= t_end) return;

  const int w = threadIdx.x >> 6;
  const int l = lane_id();
  const int n = l & 15;
  const int kg = l >> 4;

  i32x4 areg[RT][NCH];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const i32x4 *src = (const i32x4 *)(a.table + ((int64_t)stream * a.row_tiles + rt) * (NCH * 64 * 16));
#pragma unroll
    for (int c = 0; c < NCH; ++c) areg[rt][c] = src[c * 64 + l];
  }
  f32x4 cst[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int g = 4 * rt + kg;
    cst[rt] = g < a.group ? *(const f32x4 *)(a.consts + ((int64_t)stream * a.group + g) * 4)
                          : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int64_t key0 = (int64_t)stream * a.row_tokens;
  float *out_base = a.logits + ((int64_t)b * a.n_q_heads + (int64_t)kvh * a.group) * a.seq_len;

  for (int64_t tok0 = t_begin + 16 * w; tok0 < t_end; tok0 += 64) {
    const int64_t tok = tok0 + n;
    const bool valid = tok < t_end;
    const int64_t key = key0 + (valid ? tok : t_end - 1);
    uint32_t wp[LB][NQ];
#pragma unroll
    for (int p = 0; p < LB; ++p)
#pragma unroll
      for (int qd = 0; qd < NQ; ++qd)
        wp[p][qd] = *(const uint32_t *)(a.codes + key * (LB * PB) + p * PB + 4 * (kg + 4 * qd));
    uint32_t ws[NQ];
    float gam = 0.0f;
    if constexpr (PROD) {
#pragma unroll
      for (int qd = 0; qd < NQ; ++qd) ws[qd] = *(const uint32_t *)(a.signs + key * PB + 4 * (kg + 4 * qd));
      gam = f16_bits_to_f32(a.rnorm[key]);
    }
    const float nrm = f16_bits_to_f32(a.norm[key]);

    i32x4 am[RT], aq[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) { am[rt] = i32x4{0, 0, 0, 0}; aq[rt] = i32x4{0, 0, 0, 0}; }
#pragma unroll
    for (int r = 0; r < P; ++r) {
      constexpr int dummy = 0;
      (void)dummy;
      const int sub = Walsh<LB>::subset(r);
      uint32_t wr[NQ];
#pragma unroll
      for (int qd = 0; qd < NQ; ++qd) {
        uint32_t x = 0;
#pragma unroll
        for (int p = 0; p < LB; ++p)
          if (sub & (1 << p)) x ^= wp[p][qd];
        wr[qd] = x;
      }
#pragma unroll
      for (int c = 0; c < CPP; ++c) {
        const uint32_t x = wr[c >> 1];
        const int sh = 4 * (c & 1);
        i32x4 bv = {(int)(x & (0x01010101u << sh)), (int)(x & (0x01010101u << (sh + 1))),
                    (int)(x & (0x01010101u << (sh + 2))), (int)(x & (0x01010101u << (sh + 3)))};
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) am[rt] = mfma_i8(areg[rt][r * CPP + c], bv, am[rt]);
      }
    }
    if constexpr (PROD) {
#pragma unroll
      for (int c = 0; c < CPP; ++c) {
        const uint32_t x = ws[c >> 1];
        const int sh = 4 * (c & 1);
        i32x4 bv = {(int)(x & (0x01010101u << sh)), (int)(x & (0x01010101u << (sh + 1))),
                    (int)(x & (0x01010101u << (sh + 2))), (int)(x & (0x01010101u << (sh + 3)))};
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) aq[rt] = mfma_i8(areg[rt][P * CPP + c], bv, aq[rt]);
      }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int g = 4 * rt + kg;
      const float sm = (((float)am[rt][3] * 256.0f + (float)am[rt][2]) * 256.0f + (float)am[rt][1]) * 256.0f +
                       (float)am[rt][0];
      float v = cst[rt][0] * sm - cst[rt][1];
      if constexpr (PROD) {
        const float sq = (((float)aq[rt][3] * 256.0f + (float)aq[rt][2]) * 256.0f + (float)aq[rt][1]) * 256.0f +
                         (float)aq[rt][0];
        v += gam * (cst[rt][2] * sq - cst[rt][3]);
      }
      if (valid && g < a.group) out_base[(int64_t)g * a.seq_len + tok] = a.scale * nrm * v;
    }
  }
}

template <int D, int LB, bool PROD>
hipError_t launch_t(const tqi::LogitArgs &a, hipStream_t s) {
  using L = LLayout<D, LB, PROD>;
  const int group = a.n_q_heads / a.n_kv_heads;
  const int rts = (group + 3) / 4;
  const int n_streams = a.batch * a.n_kv_heads;
  const size_t table_bytes = (size_t)n_streams * rts * L::NCH * 64 * 16;
  const size_t const_bytes = (size_t)n_streams * group * 4 * sizeof(float);
  void *ws = nullptr;
  hipError_t e = hipMallocAsync(&ws, table_bytes + const_bytes, s);
  if (e != hipSuccess) return e;
  PrepArgs pa;
  pa.q = a.q;
  pa.q_f32 = a.q_f32;
  pa.n_q_heads = a.n_q_heads;
  pa.n_kv_heads = a.n_kv_heads;
  pa.group = group;
  pa.row_tiles = rts;
  pa.pi = a.pi;
  pa.s_mat = a.s_mat;
  pa.centroids = a.centroids;
  pa.table = (int8_t *)ws;
  pa.consts = (float *)((char *)ws + table_bytes);
  hipLaunchKernelGGL((logit_prep_kernel<D, LB, PROD>), dim3(n_streams, rts), dim3(256), 0, s, pa);
  e = hipGetLastError();
  if (e == hipSuccess) {
    StreamArgs sa;
    sa.table = pa.table;
    sa.consts = pa.consts;
    sa.codes = a.codes;
    sa.signs = a.signs;
    sa.norm = a.norm;
    sa.rnorm = a.rnorm;
    sa.row_tokens = a.row_tokens;
    sa.seq_len = a.seq_len;
    sa.n_kv_heads = a.n_kv_heads;
    sa.n_q_heads = a.n_q_heads;
    sa.group = group;
    sa.row_tiles = rts;
    sa.scale = a.scale;
    sa.logits = a.logits;
    const int64_t total = (int64_t)n_streams * a.seq_len;
    const int64_t target_blocks = 4LL * tqi::device_cu_count();
    int64_t tpb = (total + target_blocks - 1) / target_blocks;
    tpb = (tpb + 63) / 64 * 64;
    if (tpb < 256) tpb = 256;
    if (tpb > 16384) tpb = 16384;
    sa.tokens_per_block = tpb;
    sa.n_splits = (int)((a.seq_len + tpb - 1) / tpb);
    const int64_t blocks = (int64_t)n_streams * sa.n_splits;
    switch (rts) {
      case 1: hipLaunchKernelGGL((logit_kernel<D, LB, PROD, 1>), dim3((unsigned)blocks), dim3(256), 0, s, sa); break;
      case 2: hipLaunchKernelGGL((logit_kernel<D, LB, PROD, 2>), dim3((unsigned)blocks), dim3(256), 0, s, sa); break;
      case 3: hipLaunchKernelGGL((logit_kernel<D, LB, PROD, 3>), dim3((unsigned)blocks), dim3(256), 0, s, sa); break;
      default: hipLaunchKernelGGL((logit_kernel<D, LB, PROD, 4>), dim3((unsigned)blocks), dim3(256), 0, s, sa); break;
    }
    e = hipGetLastError();
  }
  hipError_t e2 = hipFreeAsync(ws, s);
  return e != hipSuccess ? e : e2;
}

template <int D, bool PROD>
hipError_t launch_lb(int lb, const tqi::LogitArgs &a, hipStream_t s, bool *ok) {
  *ok = true;
  switch (lb) {
    case 1: return launch_t<D, 1, PROD>(a, s);
    case 2: return launch_t<D, 2, PROD>(a, s);
    case 3: return launch_t<D, 3, PROD>(a, s);
    case 4: return launch_t<D, 4, PROD>(a, s);
  }
  *ok = false;
  return hipSuccess;
}

}  // namespace

namespace tqi {

hipError_t launch_logits(int d, int lbits, bool prod, const LogitArgs &a, hipStream_t s,
                         bool *supported) {
  *supported = false;
  if (a.n_q_heads / a.n_kv_heads > 16) return hipSuccess;
  if (d == 128) return prod ? launch_lb<128, true>(lbits, a, s, supported)
                            : launch_lb<128, false>(lbits, a, s, supported);
  if (d == 256) return prod ? launch_lb<256, true>(lbits, a, s, supported)
                            : launch_lb<256, false>(lbits, a, s, supported);
  return hipSuccess;
}

}  // namespace tqi
