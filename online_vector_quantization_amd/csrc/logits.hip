// Attention logits straight from bit-packed keys.
//
// Page "TurboQuant 설명: 무엇인지와 LLM 메모리 6배 절약 구현 방법", closing
// paragraphs of "2단계: QJL 잔차 보정" and "TurboQuant 구현 방법": the query is
// rotated once and the logits are formed from the compressed indices, never
// reconstructing the keys:
//   logit = scale * n * ( <Pi q, c[idx]> + sqrt(pi/2)/d * gamma * <S q, s> ).
//
// Reformulation used here (exact in real arithmetic):
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
  // decode-time append (x_new == nullptr: none): one new key per stream,
  // written at token pos of the stream's rows
  const void *x_new;       // [stream][D]
  bool x_f32;
  const float *boundaries;
  const float *m_mat;      // M = S Pi^T (PROD)
  uint8_t *codes_out;
  uint16_t *norm_out, *rnorm_out;
  int64_t row_tokens, pos;
  // paged cache (block_table == nullptr: stream s owns rows
  // [s * row_tokens, (s + 1) * row_tokens)): token t of KV head h of
  // sequence b is pool row (block_table[b][t / page_tokens] * n_kv_heads + h)
  // * page_tokens + t % page_tokens
  const int32_t *block_table;
  int page_tokens, max_pages;
  int64_t pool_rows;
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

// K positions of the MFMA chunks.  Lane group kg (lanes 16 kg .. 16 kg + 15)
// of chunk c of a plane holds the 16 coordinates 32 grp + 8 i + 4 hh + t
// (i, t = 0..3) of 32-coordinate group grp, as bit hh 4 + t of byte i of the
// group's plane word.  d >= 128: the four lane groups take four different
// words and the chunk picks the nibble (hh = c & 1, grp = kg + 4 (c >> 1));
// d = 64 (one chunk per plane): lanes kg and kg ^ 1 share word kg >> 1 and
// split its nibbles (hh = kg & 1).
template <int D, int LB, bool PROD>
struct LLayout {
  static constexpr int P = Walsh<LB>::P;
  static constexpr int CPP = D / 64;                    // MFMA chunks per plane
  static constexpr int NCH = (P + (PROD ? 1 : 0)) * CPP;
  static constexpr int PB = D / 8;
  static constexpr bool SPLIT = D == 64;                // lanes split a word's nibbles
  __host__ __device__ static constexpr int half(int c, int kg) { return SPLIT ? (kg & 1) : (c & 1); }
  __host__ __device__ static constexpr int group(int c, int kg) { return SPLIT ? (kg >> 1) : kg + 4 * (c >> 1); }
};

// Query preparation for one (stream, row tile, part): part 0 builds the
// Walsh-plane chunks from q' = Pi q, part 1 the sign chunks from q'' = S q.
// NT threads (512; 256 at d = 64); RL = 2 NT / D consecutive lanes share the
// matrix rows j and j + D/2 and read their 16-byte pieces p, p + RL, ...
// (coalesced), each for all four queries, then combine their partial sums
// with lane permutes.  The fixed-point weights are formed in fp64.
template <int D>
constexpr int prep_threads() { return D >= 128 ? 512 : 256; }

// A partner lane's v for sums over aligned groups of 2, 4 or 8 lanes: the
// quad permutes [1,0,3,2] and [2,3,0,1], then the half-row mirror (lane i of
// 8 with lane 7 - i, which pairs the group's two quads); beyond 8 lanes the
// LDS permute unit (lane ^ off).
__device__ __forceinline__ float xor_lanes(float v, int off) {
  const int b = __float_as_int(v);
  if (off == 1) return __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0xB1, 0xF, 0xF, false));
  if (off == 2) return __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x4E, 0xF, 0xF, false));
  if (off == 4) return __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x141, 0xF, 0xF, false));
  return __shfl_xor(v, off, 64);
}

// One DPP step of the prep's wave reductions: v[0..3] take the maximum with
// the CTRL partner lane, v[4..7] the sum.
template <int CTRL>
__device__ __forceinline__ void wave_fold(float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float o = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v[i]), CTRL, 0xF, 0xF, false));
    v[i] = i < 4 ? fmaxf(v[i], o) : v[i] + o;
  }
}

// Decode-time append: quantise the new key of one stream and write its
// packed row at token pos, inside the prep launch so that the streaming
// kernel that follows reads it (page "TurboQuant 설명 ...": quantisation on
// every cache update, section "TurboQuant 구현 방법"; stage 1 and the QJL
// stage, sections "1단계" and "2단계").  One vector per workgroup, in fp64
// from the fp32 matrices: n = ||x|| (sum of exact squares), u = Pi x / n,
// idx_j = #{k : u_j >= t_k} (ties go up), and in inner-product mode the
// rotated residual r = u - c[idx] (same norm as u - Pi^T c[idx]), gamma =
// ||r||, sign_i = [(M r)_i >= 0]; a zero vector keeps the middle index, all
// signs 1 and gamma = 0.  Rows of Pi and M are read by RL consecutive lanes,
// as in the query projection.
__device__ __forceinline__ double shfl_xor_f64(double v, int off) {
  return __shfl_xor(v, off, 64);
}

template <int D, int LB, bool PROD>
__device__ __forceinline__ void append_key(const PrepArgs &a, int stream) {
  constexpr int NT = prep_threads<D>();
  constexpr int RL = NT / D;                // lanes per matrix row
  constexpr int NP = D / 4 / RL;            // 16-byte pieces per lane
  constexpr int K = 1 << LB;
  constexpr int RBITS = LB + (PROD ? 1 : 0);
  __shared__ __attribute__((aligned(16))) float xs[D];
  __shared__ double rs[D];
  __shared__ int rec[D];
  __shared__ double nrm[2];
  const int tid = threadIdx.x;
  const int j = tid / RL, pl = tid % RL;
  const int l = lane_id();
  const f32x4 *prow = (const f32x4 *)(a.pi + (size_t)j * D);
  if (tid < D) {
    const int64_t off = (int64_t)stream * D + tid;
    xs[tid] = a.x_f32 ? ((const float *)a.x_new)[off] : bf16_to_f32(((const uint16_t *)a.x_new)[off]);
  }
  __syncthreads();
  if (tid < 64) {                           // ||x||^2: exact squares, fp64 sums
    double s2 = 0.0;
    for (int k = l; k < D; k += 64) s2 = fma((double)xs[k], (double)xs[k], s2);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s2 += shfl_xor_f64(s2, off);
    if (l == 0) nrm[0] = sqrt(s2);
  }
  double y = 0.0;
#pragma unroll 4
  for (int i = 0; i < NP; ++i) {
    const int k0 = 4 * (pl + RL * i);
    const f32x4 m4 = prow[pl + RL * i];
#pragma unroll
    for (int e = 0; e < 4; ++e) y = fma((double)m4[e], (double)xs[k0 + e], y);
  }
#pragma unroll
  for (int off = 1; off < RL; off <<= 1) y += shfl_xor_f64(y, off);
  __syncthreads();
  const double n = nrm[0];
  const double u = n > 0.0 ? y / n : 0.0;
  int idx = 0;
#pragma unroll
  for (int k = 0; k < K - 1; ++k) idx += u >= (double)a.boundaries[k] ? 1 : 0;
  if (pl == 0) {
    rec[j] = idx;
    rs[j] = u - (double)a.centroids[idx];
  }
  __syncthreads();
  if constexpr (PROD) {
    if (tid < 64) {
      double g2 = 0.0;
      for (int k = l; k < D; k += 64) g2 = fma(rs[k], rs[k], g2);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) g2 += shfl_xor_f64(g2, off);
      if (l == 0) nrm[1] = sqrt(g2);
    }
    const f32x4 *mrow = (const f32x4 *)(a.m_mat + (size_t)j * D);
    double z = 0.0;
#pragma unroll 4
    for (int i = 0; i < NP; ++i) {
      const int k0 = 4 * (pl + RL * i);
      const f32x4 m4 = mrow[pl + RL * i];
#pragma unroll
      for (int e = 0; e < 4; ++e) z = fma((double)m4[e], rs[k0 + e], z);
    }
#pragma unroll
    for (int off = 1; off < RL; off <<= 1) z += shfl_xor_f64(z, off);
    if (pl == 0 && (n == 0.0 || z >= 0.0)) rec[j] |= 1 << LB;
    __syncthreads();
  }
  // bit planes: word p of group g holds bit p of the records 32 g .. 32 g + 31
  int64_t row = (int64_t)stream * a.row_tokens + a.pos;
  if (a.block_table != nullptr) {   // paged: the row of token pos; no write where its page is not in the pool
    const int b = stream / a.n_kv_heads, kvh = stream % a.n_kv_heads;
    const int64_t pg = a.block_table[(int64_t)b * a.max_pages + a.pos / a.page_tokens];
    row = (pg * a.n_kv_heads + kvh) * a.page_tokens + a.pos % a.page_tokens;
    if (pg < 0 || row >= a.pool_rows) return;      // uniform over the workgroup
  }
  if (tid < (D / 32) * RBITS) {
    const int g = tid / RBITS, p = tid % RBITS;
    uint32_t word = 0;
#pragma unroll 8
    for (int i = 0; i < 32; ++i) word |= (uint32_t)((rec[32 * g + i] >> p) & 1) << i;
    ((uint32_t *)(a.codes_out + row * (RBITS * D / 8)))[tid] = word;
  }
  if (tid == 0) {
    a.norm_out[row] = f64_to_f16_bits(n);
    if constexpr (PROD) a.rnorm_out[row] = f64_to_f16_bits(n > 0.0 ? nrm[1] : 0.0);
  }
}

template <int D, int LB, bool PROD>
__global__ __launch_bounds__(prep_threads<D>()) void logit_prep_kernel(PrepArgs a) {
  using L = LLayout<D, LB, PROD>;
  constexpr int K = 1 << LB;
  constexpr int P = L::P;
  constexpr int NT = prep_threads<D>();
  constexpr int RL = 2 * NT / D;            // lanes per pair of matrix rows (j, j + D/2)
  constexpr int NP = D / 4 / RL;            // 16-byte pieces per lane and row
  constexpr int NW = NT / 64;               // waves
  static_assert(RL >= 2 && RL <= 8 && NP >= 1, "prep layout");
  __shared__ __attribute__((aligned(16))) float qin[4][D];
  __shared__ float proj[4][D];
  __shared__ double beta[P];
  __shared__ __attribute__((aligned(16))) float red_max[4][NW], red_sum[4][NW];

  const int stream = blockIdx.x;
  const int rt = blockIdx.y;
  const int part = blockIdx.z;              // 0: MSE planes, 1: QJL signs, last: append
  if (part == (PROD ? 2 : 1)) {             // uniform over the workgroup
    if (rt == 0) append_key<D, LB, PROD>(a, stream);
    return;
  }
  const int b = stream / a.n_kv_heads;
  const int kvh = stream % a.n_kv_heads;
  const int tid = threadIdx.x;
  const int j = tid / RL;                   // rows j and j + D/2: each staged
  const int pl = tid % RL;                  // query read feeds two rows

  const float *mat = part == 0 ? a.pi : a.s_mat;
  const f32x4 *mrow0 = (const f32x4 *)(mat + (size_t)j * D);
  const f32x4 *mrow1 = (const f32x4 *)(mat + (size_t)(j + D / 2) * D);
  // d <= 128: the whole row slices are loaded before the first barrier;
  // larger d streams them inside the loop (register budget)
  constexpr int PRE = D <= 128 ? NP : 1;
  f32x4 row0[PRE], row1[PRE];
#pragma unroll
  for (int i = 0; i < PRE; ++i) {
    row0[i] = mrow0[pl + RL * i];
    row1[i] = mrow1[pl + RL * i];
  }

  for (int i = tid; i < 4 * D; i += NT) {
    const int g = i / D, k = i % D;
    const int gg = 4 * rt + g;
    float v = 0.0f;
    if (gg < a.group) {
      const int64_t off = ((int64_t)b * a.n_q_heads + (int64_t)kvh * a.group + gg) * D + k;
      v = a.q_f32 ? ((const float *)a.q)[off] : bf16_to_f32(((const uint16_t *)a.q)[off]);
    }
    qin[g][k] = v;
  }
  if (part == 0 && tid < P) {
    const int sub = Walsh<LB>::subset(tid);
    double acc = 0.0;
    for (int i = 0; i < K; ++i) {
      // sigma_S(i) = prod_{p in S} (2 b_p - 1) = (-1)^(|S| - popcount(i & S))
      const int sg = (__builtin_popcount(i & sub) + __builtin_popcount(sub)) & 1;
      acc += sg ? -(double)a.centroids[i] : (double)a.centroids[i];
    }
    beta[tid] = acc / K;
  }
  __syncthreads();
  // fp32 accumulation: the products are exact and the sums' rounding
  // (~1e-7 relative) is far below the logit tolerance.
  float acc0[4] = {0.0f, 0.0f, 0.0f, 0.0f}, acc1[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll (D <= 128 ? NP : 4)
  for (int i = 0; i < NP; ++i) {
    const int k0 = 4 * (pl + RL * i);
    const f32x4 m0 = D <= 128 ? row0[i < PRE ? i : 0] : mrow0[pl + RL * i];
    const f32x4 m1 = D <= 128 ? row1[i < PRE ? i : 0] : mrow1[pl + RL * i];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 qv = *(const f32x4 *)&qin[g][k0];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc0[g] = fmaf(m0[e], qv[e], acc0[g]);
        acc1[g] = fmaf(m1[e], qv[e], acc1[g]);
      }
    }
  }
  // full row sums in every lane of the row (quad permutes for the lanes of a
  // row), then max |.| and sum over the rows of this wave: the eight values
  // interleaved through DPP steps within rows of 16 lanes and four
  // readlanes (no LDS permutes); then every thread folds the waves' results
  // after one barrier
  float v[8];                               // max |q'_j| (g), sum q'_j (4 + g)
#pragma unroll
  for (int g = 0; g < 4; ++g) {
#pragma unroll
    for (int off = 1; off < RL; off <<= 1) {
      acc0[g] += xor_lanes(acc0[g], off);
      acc1[g] += xor_lanes(acc1[g], off);
    }
    if (pl == 0) {
      proj[g][j] = acc0[g];
      proj[g][j + D / 2] = acc1[g];
    }
    v[g] = fmaxf(fabsf(acc0[g]), fabsf(acc1[g]));
    v[4 + g] = pl == 0 ? acc0[g] + acc1[g] : 0.0f;
  }
  wave_fold<0xB1>(v);
  wave_fold<0x4E>(v);
  wave_fold<0x124>(v);
  wave_fold<0x128>(v);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int m = __float_as_int(v[g]), q = __float_as_int(v[4 + g]);
    v[g] = fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(m, 0)), __int_as_float(__builtin_amdgcn_readlane(m, 16))),
                 fmaxf(__int_as_float(__builtin_amdgcn_readlane(m, 32)), __int_as_float(__builtin_amdgcn_readlane(m, 48))));
    v[4 + g] = (__int_as_float(__builtin_amdgcn_readlane(q, 0)) + __int_as_float(__builtin_amdgcn_readlane(q, 16))) +
               (__int_as_float(__builtin_amdgcn_readlane(q, 32)) + __int_as_float(__builtin_amdgcn_readlane(q, 48)));
  }
  if ((tid & 63) == 0) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      red_max[g][tid >> 6] = v[g];
      red_sum[g][tid >> 6] = v[4 + g];
    }
  }
  __syncthreads();
  double mb = 0.0, sb = 0.0;
  if (part == 0) {
    for (int r = 0; r < P; ++r) {
      mb = fmax(mb, fabs(beta[r]));
      sb += beta[r];
    }
  }
  int fexp[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float mqf = red_max[g][0], sqf = red_sum[g][0];
#pragma unroll
    for (int wv = 1; wv < NW; ++wv) {
      mqf = fmaxf(mqf, red_max[g][wv]);
      sqf += red_sum[g][wv];
    }
    const double mq = mqf, sq = sqf;
    const double top = part == 0 ? mq * mb : mq;
    int e = 0;
    if (top > 0.0) frexp(top, &e);
    fexp[g] = 30 - e;               // largest weight * 2^F < 2^30
    const int gg = 4 * rt + g;
    if (tid == 0 && gg < a.group) {
      const double kappa = sqrt(M_PI / 2.0) / D;
      float *cst = a.consts + ((int64_t)stream * a.group + gg) * 4;
      if (part == 0) {
        cst[0] = (float)ldexp(2.0, -fexp[g]);
        cst[1] = (float)(sb * sq);
        if (!PROD) {
          cst[2] = 0.0f;
          cst[3] = 0.0f;
        }
      } else {
        cst[2] = (float)(ldexp(2.0, -fexp[g]) * kappa);
        cst[3] = (float)(kappa * sq);
      }
    }
  }
  // A-operand chunks of this part.  Lane l = 16 kg + 4 g + piece supplies
  // row (query g, byte piece); its byte e = 4 t + i pairs with coordinate
  // 32 grp + 8 i + 4 hh + t (LLayout), whose key byte carries weight
  // 2^(4 hh + t) (see the kernel comment).  One thread per (chunk, kg, g, t) computes
  // the 32-bit fixed-point weights of bytes 4 t .. 4 t + 3 and writes word t
  // of the four piece rows.
  int8_t *tab = a.table + ((int64_t)stream * a.row_tiles + rt) * (L::NCH * 64 * 16);
  const int c_begin = part == 0 ? 0 : P * L::CPP;
  const int c_end = part == 0 ? P * L::CPP : L::NCH;
  for (int i = c_begin * 64 + tid; i < c_end * 64; i += NT) {
    const int cidx = i / 64, kg = (i >> 4) & 3, g = (i >> 2) & 3, t = i & 3;
    const int r = cidx / L::CPP, c = cidx % L::CPP;
    const int hh = L::half(c, kg), grp = L::group(c, kg);
    const double wgt = part == 0 ? beta[r < P ? r : 0] : 1.0;
    const bool live = 4 * rt + g < a.group;
    const int s = 4 * hh + t;
    uint32_t e[4];                           // [ib]: the four digits of weight ib
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      const int j = 32 * grp + 8 * ib + 4 * hh + t;
      int n = (int)rint(ldexp(wgt * (double)proj[g][j], fexp[g] - s));
      if (s == 7) n = -n;
      if (!live) n = 0;
      // balanced signed-byte digits n = sum_p d_p 256^p, d_p in [-128, 127]
      // (|n| <= 2^30): the bytes of n + 0x80808080 are the d_p + 128, with
      // no carries, so those of (n + 0x80808080) ^ 0x80808080 are the d_p
      e[ib] = ((uint32_t)n + 0x80808080u) ^ 0x80808080u;
    }
    uint32_t words[4];                       // [piece]: digit piece of the four weights
#pragma unroll
    for (int pc = 0; pc < 4; ++pc)
      words[pc] = ((e[0] >> (8 * pc)) & 0xFFu) | (((e[1] >> (8 * pc)) & 0xFFu) << 8) |
                  (((e[2] >> (8 * pc)) & 0xFFu) << 16) | (((e[3] >> (8 * pc)) & 0xFFu) << 24);
#pragma unroll
    for (int pc = 0; pc < 4; ++pc) {
      const int l = 16 * kg + 4 * g + pc;
      *(uint32_t *)(tab + ((int64_t)cidx * 64 + l) * 16 + 4 * t) = words[pc];
    }
  }
}

struct StreamArgs {
  const int8_t *table;
  const float *consts;
  const uint8_t *codes;
  const uint16_t *norm;
  const uint16_t *rnorm;
  int64_t row_tokens, seq_len;
  int n_splits;   // blocks per stream; block j takes chunks j, j + n_splits, ...
  int n_kv_heads, n_q_heads, group, row_tiles;
  float scale;
  float *logits;
  // paged cache (PAGED kernels only): see PrepArgs
  const int32_t *block_table;
  int page_tokens, max_pages;
  int64_t pool_rows;
};

constexpr int kLogitGroups = 4;        // 16-token groups per wave and loop iteration
constexpr int kLogitBlocksPerCu = 8;   // streaming workgroups per CU the launch aims for
// The logits leave with the default (write-back) policy: L2 then writes whole
// lines back (measured 3% faster than the non-temporal policy at 8.4 M keys).
constexpr int kWriteBack = 0;


// Registers of one 16-token group as loaded by one lane: the plane words of
// its 32-coordinate group(s); in inner-product mode the last word of each
// group is the sign plane.
template <int NPL, int NQ>
struct KeyGroup {
  uint32_t w[NQ][NPL];
};

// fp16 norm and residual norm of 64 consecutive tokens, one token per lane.
// Kept apart until they are consumed, so no instruction touches a load
// result before the loop has moved on to computing.
struct NormBlock {
  uint32_t n, g;
};

template <int D, int LB, bool PROD, int RT, bool PAGED>
__global__ __launch_bounds__(256) void logit_kernel(StreamArgs a) {
  using L = LLayout<D, LB, PROD>;
  constexpr int P = L::P;
  constexpr int CPP = L::CPP;
  constexpr int NCH = L::NCH;
  constexpr int PB = L::PB;
  constexpr int NPL = LB + (PROD ? 1 : 0);  // planes per record (sign on top)
  constexpr int RB = NPL * PB;              // bytes per packed row
  constexpr int NQ = D >= 128 ? D / 128 : 1;   // plane words per lane and plane
  constexpr int U = kLogitGroups;     // 16-token groups per wave and iteration
  constexpr int NB = U / 4;              // 64-token norm blocks per iteration
  static_assert(U % 4 == 0, "groups come in fours (64 tokens)");
  __shared__ __attribute__((aligned(16))) float stage[4][4 * RT][16 * U];

  int bid = blockIdx.x;
  if ((gridDim.x & 7) == 0) {  // keep a stream's blocks on one XCD (L2)
    const int per = gridDim.x >> 3;
    bid = (bid & 7) * per + (bid >> 3);
  }
  const int stream = bid / a.n_splits;
  const int split = bid % a.n_splits;
  const int b = stream / a.n_kv_heads;
  const int kvh = stream % a.n_kv_heads;

  const int w = threadIdx.x >> 6;
  const int l = lane_id();
  const int n = l & 15;
  const int kg = l >> 4;
  // byte masks of the four B dwords at d = 64, where the nibble is per lane
  const uint32_t msplit = 0x01010101u << (4 * L::half(0, kg));

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

  // Buffer resources: SGPR bases, 32-bit per-lane offsets.  Contiguous
  // streams: the ranges end at seq_len, so loads of tokens past the stream
  // read zeros.  Paged: the ranges cover the pool; tokens past seq_len read
  // whatever rows their page holds (their logits are never stored), and a
  // page outside the pool reads zeros.  Stores past seq_len are dropped.
  const int64_t key0 = PAGED ? 0 : (int64_t)stream * a.row_tokens;
  const uint32_t nvalid = (uint32_t)a.seq_len;
  const uint32_t nrows = PAGED ? (uint32_t)a.pool_rows : nvalid;
  const i32x4 rc = make_rsrc(a.codes + key0 * RB, nrows * RB);
  const i32x4 rn = make_rsrc(a.norm + key0, nrows * 2);
  const i32x4 rg = make_rsrc(PROD ? a.rnorm + key0 : a.norm, PROD ? nrows * 2 : 0u);
  // this sequence's block-table row, read with scalar loads (entries past
  // the row read 0 through the range check)
  const i32x4 rbt = make_rsrc(PAGED ? a.block_table + (int64_t)b * a.max_pages : a.block_table,
                              PAGED ? (uint32_t)a.max_pages * 4 : 0u);
  const i32x4 ro = make_rsrc(a.logits + ((int64_t)b * a.n_q_heads + (int64_t)kvh * a.group) * a.seq_len,
                             (uint32_t)(a.group * a.seq_len * 4));
  const uint32_t t_end32 = nvalid;

  // Lane (n, kg) reads, for token n of each group, the NPL plane words of
  // its 32-coordinate group of chunk pair qd (one contiguous load: 16 bytes
  // at b = 4); lane l reads the two fp16 scalars of token l of each 64-token
  // block.
  auto load = [&](uint32_t tok0, KeyGroup<NPL, NQ>(&kgp)[U], NormBlock(&nb)[NB]) {
    // first row of the wave's 64 tokens (one page holds all of them)
    uint32_t row0 = tok0;
    if constexpr (PAGED) {
      const int pg = tq_llvm_s_buf_ld_b32(rbt, (int)(4 * (tok0 / (uint32_t)a.page_tokens)), 0);
      const uint64_t r = ((uint64_t)(uint32_t)pg * (uint32_t)a.n_kv_heads + (uint32_t)kvh) * (uint32_t)a.page_tokens +
                         tok0 % (uint32_t)a.page_tokens;
      row0 = (pg >= 0 && r < (uint64_t)a.pool_rows) ? (uint32_t)r : (uint32_t)a.pool_rows;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t tok = row0 + 16 * u + n;
#pragma unroll
      for (int qd = 0; qd < NQ; ++qd)
        buf_load_words<NPL>(rc, tok * RB + 4 * NPL * L::group(2 * qd, kg), kgp[u].w[qd]);
    }
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const uint32_t tok = row0 + 64 * q + l;
      nb[q].n = buf_load_u16(rn, 2 * tok);
      if constexpr (PROD) nb[q].g = buf_load_u16(rg, 2 * tok);
    }
  };

  // B operand of chunk c from a plane word: dword t keeps bit 4 hh + t of
  // each byte (byte value 2^(4 hh + t) * bit)
  auto expand = [&](uint32_t x, int c) -> i32x4 {
    if constexpr (L::SPLIT) {
      return {(int)(x & msplit), (int)(x & (msplit << 1)), (int)(x & (msplit << 2)), (int)(x & (msplit << 3))};
    } else {
      const int sh = 4 * (c & 1);
      return {(int)(x & (0x01010101u << sh)), (int)(x & (0x01010101u << (sh + 1))),
              (int)(x & (0x01010101u << (sh + 2))), (int)(x & (0x01010101u << (sh + 3)))};
    }
  };

  auto compute = [&](uint32_t tok0, const KeyGroup<NPL, NQ>(&kgp)[U], const NormBlock(&nb)[NB]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      i32x4 am[RT], aq[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) { am[rt] = i32x4{0, 0, 0, 0}; aq[rt] = i32x4{0, 0, 0, 0}; }
#pragma unroll
      for (int r = 0; r < P; ++r) {
        const int sub = Walsh<LB>::subset(r);
#pragma unroll
        for (int c = 0; c < CPP; ++c) {
          uint32_t x = 0;
#pragma unroll
          for (int p = 0; p < LB; ++p)
            if (sub & (1 << p)) x ^= kgp[u].w[c >> 1][p];
          const i32x4 bv = expand(x, c);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) am[rt] = mfma_i8(areg[rt][r * CPP + c], bv, am[rt]);
        }
      }
      if constexpr (PROD) {
#pragma unroll
        for (int c = 0; c < CPP; ++c) {
          const i32x4 bv = expand(kgp[u].w[c >> 1][LB], c);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) aq[rt] = mfma_i8(areg[rt][P * CPP + c], bv, aq[rt]);
        }
      }
      // scalars of token 16u + n live in lane 16 (u % 4) + n of block u / 4
      const int src = 16 * (u & 3) + n;
      const float nrm = a.scale * f16_bits_to_f32((uint16_t)__shfl((int)nb[u >> 2].n, src, 64));
      const float gam = PROD ? f16_bits_to_f32((uint16_t)__shfl((int)nb[u >> 2].g, src, 64)) : 0.0f;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float sm = (((float)am[rt][3] * 256.0f + (float)am[rt][2]) * 256.0f + (float)am[rt][1]) * 256.0f +
                         (float)am[rt][0];
        float v = cst[rt][0] * sm - cst[rt][1];
        if constexpr (PROD) {
          const float sq = (((float)aq[rt][3] * 256.0f + (float)aq[rt][2]) * 256.0f + (float)aq[rt][1]) * 256.0f +
                           (float)aq[rt][0];
          v += gam * (cst[rt][2] * sq - cst[rt][3]);
        }
        stage[w][4 * rt + kg][16 * u + n] = nrm * v;
      }
    }
    // Each lane stores 4 consecutive logits of one query: one 16-byte store,
    // plus three 4-byte stores that only the lane straddling the end of the
    // sequence uses (its first 1-3 tokens).  Every other unused store gets an
    // out-of-range offset and is dropped, so the same stores are issued on
    // every path: the compiler then waits for the next iteration's loads
    // without also waiting for these stores.
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
      for (int c = 0; c < U / 4; ++c) {
        const int g = 4 * rt + kg;
        const uint32_t t4 = 4 * n + 64 * c;          // token offset within the iteration
        const f32x4 v = *(const f32x4 *)&stage[w][4 * rt + kg][t4];
        const uint32_t tok = tok0 + t4;
        const uint32_t off = 4u * ((uint32_t)g * nvalid + tok);
        const bool live = g < a.group;
        const bool all4 = tok + 3 < t_end32;
        buf_store_f32x4<kWriteBack>(ro, live && all4 ? off : kNoStore, v);
#pragma unroll
        for (int e = 0; e < 3; ++e)
          buf_store_f32<kWriteBack>(ro, (live && !all4 && tok + e < t_end32) ? off + 4 * e : kNoStore, v[e]);
      }
    }
  };

  // The blocks of a stream take its chunks of 4 x 16U tokens round-robin
  // (block j: chunks j, j + n_splits, ...), so the blocks running at any
  // moment stream through adjacent memory instead of n_splits distant
  // ranges in lockstep.  Wave w of a block takes the w-th 16U tokens of each
  // chunk.  Loop bounds are wave-uniform (scalar).
  const uint32_t stride = 4 * 16 * U * (uint32_t)a.n_splits;
  uint32_t base = (uint32_t)__builtin_amdgcn_readfirstlane((int)(16 * U * (4 * split + w)));
  // Ping-pong over two register sets: the next iteration's loads are issued
  // before the current one is consumed.  The scheduling barriers keep each
  // prefetch ahead of the compute that hides its latency.
  KeyGroup<NPL, NQ> bufa[U], bufb[U];
  NormBlock na[NB], nbb[NB];
  load(base, bufa, na);
  // Range-dropped stores: on entry, as on every later iteration, stores
  // follow the pending loads, so the first wait counts them too (the
  // compiler merges the counts of both paths into the loop).
#pragma unroll
  for (int i = 0; i < RT * U; ++i) buf_store_f32<kWriteBack>(ro, kNoStore + 4 * i, 0.0f);
  while (base < t_end32) {
    load(base + stride, bufb, nbb);
    __builtin_amdgcn_sched_barrier(0);
    compute(base, bufa, na);
    base += stride;
    if (base >= t_end32) break;
    load(base + stride, bufa, na);
    __builtin_amdgcn_sched_barrier(0);
    compute(base, bufb, nbb);
    base += stride;
  }
}

template <int D, int LB, bool PROD>
hipError_t launch_t(const tqi::LogitArgs &a, hipStream_t s) {
  using L = LLayout<D, LB, PROD>;
  const int group = a.n_q_heads / a.n_kv_heads;
  const int rts = (group + 3) / 4;
  const int n_streams = a.batch * a.n_kv_heads;
  const size_t table_bytes = (size_t)n_streams * rts * L::NCH * 64 * 16;
  // query tables and constants live in the caller's workspace; without it
  // nothing is launched
  if (a.workspace == nullptr ||
      a.workspace_bytes < tqi::logits_workspace_bytes(D, LB, PROD, n_streams, group))
    return hipErrorInvalidValue;
  void *ws = a.workspace;
  hipError_t e = hipSuccess;
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
  pa.consts = (float *)((char *)ws + tqi::ws_align(table_bytes));
  pa.x_new = a.x_new;
  pa.x_f32 = a.x_f32;
  pa.boundaries = a.boundaries;
  pa.m_mat = a.m_mat;
  pa.codes_out = a.codes_out;
  pa.norm_out = a.norm_out;
  pa.rnorm_out = a.rnorm_out;
  pa.row_tokens = a.row_tokens;
  pa.pos = a.pos;
  pa.block_table = a.block_table;
  pa.page_tokens = a.page_tokens;
  pa.max_pages = a.max_pages;
  pa.pool_rows = a.pool_rows;
  const int parts = (PROD ? 2 : 1) + (a.x_new != nullptr ? 1 : 0);
  if (a.run_prep) {
    hipLaunchKernelGGL((logit_prep_kernel<D, LB, PROD>), dim3(n_streams, rts, parts),
                       dim3(prep_threads<D>()), 0,
                       s, pa);
    e = hipGetLastError();
  }
  if (e == hipSuccess && a.run_stream) {
    StreamArgs sa;
    sa.table = pa.table;
    sa.consts = pa.consts;
    sa.codes = a.codes;
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
    const int64_t target_blocks = (int64_t)kLogitBlocksPerCu * tqi::device_cu_count();
    const int64_t n_chunks = (a.seq_len + 4 * 16 * kLogitGroups - 1) / (4 * 16 * kLogitGroups);
    int64_t splits = (target_blocks + n_streams - 1) / n_streams;
    if (splits > n_chunks) splits = n_chunks;
    if (splits < 1) splits = 1;
    sa.n_splits = (int)splits;
    const int64_t blocks = (int64_t)n_streams * sa.n_splits;
    sa.block_table = a.block_table;
    sa.page_tokens = a.page_tokens;
    sa.max_pages = a.max_pages;
    sa.pool_rows = a.pool_rows;
    if (a.block_table != nullptr) {
      switch (rts) {
        case 1: hipLaunchKernelGGL((logit_kernel<D, LB, PROD, 1, true>), dim3((unsigned)blocks), dim3(256), 0, s, sa); break;
        case 2: hipLaunchKernelGGL((logit_kernel<D, LB, PROD, 2, true>), dim3((unsigned)blocks), dim3(256), 0, s, sa); break;
        case 3: hipLaunchKernelGGL((logit_kernel<D, LB, PROD, 3, true>), dim3((unsigned)blocks), dim3(256), 0, s, sa); break;
        default: hipLaunchKernelGGL((logit_kernel<D, LB, PROD, 4, true>), dim3((unsigned)blocks), dim3(256), 0, s, sa); break;
      }
    } else {
      switch (rts) {
        case 1: hipLaunchKernelGGL((logit_kernel<D, LB, PROD, 1, false>), dim3((unsigned)blocks), dim3(256), 0, s, sa); break;
        case 2: hipLaunchKernelGGL((logit_kernel<D, LB, PROD, 2, false>), dim3((unsigned)blocks), dim3(256), 0, s, sa); break;
        case 3: hipLaunchKernelGGL((logit_kernel<D, LB, PROD, 3, false>), dim3((unsigned)blocks), dim3(256), 0, s, sa); break;
        default: hipLaunchKernelGGL((logit_kernel<D, LB, PROD, 4, false>), dim3((unsigned)blocks), dim3(256), 0, s, sa); break;
      }
    }
    e = hipGetLastError();
  }
  return e;
}

template <int D, bool PROD>
hipError_t launch_lb(int lb, const tqi::LogitArgs &a, hipStream_t s) {
  switch (lb) {
    case 1: return launch_t<D, 1, PROD>(a, s);
    case 2: return launch_t<D, 2, PROD>(a, s);
    case 3: return launch_t<D, 3, PROD>(a, s);
    case 4: return launch_t<D, 4, PROD>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

namespace tqi {

bool logits_supported(int d, int lbits, bool prod, int group, int64_t seq_len) {
  if (d != 64 && d != 128 && d != 256) return false;
  if (lbits < 1 || lbits > 4 || group < 1 || group > 16) return false;
  // The streaming kernel addresses one stream's codes with 32-bit byte
  // offsets, and its prefetch runs up to one block stride (<= seq_len + 255
  // tokens) past the end, which must not wrap.  Its logit stores drop
  // lanes through the offset 2^31 (kNoStore), so the logits of one stream
  // (group x seq_len fp32) must stay below 2^31 bytes.
  if ((2 * seq_len + 256) * (int64_t)((lbits + (prod ? 1 : 0)) * d / 8) >= (1LL << 32)) return false;
  if ((int64_t)group * seq_len * 4 >= (1LL << 31)) return false;
  return true;
}

size_t logits_workspace_bytes(int d, int lbits, bool prod, int64_t n_streams, int group) {
  const int64_t rts = (group + 3) / 4;
  const int64_t nch = ((1 << (lbits - 1)) + (prod ? 1 : 0)) * (d / 64);
  const size_t table = (size_t)(n_streams * rts * nch * 64 * 16);
  return ws_align(table) + ws_align((size_t)n_streams * group * 4 * sizeof(float));
}

hipError_t launch_logits(int d, int lbits, bool prod, const LogitArgs &a, hipStream_t s) {
  if (d == 64) return prod ? launch_lb<64, true>(lbits, a, s) : launch_lb<64, false>(lbits, a, s);
  if (d == 128) return prod ? launch_lb<128, true>(lbits, a, s) : launch_lb<128, false>(lbits, a, s);
  if (d == 256) return prod ? launch_lb<256, true>(lbits, a, s) : launch_lb<256, false>(lbits, a, s);
  return hipErrorInvalidValue;
}

}  // namespace tqi
