// Decode attention output from packed MSE-mode values.
//
// Page "TurboQuant 설명: 무엇인지와 LLM 메모리 6배 절약 구현 방법": the KV cache
// holds the key and the value vectors (section "TurboQuant란 무엇인가요?") and
// attention runs from the compressed indices without a full dequantisation
// (section "2단계: QJL 잔차 보정", closing paragraph).  The output of query head
// h is o = sum_t p_t v_hat_t, p = softmax(l_h) over the valid tokens, with
// v_hat_t = n_t Pi^T c[idx_t].  Since Pi^T is linear it is applied once per
// query: o = Pi^T (sum_t e_t n_t c[idx_t]) / sum_t e_t, e_t = exp(l_t - max l).
//
// Design (gfx950):
// * partial kernel: a workgroup owns one split of one (batch, KV head) stream
//   and all G query heads of that KV head.  Each wave walks 64-token chunks
//   with a running softmax: lane t loads token t's packed row, norm and
//   logits (the next chunk's loads fly during this chunk's work), the wave
//   takes the chunk maximum per head, rescales what it holds when the
//   maximum rises, and stages the token's plane words and weights e n in LDS,
//   transposed so that one 16-byte read gives four tokens.  Every lane then
//   accumulates its coordinate pairs (one pair for d = 128, two for 256; at
//   d = 64 one pair over half the chunk's tokens, the two halves summed at
//   the end) over the chunk; a pair's two centroid values come from one read
//   of a K^2-entry table.  The waves meet at the end and leave (max, sum e,
//   accumulator) per head and split.
// * combine kernel: one workgroup per query head rescales the splits to the
//   common maximum, divides by the total weight and applies Pi^T; every load
//   it needs is issued before its first barrier.
// The call reads the packed values (b d / 8 + 2 B per token) and the logits
// (4 B per token and head) once.  The accumulation costs G fused multiply-adds
// per value coordinate and head on the vector ALUs, which bounds it before
// HBM does for G >= 4 heads per KV head.
#include <cfloat>
#include <mutex>

#include "tq_device.h"
#include "tq_internal.h"

namespace {

using namespace tqd;

constexpr int kAttWaves = 4;         // waves per split workgroup
constexpr int kAttBlocksPerCu = 2;   // split workgroups per CU the launch aims for
constexpr int kAttThreads = 64 * kAttWaves;
constexpr int kChunk = 64;          // tokens per wave step (one per lane)

struct PartArgs {
  const float *logits;      // [batch][n_q_heads][seq_len]
  const uint8_t *codes;
  const uint16_t *norm;
  const float *centroids;
  int64_t row_tokens, seq_len, tokens_per_split;
  int n_splits, n_kv_heads, n_q_heads, group;
  float *part;              // [stream][split][G][D + 2]: max, sum e, accumulator
};

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float lane_of(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Maxima (sums) over the wave of N values at once, every lane gets them: DPP
// steps within rows of 16 lanes (quad permutes, row rotations by 4 and 8),
// then the four row results read as scalars.  The N reductions are
// interleaved so their latencies overlap; nothing goes through LDS.
template <int N>
__device__ __forceinline__ void wave_max_n(float (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], dpp<0xB1>(v[i]));
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], dpp<0x4E>(v[i]));
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], dpp<0x124>(v[i]));
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], dpp<0x128>(v[i]));
#pragma unroll
  for (int i = 0; i < N; ++i)
    v[i] = fmaxf(fmaxf(lane_of(v[i], 0), lane_of(v[i], 16)), fmaxf(lane_of(v[i], 32), lane_of(v[i], 48)));
}

template <int N>
__device__ __forceinline__ void wave_sum_n(float (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp<0xB1>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp<0x4E>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp<0x124>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp<0x128>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = (lane_of(v[i], 0) + lane_of(v[i], 16)) + (lane_of(v[i], 32) + lane_of(v[i], 48));
}

__device__ __forceinline__ float wave_max(float v) {
  float a[1] = {v};
  wave_max_n(a);
  return a[0];
}

__device__ __forceinline__ float wave_sum(float v) {
  float a[1] = {v};
  wave_sum_n(a);
  return a[0];
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One token's packed row (RW words): 16-byte loads when the row is a whole
// number of them, else (d = 64 at an odd bit width) 4- to 12-byte loads.
template <int RW>
__device__ __forceinline__ void load_row(i32x4 rc, uint32_t off, uint32_t (&out)[RW]) {
  if constexpr (RW % 4 == 0) {
#pragma unroll
    for (int i = 0; i < RW / 4; ++i) {
      const i32x4 v = tq_llvm_buf_ld_b128(rc, (int)(off + 16 * i), 0, 0);
#pragma unroll
      for (int k = 0; k < 4; ++k) out[4 * i + k] = (uint32_t)v[k];
    }
  } else {
    buf_load_words<RW, 0>(rc, off, out);
  }
}

template <int D, int LB, int G>
__global__ __launch_bounds__(kAttThreads) void attend_partial_kernel(PartArgs a) {
  constexpr int K = 1 << LB;
  constexpr int RB = LB * D / 8;          // packed bytes per token
  constexpr int RW = RB / 4;              // ... in words
  // d >= 128: every lane owns D / 64 coordinates and takes all the chunk's
  // tokens; d = 64: lanes l and l + 32 own the same two coordinates and take
  // the first and the second half of the chunk's tokens
  constexpr int TH = D == 64 ? 2 : 1;     // token halves
  constexpr int CPL = TH * D / 64;        // coordinates per lane (2 or 4)
  constexpr int NW = kAttThreads / 64;
  constexpr int CS = kChunk + 4;          // row stride of the transposed stage (words), padded against conflicts
  static_assert(RB % 4 == 0 && CPL % 2 == 0 && CPL * 64 == TH * D, "layout");
  __shared__ float2 ptab[K * K];          // (c[i0], c[i1]) of a coordinate pair
  __shared__ __attribute__((aligned(16))) uint32_t cwt[NW][RW][CS];   // [word][token]
  __shared__ __attribute__((aligned(16))) float wtt[NW][G][CS];       // [head][token]
  __shared__ float redm[NW][G];
  __shared__ float reds[NW][G];
  __shared__ float accs[G][D];

  const int split = blockIdx.x % a.n_splits;
  const int stream = blockIdx.x / a.n_splits;
  const int b = stream / a.n_kv_heads;
  const int kvh = stream % a.n_kv_heads;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = lane_id();

  const int64_t t_begin = (int64_t)split * a.tokens_per_split;
  int64_t t_end = t_begin + a.tokens_per_split;
  if (t_end > a.seq_len) t_end = a.seq_len;
  const int n_tok = (int)(t_end - t_begin);
  const float *lrow[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int gg = g < a.group ? g : 0;
    lrow[g] = a.logits + ((int64_t)b * a.n_q_heads + (int64_t)kvh * a.group + gg) * a.seq_len + t_begin;
  }
  const int64_t row0 = (int64_t)stream * a.row_tokens + t_begin;
  const i32x4 rc = make_rsrc(a.codes + row0 * RB, (uint32_t)n_tok * RB);
  const i32x4 rn = make_rsrc(a.norm + row0, (uint32_t)n_tok * 2u);

  // Per chunk, lane l owns token c0 + l; past the split's end the codes read
  // as zeros and the token gets no weight.
  uint32_t rw[RW];
  float rl[G];
  uint16_t rnb = 0;
  auto load_chunk = [&](int c0) __attribute__((always_inline)) {
    const int t = c0 + l;
    load_row<RW>(rc, (uint32_t)t * RB, rw);
    rnb = buf_load_u16<0>(rn, 2u * (uint32_t)t);
    const int tc = t < n_tok ? t : n_tok - 1;
#pragma unroll
    for (int g = 0; g < G; ++g) rl[g] = lrow[g][tc];
  };
  if (kChunk * w < n_tok) load_chunk(kChunk * w);

  // pair table: bits 2p and 2p+1 of the index are plane p of the even and of
  // the odd coordinate
  for (int e = tid; e < K * K; e += kAttThreads) {
    int i0 = 0, i1 = 0;
#pragma unroll
    for (int p = 0; p < LB; ++p) {
      i0 |= ((e >> (2 * p)) & 1) << p;
      i1 |= ((e >> (2 * p + 1)) & 1) << p;
    }
    ptab[e] = make_float2(a.centroids[i0], a.centroids[i1]);
  }
  __syncthreads();

  const int lc = l % (64 / TH);           // coordinate slot of this lane
  const int th = l / (64 / TH);           // its token half
  const int grp = CPL * lc / 32;          // coordinate group of this lane
  const int boff = CPL * lc % 32;         // bit of its first coordinate
  float acc[G][CPL];
  float esum[G], mrun[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    esum[g] = 0.0f;
    mrun[g] = -INFINITY;
#pragma unroll
    for (int i = 0; i < CPL; ++i) acc[g][i] = 0.0f;
  }

  for (int c0 = kChunk * w; c0 < n_tok; c0 += kChunk * NW) {
    const bool valid = c0 + l < n_tok;
    // running softmax: chunk maximum, rescale of what the wave holds (a
    // head with no finite logit yet keeps factor 1 and weight 0)
    float e[G], lv[G], cm[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      lv[g] = (valid && g < a.group) ? rl[g] : -INFINITY;
      cm[g] = lv[g];
    }
    wave_max_n(cm);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float nm = fmaxf(mrun[g], cm[g]);
      const bool live = nm != -INFINITY;
      const float sc = __expf(live ? mrun[g] - nm : 0.0f);
      esum[g] *= sc;
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc[g][i] *= sc;
      mrun[g] = nm;
      e[g] = __expf(live ? lv[g] - nm : -INFINITY);
    }
    const float n = f16_bits_to_f32(rnb);
#pragma unroll
    for (int i = 0; i < RW; ++i) cwt[w][i][l] = rw[i];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      esum[g] += e[g];
      wtt[w][g][l] = e[g] * n;
    }
    if (c0 + kChunk * NW < n_tok) load_chunk(c0 + kChunk * NW);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // accumulate the chunk (this lane's half of it), four tokens per LDS read
#pragma unroll 2
    for (int t4 = th * (kChunk / 4 / TH); t4 < (th + 1) * (kChunk / 4 / TH); ++t4) {
      u32x4 pw[LB];
#pragma unroll
      for (int p = 0; p < LB; ++p) pw[p] = *(const u32x4 *)&cwt[w][LB * grp + p][4 * t4];
      f32x4 wg[G];
#pragma unroll
      for (int g = 0; g < G; ++g) wg[g] = *(const f32x4 *)&wtt[w][g][4 * t4];
      // all table reads of the four tokens first, then their products
      float2 cv[4][CPL / 2];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int q = 0; q < CPL / 2; ++q) {
          // bitfield extracts and shift-ors: 2 LB VALU operations per pair
          uint32_t pidx = __builtin_amdgcn_ubfe(pw[0][j], boff + 2 * q, 2);
#pragma unroll
          for (int p = 1; p < LB; ++p) pidx |= __builtin_amdgcn_ubfe(pw[p][j], boff + 2 * q, 2) << (2 * p);
          cv[j][q] = ptab[pidx];
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int q = 0; q < CPL / 2; ++q) {
#pragma unroll
          for (int g = 0; g < G; ++g) {
            acc[g][2 * q] = fmaf(wg[g][j], cv[j][q].x, acc[g][2 * q]);
            acc[g][2 * q + 1] = fmaf(wg[g][j], cv[j][q].y, acc[g][2 * q + 1]);
          }
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // the waves meet: common maximum per head, each wave's share rescaled to it
  if (l == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) redm[w][g] = mrun[g];
  }
  __syncthreads();
  wave_sum_n(esum);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float v = redm[0][g];
#pragma unroll
    for (int i = 1; i < NW; ++i) v = fmaxf(v, redm[i][g]);
    const float f = mrun[g] == -INFINITY ? 0.0f : __expf(mrun[g] - v);
    if (l == 0) reds[w][g] = esum[g] * f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      acc[g][i] *= f;
      if constexpr (TH == 2) acc[g][i] += __shfl_xor(acc[g][i], 32, 64);   // the two token halves
    }
  }
  for (int i = 0; i < NW; ++i) {
    if (w == i && th == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int c = 0; c < CPL; ++c) accs[g][CPL * lc + c] = (i == 0 ? 0.0f : accs[g][CPL * lc + c]) + acc[g][c];
    }
    __syncthreads();
  }
  float *dst = a.part + (((int64_t)stream * a.n_splits + split) * G) * (D + 2);
  for (int i = tid; i < G * (D + 2); i += kAttThreads) {
    const int g = i / (D + 2), j = i % (D + 2);
    float v;
    if (j == 0) {
      v = redm[0][g];
#pragma unroll
      for (int k = 1; k < NW; ++k) v = fmaxf(v, redm[k][g]);
    } else if (j == 1) {
      v = 0.0f;
#pragma unroll
      for (int k = 0; k < NW; ++k) v += reds[k][g];
    } else {
      v = accs[g][j - 2];
    }
    dst[i] = v;
  }
}

// MFMA form of the split kernel, for G >= 4 query heads per KV head.  Per
// 16-token step and 32-coordinate group, a 16x16x32 fp16 MFMA forms
// D[m][n] = sum_k A[m][k] B[k][n] with
//   k = 2 tok + s   (tok: the step's 16 tokens, s: coordinate of the pair),
//   n = pair p of the group (coordinates 2p, 2p + 1),
//   m = 2 h + s'    (head h, coordinate parity s'),
//   A[m][k] = W[h][tok] if s = s' else 0,   B[k][n] = c[idx(tok, 2n + s)],
// so D[2h + s'][n] = sum_tok W[h][tok] c[idx(tok, 2n + s')].  At staging the
// lane that loaded a token turns its bit planes into one byte per pair (the
// pair's 2 LB index bits, spread with shifts and masks, four pairs a word) and
// stores them transposed by token; a lane's B fragment (four tokens of one
// pair) is then one 16-byte read, four byte extracts and eight 4-byte reads
// of the hi and lo pair tables.  Its A fragment is one read of the staged
// weights.  The running maximum is taken over
// l + ln n, so the weights W = e n lie in [0, 1]; weights and centroids are
// split into fp16 hi + lo and three products (hi hi, hi lo, lo hi) keep about
// 22 bits.
template <int D, int LB, int G>
__global__ __launch_bounds__(kAttThreads) void attend_mfma_kernel(PartArgs a) {
  constexpr int K = 1 << LB;
  constexpr int RB = LB * D / 8;          // packed bytes per token
  constexpr int NW = kAttThreads / 64;
  constexpr int MT = (2 * G + 15) / 16;   // 16-row tiles of (head, parity)
  constexpr int NG = D / 32;              // coordinate groups, 16 pairs each
  constexpr int CS = kChunk + 4;
  constexpr int PQ = D / 8;              // words of pair bytes per token
  constexpr int PS = LB <= 3 ? 2 : 0;     // pair bytes hold idx * 4 when it fits
  constexpr int RW = RB / 4;              // packed words per token
  static_assert(G >= 4 && RB % 4 == 0, "layout");
  __shared__ uint32_t tabh[K * K];        // hi of (c[i0], c[i1]) as an fp16 pair
  __shared__ uint32_t tabl[K * K];        // lo of the same
  // per wave: pair bytes [pair quad][token], then fp16 weights
  // [hi/lo][head][token] with row G = 0; reused for the waves' slabs at the end
  constexpr int SW = CS * (PQ + 2 * (G + 1));
  __shared__ __attribute__((aligned(16))) uint32_t stage[NW][SW];
  __shared__ float scs[NW][8 * MT];       // per-head factor read by lane-dependent head
  __shared__ float redm[NW][G];
  __shared__ float reds[NW][G];

  const int split = blockIdx.x % a.n_splits;
  const int stream = blockIdx.x / a.n_splits;
  const int b = stream / a.n_kv_heads;
  const int kvh = stream % a.n_kv_heads;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = lane_id();
  const int q = l >> 4, pn = l & 15;      // MFMA lane coordinates
  uint32_t *const pqt = &stage[w][0];                 // [PQ][CS]
  uint32_t *const awh = &stage[w][PQ * CS];           // [G + 1][CS]
  uint32_t *const awl = &stage[w][(PQ + G + 1) * CS]; // [G + 1][CS]

  const int64_t t_begin = (int64_t)split * a.tokens_per_split;
  int64_t t_end = t_begin + a.tokens_per_split;
  if (t_end > a.seq_len) t_end = a.seq_len;
  const int n_tok = (int)(t_end - t_begin);
  const float *lrow[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int gg = g < a.group ? g : 0;
    lrow[g] = a.logits + ((int64_t)b * a.n_q_heads + (int64_t)kvh * a.group + gg) * a.seq_len + t_begin;
  }
  const int64_t row0 = (int64_t)stream * a.row_tokens + t_begin;
  const i32x4 rc = make_rsrc(a.codes + row0 * RB, (uint32_t)n_tok * RB);
  const i32x4 rn = make_rsrc(a.norm + row0, (uint32_t)n_tok * 2u);

  uint32_t rw[RW];
  float rl[G];
  uint16_t rnb = 0;
  auto load_chunk = [&](int c0) __attribute__((always_inline)) {
    const int t = c0 + l;
    load_row<RW>(rc, (uint32_t)t * RB, rw);
    rnb = buf_load_u16<0>(rn, 2u * (uint32_t)t);
    const int tc = t < n_tok ? t : n_tok - 1;
#pragma unroll
    for (int g = 0; g < G; ++g) rl[g] = lrow[g][tc];
  };
  if (kChunk * w < n_tok) load_chunk(kChunk * w);

  for (int e = tid; e < K * K; e += kAttThreads) {
    int i0 = 0, i1 = 0;
#pragma unroll
    for (int p = 0; p < LB; ++p) {
      i0 |= ((e >> (2 * p)) & 1) << p;
      i1 |= ((e >> (2 * p + 1)) & 1) << p;
    }
    const float c0 = a.centroids[i0], c1 = a.centroids[i1];
    const _Float16 h0 = (_Float16)c0, h1 = (_Float16)c1;
    const _Float16 l0 = (_Float16)(c0 - (float)h0), l1 = (_Float16)(c1 - (float)h1);
    tabh[e] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    tabl[e] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
  }
  for (int i = tid; i < NW * 2 * CS; i += kAttThreads)
    stage[i / (2 * CS)][PQ * CS + (((i / CS) % 2) * (G + 1) + G) * CS + i % CS] = 0u;
  if (tid < NW * 8 * MT) scs[tid / (8 * MT)][tid % (8 * MT)] = 1.0f;
  __syncthreads();

  f32x4 acc[MT][NG];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < NG; ++j) acc[mt][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float esum[G], mrun[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    esum[g] = 0.0f;
    mrun[g] = -INFINITY;
  }

  for (int c0 = kChunk * w; c0 < n_tok; c0 += kChunk * NW) {
    const bool valid = c0 + l < n_tok;
    const float n = f16_bits_to_f32(rnb);
    const float lnn = __logf(fmaxf(n, 0x1p-24f));     // n = 0 gives weight 0 whatever the shift
    float sc[G], lv[G], cm[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      lv[g] = (valid && g < a.group) ? rl[g] : -INFINITY;
      cm[g] = lv[g] + lnn;
    }
    wave_max_n(cm);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      // a head with no finite logit yet keeps factor 1 and weight 0
      const float nm = fmaxf(mrun[g], cm[g]);
      const bool live = nm != -INFINITY;
      sc[g] = __expf(live ? mrun[g] - nm : 0.0f);
      esum[g] *= sc[g];
      mrun[g] = nm;
      const float e = __expf(live ? lv[g] - nm : -INFINITY);
      esum[g] += e;
      const float wgt = e * n;
      const _Float16 hi = (_Float16)wgt;
      const _Float16 lo = (_Float16)(wgt - (float)hi);
      awh[g * CS + l] = __builtin_bit_cast(uint16_t, hi);
      awl[g * CS + l] = __builtin_bit_cast(uint16_t, lo);
    }
    if (l == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) scs[w][g] = sc[g];
    }
    // pair bytes: byte k of word 4 j + o holds the index bits of pair
    // 4 k + o of group j (bits 2p, 2p + 1 = plane p of its two coordinates),
    // times 4 when that fits in a byte.  Pair 4 k + o sits at bit 8 k + 2 o of
    // every plane word, so each plane costs one shift and one masked or.
#pragma unroll
    for (int j = 0; j < NG; ++j) {
#pragma unroll
      for (int o = 0; o < 4; ++o) {
        uint32_t pb = 0;
#pragma unroll
        for (int p = 0; p < LB; ++p) {
          const int wi = LB * j + p;
          const uint32_t x = rw[wi];
          const int sh = 2 * p + PS - 2 * o;              // where the pair's bits go
          const uint32_t y = sh >= 0 ? x << sh : x >> -sh;
          pb |= y & (0x03030303u << (2 * p + PS));
        }
        pqt[(4 * j + o) * CS + l] = pb;
      }
    }
    if (c0 + kChunk * NW < n_tok) load_chunk(c0 + kChunk * NW);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // rows 4q + r of tile mt hold head 8 mt + 2 q + r / 2
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const float f0 = scs[w][8 * mt + 2 * q], f1 = scs[w][8 * mt + 2 * q + 1];
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        acc[mt][j][0] *= f0;
        acc[mt][j][1] *= f0;
        acc[mt][j][2] *= f1;
        acc[mt][j][3] *= f1;
      }
    }
    // Per 16-token step: every LDS read of the step first (A rows, pair
    // bytes of all groups, then all table entries), then the MFMAs with the
    // groups interleaved so that no product waits on the previous one.
#pragma unroll
    for (int st = 0; st < kChunk / 16; ++st) {
      const int tb = 16 * st + 4 * q;     // this lane's four tokens
      u32x4 xh[MT], xl[MT], pv[NG];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        // A row 16 mt + pn is head (16 mt + pn) / 2 on its parity's half of
        // each k pair (rows past the heads read the zero row)
        const int hr = (16 * mt + pn) >> 1;
        const int row = hr < G ? hr : G;
        xh[mt] = *(const u32x4 *)&awh[row * CS + tb];
        xl[mt] = *(const u32x4 *)&awl[row * CS + tb];
      }
#pragma unroll
      for (int j = 0; j < NG; ++j) pv[j] = *(const u32x4 *)&pqt[(4 * j + (pn & 3)) * CS + tb];
      u32x4 bh[NG], bl[NG];
#pragma unroll
      for (int j = 0; j < NG; ++j) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t pb = __builtin_amdgcn_ubfe(pv[j][t], 8 * (pn >> 2), 8);
          const uint32_t off = PS == 2 ? pb : pb << 2;          // byte offset into the tables
          bh[j][t] = *(const uint32_t *)((const char *)tabh + off);
          bl[j][t] = *(const uint32_t *)((const char *)tabl + off);
        }
      }
      half8 ah[MT], al[MT];
      const int sh = 16 * (pn & 1);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xh[mt][i] <<= sh;
          xl[mt][i] <<= sh;
        }
        ah[mt] = __builtin_bit_cast(half8, xh[mt]);
        al[mt] = __builtin_bit_cast(half8, xl[mt]);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int j = 0; j < NG; ++j)
          acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[mt], __builtin_bit_cast(half8, bh[j]), acc[mt][j], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < NG; ++j)
          acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[mt], __builtin_bit_cast(half8, bl[j]), acc[mt][j], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < NG; ++j)
          acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[mt], __builtin_bit_cast(half8, bh[j]), acc[mt][j], 0, 0, 0);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // the waves meet: common maximum per head, each wave's share rescaled to it
  if (l == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) redm[w][g] = mrun[g];
  }
  __syncthreads();
  float fw[G];
  wave_sum_n(esum);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float v = redm[0][g];
#pragma unroll
    for (int i = 1; i < NW; ++i) v = fmaxf(v, redm[i][g]);
    fw[g] = mrun[g] == -INFINITY ? 0.0f : __expf(mrun[g] - v);
    if (l == 0) reds[w][g] = esum[g] * fw[g];
  }
  // each wave leaves its rescaled share in its own slab (the staging
  // memory, free now), then every thread sums the slabs for its outputs
  float *slab = (float *)&stage[0][0];                    // [NW][G][D]
  static_assert(G * D <= SW, "slab fits");
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int g = 8 * mt + 2 * q + r / 2;
      if (g < G) {
        float f = fw[0];
#pragma unroll
        for (int gg = 1; gg < G; ++gg) f = g == gg ? fw[gg] : f;
#pragma unroll
        for (int j = 0; j < NG; ++j) slab[(w * G + g) * D + 32 * j + 2 * pn + (r & 1)] = acc[mt][j][r] * f;
      }
    }
  }
  __syncthreads();
  float *dst = a.part + (((int64_t)stream * a.n_splits + split) * G) * (D + 2);
  for (int i = tid; i < G * (D + 2); i += kAttThreads) {
    const int g = i / (D + 2), j = i % (D + 2);
    float v;
    if (j == 0) {
      v = redm[0][g];
#pragma unroll
      for (int k = 1; k < NW; ++k) v = fmaxf(v, redm[k][g]);
    } else if (j == 1) {
      v = 0.0f;
#pragma unroll
      for (int k = 0; k < NW; ++k) v += reds[k][g];
    } else {
      v = 0.0f;
#pragma unroll
      for (int k = 0; k < NW; ++k) v += slab[(k * G + g) * D + j - 2];
    }
    dst[i] = v;
  }
}

struct CombArgs {
  const float *part;
  const float *pi;
  int64_t n_rows;           // batch * n_q_heads
  int n_splits, n_kv_heads, n_q_heads, group, gbucket;
  void *out;
  bool out_f32;
};

// One workgroup per query head, 4 groups of D threads: group q takes the
// splits i = q (mod 4), then rows [q D/4, (q+1) D/4) of Pi; the groups meet
// in LDS.  The Pi rows, the first kPre splits' accumulators and the split
// maxima and sums are all requested before the first barrier, so the kernel
// waits on memory about once.
constexpr int kPre = 16;

template <int D>
__global__ __launch_bounds__(4 * D) void attend_combine_kernel(CombArgs a) {
  constexpr int NWC = 4 * D / 64;
  __shared__ float fac[256];
  __shared__ float red[NWC];
  __shared__ float red2[NWC];
  __shared__ __attribute__((aligned(16))) float sum4[4][D];
  __shared__ __attribute__((aligned(16))) float r[D];
  const int64_t row = blockIdx.x;         // b * n_q_heads + h
  const int tid = threadIdx.x;
  const int wv = tid >> 6, l = lane_id();
  const int q = tid / D, j = tid % D;
  const int64_t b = row / a.n_q_heads;
  const int h = (int)(row % a.n_q_heads);
  const int kvh = h / a.group, g = h % a.group;
  const int64_t stream = b * a.n_kv_heads + kvh;
  const int64_t sstride = (int64_t)a.gbucket * (D + 2);
  const float *src = a.part + (stream * a.n_splits * a.gbucket + g) * (D + 2);
  const int ns = a.n_splits;              // <= 256 <= 4 D
  if (ns == 0) {                          // no token at all: the output is zero
    if (q == 0) {
      if (a.out_f32)
        ((float *)a.out)[row * D + j] = 0.0f;
      else
        ((uint16_t *)a.out)[row * D + j] = 0;
    }
    return;
  }

  // Loads with clamped indices and a select after them, so none of them
  // sits behind a branch.
  float pv[D / 4];
#pragma unroll
  for (int k = 0; k < D / 4; ++k) pv[k] = a.pi[(size_t)(q * (D / 4) + k) * D + j];
  float av[kPre];
#pragma unroll
  for (int k = 0; k < kPre; ++k) {
    const int i = q + 4 * k;
    const float x = src[(i < ns ? i : ns - 1) * sstride + 2 + j];
    av[k] = i < ns ? x : 0.0f;
  }
  const int ts = tid < ns ? tid : ns - 1;
  const float fm0 = src[ts * sstride];
  const float fs0 = src[ts * sstride + 1];
  const float fm = tid < ns ? fm0 : -INFINITY;
  const float fs = tid < ns ? fs0 : 0.0f;

  // common maximum, then the rescaled total weight
  float v = wave_max(fm);
  if (l == 0) red[wv] = v;
  __syncthreads();
  float mm = red[0];
#pragma unroll
  for (int i = 1; i < NWC; ++i) mm = fmaxf(mm, red[i]);
  const float f = (mm == -INFINITY || fm == -INFINITY) ? 0.0f : expf(fm - mm);
  if (tid < ns) fac[tid] = f;
  v = wave_sum(fs * f);
  if (l == 0) red2[wv] = v;
  __syncthreads();
  float o = 0.0f;
  if (mm != -INFINITY) {                  // uniform over the workgroup
    float ssum = 0.0f;
#pragma unroll
    for (int i = 0; i < NWC; ++i) ssum += red2[i];
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
      const int i = q + 4 * k;
      acc = fmaf(av[k], fac[i < ns ? i : 0], acc);     // av is 0 past ns
    }
    for (int i = q + 4 * kPre; i < ns; i += 4) acc = fmaf(src[i * sstride + 2 + j], fac[i], acc);
    sum4[q][j] = acc;
    __syncthreads();
    if (q == 0) r[j] = (sum4[0][j] + sum4[1][j] + sum4[2][j] + sum4[3][j]) / ssum;
    __syncthreads();
    // o = Pi^T r: o_j = sum_k Pi[k][j] r_k, a quarter of the rows per group
    float oq = 0.0f;
#pragma unroll
    for (int k = 0; k < D / 4; k += 4) {
      const f32x4 rv = *(const f32x4 *)&r[q * (D / 4) + k];
      oq = fmaf(pv[k], rv[0], oq);
      oq = fmaf(pv[k + 1], rv[1], oq);
      oq = fmaf(pv[k + 2], rv[2], oq);
      oq = fmaf(pv[k + 3], rv[3], oq);
    }
    sum4[q][j] = oq;
    __syncthreads();
    o = sum4[0][j] + sum4[1][j] + sum4[2][j] + sum4[3][j];
  }
  if (q == 0) {
    if (a.out_f32)
      ((float *)a.out)[row * D + j] = o;
    else
      ((uint16_t *)a.out)[row * D + j] = f32_to_bf16_bits(o);
  }
}

// Token splits of one call: a few workgroups per CU in all, at least 256
// tokens each, a whole number of chunks per split.
struct AttendPlan {
  int64_t splits, tps;
};

AttendPlan attend_plan(int64_t n_streams, int64_t seq_len) {
  const int64_t cus = tqi::device_cu_count();
  int64_t splits = (kAttBlocksPerCu * cus + n_streams - 1) / n_streams;
  const int64_t max_splits = (seq_len + 255) / 256;
  if (splits > max_splits) splits = max_splits;
  if (splits > 256) splits = 256;
  if (splits < 1) splits = 1;
  int64_t tps = (seq_len + splits - 1) / splits;
  tps = (tps + kChunk - 1) / kChunk * kChunk;
  AttendPlan p;
  p.tps = tps;
  p.splits = seq_len > 0 ? (seq_len + tps - 1) / tps : 0;
  return p;
}

int group_bucket(int group) {
  return group <= 1 ? 1 : group <= 2 ? 2 : group <= 4 ? 4 : group <= 8 ? 8 : 16;
}

template <int D, int LB, int G>
hipError_t launch_t(const tqi::AttendArgs &aa, hipStream_t s) {
  const int group = aa.n_q_heads / aa.n_kv_heads;
  const int64_t n_streams = (int64_t)aa.batch * aa.n_kv_heads;
  const AttendPlan plan = attend_plan(n_streams, aa.seq_len);
  const int64_t splits = plan.splits, tps = plan.tps;
  const size_t bytes = (size_t)n_streams * splits * G * (D + 2) * sizeof(float);
  if (aa.workspace_bytes < bytes || (bytes > 0 && aa.workspace == nullptr))   // checked by the caller
    return hipErrorInvalidValue;
  float *part = (float *)aa.workspace;
  hipError_t e = hipSuccess;
  if (splits > 0) {
    PartArgs pa;
    pa.logits = aa.logits;
    pa.codes = aa.codes;
    pa.norm = aa.norm;
    pa.centroids = aa.centroids;
    pa.row_tokens = aa.row_tokens;
    pa.seq_len = aa.seq_len;
    pa.tokens_per_split = tps;
    pa.n_splits = (int)splits;
    pa.n_kv_heads = aa.n_kv_heads;
    pa.n_q_heads = aa.n_q_heads;
    pa.group = group;
    pa.part = part;
    if constexpr (G >= 4)
      hipLaunchKernelGGL((attend_mfma_kernel<D, LB, G>), dim3((unsigned)(n_streams * splits)), dim3(kAttThreads),
                         0, s, pa);
    else
      hipLaunchKernelGGL((attend_partial_kernel<D, LB, G>), dim3((unsigned)(n_streams * splits)), dim3(kAttThreads),
                         0, s, pa);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  CombArgs ca;
  ca.part = part;
  ca.pi = aa.pi;
  ca.n_rows = (int64_t)aa.batch * aa.n_q_heads;
  ca.n_splits = (int)splits;
  ca.n_kv_heads = aa.n_kv_heads;
  ca.n_q_heads = aa.n_q_heads;
  ca.group = group;
  ca.gbucket = G;
  ca.out = aa.out;
  ca.out_f32 = aa.out_f32;
  hipLaunchKernelGGL((attend_combine_kernel<D>), dim3((unsigned)ca.n_rows), dim3(4 * D), 0, s, ca);
  return hipGetLastError();
}

template <int D, int LB>
hipError_t launch_g(const tqi::AttendArgs &a, hipStream_t s) {
  switch (group_bucket(a.n_q_heads / a.n_kv_heads)) {
    case 1: return launch_t<D, LB, 1>(a, s);
    case 2: return launch_t<D, LB, 2>(a, s);
    case 4: return launch_t<D, LB, 4>(a, s);
    case 8: return launch_t<D, LB, 8>(a, s);
  }
  return launch_t<D, LB, 16>(a, s);
}

template <int D>
hipError_t launch_lb(int lb, const tqi::AttendArgs &a, hipStream_t s) {
  switch (lb) {
    case 1: return launch_g<D, 1>(a, s);
    case 2: return launch_g<D, 2>(a, s);
    case 3: return launch_g<D, 3>(a, s);
    case 4: return launch_g<D, 4>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

namespace tqi {

bool attend_supported(int d, int lbits, int group, int64_t seq_len) {
  if (d != 64 && d != 128 && d != 256) return false;
  if (lbits < 1 || lbits > 4 || group < 1 || group > 16) return false;
  // 32-bit byte offsets within one split of the packed values (plus a chunk)
  const int64_t rb = (int64_t)lbits * d / 8;
  return (seq_len + kChunk) * rb < (1LL << 31);
}

size_t attend_workspace_bytes(int d, int lbits, int batch, int n_q_heads, int n_kv_heads, int64_t seq_len) {
  (void)lbits;
  const int64_t n_streams = (int64_t)batch * n_kv_heads;
  const int g = group_bucket(n_q_heads / n_kv_heads);
  const AttendPlan plan = attend_plan(n_streams, seq_len);
  return ws_align((size_t)n_streams * plan.splits * g * (d + 2) * sizeof(float));
}

hipError_t launch_attend(int d, int lbits, const AttendArgs &a, hipStream_t s) {
  if (d == 64) return launch_lb<64>(lbits, a, s);
  if (d == 128) return launch_lb<128>(lbits, a, s);
  if (d == 256) return launch_lb<256>(lbits, a, s);
  return hipErrorInvalidValue;
}

}  // namespace tqi

// Per-split partials of tq_attn_output_noalloc: a fixed array in device
// memory instead of a caller workspace (each device that runs the library
// holds its own copy until the process ends).  Host code never passes the
// array's name to a kernel: that name is a host-side stand-in, not a device
// address; the device address comes from hipGetSymbolAddress below.
static __device__ __align__(256) unsigned char scratch[tqi::kNoAllocScratchBytes];

namespace tqi {

hipError_t noalloc_scratch(void **out) {
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {        // once per device, with that device current
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace tqi
