// Top-k inner-product search over a quantised database.
//
// Page "TurboQuant 설명: 무엇인지와 LLM 메모리 6배 절약 구현 방법", sections
// "벤치마크 및 실제 성능" (top-k recall of vector search at d = 200 without
// dataset-specific codebooks) and "응용 분야 및 미래 영향" (vector databases):
// score(q, x) = scale * n * <Pi q, c[idx]>, with the query rotated once.
//
// Design (gfx950): the dense score matrix of a large search does not fit in
// memory, so selection is fused into the scoring kernel.
// * prep: q' = Pi q per query (fp64 accumulate), scaled by a power of two and
//   split into fp16 hi + lo.
// * score: a workgroup owns 256 queries (8 waves x 32) and one slice of the
//   database.  Each 32-key tile is decoded once into LDS (centroid values as
//   fp16 hi + lo) and multiplied on the 32x32x16 fp16 MFMA by every wave's
//   stationary query fragments: hi*hi first, hi*lo + lo*hi only where some
//   lane's score could still enter its list (a rigorous margin covers the lo
//   products).  In the accumulator layout a lane holds one query and 16 keys;
//   passing scores go to per-lane candidate slots, merged into the query's
//   sorted list of 16 in LDS when the slots fill.
// * two passes: a sample pass over the first 1/16 of the keys, whose merged
//   topk-th scores seed the lists' bounds for the main pass over the rest.
// * merge: per query, the sorted lists of all database slices of both passes
//   are merged; ties go to the smaller key index.
#include <cfloat>

#include "tq_device.h"
#include "tq_internal.h"

namespace {

using namespace tqd;

constexpr int kTop = 16;               // list length kept per lane (topk <= 16)
constexpr int kCand = 8;               // candidate slots per lane between list updates
constexpr int kEmptyKey = 0x3FFFFFFF;  // key index of an empty list entry (score -FLT_MAX)
constexpr int kSearchThreads = 512;    // 8 waves
constexpr int kSearchQueries = 32 * (kSearchThreads / 64);   // queries per workgroup
constexpr float kCenScale = 1024.0f;

struct QPrepArgs {
  const void *q;
  bool q_f32;
  int64_t n_queries;  // batch * n_q_heads
  const float *pi;
  _Float16 *qh;       // [n_queries][D]
  _Float16 *ql;
  float *qfac;        // [n_queries]: 1 / (query scale * centroid scale)
};

// One workgroup rotates kPrepQueries queries; thread j owns row j of Pi and
// accumulates q'_j = sum_k Pi[j][k] q[k] for each of them in k order (fp64;
// the products of fp32 values are exact).
constexpr int kPrepQueries = 16;

template <int D>
__global__ __launch_bounds__(D) void search_prep_kernel(QPrepArgs a) {
  constexpr int QB = kPrepQueries;
  __shared__ __attribute__((aligned(16))) float qin[QB][D];
  __shared__ double red[QB][D / 64];
  const int64_t q0 = (int64_t)blockIdx.x * QB;
  const int j = threadIdx.x;
  for (int i = j; i < QB * D; i += D) {
    const int qi = i / D, k = i % D;
    const int64_t g = q0 + qi;
    float v = 0.0f;
    if (g < a.n_queries)
      v = a.q_f32 ? ((const float *)a.q)[g * D + k] : bf16_to_f32(((const uint16_t *)a.q)[g * D + k]);
    qin[qi][k] = v;
  }
  __syncthreads();
  double acc[QB];
#pragma unroll
  for (int qi = 0; qi < QB; ++qi) acc[qi] = 0.0;
  const f32x4 *row = (const f32x4 *)(a.pi + (size_t)j * D);
  for (int k4 = 0; k4 < D / 4; ++k4) {
    const f32x4 p = row[k4];
#pragma unroll
    for (int qi = 0; qi < QB; ++qi) {
      const f32x4 x = *(const f32x4 *)&qin[qi][4 * k4];
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[qi] = fma((double)p[c], (double)x[c], acc[qi]);
    }
  }
  // per query: largest |q'_j| over the rows
  const int wv = j >> 6;
#pragma unroll
  for (int qi = 0; qi < QB; ++qi) {
    double mx = fabs(acc[qi]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmax(mx, __shfl_xor(mx, off));
    if ((j & 63) == 0) red[qi][wv] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int qi = 0; qi < QB; ++qi) {
    const int64_t g = q0 + qi;
    if (g >= a.n_queries) break;
    double mx = red[qi][0];
#pragma unroll
    for (int i = 1; i < D / 64; ++i) mx = fmax(mx, red[qi][i]);
    int e = 0;
    if (mx > 0.0) frexp(mx, &e);
    const double sc = ldexp(1.0, 15 - e);   // largest |q'| lands in [2^14, 2^15)
    const float v = (float)(acc[qi] * sc);
    const _Float16 hv = (_Float16)v;
    a.qh[g * D + j] = hv;
    a.ql[g * D + j] = (_Float16)(v - (float)hv);
    if (j == 0) a.qfac[g] = (float)(1.0 / (sc * (double)kCenScale));
  }
}

struct ScoreArgs {
  const _Float16 *qh;
  const _Float16 *ql;
  const float *qfac;
  const float *centroids;
  const uint8_t *codes;
  const uint16_t *norm;
  int64_t row_tokens, seq_len, keys_per_split, n_rows;
  int64_t key_base;   // this pass scores keys [key_base, key_base + seq_len)
  int n_splits, q_tiles, n_kv_heads, n_q_heads, group, topk;
  int split_base;     // its lists are splits [split_base, split_base + n_splits)
  float scale;
  const float *seed;  // [query][topk] scores whose last is a lower bound of the
                      // query's topk-th best (nullptr: none)
  float *part_val;    // [split][query][kTop]; the first topk of each list are exact
  int32_t *part_idx;
};

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// A list entry (score s, key index i < 2^30) packed into one 64-bit word
// whose unsigned order is the list order: higher score first, then the
// smaller index.  The top two bits are clear and the exponent field is never
// all ones or zero for finite or infinite scores, so the word read as an fp64
// value is a positive normal number and fp64 max/min order it the same way.
__device__ __forceinline__ double pack_entry(float s, int i) {
  const uint32_t b = __float_as_uint(s + 0.0f);      // -0 -> +0: equal scores tie on the index
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  const uint64_t w = ((uint64_t)ord << 30) | (uint64_t)(0x3FFFFFFFu - ((uint32_t)i & 0x3FFFFFFFu));
  return __longlong_as_double((long long)w);
}

__device__ __forceinline__ void unpack_entry(double e, float &s, int &i) {
  const uint64_t w = (uint64_t)__double_as_longlong(e);
  const uint32_t ord = (uint32_t)(w >> 30);
  s = __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
  i = (int)(0x3FFFFFFFu - ((uint32_t)w & 0x3FFFFFFFu));
}

// Insert x into a descending list of packed entries (branch-free).
__device__ __forceinline__ void list_insert(double (&e)[kTop], double x) {
#pragma unroll
  for (int j = kTop - 1; j > 0; --j) e[j] = fmax(e[j], fmin(x, e[j - 1]));
  e[0] = fmax(e[0], x);
}

template <int D, int LB>
struct SearchTile {
  static constexpr int K = 1 << LB;
  static constexpr int PITCH = D + 8;      // halves per decoded key row (16-byte pad)
  static constexpr int CPT = D / 16;       // coordinates a thread decodes per tile
  static constexpr int ROWB = LB * D / 8;  // packed bytes per key
};

// Spread the 2-bit groups of the low 2*NP bits of x to a 4-bit pitch.
template <int NP>
__device__ __forceinline__ uint32_t spread2(uint32_t x) {
  if constexpr (NP == 8) {
    x &= 0xFFFFu;
    x = (x | (x << 8)) & 0x00FF00FFu;
  } else if constexpr (NP == 4) {
    x &= 0xFFu;
  } else {
    static_assert(NP == 2, "pairs per thread");
    x &= 0xFu;
  }
  x = (x | (x << 4)) & 0x0F0F0F0Fu;
  x = (x | (x << 2)) & 0x33333333u;
  return x;
}

// Decode the coordinates [CPT*c, CPT*c + CPT) of one key from its bit-plane
// words into fp16 hi and lo halves through the pair tables (hi table at
// tab[0, K*K), lo table at tab[K*K, 2*K*K)).
template <int D, int LB>
__device__ __forceinline__ void decode_pairs(const uint32_t (&pw)[LB], int c, const uint32_t *tab,
                                             _Float16 *hrow, _Float16 *lrow) {
  constexpr int CPT = SearchTile<D, LB>::CPT;
  constexpr int NP = CPT / 2;
  constexpr int KK = 1 << (2 * LB);
  const int boff = (CPT * c) & 31;
  // z01 (and z23) hold the pair index bits of planes 0-1 (2-3) at a 4-bit pitch
  uint32_t z01 = spread2<NP>(pw[0] >> boff);
  if constexpr (LB >= 2) z01 |= spread2<NP>(pw[1] >> boff) << 2;
  uint32_t z23 = 0;
  if constexpr (LB >= 3) z23 = spread2<NP>(pw[2] >> boff);
  if constexpr (LB >= 4) z23 |= spread2<NP>(pw[3] >> boff) << 2;
  uint32_t hw[NP], lw[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    uint32_t pidx = (z01 >> (4 * k)) & 15u;
    if constexpr (LB >= 3) pidx |= ((z23 >> (4 * k)) & 15u) << 4;
    hw[k] = tab[pidx];
    lw[k] = tab[KK + pidx];
  }
  if constexpr (NP == 2) {                 // d = 64: four coordinates
    *(uint2 *)hrow = make_uint2(hw[0], hw[1]);
    *(uint2 *)lrow = make_uint2(lw[0], lw[1]);
  } else {
#pragma unroll
    for (int k = 0; k < NP; k += 4) {
      *(uint4 *)(hrow + 2 * k) = make_uint4(hw[k], hw[k + 1], hw[k + 2], hw[k + 3]);
      *(uint4 *)(lrow + 2 * k) = make_uint4(lw[k], lw[k + 1], lw[k + 2], lw[k + 3]);
    }
  }
}

template <int D, int LB>
__global__ __launch_bounds__(kSearchThreads) void search_score_kernel(ScoreArgs a) {
  using T = SearchTile<D, LB>;
  constexpr int K = T::K;
  constexpr int KS = D / 16;
  constexpr int PITCH = T::PITCH;
  constexpr int CPT = T::CPT;
  constexpr int ROWB = T::ROWB;
  constexpr int NW = kSearchThreads / 64;
  __shared__ uint32_t ptab[2 * K * K];
  __shared__ __attribute__((aligned(16))) float kn[3][32];   // norms of tiles t, t+1, t+2 (mod 3)
  // Two statically distinct tile buffers, so that the decode of the next
  // tile can be interleaved with the products on the current one.
  __shared__ __attribute__((aligned(16))) _Float16 ch0[32 * PITCH], ch1[32 * PITCH];
  __shared__ __attribute__((aligned(16))) _Float16 cl0[32 * PITCH], cl1[32 * PITCH];
  // Per query (32 per wave): one sorted list of kTop packed entries, shared
  // by the two half-wave lanes that hold the query's scores, and kCand
  // candidate slots per lane; query-minor, so a row is one line per wave.
  __shared__ double qlist[NW * kTop * 32];
  __shared__ double qslot[NW * 2 * kCand * 32];

  const int split = blockIdx.x % a.n_splits;
  const int rest = blockIdx.x / a.n_splits;
  const int qt = rest % a.q_tiles;
  const int stream = rest / a.q_tiles;
  const int b = stream / a.n_kv_heads;
  const int kvh = stream % a.n_kv_heads;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = lane_id();
  const int m = l & 31;
  const int h = l >> 5;

  const int gq = qt * kSearchQueries + 32 * w + m;      // query within the GQA group
  const bool qvalid = gq < a.group;
  const int64_t qglob = (int64_t)b * a.n_q_heads + (int64_t)kvh * a.group + (qvalid ? gq : 0);
  // A negative scale reverses the order: the query is negated instead, which
  // is exact, and |scale| applied afterwards.
  const uint32_t qsign = a.scale < 0.0f ? 0x80008000u : 0u;
  half8 qh[KS], ql[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    i32x4 vh = {}, vl = {};
    if (qvalid) {
      vh = *(const i32x4 *)(a.qh + qglob * D + 16 * s + 8 * h);
      vl = *(const i32x4 *)(a.ql + qglob * D + 16 * s + 8 * h);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) { vh[j] ^= (int)qsign; vl[j] ^= (int)qsign; }
    __builtin_memcpy(&qh[s], &vh, 16);
    __builtin_memcpy(&ql[s], &vl, 16);
  }
  const float qf = qvalid ? a.qfac[qglob] * fabsf(a.scale) : 0.0f;

  // pair tables: bits 2p and 2p+1 of the entry index are plane p of the even
  // and of the odd coordinate of a pair; hi halves, then lo halves
  for (int e = tid; e < K * K; e += kSearchThreads) {
    uint32_t i0 = 0, i1 = 0;
#pragma unroll
    for (int p = 0; p < LB; ++p) {
      i0 |= ((e >> (2 * p)) & 1u) << p;
      i1 |= ((e >> (2 * p + 1)) & 1u) << p;
    }
    uint32_t hw = 0, lw = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float cv = a.centroids[j ? i1 : i0] * kCenScale;
      const _Float16 hv = (_Float16)cv;
      const _Float16 lv = (_Float16)(cv - (float)hv);
      uint16_t hb, lb;
      __builtin_memcpy(&hb, &hv, 2);
      __builtin_memcpy(&lb, &lv, 2);
      hw |= (uint32_t)hb << (16 * j);
      lw |= (uint32_t)lb << (16 * j);
    }
    ptab[e] = hw;
    ptab[K * K + e] = lw;
  }

  const int64_t k_begin = (int64_t)split * a.keys_per_split;
  int64_t k_end = k_begin + a.keys_per_split;
  if (k_end > a.seq_len) k_end = a.seq_len;
  const int n_keys = (int)(k_end - k_begin);
  const int64_t key0 = (int64_t)stream * a.row_tokens + a.key_base + k_begin;
  // Keys past the split's end fall outside these ranges and load as zero.
  const i32x4 rcode = make_rsrc(a.codes + key0 * ROWB, (uint32_t)n_keys * ROWB);
  const i32x4 rnrm = make_rsrc(a.norm + key0, (uint32_t)n_keys * 2u);

  // decode role: key v of a tile, coordinates [CPT*c, CPT*c + CPT)
  const int dv = tid >> 4;
  const int dc = tid & 15;
  const uint32_t code_off = (uint32_t)dv * ROWB + 4u * LB * (uint32_t)((CPT * dc) >> 5);
  uint32_t pw[LB];
  uint16_t nb = 0;
  auto load_tile = [&](int t0) __attribute__((always_inline)) {
    buf_load_words<LB, 0>(rcode, (uint32_t)t0 * ROWB + code_off, pw);
    nb = buf_load_u16<0>(rnrm, 2u * (uint32_t)(t0 + dv));
  };
  // Branch-free, so that the decode can be interleaved with the products.  A
  // key past the end gets a NaN norm, so none of its scores passes a test.
  auto decode_tile = [&](int t0, _Float16 *dh, _Float16 *dl, float *dn) __attribute__((always_inline)) {
    decode_pairs<D, LB>(pw, dc, ptab, dh + dv * PITCH + CPT * dc, dl + dv * PITCH + CPT * dc);
    dn[dv] = t0 + dv < n_keys ? f16_bits_to_f32(nb) : __builtin_nanf("");   // same value from 16 lanes
  };

  // A score s = (acc * norm) * qf enters the query's list only if s > thr,
  // the list's current topk-th best.  The products are first tested against
  // thq, a bound a little below thr / qf, so the exact test runs only on the
  // few that pass.  qf == 0 (invalid lane or zero scale) gives -inf or NaN:
  // all scores tie at zero and the first keys stay, as the order requires.
  double *lq = qlist + (w * kTop) * 32 + m;
  double *sq = qslot + ((w * 2 + h) * kCand) * 32 + m;
  {
    const double empty = pack_entry(-FLT_MAX, kEmptyKey);
#pragma unroll
    for (int j = 0; j < kTop; ++j) lq[32 * j] = empty;     // both half-lanes store the same
  }
  // A seed (the topk-th best over a sample of the keys scored before) is a
  // lower bound of the final topk-th best: a key at or below it cannot
  // make the top-k (the sample's keys have smaller indices and win ties).
  const float seed = (a.seed != nullptr && qvalid)
                         ? a.seed[((int64_t)stream * a.group + gq) * a.topk + a.topk - 1] : -FLT_MAX;
  float thr = qvalid ? seed : FLT_MAX;
  float thq = -INFINITY;
  int cnt = 0;
  auto set_bound = [&]() __attribute__((always_inline)) {
    const float t = thr / qf;
    thq = t - fabsf(t) * 0x1p-20f;
  };
  set_bound();
  // Both half-lanes of a query merge the slots of both into the shared list
  // (the same work on the same data) and store the same result.
  auto flush = [&]() __attribute__((always_inline)) {
    const int cnt_o = __shfl_xor(cnt, 32);
    double e[kTop];
#pragma unroll
    for (int j = 0; j < kTop; ++j) e[j] = lq[32 * j];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int ch = hh == h ? cnt : cnt_o;
      const double *src_s = qslot + ((w * 2 + hh) * kCand) * 32 + m;
#pragma unroll 1
      for (int s = 0; s < kCand; ++s)
        if (s < ch) list_insert(e, src_s[32 * s]);
    }
#pragma unroll
    for (int j = 0; j < kTop; ++j) lq[32 * j] = e[j];
    cnt = 0;
    // The bound is the topk-th best: the merge reads no further down a list.
    float t;
    int ix;
    unpack_entry(lq[32 * (a.topk - 1)], t, ix);
    thr = qvalid ? fmaxf(t, seed) : FLT_MAX;
    set_bound();
  };
  // Products on a tile held in (sh, sl), norms sn: the hi x hi product
  // first, then, only where some lane's score could pass its bound, the two
  // lo products.  The lo halves are at most 2^-11 of their hi halves (fp16
  // rounding; the query's subnormal halves add an absolute term below
  // 2^-17 max|c|), so the three-product sum differs from hi x hi by at most
  // 2^-10 sum_k |qh_k| |ch_k| <= 2^-10 max|c| ||qh||_1 (scaled centroids);
  // marg adds 1/8 of that for the fp32 roundings of both sums (products
  // are exact, at most 64 roundings of 2^-24 each, relative to the same
  // sum).  A lane whose hi x hi product plus marg does not pass cannot pass
  // with all three.  Returns whether the three products were formed.
  const int h4 = 4 * h;
  float marg;
  {
    float q1 = 0.0f;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i) q1 += fabsf((float)qh[s][i]);
    q1 += __shfl_xor(q1, 32);                         // the other half of the coordinates
    const float cmax = fmaxf(fabsf(a.centroids[0]), fabsf(a.centroids[K - 1])) * kCenScale;
    marg = 0x1.2p-10f * cmax * q1;
  }
  auto products = [&](const _Float16 *sh, const _Float16 *sl, const float *sn, bool &exact)
      __attribute__((always_inline)) {
    f32x16 acc = {};
    const _Float16 *hb = sh + m * PITCH + 8 * h;
    const _Float16 *lb = sl + m * PITCH + 8 * h;
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = mfma32(*(const half8 *)(hb + 16 * s), qh[s], acc);
    bool pass = false;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 k4 = *(const f32x4 *)&sn[8 * g + h4];
#pragma unroll
      for (int j = 0; j < 4; ++j) pass = pass || (acc[4 * g + j] + marg) * k4[j] > thq;
    }
    exact = __ballot(pass) != 0;
    if (exact) {
      // fragments of four K steps in flight at a time (register budget)
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const half8 ah = *(const half8 *)(hb + 16 * s);
        const half8 al = *(const half8 *)(lb + 16 * s);
        acc = mfma32(al, qh[s], acc);
        acc = mfma32(ah, ql[s], acc);
        if ((s & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      }
    }
    return acc;
  };
  // selection on tile t0 (three-product scores); lane (m, h) holds query m
  // and keys 8*(r/4) + 4*h + r%4 of the tile
  auto select = [&](const f32x16 &acc, int t0, const float *sn) __attribute__((always_inline)) {
    float pr[16];
    uint64_t rm[16];      // per row: lanes whose product passes the bound
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 k4 = *(const f32x4 *)&sn[8 * g + h4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pr[4 * g + j] = acc[4 * g + j] * k4[j];
        rm[4 * g + j] = __ballot(pr[4 * g + j] > thq);
      }
    }
    // Few rows have candidates once the lists are warm: a scalar loop visits
    // only rows with a passing lane, and room is made before each append.
    uint64_t any = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) any |= rm[r];
    if (any != 0) {
      uint32_t act = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) act |= (rm[r] != 0 ? 1u : 0u) << r;
      while (act != 0) {
        const int r = __builtin_ctz(act);
        act &= act - 1;
        if (__ballot(cnt >= kCand) != 0) flush();
        const float v = pr[r];
        if (v > thq) {
          const int kb = (int)(a.key_base + k_begin) + t0 + 8 * (r >> 2) + (r & 3);
          sq[32 * cnt] = pack_entry(v * qf, kb + h4);
          ++cnt;
        }
      }
    }
  };

  // The two waves that share a SIMD (w and w + 4 when waves are dealt round
  // robin, 2k and 2k + 1 when dealt in pairs) take each tile period in
  // opposite orders:
  //   first wave:  products(t), select(t), decode(t + 1)
  //   second wave: select(t - 1), decode(t + 1), products(t)
  // with one barrier per tile.  gfx950 does not run one wave's MFMA alongside
  // another wave's VALU work on the same SIMD, so the skew does not hide
  // VALU time; it keeps the two waves from contending for the matrix unit,
  // LDS and the barrier at the same moments.  Tile buffers alternate; norms rotate over
  // three buffers, so the second wave's select(t - 1) never reads the norms
  // that decode(t + 1) writes.
  // A tile whose products stopped at hi x hi has no lane that passes (the
  // bounds only rise), so its selection is skipped.
  const bool mfma_first = ((w ^ (w >> 2)) & 1) == 0;
  f32x16 pend = {};                    // second wave: products of the previous tile
  bool pend_exact = false;
  auto step = [&](int t0, const _Float16 *sh, const _Float16 *sl, _Float16 *dh, _Float16 *dl)
      __attribute__((always_inline)) {
    const int ti = t0 >> 5;
    float *kn_cur = kn[ti % 3];
    float *kn_next = kn[(ti + 1) % 3];
    if (mfma_first) {
      bool exact;
      const f32x16 acc = products(sh, sl, kn_cur, exact);
      if (exact) select(acc, t0, kn_cur);
      decode_tile(t0 + 32, dh, dl, kn_next);
      load_tile(t0 + 64);
    } else {
      if (t0 > 0 && pend_exact) select(pend, t0 - 32, kn[(ti + 2) % 3]);
      decode_tile(t0 + 32, dh, dl, kn_next);
      load_tile(t0 + 64);
      pend = products(sh, sl, kn_cur, pend_exact);
    }
    __syncthreads();
  };

  load_tile(0);
  __syncthreads();                     // pair table ready
  decode_tile(0, ch0, cl0, kn[0]);
  load_tile(32);
  __syncthreads();
  int t_last = 0;
  for (int t0 = 0; t0 < n_keys; t0 += 64) {
    step(t0, ch0, cl0, ch1, cl1);      // tile t0 in buffer 0, decode t0 + 32 into 1
    t_last = t0;
    if (t0 + 32 >= n_keys) break;
    step(t0 + 32, ch1, cl1, ch0, cl0);
    t_last = t0 + 32;
  }
  if (!mfma_first && n_keys > 0 && pend_exact) select(pend, t_last, kn[(t_last >> 5) % 3]);
  if (__ballot(cnt > 0) != 0) flush();
  if (h == 0 && qvalid) {
    const int64_t qrow = (int64_t)stream * a.group + gq;
    float *outv = a.part_val + ((int64_t)(a.split_base + split) * a.n_rows + qrow) * kTop;
    int32_t *outi = a.part_idx + ((int64_t)(a.split_base + split) * a.n_rows + qrow) * kTop;
#pragma unroll
    for (int j = 0; j < kTop; ++j) {
      float s;
      int ix;
      unpack_entry(lq[32 * j], s, ix);
      outv[j] = s;
      outi[j] = ix;
    }
  }
}

struct MergeArgs {
  const float *part_val;
  const int32_t *part_idx;
  int64_t n_rows;      // n_streams * group
  int n_splits, topk, group, n_q_heads, n_kv_heads;
  float *out_val;
  int32_t *out_idx;
};

// One wave per query: lane s holds the head of split s's sorted list, and
// each output is the best head (wave butterfly; ties on the key index, then
// on the split); the winning lane moves to its next entry.
__global__ __launch_bounds__(256) void search_merge_kernel(MergeArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  if (row >= a.n_rows) return;
  const bool has = lane < a.n_splits;
  const int64_t base = ((int64_t)(has ? lane : 0) * a.n_rows + row) * kTop;
  const float *pv = a.part_val + base;
  const int32_t *pi = a.part_idx + base;
  int pos = 0;
  float hv = has ? pv[0] : -INFINITY;
  int hi = has ? pi[0] : 0x7FFFFFFF;
  const int64_t stream = row / a.group;
  const int g = (int)(row % a.group);
  const int64_t b = stream / a.n_kv_heads;
  const int kvh = (int)(stream % a.n_kv_heads);
  const int64_t orow = b * a.n_q_heads + (int64_t)kvh * a.group + g;
  for (int i = 0; i < a.topk; ++i) {
    float bv = hv;
    int bi = hi, bl = lane;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      const int ol = __shfl_xor(bl, off);
      if (better(ov, oi, bv, bi) || (ov == bv && oi == bi && ol < bl)) { bv = ov; bi = oi; bl = ol; }
    }
    if (lane == 0) {
      a.out_val[orow * a.topk + i] = bv;
      a.out_idx[orow * a.topk + i] = bi;
    }
    if (lane == bl) {
      ++pos;
      hv = pos < kTop ? pv[pos] : -INFINITY;
      hi = pos < kTop ? pi[pos] : 0x7FFFFFFF;
    }
  }
}

// Launch plan of one search call.  A sample pass scores the first
// 1/16 of every stream's keys exactly and merges its lists into a seed, the
// topk-th best of the sample per query; the main pass scores the rest with
// the lists' bounds starting at the seed, so that after the sample almost
// no tile needs more than the hi x hi product.  A final merge takes the
// lists of both passes.  Each pass has its own key splits (so that the
// workgroups fill the chip in whole rounds: the cost of a split count is
// (rounds of resident workgroups) x (tiles per split + a fixed allowance for
// filling the lists)); together at most 64 (lanes of the merge).
struct SearchPass {
  int64_t key_base, seq_len, splits, kps;
};

struct SearchPlan {
  SearchPass sample, main;
  int64_t n_rows, n_queries, q_tiles;
  size_t qbytes, qfac_off, seed_val_off, seed_idx_off, pv_off, pi_off, bytes;
};

SearchPass plan_pass(int64_t base_blocks, int64_t key_base, int64_t seq_len, int64_t cap) {
  SearchPass p;
  p.key_base = key_base;
  p.seq_len = seq_len;
  const int64_t cus = tqi::device_cu_count();
  const int64_t n_tiles = (seq_len + 31) / 32;
  int64_t max_splits = (seq_len + 4095) / 4096;
  if (max_splits > cap) max_splits = cap;
  if (max_splits < 1) max_splits = 1;
  int64_t splits = 1, best = -1;
  for (int64_t sp = 1; sp <= max_splits; ++sp) {
    const int64_t rounds = (base_blocks * sp + cus - 1) / cus;
    const int64_t cost = rounds * ((n_tiles + sp - 1) / sp + 16);
    if (best < 0 || cost < best) { best = cost; splits = sp; }
  }
  int64_t kps = (seq_len + splits - 1) / splits;
  kps = (kps + 31) / 32 * 32;
  p.kps = kps > 0 ? kps : 32;
  p.splits = seq_len > 0 ? (seq_len + p.kps - 1) / p.kps : 0;
  return p;
}

SearchPlan search_plan(int batch, int n_q_heads, int n_kv_heads, int64_t seq_len, int d) {
  SearchPlan p;
  const int group = n_q_heads / n_kv_heads;
  const int64_t n_streams = (int64_t)batch * n_kv_heads;
  p.n_queries = (int64_t)batch * n_q_heads;
  p.q_tiles = (group + kSearchQueries - 1) / kSearchQueries;
  const int64_t base_blocks = n_streams * p.q_tiles;
  // sample: a whole number of 32-key tiles, none below 1024 keys
  const int64_t n_sample = seq_len >= 1024 ? ((seq_len + 15) / 16 + 31) / 32 * 32 : 0;
  p.sample = plan_pass(base_blocks, 0, n_sample, 16);
  p.main = plan_pass(base_blocks, n_sample, seq_len - n_sample, 64 - p.sample.splits);
  p.n_rows = n_streams * group;
  const int64_t total = p.sample.splits + p.main.splits;
  p.qbytes = tqi::ws_align((size_t)p.n_queries * d * sizeof(_Float16));
  p.qfac_off = 2 * p.qbytes;
  p.seed_val_off = p.qfac_off + tqi::ws_align((size_t)p.n_queries * sizeof(float));
  const size_t seed_bytes = p.sample.splits > 0 ? tqi::ws_align((size_t)p.n_rows * kTop * sizeof(float)) : 0;
  p.seed_idx_off = p.seed_val_off + seed_bytes;
  p.pv_off = p.seed_idx_off + seed_bytes;
  p.pi_off = p.pv_off + tqi::ws_align((size_t)total * p.n_rows * kTop * sizeof(float));
  p.bytes = p.pi_off + tqi::ws_align((size_t)total * p.n_rows * kTop * sizeof(int32_t));
  return p;
}

template <int D, int LB>
hipError_t launch_t(const tqi::SearchArgs &sa, hipStream_t s) {
  const tqi::LogitArgs &a = sa.base;
  const int group = a.n_q_heads / a.n_kv_heads;
  const int64_t n_streams = (int64_t)a.batch * a.n_kv_heads;
  const SearchPlan plan = search_plan(a.batch, a.n_q_heads, a.n_kv_heads, a.seq_len, D);
  const int64_t n_queries = plan.n_queries;
  const int q_tiles = (int)plan.q_tiles;
  const int64_t base_blocks = n_streams * q_tiles;
  // Key indices fit the packed list entries (30 bits); per-split byte offsets
  // of the packed codes stay below 2^31 (both checked by search_supported).
  const int64_t n_rows = plan.n_rows;
  if (a.workspace_bytes < plan.bytes || (plan.bytes > 0 && a.workspace == nullptr)) return hipErrorInvalidValue;
  char *ws = (char *)a.workspace;
  hipError_t e = hipSuccess;
  QPrepArgs pa;
  pa.q = a.q;
  pa.q_f32 = a.q_f32;
  pa.n_queries = n_queries;
  pa.pi = a.pi;
  pa.qh = (_Float16 *)ws;
  pa.ql = (_Float16 *)(ws + plan.qbytes);
  pa.qfac = (float *)(ws + plan.qfac_off);
  float *seed_val = (float *)(ws + plan.seed_val_off);
  int32_t *seed_idx = (int32_t *)(ws + plan.seed_idx_off);
  float *pv = (float *)(ws + plan.pv_off);
  int32_t *pi = (int32_t *)(ws + plan.pi_off);
  hipLaunchKernelGGL((search_prep_kernel<D>), dim3((unsigned)((n_queries + kPrepQueries - 1) / kPrepQueries)),
                     dim3(D), 0, s, pa);
  e = hipGetLastError();
  auto score = [&](const SearchPass &ps, int split_base, const float *seed) {
    ScoreArgs sc;
    sc.qh = pa.qh;
    sc.ql = pa.ql;
    sc.qfac = pa.qfac;
    sc.centroids = a.centroids;
    sc.codes = a.codes;
    sc.norm = a.norm;
    sc.row_tokens = a.row_tokens;
    sc.seq_len = ps.seq_len;
    sc.keys_per_split = ps.kps;
    sc.n_rows = n_rows;
    sc.key_base = ps.key_base;
    sc.n_splits = (int)ps.splits;
    sc.q_tiles = q_tiles;
    sc.n_kv_heads = a.n_kv_heads;
    sc.n_q_heads = a.n_q_heads;
    sc.group = group;
    sc.split_base = split_base;
    sc.scale = a.scale;
    sc.topk = sa.topk;
    sc.seed = seed;
    sc.part_val = pv;
    sc.part_idx = pi;
    hipLaunchKernelGGL((search_score_kernel<D, LB>), dim3((unsigned)(base_blocks * ps.splits)),
                       dim3(kSearchThreads), 0, s, sc);
    return hipGetLastError();
  };
  auto merge = [&](int n_splits, float *out_val, int32_t *out_idx) {
    MergeArgs ma;
    ma.part_val = pv;
    ma.part_idx = pi;
    ma.n_rows = n_rows;
    ma.n_splits = n_splits;
    ma.topk = sa.topk;
    ma.group = group;
    ma.n_q_heads = a.n_q_heads;
    ma.n_kv_heads = a.n_kv_heads;
    ma.out_val = out_val;
    ma.out_idx = out_idx;
    hipLaunchKernelGGL(search_merge_kernel, dim3((unsigned)((n_rows + 3) / 4)), dim3(256), 0, s, ma);
    return hipGetLastError();
  };
  // (the main pass is never empty: the sample is at most seq_len / 16 + 32
  // keys, and a call has seq_len >= topk >= 1)
  const int ns = (int)plan.sample.splits;
  if (e == hipSuccess && ns > 0) e = score(plan.sample, 0, nullptr);
  if (e == hipSuccess && ns > 0) e = merge(ns, seed_val, seed_idx);
  if (e == hipSuccess) e = score(plan.main, ns, ns > 0 ? seed_val : nullptr);
  if (e == hipSuccess) e = merge(ns + (int)plan.main.splits, a.logits, sa.topk_idx);
  return e;
}

template <int D>
hipError_t launch_lb(int lb, const tqi::SearchArgs &a, hipStream_t s) {
  switch (lb) {
    case 1: return launch_t<D, 1>(a, s);
    case 2: return launch_t<D, 2>(a, s);
    case 3: return launch_t<D, 3>(a, s);
    case 4: return launch_t<D, 4>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

namespace tqi {

bool search_supported(int d, int lbits, int topk, int batch, int n_q_heads, int n_kv_heads, int64_t seq_len) {
  if (d != 64 && d != 128 && d != 256) return false;
  if (lbits < 1 || lbits > 4 || topk < 1 || topk > kTop) return false;
  if (seq_len >= (1LL << 30)) return false;        // key index in 30 bits of a list entry
  // per-split byte offsets of the packed codes (one split plus one tile of
  // prefetch) below 2^31
  const SearchPlan p = search_plan(batch, n_q_heads, n_kv_heads, seq_len, d);
  const int64_t kps = p.main.kps > p.sample.kps ? p.main.kps : p.sample.kps;
  return (kps + 64) * (int64_t)(lbits * d / 8) < (1LL << 31);
}

size_t search_workspace_bytes(int d, int lbits, int batch, int n_q_heads, int n_kv_heads, int64_t seq_len) {
  (void)lbits;
  return search_plan(batch, n_q_heads, n_kv_heads, seq_len, d).bytes;
}

hipError_t launch_search(int d, int lbits, const SearchArgs &a, hipStream_t s) {
  if (d == 64) return launch_lb<64>(lbits, a, s);
  if (d == 128) return launch_lb<128>(lbits, a, s);
  if (d == 256) return launch_lb<256>(lbits, a, s);
  return hipErrorInvalidValue;
}

}  // namespace tqi
