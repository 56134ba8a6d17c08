// Attention logits straight from polar-format keys (the PolarQuant variant
// of stage 1: page "TurboQuant 설명: 무엇인지와 LLM 메모리 6배 절약 구현 방법",
// section "1단계: 무작위 회전 + PolarQuant 압축"; the query is rotated once and
// the logits come from the indices, closing paragraph of "2단계: QJL 잔차 보정"
// and "TurboQuant 구현 방법"):
//   logit = scale * n16 * <Pi q, y_hat>,
// y_hat the unit vector the key's angles describe.  Every coordinate of y_hat
// is a product of one cos or sin per level along the path from the top of
// the angle tree, so no key is reconstructed in memory:
// * a query preparation launch writes q' = Pi q of every query head (fp32
//   sums of exact fp32 products) and the cos/sin of every centroid angle
//   (sector midpoints 2 pi (j + 1/2) / 16 of level 1, the codebook angles of
//   levels 2..L, in fp64, rounded once) to the caller's workspace;
// * the streaming launch gives every key one thread: it walks the levels
//   above 4 top-down to the d/16 radii of level 4, then each subtree of
//   16 coordinates down to its coordinates, and accumulates them against
//   the group's rotated queries, which every thread reads at the same LDS
//   address (broadcast).
// The cos/sin tables sit in LDS as (cos, sin) pairs: 16 for level 1 (32
// banks, so any mix of indices is conflict-free) and 4 per higher level.
#include "tq_device.h"
#include "tq_internal.h"

namespace {

using namespace tqd;

constexpr int kPolarThreads = 256;     // one key per thread

template <int D>
struct PLayout {
  static constexpr int L = D == 64 ? 6 : (D == 128 ? 7 : 8);  // levels
  static constexpr int RB = 3 * D / 8;                         // bytes per key
  static constexpr int W = RB / 4;                             // words per key
  static constexpr int UW = D / 16;                            // first word of the higher-level planes
  static constexpr int NT = 16 + 4 * (L - 1);                  // (cos, sin) pairs
  static constexpr int NR = D / 16;                            // level-4 radii (subtrees)
  // first slot of the angles of level l >= 2 among the higher indices
  __host__ __device__ static constexpr int slot(int level) { return D / 2 - (D >> (level - 1)); }
};

struct PolarPrepArgs {
  const void *q;
  bool q_f32;
  int n_q_heads, n_kv_heads, group;
  const float *pi;
  const float *centroids;   // levels 2..L, 4 angles each
  float *qrot;              // [stream][group][D]
  float *trig;              // [NT][2]
};

// One workgroup per (stream, query of its group): thread j < D forms
// (Pi q)_j from row j of Pi; workgroup 0 also writes the cos/sin table.
template <int D>
__global__ __launch_bounds__(kPolarThreads) void polar_prep_kernel(PolarPrepArgs a) {
  using P = PLayout<D>;
  __shared__ __attribute__((aligned(16))) float qs[D];
  const int stream = blockIdx.x / a.group;
  const int g = blockIdx.x % a.group;
  const int b = stream / a.n_kv_heads, kvh = stream % a.n_kv_heads;
  const int tid = threadIdx.x;
  const int64_t qoff = ((int64_t)b * a.n_q_heads + (int64_t)kvh * a.group + g) * D;
  for (int k = tid; k < D; k += kPolarThreads)
    qs[k] = a.q_f32 ? ((const float *)a.q)[qoff + k] : bf16_to_f32(((const uint16_t *)a.q)[qoff + k]);
  if (blockIdx.x == 0 && tid < P::NT) {
    double ang;
    if (tid < 16) {
      ang = 2.0 * M_PI * (tid + 0.5) / 16.0;
    } else {
      ang = (double)a.centroids[tid - 16];
    }
    a.trig[2 * tid] = (float)cos(ang);
    a.trig[2 * tid + 1] = (float)sin(ang);
  }
  __syncthreads();
  if (tid < D) {
    const f32x4 *row = (const f32x4 *)(a.pi + (size_t)tid * D);
    float acc = 0.0f;
#pragma unroll 8
    for (int k = 0; k < D / 4; ++k) {
      const f32x4 m = row[k];
      const f32x4 v = *(const f32x4 *)&qs[4 * k];
      acc = fmaf(m[0], v[0], acc);
      acc = fmaf(m[1], v[1], acc);
      acc = fmaf(m[2], v[2], acc);
      acc = fmaf(m[3], v[3], acc);
    }
    a.qrot[((int64_t)stream * a.group + g) * D + tid] = acc;
  }
}

struct PolarStreamArgs {
  const float *qrot;
  const float *trig;
  const uint8_t *codes;
  const uint16_t *norm;
  int64_t row_tokens, seq_len;
  int n_q_heads, n_kv_heads, group;
  int blocks_per_stream;
  float scale;
  float *logits;
};

// Bits 0..7 of x moved to bits 0, 4, ..., 28.
__device__ __forceinline__ uint32_t spread_nibbles(uint32_t x) {
  x &= 0xFFu;
  x = (x | (x << 12)) & 0x000F000Fu;
  x = (x | (x << 6)) & 0x03030303u;
  x = (x | (x << 3)) & 0x11111111u;
  return x;
}

// 2-bit index of higher slot s from its group's two plane words
__device__ __forceinline__ uint32_t upper_index(uint32_t p0, uint32_t p1, int bit) {
  return ((p0 >> bit) & 1u) | (((p1 >> bit) & 1u) << 1);
}

template <int D, int NQ>
__global__ __launch_bounds__(kPolarThreads) void polar_logit_kernel(PolarStreamArgs a) {
  using P = PLayout<D>;
  __shared__ __attribute__((aligned(16))) float qs[NQ][D];
  __shared__ __attribute__((aligned(16))) float2 trig[P::NT];
  // the keys' words and level-4 radii, word-major so that the threads of a
  // wave read consecutive banks
  __shared__ uint32_t wl[P::W][kPolarThreads];
  __shared__ float rl[P::NR][kPolarThreads];
  const int stream = blockIdx.x / a.blocks_per_stream;
  const int kb = blockIdx.x % a.blocks_per_stream;
  const int tid = threadIdx.x;
  const int b = stream / a.n_kv_heads, kvh = stream % a.n_kv_heads;
  for (int i = tid; i < NQ * D; i += kPolarThreads) {
    const int g = i / D, k = i % D;
    qs[g][k] = g < a.group ? a.qrot[((int64_t)stream * a.group + g) * D + k] : 0.0f;
  }
  if (tid < P::NT) trig[tid] = make_float2(a.trig[2 * tid], a.trig[2 * tid + 1]);

  // the stream's packed keys (the first seq_len rows) and its logits; a key
  // past seq_len reads zeros and stores nothing
  const int64_t t = (int64_t)kb * kPolarThreads + tid;
  const bool live = t < a.seq_len;
  const i32x4 rc = make_rsrc(a.codes + (size_t)stream * a.row_tokens * P::RB, (uint32_t)(a.seq_len * P::RB));
  const i32x4 rn = make_rsrc(a.norm + (size_t)stream * a.row_tokens, (uint32_t)(a.seq_len * 2));
  const uint32_t off = live ? (uint32_t)(t * P::RB) : kNoStore;
  uint32_t w[P::W];
  if constexpr (P::W == 6) {
    uint32_t x[2], y[4];
    buf_load_words<2>(rc, off, x);
    buf_load_words<4>(rc, off + 8, y);
    w[0] = x[0]; w[1] = x[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[2 + i] = y[i];
  } else {
#pragma unroll
    for (int c = 0; c < P::W / 4; ++c) {
      uint32_t y[4];
      buf_load_words<4>(rc, off + 16 * c, y);
#pragma unroll
      for (int i = 0; i < 4; ++i) w[4 * c + i] = y[i];
    }
  }
  const float nrm = f16_bits_to_f32(buf_load_u16(rn, live ? (uint32_t)(t * 2) : kNoStore));
#pragma unroll
  for (int i = 0; i < P::W; ++i) wl[i][tid] = w[i];
  __syncthreads();

  // radii of level 4, top-down from radius 1 (in place: node i of a level
  // becomes nodes 2i and 2i + 1 of the next one down)
  {
    float r[P::NR];
    r[0] = 1.0f;
#pragma unroll
    for (int level = P::L; level >= 5; --level) {
      const int cnt = D >> level;
#pragma unroll
      for (int i = cnt - 1; i >= 0; --i) {
        const int sl = P::slot(level) + i;
        const int wd = P::UW + 2 * (sl / 32);
        const float2 cs = trig[16 + 4 * (level - 2) + upper_index(w[wd], w[wd + 1], sl % 32)];
        const float v = r[i];
        r[2 * i + 1] = v * cs.y;
        r[2 * i] = v * cs.x;
      }
    }
#pragma unroll
    for (int m = 0; m < P::NR; ++m) rl[m][tid] = r[m];
  }

  // one subtree of 16 coordinates at a time: level 4 angle m, level 3
  // angles 2m, 2m + 1, level 2 angles 4m .. 4m + 3, level-1 pairs 8m .. 8m + 7
  float acc[NQ];
#pragma unroll
  for (int g = 0; g < NQ; ++g) acc[g] = 0.0f;
#pragma unroll 1
  for (int m = 0; m < P::NR; ++m) {
    const float r4 = rl[m][tid];
    float r3[2], r2[4], r1[8];
    {
      const int sl = P::slot(4) + m;
      const int wd = P::UW + 2 * (sl >> 5);
      const float2 cs = trig[16 + 4 * 2 + upper_index(wl[wd][tid], wl[wd + 1][tid], sl & 31)];
      r3[0] = r4 * cs.x;
      r3[1] = r4 * cs.y;
    }
    {
      const int sl = P::slot(3) + 2 * m;              // even: both angles in one group
      const int wd = P::UW + 2 * (sl >> 5);
      const uint32_t p0 = wl[wd][tid], p1 = wl[wd + 1][tid];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float2 cs = trig[16 + 4 * 1 + upper_index(p0, p1, (sl & 31) + i)];
        r2[2 * i] = r3[i] * cs.x;
        r2[2 * i + 1] = r3[i] * cs.y;
      }
    }
    {
      const int sl = P::slot(2) + 4 * m;              // a multiple of 4: one group
      const int wd = P::UW + 2 * (sl >> 5);
      const uint32_t p0 = wl[wd][tid], p1 = wl[wd + 1][tid];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float2 cs = trig[16 + upper_index(p0, p1, (sl & 31) + i)];
        r1[2 * i] = r2[i] * cs.x;
        r1[2 * i + 1] = r2[i] * cs.y;
      }
    }
    // level-1 sector indices of the 8 pairs as the nibbles of one word
    // (plane p of group g at word 4 g + p)
    const int grp = m >> 2, sh = 8 * (m & 3);
    const uint32_t nib = spread_nibbles(wl[4 * grp][tid] >> sh) | (spread_nibbles(wl[4 * grp + 1][tid] >> sh) << 1) |
                         (spread_nibbles(wl[4 * grp + 2][tid] >> sh) << 2) |
                         (spread_nibbles(wl[4 * grp + 3][tid] >> sh) << 3);
    float y[16];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float2 cs = trig[(nib >> (4 * k)) & 15u];
      y[2 * k] = r1[k] * cs.x;
      y[2 * k + 1] = r1[k] * cs.y;
    }
#pragma unroll
    for (int g = 0; g < NQ; ++g) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 qv = *(const f32x4 *)&qs[g][16 * m + 4 * j];
        acc[g] = fmaf(qv[0], y[4 * j], acc[g]);
        acc[g] = fmaf(qv[1], y[4 * j + 1], acc[g]);
        acc[g] = fmaf(qv[2], y[4 * j + 2], acc[g]);
        acc[g] = fmaf(qv[3], y[4 * j + 3], acc[g]);
      }
    }
  }

  // logits [batch][n_q_heads][seq_len]: this stream's group of rows
  float *lbase = a.logits + ((int64_t)b * a.n_q_heads + (int64_t)kvh * a.group) * a.seq_len;
  const i32x4 ro = make_rsrc(lbase, (uint32_t)(a.group * a.seq_len * 4));
  const float f = nrm * a.scale;
#pragma unroll
  for (int g = 0; g < NQ; ++g) {
    if (g < a.group)
      buf_store_f32(ro, live ? (uint32_t)((g * a.seq_len + t) * 4) : kNoStore, acc[g] * f);
  }
}

template <int D>
hipError_t launch_d(const tqi::LogitArgs &a, hipStream_t s) {
  const int group = a.n_q_heads / a.n_kv_heads;
  const int n_streams = a.batch * a.n_kv_heads;
  if (a.workspace == nullptr ||
      a.workspace_bytes < tqi::polar_logits_workspace_bytes(D, n_streams, group))
    return hipErrorInvalidValue;
  float *qrot = (float *)a.workspace;
  float *trig = (float *)((char *)a.workspace + tqi::ws_align((size_t)n_streams * group * D * sizeof(float)));
  PolarPrepArgs pa;
  pa.q = a.q;
  pa.q_f32 = a.q_f32;
  pa.n_q_heads = a.n_q_heads;
  pa.n_kv_heads = a.n_kv_heads;
  pa.group = group;
  pa.pi = a.pi;
  pa.centroids = a.centroids;
  pa.qrot = qrot;
  pa.trig = trig;
  hipLaunchKernelGGL((polar_prep_kernel<D>), dim3((unsigned)(n_streams * group)), dim3(kPolarThreads), 0, s, pa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  PolarStreamArgs sa;
  sa.qrot = qrot;
  sa.trig = trig;
  sa.codes = a.codes;
  sa.norm = a.norm;
  sa.row_tokens = a.row_tokens;
  sa.seq_len = a.seq_len;
  sa.n_q_heads = a.n_q_heads;
  sa.n_kv_heads = a.n_kv_heads;
  sa.group = group;
  sa.blocks_per_stream = (int)((a.seq_len + kPolarThreads - 1) / kPolarThreads);
  sa.scale = a.scale;
  sa.logits = a.logits;
  const int64_t blocks = (int64_t)n_streams * sa.blocks_per_stream;
  if (group <= 4)
    hipLaunchKernelGGL((polar_logit_kernel<D, 4>), dim3((unsigned)blocks), dim3(kPolarThreads), 0, s, sa);
  else if (group <= 8)
    hipLaunchKernelGGL((polar_logit_kernel<D, 8>), dim3((unsigned)blocks), dim3(kPolarThreads), 0, s, sa);
  else
    hipLaunchKernelGGL((polar_logit_kernel<D, 16>), dim3((unsigned)blocks), dim3(kPolarThreads), 0, s, sa);
  return hipGetLastError();
}

}  // namespace

namespace tqi {

bool polar_logits_supported(int d, int group, int64_t seq_len, int64_t n_streams) {
  if (d != 64 && d != 128 && d != 256) return false;
  if (group < 1 || group > 16) return false;
  // 32-bit byte ranges of one stream's codes and logits, and the grid size
  if (seq_len * (3 * d / 8) >= (1LL << 31)) return false;
  if ((int64_t)group * seq_len * 4 >= (1LL << 31)) return false;
  if (n_streams * ((seq_len + kPolarThreads - 1) / kPolarThreads) >= (1LL << 31)) return false;
  return true;
}

size_t polar_logits_workspace_bytes(int d, int64_t n_streams, int group) {
  const int levels = d == 64 ? 6 : (d == 128 ? 7 : 8);
  return ws_align((size_t)n_streams * group * d * sizeof(float)) + ws_align((size_t)(16 + 4 * (levels - 1)) * 8);
}

hipError_t launch_polar_logits(int d, const LogitArgs &a, hipStream_t s) {
  if (d == 64) return launch_d<64>(a, s);
  if (d == 128) return launch_d<128>(a, s);
  if (d == 256) return launch_d<256>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace tqi
