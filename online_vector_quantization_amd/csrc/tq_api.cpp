// C ABI entry points on the device: argument validation and dispatch to the
// gfx950 kernels.  Declarations, layouts and error behaviour: include/tq.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <map>
#include <mutex>
#include <utility>

#include "tq.h"
#include "tq_internal.h"

namespace tqi {

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cu = 0;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
    cu = 256;
  if (dev < 64) cache[dev].store(cu, std::memory_order_relaxed);
  return cu;
}

hipError_t workspace(hipStream_t s, size_t bytes, void **out) {
  struct Buf {
    void *ptr = nullptr;
    size_t size = 0;
  };
  static std::mutex mu;
  static std::map<std::pair<int, hipStream_t>, Buf> bufs;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  Buf &b = bufs[std::make_pair(dev, s)];
  if (b.size < bytes) {
    if (b.ptr != nullptr) {
      e = hipStreamSynchronize(s);
      if (e != hipSuccess) return e;
      e = hipFree(b.ptr);
      if (e != hipSuccess) return e;
      b.ptr = nullptr;
      b.size = 0;
    }
    size_t want = bytes + bytes / 4;
    want = (want + (1u << 20) - 1) & ~(size_t)((1u << 20) - 1);
    e = hipMalloc(&b.ptr, want);
    if (e != hipSuccess) {
      b.ptr = nullptr;
      return e;
    }
    b.size = want;
  }
  *out = b.ptr;
  return hipSuccess;
}

}  // namespace tqi

namespace {

// Lloyd-Max bits for (bits, mode), or -1 when the pair is invalid.
int lloyd_bits(const tq_params *p) {
  if (p->mode == TQ_MODE_MSE) return (p->bits >= 1 && p->bits <= 4) ? p->bits : -1;
  if (p->mode == TQ_MODE_PROD) return (p->bits >= 2 && p->bits <= 5) ? p->bits - 1 : -1;
  if (p->mode == TQ_MODE_POLAR) return p->bits == 3 ? 2 : -1;   // 2 bits per higher-level angle
  return -1;
}

bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }

tq_status check_params(const tq_params *p) {
  if (p == nullptr) return TQ_ERR_INVALID;
  if (p->reserved != 0 || p->d <= 0) return TQ_ERR_INVALID;
  if (lloyd_bits(p) < 0) return TQ_ERR_INVALID;
  if (p->pi == nullptr || p->centroids == nullptr || p->boundaries == nullptr) return TQ_ERR_INVALID;
  return TQ_OK;
}

tq_status hip_status(hipError_t e) { return e == hipSuccess ? TQ_OK : TQ_ERR_HIP; }

}  // namespace

extern "C" tq_status tq_quantize_kv(const tq_params *p, const void *x, int32_t x_dtype,
                                    int64_t n_vec, int64_t x_row_stride, const tq_packed *out,
                                    int64_t out_offset, void *stream) {
  tq_status st = check_params(p);
  if (st != TQ_OK) return st;
  const bool prod = p->mode == TQ_MODE_PROD;
  if (out == nullptr || n_vec < 0 || out_offset < 0) return TQ_ERR_INVALID;
  if (x_dtype != TQ_F32 && x_dtype != TQ_BF16) return TQ_ERR_INVALID;
  if (n_vec == 0) return TQ_OK;
  if (x == nullptr || out->codes == nullptr || out->norm == nullptr) return TQ_ERR_INVALID;
  if (x_row_stride < p->d) return TQ_ERR_INVALID;
  if (prod && (p->qjl_rot == nullptr || out->rnorm == nullptr)) return TQ_ERR_INVALID;
  const int esz = x_dtype == TQ_F32 ? 4 : 2;
  if (!aligned16(x) || (x_row_stride * esz) % 16 != 0) return TQ_ERR_UNSUPPORTED;
  if ((uintptr_t)out->codes & 3u) return TQ_ERR_UNSUPPORTED;
  tqi::QuantizeArgs a;
  a.x = x;
  a.n_vec = n_vec;
  a.x_stride = x_row_stride;
  a.pi = p->pi;
  a.m = p->qjl_rot;
  a.centroids = p->centroids;
  a.boundaries = p->boundaries;
  a.codes = out->codes;
  a.norm = out->norm;
  a.rnorm = out->rnorm;
  a.out_offset = out_offset;
  bool ok = false;
  hipError_t e;
  if (p->mode == TQ_MODE_POLAR)
    e = tqi::launch_quantize_polar(p->d, x_dtype == TQ_F32, a, (hipStream_t)stream, &ok);
  else
    e = tqi::launch_quantize(p->d, lloyd_bits(p), prod, x_dtype == TQ_F32, a, (hipStream_t)stream, &ok);
  if (!ok) return TQ_ERR_UNSUPPORTED;
  return hip_status(e);
}

extern "C" tq_status tq_attn_logits(const tq_params *p, const void *q, int32_t q_dtype,
                                    int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                    const tq_packed *k, int64_t row_tokens, int64_t seq_len,
                                    float scale, float *logits, int32_t topk, int32_t *topk_idx,
                                    void *stream) {
  tq_status st = check_params(p);
  if (st != TQ_OK) return st;
  if (p->mode == TQ_MODE_POLAR) return TQ_ERR_UNSUPPORTED;
  const bool prod = p->mode == TQ_MODE_PROD;
  if (k == nullptr || batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || topk < 0) return TQ_ERR_INVALID;
  if (n_q_heads % n_kv_heads != 0) return TQ_ERR_INVALID;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return TQ_ERR_INVALID;
  if (seq_len < 0 || row_tokens < seq_len) return TQ_ERR_INVALID;
  if (batch == 0 || seq_len == 0) return TQ_OK;
  if (q == nullptr || logits == nullptr || k->codes == nullptr || k->norm == nullptr) return TQ_ERR_INVALID;
  if (prod && (p->qjl == nullptr || k->rnorm == nullptr)) return TQ_ERR_INVALID;
  if (topk > 0 && (topk_idx == nullptr || seq_len < topk)) return TQ_ERR_INVALID;
  if ((uintptr_t)k->codes & 3u) return TQ_ERR_UNSUPPORTED;
  tqi::LogitArgs a;
  a.q = q;
  a.q_f32 = q_dtype == TQ_F32;
  a.batch = batch;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.pi = p->pi;
  a.s_mat = p->qjl;
  a.centroids = p->centroids;
  a.codes = k->codes;
  a.norm = k->norm;
  a.rnorm = k->rnorm;
  a.row_tokens = row_tokens;
  a.seq_len = seq_len;
  a.scale = scale;
  a.logits = logits;
  bool ok = false;
  hipError_t e;
  if (topk > 0) {
    if (prod) return TQ_ERR_UNSUPPORTED;
    tqi::SearchArgs sa;
    sa.base = a;
    sa.topk = topk;
    sa.topk_idx = topk_idx;
    e = tqi::launch_search(p->d, lloyd_bits(p), sa, (hipStream_t)stream, &ok);
  } else {
    e = tqi::launch_logits(p->d, lloyd_bits(p), prod, a, (hipStream_t)stream, &ok);
  }
  if (!ok) return TQ_ERR_UNSUPPORTED;
  return hip_status(e);
}

extern "C" tq_status tq_append_attn_logits(const tq_params *p, const void *x_new, int32_t x_dtype,
                                           const void *q, int32_t q_dtype, int32_t batch,
                                           int32_t n_q_heads, int32_t n_kv_heads, const tq_packed *k,
                                           int64_t row_tokens, int64_t pos, float scale, float *logits,
                                           void *stream) {
  tq_status st = check_params(p);
  if (st != TQ_OK) return st;
  if (p->mode == TQ_MODE_POLAR) return TQ_ERR_UNSUPPORTED;
  const bool prod = p->mode == TQ_MODE_PROD;
  if (k == nullptr || batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0) return TQ_ERR_INVALID;
  if (n_q_heads % n_kv_heads != 0) return TQ_ERR_INVALID;
  if ((q_dtype != TQ_F32 && q_dtype != TQ_BF16) || (x_dtype != TQ_F32 && x_dtype != TQ_BF16))
    return TQ_ERR_INVALID;
  if (pos < 0 || pos >= row_tokens) return TQ_ERR_INVALID;
  if (batch == 0) return TQ_OK;
  if (x_new == nullptr || q == nullptr || logits == nullptr || k->codes == nullptr || k->norm == nullptr)
    return TQ_ERR_INVALID;
  if (prod && (p->qjl == nullptr || p->qjl_rot == nullptr || k->rnorm == nullptr)) return TQ_ERR_INVALID;
  if ((uintptr_t)k->codes & 3u) return TQ_ERR_UNSUPPORTED;
  tqi::LogitArgs a;
  a.q = q;
  a.q_f32 = q_dtype == TQ_F32;
  a.batch = batch;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.pi = p->pi;
  a.s_mat = p->qjl;
  a.centroids = p->centroids;
  a.codes = k->codes;
  a.norm = k->norm;
  a.rnorm = k->rnorm;
  a.row_tokens = row_tokens;
  a.seq_len = pos + 1;
  a.scale = scale;
  a.logits = logits;
  a.x_new = x_new;
  a.x_f32 = x_dtype == TQ_F32;
  a.boundaries = p->boundaries;
  a.m_mat = p->qjl_rot;
  a.codes_out = k->codes;
  a.norm_out = k->norm;
  a.rnorm_out = k->rnorm;
  a.pos = pos;
  bool ok = false;
  const hipError_t e = tqi::launch_logits(p->d, lloyd_bits(p), prod, a, (hipStream_t)stream, &ok);
  if (!ok) return TQ_ERR_UNSUPPORTED;
  return hip_status(e);
}

extern "C" tq_status tq_attn_output(const tq_params *p, const float *logits, int32_t batch,
                                    int32_t n_q_heads, int32_t n_kv_heads, const tq_packed *v,
                                    int64_t row_tokens, int64_t seq_len, void *out, int32_t out_dtype,
                                    void *stream) {
  tq_status st = check_params(p);
  if (st != TQ_OK) return st;
  if (p->mode == TQ_MODE_POLAR) return TQ_ERR_UNSUPPORTED;
  if (v == nullptr || batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0) return TQ_ERR_INVALID;
  if (n_q_heads % n_kv_heads != 0) return TQ_ERR_INVALID;
  if (out_dtype != TQ_F32 && out_dtype != TQ_BF16) return TQ_ERR_INVALID;
  if (seq_len < 0 || row_tokens < seq_len) return TQ_ERR_INVALID;
  if (batch == 0) return TQ_OK;
  if (out == nullptr) return TQ_ERR_INVALID;
  if (seq_len > 0 && (logits == nullptr || v->codes == nullptr || v->norm == nullptr)) return TQ_ERR_INVALID;
  if (p->mode != TQ_MODE_MSE) return TQ_ERR_UNSUPPORTED;
  if ((uintptr_t)v->codes & 15u) return TQ_ERR_UNSUPPORTED;
  tqi::AttendArgs a;
  a.logits = logits;
  a.batch = batch;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.pi = p->pi;
  a.centroids = p->centroids;
  a.codes = v->codes;
  a.norm = v->norm;
  a.row_tokens = row_tokens;
  a.seq_len = seq_len;
  a.out = out;
  a.out_f32 = out_dtype == TQ_F32;
  bool ok = false;
  hipError_t e = tqi::launch_attend(p->d, lloyd_bits(p), a, (hipStream_t)stream, &ok);
  if (!ok) return TQ_ERR_UNSUPPORTED;
  return hip_status(e);
}

extern "C" tq_status tq_dequantize(const tq_params *p, const tq_packed *k, int64_t n_vec, void *out,
                                   int32_t out_dtype, void *stream) {
  tq_status st = check_params(p);
  if (st != TQ_OK) return st;
  const bool prod = p->mode == TQ_MODE_PROD;
  if (k == nullptr || n_vec < 0) return TQ_ERR_INVALID;
  if (out_dtype != TQ_F32 && out_dtype != TQ_BF16) return TQ_ERR_INVALID;
  if (n_vec == 0) return TQ_OK;
  if (out == nullptr || k->codes == nullptr || k->norm == nullptr) return TQ_ERR_INVALID;
  if (prod && (p->qjl == nullptr || k->rnorm == nullptr)) return TQ_ERR_INVALID;
  tqi::DequantArgs a;
  a.pi = p->pi;
  a.s_mat = p->qjl;
  a.centroids = p->centroids;
  a.codes = k->codes;
  a.norm = k->norm;
  a.rnorm = k->rnorm;
  a.n_vec = n_vec;
  a.out = out;
  a.out_f32 = out_dtype == TQ_F32;
  bool ok = false;
  hipError_t e;
  if (p->mode == TQ_MODE_POLAR) {
    if (!aligned16(k->codes)) return TQ_ERR_UNSUPPORTED;
    e = tqi::launch_dequant_polar(p->d, a, (hipStream_t)stream, &ok);
  } else {
    e = tqi::launch_dequant(p->d, lloyd_bits(p), prod, a, (hipStream_t)stream, &ok);
  }
  if (!ok) return TQ_ERR_UNSUPPORTED;
  return hip_status(e);
}
