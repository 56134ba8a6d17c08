// C ABI entry points on the device: argument validation and dispatch to the
// gfx950 kernels.  Declarations, layouts and error behaviour: include/tq.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

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

// Argument checks common to the logit, append and search calls (before any
// shape or workspace check).
tq_status check_logit_args(const tq_params *p, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                           int64_t seq_len, int32_t topk) {
  tq_status st = check_params(p);
  if (st != TQ_OK) return st;
  if (batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || topk < 0 || seq_len < 0) return TQ_ERR_INVALID;
  if (n_q_heads % n_kv_heads != 0) return TQ_ERR_INVALID;
  return TQ_OK;
}

// TQ_OK when a kernel takes the shape, TQ_ERR_UNSUPPORTED otherwise.
tq_status logits_shape(const tq_params *p, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                       int64_t seq_len, int32_t topk) {
  if (p->mode == TQ_MODE_POLAR) {
    if (topk > 0) return TQ_ERR_UNSUPPORTED;
    return tqi::polar_logits_supported(p->d, n_q_heads / n_kv_heads, seq_len, (int64_t)batch * n_kv_heads)
               ? TQ_OK : TQ_ERR_UNSUPPORTED;
  }
  const bool prod = p->mode == TQ_MODE_PROD;
  if (topk > 0) {
    if (prod) return TQ_ERR_UNSUPPORTED;
    return tqi::search_supported(p->d, lloyd_bits(p), topk, batch, n_q_heads, n_kv_heads, seq_len)
               ? TQ_OK : TQ_ERR_UNSUPPORTED;
  }
  return tqi::logits_supported(p->d, lloyd_bits(p), prod, n_q_heads / n_kv_heads, seq_len) ? TQ_OK
                                                                                           : TQ_ERR_UNSUPPORTED;
}

size_t logits_ws_bytes(const tq_params *p, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                       int64_t seq_len, int32_t topk) {
  if (batch == 0 || seq_len == 0) return 0;
  if (p->mode == TQ_MODE_POLAR)
    return tqi::polar_logits_workspace_bytes(p->d, (int64_t)batch * n_kv_heads, n_q_heads / n_kv_heads);
  if (topk > 0) return tqi::search_workspace_bytes(p->d, lloyd_bits(p), batch, n_q_heads, n_kv_heads, seq_len);
  return tqi::logits_workspace_bytes(p->d, lloyd_bits(p), p->mode == TQ_MODE_PROD,
                                     (int64_t)batch * n_kv_heads, n_q_heads / n_kv_heads);
}

tq_status check_attend_args(const tq_params *p, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                            int64_t seq_len) {
  tq_status st = check_params(p);
  if (st != TQ_OK) return st;
  if (batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || seq_len < 0) return TQ_ERR_INVALID;
  if (n_q_heads % n_kv_heads != 0) return TQ_ERR_INVALID;
  if (p->mode != TQ_MODE_MSE) return TQ_ERR_UNSUPPORTED;
  return tqi::attend_supported(p->d, lloyd_bits(p), n_q_heads / n_kv_heads, seq_len) ? TQ_OK
                                                                                     : TQ_ERR_UNSUPPORTED;
}

// A workspace of `need` bytes: NULL is fine when nothing is needed;
// otherwise at least `need` bytes, 256-byte aligned.
tq_status check_workspace(const void *ws, size_t have, size_t need) {
  if (need == 0) return TQ_OK;
  if (ws == nullptr || have < need) return TQ_ERR_INVALID;
  if ((uintptr_t)ws & 255u) return TQ_ERR_UNSUPPORTED;
  return TQ_OK;
}

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

extern "C" tq_status tq_attn_logits_workspace_size(const tq_params *p, int32_t batch, int32_t n_q_heads,
                                                   int32_t n_kv_heads, int64_t seq_len, int32_t topk,
                                                   size_t *bytes) {
  if (bytes == nullptr) return TQ_ERR_INVALID;
  *bytes = 0;
  tq_status st = check_logit_args(p, batch, n_q_heads, n_kv_heads, seq_len, topk);
  if (st != TQ_OK) return st;
  st = logits_shape(p, batch, n_q_heads, n_kv_heads, seq_len, topk);
  if (st != TQ_OK) return st;
  *bytes = logits_ws_bytes(p, batch, n_q_heads, n_kv_heads, seq_len, topk);
  return TQ_OK;
}

extern "C" tq_status tq_attn_logits(const tq_params *p, const void *q, int32_t q_dtype,
                                    int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                    const tq_packed *k, int64_t row_tokens, int64_t seq_len,
                                    float scale, float *logits, int32_t topk, int32_t *topk_idx,
                                    void *workspace, size_t workspace_bytes, void *stream) {
  tq_status st = check_logit_args(p, batch, n_q_heads, n_kv_heads, seq_len, topk);
  if (st != TQ_OK) return st;
  const bool prod = p->mode == TQ_MODE_PROD;
  if (k == nullptr || row_tokens < seq_len) return TQ_ERR_INVALID;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return TQ_ERR_INVALID;
  st = logits_shape(p, batch, n_q_heads, n_kv_heads, seq_len, topk);
  if (st != TQ_OK) return st;
  if (batch == 0 || seq_len == 0) return TQ_OK;
  if (q == nullptr || logits == nullptr || k->codes == nullptr || k->norm == nullptr) return TQ_ERR_INVALID;
  if (prod && (p->qjl == nullptr || k->rnorm == nullptr)) return TQ_ERR_INVALID;
  if (topk > 0 && (topk_idx == nullptr || seq_len < topk)) return TQ_ERR_INVALID;
  st = check_workspace(workspace, workspace_bytes, logits_ws_bytes(p, batch, n_q_heads, n_kv_heads, seq_len, topk));
  if (st != TQ_OK) return st;
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
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  hipError_t e;
  if (topk > 0) {
    tqi::SearchArgs sa;
    sa.base = a;
    sa.topk = topk;
    sa.topk_idx = topk_idx;
    e = tqi::launch_search(p->d, lloyd_bits(p), sa, (hipStream_t)stream);
  } else if (p->mode == TQ_MODE_POLAR) {
    e = tqi::launch_polar_logits(p->d, a, (hipStream_t)stream);
  } else {
    e = tqi::launch_logits(p->d, lloyd_bits(p), prod, a, (hipStream_t)stream);
  }
  return hip_status(e);
}

extern "C" tq_status tq_append_attn_logits(const tq_params *p, const void *x_new, int32_t x_dtype,
                                           const void *q, int32_t q_dtype, int32_t batch,
                                           int32_t n_q_heads, int32_t n_kv_heads, const tq_packed *k,
                                           int64_t row_tokens, int64_t pos, float scale, float *logits,
                                           void *workspace, size_t workspace_bytes, void *stream) {
  tq_status st = check_logit_args(p, batch, n_q_heads, n_kv_heads, 0, 0);
  if (st != TQ_OK) return st;
  const bool prod = p->mode == TQ_MODE_PROD;
  if (k == nullptr) return TQ_ERR_INVALID;
  if ((q_dtype != TQ_F32 && q_dtype != TQ_BF16) || (x_dtype != TQ_F32 && x_dtype != TQ_BF16))
    return TQ_ERR_INVALID;
  if (pos < 0 || pos >= row_tokens) return TQ_ERR_INVALID;
  if (p->mode == TQ_MODE_POLAR) return TQ_ERR_UNSUPPORTED;   // dense one-shot logits only
  st = logits_shape(p, batch, n_q_heads, n_kv_heads, pos + 1, 0);
  if (st != TQ_OK) return st;
  if (batch == 0) return TQ_OK;
  if (x_new == nullptr || q == nullptr || logits == nullptr || k->codes == nullptr || k->norm == nullptr)
    return TQ_ERR_INVALID;
  if (prod && (p->qjl == nullptr || p->qjl_rot == nullptr || k->rnorm == nullptr)) return TQ_ERR_INVALID;
  st = check_workspace(workspace, workspace_bytes, logits_ws_bytes(p, batch, n_q_heads, n_kv_heads, pos + 1, 0));
  if (st != TQ_OK) return st;
  if ((uintptr_t)k->codes & 3u) return TQ_ERR_UNSUPPORTED;
  tqi::LogitArgs a;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
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
  return hip_status(tqi::launch_logits(p->d, lloyd_bits(p), prod, a, (hipStream_t)stream));
}

namespace {

// Checks of a paged call: the table and page shape, tokens within the table,
// the pool's codes addressable with 32-bit offsets (plus one block of
// prefetch).  On success fills the paged fields of `a`.
tq_status paged_args(const tq_params *p, int32_t batch, int32_t n_kv_heads, const tq_pages *pg,
                     int64_t tokens, tqi::LogitArgs &a) {
  if (pg == nullptr || pg->block_table == nullptr) return TQ_ERR_INVALID;
  if (pg->page_tokens <= 0 || pg->page_tokens % 64 != 0 || pg->max_pages <= 0 || pg->n_pages <= 0)
    return TQ_ERR_INVALID;
  if (tokens > (int64_t)pg->max_pages * pg->page_tokens) return TQ_ERR_INVALID;
  const int64_t rows = pg->n_pages * n_kv_heads * (int64_t)pg->page_tokens;
  const int64_t rb = (int64_t)p->bits * p->d / 8;
  if ((rows + 64) * rb >= (1LL << 31) || rows >= (1LL << 31)) return TQ_ERR_UNSUPPORTED;
  (void)batch;
  a.block_table = pg->block_table;
  a.page_tokens = pg->page_tokens;
  a.max_pages = pg->max_pages;
  a.pool_rows = rows;
  a.row_tokens = 0;
  return TQ_OK;
}

}  // namespace

extern "C" tq_status tq_attn_logits_paged(const tq_params *p, const void *q, int32_t q_dtype, int32_t batch,
                                          int32_t n_q_heads, int32_t n_kv_heads, const tq_packed *pool,
                                          const tq_pages *pages, int64_t seq_len, float scale, float *logits,
                                          void *workspace, size_t workspace_bytes, void *stream) {
  tq_status st = check_logit_args(p, batch, n_q_heads, n_kv_heads, seq_len, 0);
  if (st != TQ_OK) return st;
  const bool prod = p->mode == TQ_MODE_PROD;
  if (pool == nullptr) return TQ_ERR_INVALID;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return TQ_ERR_INVALID;
  if (p->mode == TQ_MODE_POLAR) return TQ_ERR_UNSUPPORTED;   // dense one-shot logits only
  st = logits_shape(p, batch, n_q_heads, n_kv_heads, seq_len, 0);
  if (st != TQ_OK) return st;
  tqi::LogitArgs a;
  st = paged_args(p, batch, n_kv_heads, pages, seq_len, a);
  if (st != TQ_OK) return st;
  if (batch == 0 || seq_len == 0) return TQ_OK;
  if (q == nullptr || logits == nullptr || pool->codes == nullptr || pool->norm == nullptr) return TQ_ERR_INVALID;
  if (prod && (p->qjl == nullptr || pool->rnorm == nullptr)) return TQ_ERR_INVALID;
  st = check_workspace(workspace, workspace_bytes, logits_ws_bytes(p, batch, n_q_heads, n_kv_heads, seq_len, 0));
  if (st != TQ_OK) return st;
  if ((uintptr_t)pool->codes & 3u) return TQ_ERR_UNSUPPORTED;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  a.q = q;
  a.q_f32 = q_dtype == TQ_F32;
  a.batch = batch;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.pi = p->pi;
  a.s_mat = p->qjl;
  a.centroids = p->centroids;
  a.codes = pool->codes;
  a.norm = pool->norm;
  a.rnorm = pool->rnorm;
  a.seq_len = seq_len;
  a.scale = scale;
  a.logits = logits;
  return hip_status(tqi::launch_logits(p->d, lloyd_bits(p), prod, a, (hipStream_t)stream));
}

extern "C" tq_status tq_append_attn_logits_paged(const tq_params *p, const void *x_new, int32_t x_dtype,
                                                 const void *q, int32_t q_dtype, int32_t batch, int32_t n_q_heads,
                                                 int32_t n_kv_heads, const tq_packed *pool, const tq_pages *pages,
                                                 int64_t pos, float scale, float *logits, void *workspace,
                                                 size_t workspace_bytes, void *stream) {
  tq_status st = check_logit_args(p, batch, n_q_heads, n_kv_heads, 0, 0);
  if (st != TQ_OK) return st;
  const bool prod = p->mode == TQ_MODE_PROD;
  if (pool == nullptr || pos < 0) return TQ_ERR_INVALID;
  if ((q_dtype != TQ_F32 && q_dtype != TQ_BF16) || (x_dtype != TQ_F32 && x_dtype != TQ_BF16))
    return TQ_ERR_INVALID;
  if (p->mode == TQ_MODE_POLAR) return TQ_ERR_UNSUPPORTED;   // dense one-shot logits only
  st = logits_shape(p, batch, n_q_heads, n_kv_heads, pos + 1, 0);
  if (st != TQ_OK) return st;
  tqi::LogitArgs a;
  st = paged_args(p, batch, n_kv_heads, pages, pos + 1, a);
  if (st != TQ_OK) return st;
  if (batch == 0) return TQ_OK;
  if (x_new == nullptr || q == nullptr || logits == nullptr || pool->codes == nullptr || pool->norm == nullptr)
    return TQ_ERR_INVALID;
  if (prod && (p->qjl == nullptr || p->qjl_rot == nullptr || pool->rnorm == nullptr)) return TQ_ERR_INVALID;
  st = check_workspace(workspace, workspace_bytes, logits_ws_bytes(p, batch, n_q_heads, n_kv_heads, pos + 1, 0));
  if (st != TQ_OK) return st;
  if ((uintptr_t)pool->codes & 3u) return TQ_ERR_UNSUPPORTED;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  a.q = q;
  a.q_f32 = q_dtype == TQ_F32;
  a.batch = batch;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.pi = p->pi;
  a.s_mat = p->qjl;
  a.centroids = p->centroids;
  a.codes = pool->codes;
  a.norm = pool->norm;
  a.rnorm = pool->rnorm;
  a.seq_len = pos + 1;
  a.scale = scale;
  a.logits = logits;
  a.x_new = x_new;
  a.x_f32 = x_dtype == TQ_F32;
  a.boundaries = p->boundaries;
  a.m_mat = p->qjl_rot;
  a.codes_out = pool->codes;
  a.norm_out = pool->norm;
  a.rnorm_out = pool->rnorm;
  a.pos = pos;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  return hip_status(tqi::launch_logits(p->d, lloyd_bits(p), prod, a, (hipStream_t)stream));
}

extern "C" tq_status tq_prepare_queries(const tq_params *p, const void *q, int32_t q_dtype, int32_t batch,
                                        int32_t n_q_heads, int32_t n_kv_heads, void *workspace,
                                        size_t workspace_bytes, void *stream) {
  tq_status st = check_logit_args(p, batch, n_q_heads, n_kv_heads, 1, 0);
  if (st != TQ_OK) return st;
  const bool prod = p->mode == TQ_MODE_PROD;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return TQ_ERR_INVALID;
  if (p->mode == TQ_MODE_POLAR) return TQ_ERR_UNSUPPORTED;   // dense one-shot logits only
  st = logits_shape(p, batch, n_q_heads, n_kv_heads, 1, 0);
  if (st != TQ_OK) return st;
  if (batch == 0) return TQ_OK;
  if (q == nullptr) return TQ_ERR_INVALID;
  if (prod && p->qjl == nullptr) return TQ_ERR_INVALID;
  st = check_workspace(workspace, workspace_bytes, logits_ws_bytes(p, batch, n_q_heads, n_kv_heads, 1, 0));
  if (st != TQ_OK) return st;
  tqi::LogitArgs a;
  a.q = q;
  a.q_f32 = q_dtype == TQ_F32;
  a.batch = batch;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.pi = p->pi;
  a.s_mat = p->qjl;
  a.centroids = p->centroids;
  a.codes = nullptr;
  a.norm = nullptr;
  a.rnorm = nullptr;
  a.row_tokens = 0;
  a.seq_len = 0;
  a.scale = 0.0f;
  a.logits = nullptr;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  a.run_stream = false;
  return hip_status(tqi::launch_logits(p->d, lloyd_bits(p), prod, a, (hipStream_t)stream));
}

extern "C" tq_status tq_attn_logits_prepared(const tq_params *p, int32_t batch, int32_t n_q_heads,
                                             int32_t n_kv_heads, const tq_packed *k, int64_t row_tokens,
                                             const tq_pages *pages, int64_t seq_len, float scale, float *logits,
                                             const void *workspace, size_t workspace_bytes, void *stream) {
  tq_status st = check_logit_args(p, batch, n_q_heads, n_kv_heads, seq_len, 0);
  if (st != TQ_OK) return st;
  const bool prod = p->mode == TQ_MODE_PROD;
  if (k == nullptr) return TQ_ERR_INVALID;
  if (pages == nullptr && row_tokens < seq_len) return TQ_ERR_INVALID;
  if (p->mode == TQ_MODE_POLAR) return TQ_ERR_UNSUPPORTED;   // dense one-shot logits only
  st = logits_shape(p, batch, n_q_heads, n_kv_heads, seq_len, 0);
  if (st != TQ_OK) return st;
  tqi::LogitArgs a;
  if (pages != nullptr) {
    st = paged_args(p, batch, n_kv_heads, pages, seq_len, a);
    if (st != TQ_OK) return st;
  } else {
    a.row_tokens = row_tokens;
  }
  if (batch == 0 || seq_len == 0) return TQ_OK;
  if (logits == nullptr || k->codes == nullptr || k->norm == nullptr) return TQ_ERR_INVALID;
  if (prod && k->rnorm == nullptr) return TQ_ERR_INVALID;
  st = check_workspace(workspace, workspace_bytes, logits_ws_bytes(p, batch, n_q_heads, n_kv_heads, seq_len, 0));
  if (st != TQ_OK) return st;
  if ((uintptr_t)k->codes & 3u) return TQ_ERR_UNSUPPORTED;
  a.q = nullptr;
  a.q_f32 = false;
  a.batch = batch;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.pi = p->pi;
  a.s_mat = p->qjl;
  a.centroids = p->centroids;
  a.codes = k->codes;
  a.norm = k->norm;
  a.rnorm = k->rnorm;
  a.seq_len = seq_len;
  a.scale = scale;
  a.logits = logits;
  // the streaming launch only reads the tables
  a.workspace = const_cast<void *>(workspace);
  a.workspace_bytes = workspace_bytes;
  a.run_prep = false;
  return hip_status(tqi::launch_logits(p->d, lloyd_bits(p), prod, a, (hipStream_t)stream));
}

extern "C" tq_status tq_attn_output_workspace_size(const tq_params *p, int32_t batch, int32_t n_q_heads,
                                                   int32_t n_kv_heads, int64_t seq_len, size_t *bytes) {
  if (bytes == nullptr) return TQ_ERR_INVALID;
  *bytes = 0;
  const tq_status st = check_attend_args(p, batch, n_q_heads, n_kv_heads, seq_len);
  if (st != TQ_OK) return st;
  if (batch > 0)
    *bytes = tqi::attend_workspace_bytes(p->d, lloyd_bits(p), batch, n_q_heads, n_kv_heads, seq_len);
  return TQ_OK;
}

namespace {

// tq_attn_output and its no-allocation variant: the same validation, the
// same kernels; `noalloc` takes the library's fixed array as the workspace.
tq_status attn_output_call(const tq_params *p, const float *logits, int32_t batch, int32_t n_q_heads,
                           int32_t n_kv_heads, const tq_packed *v, int64_t row_tokens, int64_t seq_len,
                           void *out, int32_t out_dtype, void *workspace, size_t workspace_bytes,
                           bool noalloc, void *stream) {
  tq_status st = check_params(p);
  if (st != TQ_OK) return st;
  if (v == nullptr || row_tokens < seq_len) return TQ_ERR_INVALID;
  if (out_dtype != TQ_F32 && out_dtype != TQ_BF16) return TQ_ERR_INVALID;
  st = check_attend_args(p, batch, n_q_heads, n_kv_heads, seq_len);
  if (st != TQ_OK) return st;
  if (batch == 0) return TQ_OK;
  if (out == nullptr) return TQ_ERR_INVALID;
  if (seq_len > 0 && (logits == nullptr || v->codes == nullptr || v->norm == nullptr)) return TQ_ERR_INVALID;
  const size_t need = tqi::attend_workspace_bytes(p->d, lloyd_bits(p), batch, n_q_heads, n_kv_heads, seq_len);
  if (noalloc) {
    if (need > tqi::kNoAllocScratchBytes) return TQ_ERR_UNSUPPORTED;
  } else {
    st = check_workspace(workspace, workspace_bytes, need);
    if (st != TQ_OK) return st;
  }
  if ((uintptr_t)v->codes & 15u) return TQ_ERR_UNSUPPORTED;
  if (noalloc) {
    const hipError_t e = tqi::noalloc_scratch(&workspace);
    if (e != hipSuccess) return TQ_ERR_HIP;
    workspace_bytes = tqi::kNoAllocScratchBytes;
  }
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
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  return hip_status(tqi::launch_attend(p->d, lloyd_bits(p), a, (hipStream_t)stream));
}

}  // namespace

extern "C" tq_status tq_attn_output(const tq_params *p, const float *logits, int32_t batch,
                                    int32_t n_q_heads, int32_t n_kv_heads, const tq_packed *v,
                                    int64_t row_tokens, int64_t seq_len, void *out, int32_t out_dtype,
                                    void *workspace, size_t workspace_bytes, void *stream) {
  return attn_output_call(p, logits, batch, n_q_heads, n_kv_heads, v, row_tokens, seq_len, out, out_dtype,
                          workspace, workspace_bytes, false, stream);
}

extern "C" tq_status tq_attn_output_noalloc(const tq_params *p, const float *logits, int32_t batch,
                                            int32_t n_q_heads, int32_t n_kv_heads, const tq_packed *v,
                                            int64_t row_tokens, int64_t seq_len, void *out, int32_t out_dtype,
                                            void *stream) {
  return attn_output_call(p, logits, batch, n_q_heads, n_kv_heads, v, row_tokens, seq_len, out, out_dtype,
                          nullptr, 0, true, stream);
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

extern "C" tq_status tq_probe_sink_words(int64_t *words) {
  if (words == nullptr) return TQ_ERR_INVALID;
  *words = (int64_t)tqi::probe_blocks() * 4;
  return TQ_OK;
}

extern "C" tq_status tq_probe(int32_t kind, void *buf, int64_t bytes, int32_t iters, uint32_t *sink,
                              int64_t sink_words, void *stream) {
  if (kind < TQ_PROBE_READ || kind > TQ_PROBE_MFMA_I8 || sink == nullptr) return TQ_ERR_INVALID;
  if (sink_words < (int64_t)tqi::probe_blocks() * 4) return TQ_ERR_INVALID;
  if (kind <= TQ_PROBE_WRITE && (buf == nullptr || bytes < 16 || bytes % 16 != 0 || ((uintptr_t)buf & 15u)))
    return TQ_ERR_INVALID;
  if (kind >= TQ_PROBE_MFMA_F16 && iters <= 0) return TQ_ERR_INVALID;
  return hip_status(tqi::launch_probe(kind, buf, bytes, iters, sink, (hipStream_t)stream));
}
