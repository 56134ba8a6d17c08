// Internal launch interface between the C ABI (tq_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq.h"

namespace tqi {

struct QuantizeArgs {
  const void *x;
  int64_t n_vec;
  int64_t x_stride;      // elements
  const float *pi;
  const float *m;        // qjl_rot (PROD)
  const float *centroids;
  const float *boundaries;
  uint8_t *codes;
  uint16_t *norm;
  uint16_t *rnorm;
  int64_t out_offset;
};

hipError_t launch_quantize(int d, int lbits, bool prod, bool in_f32, const QuantizeArgs &a,
                           hipStream_t s, bool *supported);
// polar format (d = 128): boundaries = the angle boundaries of levels 2..log2 d
hipError_t launch_quantize_polar(int d, bool in_f32, const QuantizeArgs &a, hipStream_t s, bool *supported);

struct LogitArgs {
  const void *q;
  bool q_f32;
  int batch, n_q_heads, n_kv_heads;
  const float *pi;
  const float *s_mat;    // S (PROD)
  const float *centroids;
  const uint8_t *codes;
  const uint16_t *norm;
  const uint16_t *rnorm;
  int64_t row_tokens, seq_len;
  float scale;
  float *logits;
  // decode-time append (x_new == nullptr: none): the new key of every stream
  // is quantised into token pos = seq_len - 1 before the logits are formed
  const void *x_new = nullptr;
  bool x_f32 = false;
  const float *boundaries = nullptr;
  const float *m_mat = nullptr;
  uint8_t *codes_out = nullptr;
  uint16_t *norm_out = nullptr;
  uint16_t *rnorm_out = nullptr;
  int64_t pos = 0;
  // paged cache (block_table == nullptr: contiguous rows per stream)
  const int32_t *block_table = nullptr;
  int page_tokens = 0, max_pages = 0;
  int64_t pool_rows = 0;
  // caller-owned device scratch (query tables; for top-k also partial lists)
  void *workspace = nullptr;
  size_t workspace_bytes = 0;
  // dense logits run two launches: the query preparation, which writes the
  // tables into the workspace, and the streaming launch, which reads them;
  // either can run alone (q is unused without the first, codes and logits
  // without the second)
  bool run_prep = true, run_stream = true;
};

// Shapes the dense logit kernels take (GQA group <= 16, d in {64, 128, 256},
// 32-bit byte offsets of one stream's codes and logits below 2^31).
bool logits_supported(int d, int lbits, bool prod, int group, int64_t seq_len);
size_t logits_workspace_bytes(int d, int lbits, bool prod, int64_t n_streams, int group);
hipError_t launch_logits(int d, int lbits, bool prod, const LogitArgs &a, hipStream_t s);

// Dense logits from polar-format keys (d in {64, 128, 256}, GQA group <= 16,
// 32-bit byte ranges of one stream's codes and logits): query preparation
// and streaming launch; the workspace holds the rotated queries and the
// cos/sin table of the centroid angles.
bool polar_logits_supported(int d, int group, int64_t seq_len, int64_t n_streams);
size_t polar_logits_workspace_bytes(int d, int64_t n_streams, int group);
hipError_t launch_polar_logits(int d, const LogitArgs &a, hipStream_t s);

struct SearchArgs {
  LogitArgs base;
  int topk;
  int32_t *topk_idx;
};

// Top-k search: shapes it takes and the scratch it needs on the current device.
bool search_supported(int d, int lbits, int topk, int batch, int n_q_heads, int n_kv_heads, int64_t seq_len);
size_t search_workspace_bytes(int d, int lbits, int batch, int n_q_heads, int n_kv_heads, int64_t seq_len);
hipError_t launch_search(int d, int lbits, const SearchArgs &a, hipStream_t s);

struct DequantArgs {
  const float *pi;
  const float *s_mat;
  const float *centroids;
  const uint8_t *codes;
  const uint16_t *norm;
  const uint16_t *rnorm;
  int64_t n_vec;
  void *out;
  bool out_f32;
};

hipError_t launch_dequant(int d, int lbits, bool prod, const DequantArgs &a, hipStream_t s,
                          bool *supported);
// polar format (d = 128): centroids = the angle centroids of levels 2..log2 d
hipError_t launch_dequant_polar(int d, const DequantArgs &a, hipStream_t s, bool *supported);

struct AttendArgs {
  const float *logits;   // [batch][n_q_heads][seq_len]
  int batch, n_q_heads, n_kv_heads;
  const float *pi;
  const float *centroids;
  const uint8_t *codes;
  const uint16_t *norm;
  int64_t row_tokens, seq_len;
  void *out;             // [batch][n_q_heads][d]
  bool out_f32;
  void *workspace = nullptr;   // caller-owned device scratch (per-split partials)
  size_t workspace_bytes = 0;
};

bool attend_supported(int d, int lbits, int group, int64_t seq_len);

// Fixed device array behind tq_attn_output_noalloc: its size, and its device
// address on the current device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = TQ_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
hipError_t noalloc_scratch(void **out);
size_t attend_workspace_bytes(int d, int lbits, int batch, int n_q_heads, int n_kv_heads, int64_t seq_len);
hipError_t launch_attend(int d, int lbits, const AttendArgs &a, hipStream_t s);

// Ceiling probes (probes.hip): kind 0 read stream, 1 write stream, 2 fp16
// MFMA loop, 3 int8 MFMA loop; probe_blocks() workgroups of 4 waves.
int probe_blocks();
hipError_t launch_probe(int kind, void *buf, int64_t bytes, int iters, uint32_t *sink, hipStream_t s);

// Compute units of the current device (cached per device; 256 when the
// runtime cannot say).
int device_cu_count();

// Bytes rounded up to the 256-byte alignment of every workspace piece.
constexpr size_t ws_align(size_t bytes) { return (bytes + 255) & ~(size_t)255; }

}  // namespace tqi
