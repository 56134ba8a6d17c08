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
};

hipError_t launch_logits(int d, int lbits, bool prod, const LogitArgs &a, hipStream_t s,
                         bool *supported);

struct SearchArgs {
  LogitArgs base;
  int topk;
  int32_t *topk_idx;
};

hipError_t launch_search(int d, int lbits, const SearchArgs &a, hipStream_t s, bool *supported);

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
};

hipError_t launch_attend(int d, int lbits, const AttendArgs &a, hipStream_t s, bool *supported);

int device_cu_count();

// Scratch memory for one call on stream `s` of the current device.  The
// library keeps one buffer per (device, stream), grows it with hipMalloc when
// a call needs more (after synchronising that stream, whose queued work may
// still read the old buffer) and keeps it until the process ends.  Work on
// one stream runs in order, so successive calls on it can share the buffer.
hipError_t workspace(hipStream_t s, size_t bytes, void **out);

}  // namespace tqi
