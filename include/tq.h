/* tq.h - C ABI of the MI355X (gfx950) online KV-cache vector quantizer.
 *
 * Method: page "TurboQuant 설명: 무엇인지와 LLM 메모리 6배 절약 구현 방법"
 * (a2a-mcp.org).  Stage 1 ("1단계: 무작위 회전 + PolarQuant 압축"): normalise
 * each vector, rotate it with one seeded random orthogonal matrix (QR of a
 * Gaussian matrix), map every rotated coordinate to the nearest Lloyd-Max
 * centroid of the Beta((d-1)/2,(d-1)/2) law.  Stage 2 ("2단계: QJL 잔차 보정"):
 * keep the sign of each coordinate of a Gaussian projection of the stage-1
 * residual, which makes inner products unbiased.  Attention logits are formed
 * straight from the packed indices against a query rotated once (closing
 * paragraphs of "2단계" and "TurboQuant 구현 방법").
 *
 * Conventions shared by every call
 *   - Every call returns tq_status (TQ_OK = 0, negative = error) and never
 *     throws.  Arguments are validated on the host before anything is
 *     launched; a failed validation launches nothing and writes nothing.
 *   - Pointers are owned by the caller and borrowed for the duration of the
 *     call (device pointers until the work queued on `stream` completes).
 *     Host pointers are plain host memory; device pointers are HIP device
 *     memory of the current device.
 *   - Device work is queued asynchronously on the caller's `stream` (a
 *     hipStream_t passed as void*, NULL = the null stream).  Launch errors
 *     return TQ_ERR_HIP; faults inside a kernel surface at the caller's next
 *     synchronisation, as with any HIP launch.
 *   - The library never allocates or frees memory, never synchronises and
 *     keeps no state between calls (apart from a per-device cache of the
 *     compute-unit count, set once, and the fixed per-device array that
 *     tq_attn_output_noalloc uses instead of a workspace).  Calls that need device scratch memory
 *     (the logit calls: query tables; top-k: partial lists; tq_attn_output:
 *     per-split partials) take a
 *     caller-owned `workspace` of `workspace_bytes` bytes: 256-byte aligned
 *     device memory of at least the size the matching *_workspace_size query
 *     gives for the same arguments on the current device.  It is borrowed
 *     until the queued work completes, so calls that may overlap in time
 *     (other streams, other host threads) need workspaces of their own.  A
 *     NULL workspace is accepted where the query returns 0.
 *   - Calls are reentrant and thread-safe: nothing is shared between calls
 *     except what the caller passes in (tq_attn_output_noalloc excepted: its
 *     calls share the array, see there).
 *
 * Packed format of one vector (d coordinates, b total bits per coordinate)
 *   mode TQ_MODE_MSE : b' = b Lloyd-Max bits.     1 <= b <= 4
 *   mode TQ_MODE_PROD: b' = b - 1 Lloyd-Max bits + 1 QJL sign bit. 2 <= b <= 5
 *   record: every coordinate carries b bits: bits 0..b'-1 hold its Lloyd-Max
 *           index idx_j = #{k : y_j >= t_k} (y = Pi x / ||x||, t the Lloyd-Max
 *           boundaries) and, in PROD mode, bit b' holds its QJL sign bit
 *           [(S r)_j >= 0] with r = u - Pi^T c_hat, u = x / ||x||.
 *   codes : b * d/8 bytes: the records as word-interleaved bit planes.
 *           Coordinates go in groups of 32; group g holds b little-endian
 *           32-bit words, one per plane, at bytes 4(b g + p) .. 4(b g + p) + 3,
 *           and bit i of the word of plane p is bit p of the record of
 *           coordinate 32g + i.
 *   norm  : fp16 bits (round to nearest even) of ||x||_2.
 *   rnorm : (PROD) fp16 bits of gamma = ||r||_2.
 *   A zero vector gets idx_j = 2^(b'-1), all sign bits 1 and gamma = 0.
 *   Reconstruction: x_hat = norm * (Pi^T c_hat + sqrt(pi/2)/d * rnorm * S^T s),
 *   s = 2*sign_bit - 1.  A row is b*d/8 + 2 (MSE) or b*d/8 + 4 (PROD) bytes.
 *
 * Polar format (mode TQ_MODE_POLAR, b = 3, d a power of two >= 64): the
 * PolarQuant variant of stage 1 (page section "1단계": the unit vector is
 * paired recursively into polar form).  y = Pi x / ||x||; level 1 turns the
 * pairs (y_2i, y_2i+1) into angles phi_i = atan2(y_2i+1, y_2i) in [0, 2 pi),
 * level l >= 2 the pairs of level-(l-1) radii (rho_2i, rho_2i+1) into angles
 * psi_i = atan2(rho_2i+1, rho_2i) in [0, pi/2].  phi gets 4 bits: sector
 * floor(16 phi / (2 pi)); psi gets 2 bits: #{k : psi >= t_k} against the 3
 * boundaries of its level (tq_make_polar_codebook); an angle of a zero pair
 * or block is 0.
 *   codes : 3 d/8 bytes: the d/2 level-1 indices as 4 bit planes over groups
 *           of 32 slots (group g, plane p at word 4 g + p), then the d/2 - 1
 *           higher indices in level order (level 2 first) plus one zero slot
 *           as 2 bit planes (group g, plane p at word d/16 + 2 g + p).
 *   norm  : fp16 bits of ||x||_2 (no rnorm).
 *   Reconstruction: y_hat from the centroid angles from the top (radius 1)
 *   down, x_hat = norm * Pi^T y_hat; level-1 centroids are the sector
 *   midpoints 2 pi (j + 1/2) / 16.
 *   tq_params.centroids / boundaries hold the levels 2..log2(d) codebooks,
 *   4 centroids and 3 boundaries per level (angles, fp32), level 2 first.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t tq_status;

enum {
  TQ_OK = 0,
  TQ_ERR_INVALID = -1,        /* NULL pointer, negative size, bad enum value   */
  TQ_ERR_UNSUPPORTED = -2,    /* valid request the library has no kernel for  */
  TQ_ERR_NO_CONVERGENCE = -3, /* Lloyd-Max solver did not settle               */
  TQ_ERR_HIP = -4             /* a HIP runtime call or launch failed           */
};

enum { TQ_MODE_MSE = 0, TQ_MODE_PROD = 1, TQ_MODE_POLAR = 2 };
enum { TQ_F32 = 0, TQ_BF16 = 1 };
enum { TQ_KIND_PI = 0, TQ_KIND_S = 1, TQ_KIND_M = 2 };

/* Lloyd-Max codebook for one coordinate of a rotated unit vector in R^d
 * (page section "1단계": Beta((d-1)/2,(d-1)/2) law on [-1,1], codebook
 * precomputed per dimension and bit width; section "TurboQuant 구현 방법").
 * Host only, fp64.  The density is integrated numerically (composite
 * Gauss-Legendre in the angle x = sin(phi)); the fixed point is found by
 * Lloyd iterations followed by Newton steps and is returned exactly
 * antisymmetric (c[k] = -c[K-1-k], middle boundary 0).
 *   d            dimension, d >= 3
 *   bits         Lloyd-Max bits b', 1..8; K = 2^bits levels
 *   centroids    out, K doubles, ascending
 *   boundaries   out, K-1 doubles, midpoints of adjacent centroids
 *   mse_per_coord out (may be NULL): E[(X - Q(X))^2] of one coordinate
 * Errors: TQ_ERR_INVALID (bad d/bits/NULL), TQ_ERR_NO_CONVERGENCE. */
tq_status tq_make_codebook(int32_t d, int32_t bits, double *centroids, double *boundaries,
                           double *mse_per_coord);

/* Angle codebooks of the polar format (page section "1단계": the angle laws
 * are concentrated and known, so Lloyd-Max codebooks are precomputed).  At
 * level l >= 2 an angle splits two radii spanning k = 2^(l-1) dimensions
 * each; for a uniform point on the sphere sin^2 psi ~ Beta(k/2, k/2), density
 * proportional to (sin psi cos psi)^(k-1) on [0, pi/2].  Host only, fp64:
 * composite Gauss-Legendre quadrature and Lloyd iteration, returned exactly
 * symmetric about pi/4.
 *   d            a power of two >= 64
 *   centroids    out, 4 (log2 d - 1) doubles: levels 2..log2 d, ascending
 *   boundaries   out, 3 (log2 d - 1) doubles, midpoints of adjacent centroids
 * Errors: TQ_ERR_INVALID, TQ_ERR_NO_CONVERGENCE. */
tq_status tq_make_polar_codebook(int32_t d, double *centroids, double *boundaries);

/* Seeded random matrices (page sections "1단계" and "2단계").  Host only, fp64,
 * row-major d x d written to `out`.
 *   kind TQ_KIND_PI: Pi = Q diag(sign R_ii) (sign(0)=+1) from the QR
 *                    factorisation G = QR of the Gaussian matrix of stream 0;
 *                    Haar distributed; the rotation is y = Pi x.
 *   kind TQ_KIND_S : S, i.i.d. N(0,1) from stream 1 (m = d rows, no QR).
 *   kind TQ_KIND_M : M = S Pi^T (QJL projection in the rotated domain).
 * Gaussian stream k of seed s: SplitMix64 started at state 2s+k, uniforms
 * ((w >> 11) + 0.5) * 2^-53, Box-Muller pairs (cos first), row-major fill.
 * Errors: TQ_ERR_INVALID (d < 2, d > 4096, bad kind, NULL). */
tq_status tq_make_rotation(int32_t d, uint64_t seed, int32_t kind, double *out);

/* Device-side parameters of one quantizer: fp32 copies of the host tables.
 * All pointers are device memory, row-major d x d matrices. */
typedef struct tq_params {
  int32_t d;                /* 64, 128 or 256 (see each call for support)  */
  int32_t bits;             /* total bits per coordinate b                 */
  int32_t mode;             /* TQ_MODE_MSE or TQ_MODE_PROD                 */
  int32_t reserved;         /* must be 0                                   */
  const float *pi;          /* Pi                                          */
  const float *qjl;         /* S (PROD; may be NULL in MSE)                */
  const float *qjl_rot;     /* M = S Pi^T (PROD; may be NULL in MSE)       */
  const float *centroids;   /* 2^b' ascending, antisymmetric               */
  const float *boundaries;  /* 2^b' - 1 ascending                          */
} tq_params;

/* Packed vectors, structure of arrays.  Vector i occupies codes[i*b*d/8 ..]
 * (4-byte aligned rows), norm[i] and rnorm[i] (device memory). */
typedef struct tq_packed {
  uint8_t *codes;
  uint16_t *norm;
  uint16_t *rnorm;          /* PROD only; NULL in MSE                      */
} tq_packed;

/* Quantise n_vec vectors (page sections "1단계" and "2단계"; quantisation on
 * every cache update: "TurboQuant 구현 방법").
 *   x            device, n_vec rows of d elements (x_dtype TQ_F32 or
 *                TQ_BF16), consecutive rows x_row_stride elements apart
 *   out          packed arrays; vector i is written at index out_offset + i
 * Supported: d in {64, 128, 256} for all three modes; b' <= 4 (polar: 3
 * bits per coordinate).
 * n_vec == 0 is a no-op.  Errors: TQ_ERR_INVALID, TQ_ERR_UNSUPPORTED,
 * TQ_ERR_HIP. */
tq_status tq_quantize_kv(const tq_params *p, const void *x, int32_t x_dtype, int64_t n_vec,
                         int64_t x_row_stride, const tq_packed *out, int64_t out_offset,
                         void *stream);

/* Device scratch that tq_attn_logits needs for these arguments on the current
 * device (the same validation as the call itself: an unsupported shape
 * returns TQ_ERR_UNSUPPORTED).  Dense logits need the query tables (A
 * operands and constants of every query: a few KB per (batch, kv head)
 * stream, independent of seq_len; polar-format keys: the rotated queries and
 * the cos/sin tables of the angle codebooks); top-k search needs its rotated
 * queries and partial lists.  The other logit calls (append, paged) take the dense
 * size: this query with their batch, heads, seq_len (pos + 1) and topk = 0.
 * *bytes is 0 for empty calls.
 * Errors: TQ_ERR_INVALID, TQ_ERR_UNSUPPORTED. */
tq_status tq_attn_logits_workspace_size(const tq_params *p, int32_t batch, int32_t n_q_heads,
                                        int32_t n_kv_heads, int64_t seq_len, int32_t topk, size_t *bytes);

/* Attention logits straight from packed keys (page: the query is rotated
 * once and logits come from the indices without reconstructing the keys).
 *   q            device [batch][n_q_heads][d], q_dtype TQ_F32 or TQ_BF16
 *   k            packed keys laid out [batch][n_kv_heads][row_tokens]
 *   seq_len      valid tokens per (batch, kv head) stream, <= row_tokens
 *   scale        logit scale (e.g. 1/sqrt(d))
 *   topk == 0 :  logits  device fp32 [batch][n_q_heads][seq_len],
 *                logit = scale * <q, x_hat>; topk_idx unused (may be NULL)
 *   topk  > 0 :  vector search: for every query the topk largest logits,
 *                ties to the smaller token index, descending; logits is
 *                fp32 [batch][n_q_heads][topk] and topk_idx int32 of the same
 *                shape.  Needs seq_len >= topk.
 *   workspace    device scratch of tq_attn_logits_workspace_size bytes
 * GQA: query head h reads KV head h / (n_q_heads / n_kv_heads); n_q_heads
 * must be a multiple of n_kv_heads.  Dense logits support d in {64, 128,
 * 256}, up to 16 query heads per KV head, streams whose packed codes stay
 * under 2 GiB and whose logits (group x seq_len fp32) stay under 2 GiB, in
 * all three modes (polar keys: logit = scale * n * <Pi q, y_hat>, y_hat the
 * unit vector the key's angle codes describe, "1단계");
 * top-k supports MSE mode, d in {64, 128, 256}, topk <= 16, seq_len < 2^30.
 * seq_len == 0 is a no-op.  A workspace smaller than the query's size, or
 * NULL where it is not 0, is TQ_ERR_INVALID; a misaligned one
 * TQ_ERR_UNSUPPORTED.
 * Errors: TQ_ERR_INVALID, TQ_ERR_UNSUPPORTED, TQ_ERR_HIP. */
tq_status tq_attn_logits(const tq_params *p, const void *q, int32_t q_dtype, int32_t batch,
                         int32_t n_q_heads, int32_t n_kv_heads, const tq_packed *k,
                         int64_t row_tokens, int64_t seq_len, float scale, float *logits,
                         int32_t topk, int32_t *topk_idx, void *workspace, size_t workspace_bytes,
                         void *stream);

/* Decode step with append: quantise one new key per (batch, kv head) stream
 * into the cache at token pos, then form the logits over tokens 0..pos of
 * every stream (quantisation on every cache update, page section
 * "TurboQuant 구현 방법"; the key is quantised exactly as by tq_quantize_kv,
 * stages "1단계" and "2단계"; logits as tq_attn_logits).  The append runs
 * inside the logit call's first (query preparation) launch, so the step costs
 * no extra launch.
 *   x_new        device [batch][n_kv_heads][d], x_dtype TQ_F32 or TQ_BF16
 *   k            packed keys laid out [batch][n_kv_heads][row_tokens]; token
 *                pos of every stream is overwritten, the other rows are only
 *                read (tokens 0..pos-1 must already hold packed keys)
 *   pos          0 <= pos < row_tokens
 *   logits       device fp32 [batch][n_q_heads][pos + 1]
 *   workspace    as tq_attn_logits with seq_len = pos + 1 and topk = 0
 * The new key is quantised in fp64 from the fp32 matrices (the inner-product
 * mode needs p->qjl_rot).  Supported: as dense tq_attn_logits (d in {64,
 * 128, 256}, up to 16 query heads per KV head).  batch == 0 is a no-op.
 * Errors: TQ_ERR_INVALID, TQ_ERR_UNSUPPORTED, TQ_ERR_HIP. */
tq_status tq_append_attn_logits(const tq_params *p, const void *x_new, int32_t x_dtype,
                                const void *q, int32_t q_dtype, int32_t batch, int32_t n_q_heads,
                                int32_t n_kv_heads, const tq_packed *k, int64_t row_tokens,
                                int64_t pos, float scale, float *logits, void *workspace,
                                size_t workspace_bytes, void *stream);

/* Paged key cache (a serving cache of fixed-size pages; the page reads
 * "quantise on every cache update", section "TurboQuant 구현 방법").  The
 * pool is one tq_packed of n_pages * n_kv_heads * page_tokens rows; page g
 * holds the rows of every KV head for its tokens, head-major: token t of KV
 * head h of sequence b is pool row
 *     (block_table[b * max_pages + t / page_tokens] * n_kv_heads + h)
 *     * page_tokens + t % page_tokens.
 * Sequences own disjoint pages in any order.  A block-table entry outside
 * [0, n_pages) never faults: its rows read as zero keys and an append into
 * it writes nothing. */
typedef struct tq_pages {
  const int32_t *block_table; /* device [batch][max_pages]                        */
  int32_t page_tokens;        /* tokens per page, a positive multiple of 64       */
  int32_t max_pages;          /* block-table entries per sequence                 */
  int64_t n_pages;            /* pages in the pool                                */
} tq_pages;

/* tq_attn_logits (dense, topk = 0) over a paged key cache: the first seq_len
 * tokens of every sequence, read through its block table; logits as
 * tq_attn_logits, [batch][n_q_heads][seq_len].  Needs seq_len <=
 * max_pages * page_tokens and the pool's packed codes under 2 GiB.  Same
 * support, workspace (the dense size) and errors as tq_attn_logits. */
tq_status tq_attn_logits_paged(const tq_params *p, const void *q, int32_t q_dtype, int32_t batch,
                               int32_t n_q_heads, int32_t n_kv_heads, const tq_packed *pool,
                               const tq_pages *pages, int64_t seq_len, float scale, float *logits,
                               void *workspace, size_t workspace_bytes, void *stream);

/* tq_append_attn_logits over a paged key cache: the new key of every
 * (sequence, KV head) goes to the pool row of token pos (its page must be in
 * the block table: pos < max_pages * page_tokens), then the logits over tokens
 * 0..pos, [batch][n_q_heads][pos + 1].  Same support and errors as
 * tq_attn_logits_paged; workspace as tq_attn_logits with seq_len = pos + 1
 * and topk = 0. */
tq_status tq_append_attn_logits_paged(const tq_params *p, const void *x_new, int32_t x_dtype,
                                      const void *q, int32_t q_dtype, int32_t batch, int32_t n_q_heads,
                                      int32_t n_kv_heads, const tq_packed *pool, const tq_pages *pages,
                                      int64_t pos, float scale, float *logits, void *workspace,
                                      size_t workspace_bytes, void *stream);

/* The query rotation on its own (page: the query is rotated once, closing
 * paragraph of "2단계" and "TurboQuant 구현 방법"): the first launch of a dense
 * tq_attn_logits, which turns the queries into the tables the streaming
 * launch reads (Pi q, S q and their fixed-point weights).  One preparation
 * then serves any number of tq_attn_logits_prepared calls, e.g. over a
 * shared-prefix cache and a per-sequence cache, or over a cache scored in
 * segments.
 *   q, q_dtype, batch, n_q_heads, n_kv_heads   as tq_attn_logits
 *   workspace    device scratch of tq_attn_logits_workspace_size(p, batch,
 *                n_q_heads, n_kv_heads, 1, 0) bytes (the dense size, which
 *                does not depend on seq_len); the tables are written into it
 * Supported: as dense tq_attn_logits.  batch == 0 is a no-op.
 * Errors: TQ_ERR_INVALID, TQ_ERR_UNSUPPORTED, TQ_ERR_HIP. */
tq_status tq_prepare_queries(const tq_params *p, const void *q, int32_t q_dtype, int32_t batch,
                             int32_t n_q_heads, int32_t n_kv_heads, void *workspace, size_t workspace_bytes,
                             void *stream);

/* Dense logits from queries prepared by tq_prepare_queries: the streaming
 * launch of tq_attn_logits alone, whose results it gives bit for bit.
 *   k, row_tokens, seq_len, scale, logits   as tq_attn_logits with topk = 0
 *   pages        NULL: k holds contiguous streams of row_tokens rows;
 *                otherwise k is a paged pool read as by tq_attn_logits_paged
 *                (row_tokens is then ignored)
 *   workspace    a workspace that tq_prepare_queries filled with the same
 *                quantiser (p), batch and heads, queued before this call on
 *                this stream or completed; it is only read, so calls on
 *                several streams may share it once it is filled.  Tables of
 *                another shape or quantiser give wrong logits; every access
 *                still stays inside the workspace.
 * Supported: as dense tq_attn_logits (paged: as tq_attn_logits_paged).
 * batch == 0 or seq_len == 0 is a no-op.
 * Errors: TQ_ERR_INVALID, TQ_ERR_UNSUPPORTED, TQ_ERR_HIP. */
tq_status tq_attn_logits_prepared(const tq_params *p, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                  const tq_packed *k, int64_t row_tokens, const tq_pages *pages,
                                  int64_t seq_len, float scale, float *logits, const void *workspace,
                                  size_t workspace_bytes, void *stream);

/* Decode attention output straight from packed values (page: the KV cache
 * holds keys and values, section "TurboQuant란 무엇인가요?", and attention runs
 * from the compressed indices, section "2단계", closing paragraph; the output
 * is standard attention, softmax of the logits times the values).
 *   logits       device fp32 [batch][n_q_heads][seq_len] (e.g. the output of
 *                tq_attn_logits; -inf entries are masked tokens)
 *   v            packed MSE-mode values laid out [batch][n_kv_heads][row_tokens]
 *   out          device [batch][n_q_heads][d], out_dtype TQ_F32 or TQ_BF16:
 *                o = sum_t softmax(logits)_t v_hat_t over the seq_len tokens of
 *                the query head's KV head (GQA as in tq_attn_logits); a head
 *                whose logits are all -inf, or seq_len == 0, gives o = 0.
 *   workspace    device scratch of tq_attn_output_workspace_size bytes (the
 *                per-split partial maxima, sums and accumulators)
 * Supported: MSE mode, d in {64, 128, 256}, up to 16 query heads per KV head,
 * 16-byte aligned value codes, packed values of one stream under 2 GiB.
 * Errors: TQ_ERR_INVALID, TQ_ERR_UNSUPPORTED, TQ_ERR_HIP. */
tq_status tq_attn_output(const tq_params *p, const float *logits, int32_t batch, int32_t n_q_heads,
                         int32_t n_kv_heads, const tq_packed *v, int64_t row_tokens, int64_t seq_len,
                         void *out, int32_t out_dtype, void *workspace, size_t workspace_bytes,
                         void *stream);

/* tq_attn_output for callers that cannot allocate memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same arguments, validation, kernels and results, but the per-split
 * partials live in a fixed device array of the library instead of a caller
 * workspace.  The array holds TQ_NOALLOC_SCRATCH_BYTES (4 MiB); every device
 * the call runs on holds its own copy until the process ends (its address is
 * looked up on the first call on each device).  Calls whose
 * tq_attn_output_workspace_size exceeds that return TQ_ERR_UNSUPPORTED
 * before any launch.  Every call on one device shares the array: calls that
 * overlap in time on a device (several streams, several host threads) race
 * and give wrong results, so queue them on one stream.  Nothing in the array
 * needs clearing: every call writes all it reads.
 * Errors: TQ_ERR_INVALID, TQ_ERR_UNSUPPORTED, TQ_ERR_HIP. */
#define TQ_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
tq_status tq_attn_output_noalloc(const tq_params *p, const float *logits, int32_t batch, int32_t n_q_heads,
                                 int32_t n_kv_heads, const tq_packed *v, int64_t row_tokens, int64_t seq_len,
                                 void *out, int32_t out_dtype, void *stream);

/* Device scratch that tq_attn_output needs for these arguments on the
 * current device; 0 when seq_len or batch is 0.
 * Errors: TQ_ERR_INVALID, TQ_ERR_UNSUPPORTED. */
tq_status tq_attn_output_workspace_size(const tq_params *p, int32_t batch, int32_t n_q_heads,
                                        int32_t n_kv_heads, int64_t seq_len, size_t *bytes);

/* Reconstruct n_vec vectors (page section "2단계": reconstructed vectors).
 *   out          device [n_vec][d], out_dtype TQ_F32 or TQ_BF16
 * Supported: d in {64, 128, 256} in all three modes.
 * Errors: TQ_ERR_INVALID, TQ_ERR_UNSUPPORTED, TQ_ERR_HIP. */
tq_status tq_dequantize(const tq_params *p, const tq_packed *k, int64_t n_vec, void *out,
                        int32_t out_dtype, void *stream);

/* Ceiling probes (measurement support, not a step of the method): the best
 * this device reaches on a plain stream or instruction loop, against which
 * the hot-path kernels' rooflines are also reported.
 *   TQ_PROBE_READ      read `bytes` of `buf` once (16-byte non-temporal loads)
 *   TQ_PROBE_WRITE     write `bytes` of `buf` once (16-byte non-temporal stores)
 *   TQ_PROBE_MFMA_F16  every wave of the grid runs 4 x `iters` 32x32x16 fp16
 *                      MFMAs (32768 flops each) on registers; no memory
 *   TQ_PROBE_MFMA_I8   the same with 16x16x64 int8 MFMAs (32768 ops each)
 * The grid is tq_probe_sink_words / 4 workgroups of 4 waves; `sink` (device,
 * sink_words uint32) receives values that keep the work live.  buf: device,
 * 16-byte aligned, bytes a multiple of 16.
 * Errors: TQ_ERR_INVALID, TQ_ERR_HIP. */
enum { TQ_PROBE_READ = 0, TQ_PROBE_WRITE = 1, TQ_PROBE_MFMA_F16 = 2, TQ_PROBE_MFMA_I8 = 3 };
tq_status tq_probe_sink_words(int64_t *words);
tq_status tq_probe(int32_t kind, void *buf, int64_t bytes, int32_t iters, uint32_t *sink, int64_t sink_words,
                   void *stream);

/* Human-readable name of a status code (static string). */
const char *tq_status_string(tq_status s);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
