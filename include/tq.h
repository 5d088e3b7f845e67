/*
 * tq.h -- C ABI of libtq, the MI355X (gfx950) TurboQuant KV-cache quantizer.
 *
 * Sources (cited by short tag below):
 *   [Scratch] "TurboQuant From Scratch on Real KV Tensors -- What 3 Bits
 *             Actually Cost, and Why the Forks Beat the Paper's Layout"
 *             (www.sotaaz.com/post/turboquant-scratch-en)
 *   [README]  "turboquant-pytorch" README (github, ringlorn/turboquant-pytorch)
 *   [Fork]    "TurboQuant KV Cache Quantization (Experimental)",
 *             llama.cpp-turboquant docs/turboquant.md
 *   [Blog]    "TurboQuant: 3-Bit Compression with Zero Overhead"
 *             (cneuralnets.xyz/blog/turboquant)
 *
 * Conventions for every entry point:
 *   - Device pointers are plain HIP device addresses allocated by the caller
 *     (e.g. torch tensors' data_ptr()).  The library never allocates, frees or
 *     synchronises on the compute calls; scratch space comes from a caller
 *     workspace sized with tq_workspace_size().
 *   - `stream` is a hipStream_t (NULL = the default stream).  Kernels are
 *     enqueued on it and the call returns without waiting; faults inside a
 *     kernel surface at the caller's next synchronisation.
 *   - Arguments are validated on the host before anything is launched.  A
 *     call that returns anything but TQ_OK has launched nothing, except
 *     TQ_ERR_HIP, which reports a launch failure.  tq_last_error() gives a
 *     human-readable reason (per thread).
 *   - n = 0 rows/keys/tokens is a valid no-op that returns TQ_OK.
 *   - Non-finite inputs give unspecified (but memory-safe) outputs.
 *   - Calls are stateless and thread-safe; calls on different streams may
 *     overlap if their output buffers do not.
 *
 * Data layout (all little-endian, row-major):
 *   A "unit" is a dt-long slice of a head vector: the whole vector
 *   (dt = head_dim) or one block of the block-32 layout (dt = 32, [Scratch]
 *   §7, [Fork] "GGML Types").  A row of head_dim elements holds
 *   head_dim / dt units.
 *   codes   : [units][dt * bits / 8] bytes.  Each unit is a run of 32-
 *             coordinate groups; a group is a little-endian bit stream with
 *             coordinate j at bits [bits*j, bits*j + bits).  The stored
 *             b-bit code of coordinate i is the sign-magnitude form of its
 *             bucket index idx (0..2^b-1, ascending centroids): with
 *             h = 2^(b-1), code = idx - h if idx >= h, else
 *             2^(b-1) | (h - 1 - idx).
 *   norms   : [units] of norm_dtype (the unit's L2 norm, [Scratch] §2 step 1).
 *   qjl_bits: [units][m / 8] bytes, projection i at bit i%8 of byte i/8,
 *             1 meaning sign(+), i.e. (S r)_i >= 0.
 *   qjl_rnorm: [units] binary16, the residual norm ||r||.
 *
 * Records (flag TQ_BLOCKS; [Fork] "GGML Types" and "How it works"): instead of
 *   the two planes above, one array of 32-coordinate records in coordinate
 *   order, record g = the binary16 norm of the unit that group g belongs to,
 *   then group g's 4 * bits code bytes (14 bytes per 32 values at 3 bits, 18
 *   at 4).  With dt = 128 this is the fork's turbo3/turbo4 layout: rows walked
 *   in 128-value chunks, each its own unit, the chunk norm copied into each of
 *   its four records.  Decode scales each group by the norm in its own record.
 *   Requires norm_dtype TQ_F16, no TQ_QJL; the record array is passed as
 *   `codes` (16-byte aligned) and `norms` must be NULL.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARG = 1, /* a pointer, size, stride, alignment or flag is wrong */
  TQ_ERR_UNSUPPORTED = 2, /* a valid but unimplemented combination */
  TQ_ERR_WORKSPACE = 3,   /* workspace missing or smaller than tq_workspace_size() */
  TQ_ERR_HIP = 4          /* the HIP runtime reported an error */
} tq_status;

typedef enum { TQ_F16 = 0, TQ_F32 = 1 } tq_dtype;

enum {
  TQ_NORM_CORRECT = 1u, /* rescale the reconstructed direction to unit length ([Scratch] §6) */
  TQ_QJL = 2u,          /* add the 1-bit QJL residual stage ([Scratch] §2, [README]) */
  TQ_BLOCKS = 4u        /* codes and norms as the fork's 32-value records (see "Records" above) */
};

enum { TQ_OP_QJL_SCORES = 1, TQ_OP_DECODE_ATTN = 2, TQ_OP_MULTI_ATTN = 3 };

/*
 * Lloyd-Max codebook for one rotated coordinate, whose variance is 1/dim
 * ([Scratch] §2 step 3: computed once per bit width, no calibration).  Plain
 * host data.  unit_* are the values for the unit-variance variable
 * sqrt(dim) * coordinate; the codebook proper is unit_* / sqrt(dim).  Only the
 * first 2^bits centroids and 2^bits - 1 bounds are meaningful.  Every kernel
 * reads only these fields, so either solver below can feed any entry point.
 */
typedef struct {
  int bits;                     /* 1..8 */
  int dim;                      /* transform length the codebook is scaled for */
  double unit_centroids[256];   /* ascending, symmetric about 0 */
  double unit_bounds[255];      /* midpoints of neighbouring centroids */
  float centroids[256];         /* fp32(unit_centroids / sqrt(dim)) */
  float bounds[255];            /* fp32(unit_bounds / sqrt(dim)) */
  double distortion;            /* E[(X - Q(X))^2] for the unit-variance X the codebook was solved for */
} tq_codebook;

/*
 * Fill *out with the Lloyd-Max quantizer of N(0,1/dim) at `bits` bits.
 * Host only, float64: Lloyd's fixed-point iteration up to 4 bits, Newton's
 * method on the same conditions above (the 8-bit keys of [Scratch] §10;
 * the quantize/dequantize kernels take 1..4 and 8 bits).  bits in 1..8, dim a
 * power of two in 2..4096.  Errors: TQ_ERR_INVALID_ARG.
 */
tq_status tq_codebook_init(tq_codebook* out, int bits, int dim);

/*
 * Fill *out with the Lloyd-Max quantizer of the exact marginal of a rotated
 * unit vector ([Fork] "How it works": centroids solved for the
 * Beta((dim-1)/2, (dim-1)/2) law of one coordinate, i.e. density proportional
 * to (1 - t^2)^((dim-3)/2) on [-1, 1]; [README], stage 1 of its two-stage
 * description: the Gaussian N(0, 1/dim) of tq_codebook_init is its large-dim
 * limit).  It differs from
 * the Gaussian codebook most at small dim, e.g. the 32-coordinate blocks of
 * [Scratch] §7.  Same fields and scaling as tq_codebook_init (X = sqrt(dim) T
 * has unit variance); distortion is the MSE under this law.  Host only,
 * float64.  bits in 1..4, dim a power of two in 4..4096 (the law is
 * log-concave there, so the fixed point is unique).  Errors:
 * TQ_ERR_INVALID_ARG.
 */
tq_status tq_codebook_init_beta(tq_codebook* out, int bits, int dim);

/*
 * One quantizer (e.g. the key quantizer or the value quantizer of a cache).
 *   head_dim   elements per input row, a multiple of dt
 *   dt         transform / normalisation length: 32, 64, 128 or 256
 *   bits       1..4 or 8, must equal cb->bits; cb->dim must equal dt (QJL
 *              takes a 1..4-bit first stage)
 *   flags      any of TQ_NORM_CORRECT, TQ_QJL, TQ_BLOCKS (TQ_BLOCKS excludes TQ_QJL)
 *   qjl_m      number of QJL projections (TQ_QJL only): 32..256, multiple of 32
 *   x_dtype    element type of the input rows (TQ_F16 or TQ_F32)
 *   norm_dtype type of the stored norms (TQ_F16 or TQ_F32)
 *   cb         host pointer to the codebook
 *   signs      host pointer, dt values each exactly +1 or -1: the random
 *              diagonal D of the rotation y = H D u ([Scratch] §2 step 2)
 *   qjl_params device pointer written by tq_qjl_prepare (TQ_QJL only)
 */
typedef struct {
  int head_dim;
  int dt;
  int bits;
  unsigned flags;
  int qjl_m;
  tq_dtype x_dtype;
  tq_dtype norm_dtype;
  const tq_codebook* cb;
  const float* signs;
  const void* qjl_params;
} tq_config;

/* Bytes of device memory tq_qjl_prepare writes for (m, dt). */
size_t tq_qjl_params_size(int m, int dt);

/*
 * Prepare the QJL projection for cfg: from the host matrix S ([m][dt] fp32,
 * i.i.d. N(0,1) entries, [README] estimator) compute S~ = S D H in float64 on
 * the host and copy S~ (float64 and float32 copies) to params_dev
 * (>= tq_qjl_params_size(m, dt) bytes, 16-byte aligned).  Because H and D
 * are symmetric involutions, the residual of the unrotated unit vector
 * projects as S (u - D H c) = S~ (y - c), so the device works in the rotated
 * domain.  Set-up only: this call synchronises `stream`.
 */
tq_status tq_qjl_prepare(const tq_config* cfg, const float* S_host, void* params_dev, size_t params_bytes,
                         void* stream);

/*
 * Encode n_rows rows ([Scratch] §2 steps 1-3, [Fork] "How it works"):
 * per unit n = ||x||, u = x / n, y = H D u, idx_i = #{bounds < y_i}, codes
 * packed as described above, n stored as norm_dtype.  With TQ_QJL
 * (dt == head_dim required) also r = u - D H c[idx], qjl_rnorm = ||r|| and
 * qjl_bits = [S r >= 0].
 * Exact ties: a coordinate that lies exactly on a cell edge is equally near
 * both neighbouring centroids, and either cell may be stored.  The encoders
 * pick the half (idx >= 2^(b-1) or below) from y's sign and then the cell
 * nearer zero within it: without TQ_QJL by the float's sign bit (+0.0 takes
 * idx 2^(b-1), -0.0 takes 2^(b-1) - 1), with TQ_QJL by y > 0 (both zeros take
 * 2^(b-1) - 1).  A value on any other edge thus goes to the lower cell when
 * positive and to the upper one when negative.  (The rounded y a kernel
 * compares differs from the exact y in the last bits anyway.)
 *   x        device, rows of ld_x elements (ld_x >= head_dim); 16-byte
 *            aligned, ld_x * element size a multiple of 16 bytes
 *   codes    device, 4-byte aligned, n_rows * head_dim/dt units (TQ_BLOCKS:
 *            the records, 16-byte aligned)
 *   norms    device, aligned to norm_dtype (TQ_BLOCKS: NULL)
 *   qjl_bits, qjl_rnorm  device (TQ_QJL), otherwise ignored
 * A zero unit stores norm 0 and the codes of idx = 2^(b-1) - 1.
 * At 4 and 8 bits the encoder finds a code's cell through a uniform bin table
 * of |y| with 1.6 bins per narrowest cell; a codebook whose edges would need
 * more than 256 bins at 4 bits or 1024 at 8 (the built-in codebooks need
 * about 17 and 420) is rejected with TQ_ERR_INVALID_ARG.
 */
tq_status tq_quantize(const tq_config* cfg, const void* x, int64_t n_rows, int64_t ld_x, uint8_t* codes,
                      void* norms, uint8_t* qjl_bits, void* qjl_rnorm, void* stream);

/*
 * Decode n_rows rows ([Scratch] §2 "un-rotate", §6 norm correction,
 * [Fork] "How it works"): c = centroid(code), optional QJL correction
 * c += sqrt(pi/2) * rnorm / m * S~^T sign (in the rotated domain), optional
 * norm correction c /= ||c||, then x~ = n * D H c written as y_dtype rows of
 * stride ld_y (16-byte aligned like x).  codes and norms as for tq_quantize
 * (TQ_BLOCKS: records in codes, norms NULL).
 */
tq_status tq_dequantize(const tq_config* cfg, const uint8_t* codes, const void* norms, const uint8_t* qjl_bits,
                        const void* qjl_rnorm, int64_t n_rows, void* y, tq_dtype y_dtype, int64_t ld_y,
                        void* stream);

/*
 * QJL inner-product scores ([README] combined estimator):
 *   scores[i][j] = n_j * ( <q_i, D H c_j> + rnorm_j * sqrt(pi/2)/m * <S q_i, sign_j> )
 * for n_q query rows (q_dtype, row stride ld_q >= head_dim, head_dim == dt)
 * against n_k keys encoded with TQ_QJL.  scores: device fp32 [n_q][ld_s],
 * ld_s >= n_k.  Norm correction is not applied to scores (TQ_NORM_CORRECT
 * is rejected).  Supported: 1..3-bit MSE stage, head_dim <= 128, qjl_m <= 128
 * (TQ_ERR_UNSUPPORTED otherwise), at most 2^31 queries and keys per call.
 * ws: 256-byte aligned device workspace of
 * tq_workspace_size(TQ_OP_QJL_SCORES, cfg, n_q, n_k, 0) bytes (the queries'
 * int8 operand records and scales; contents are scratch).
 */
tq_status tq_qjl_scores(const tq_config* cfg, const void* q, tq_dtype q_dtype, int64_t n_q, int64_t ld_q,
                        const uint8_t* codes, const void* norms, const uint8_t* qjl_bits, const void* qjl_rnorm,
                        int64_t n_k, float* scores, int64_t ld_s, void* ws, size_t ws_bytes, void* stream);

/*
 * Single-token decode attention over a quantized cache ([Fork] "Fused tile
 * path": q is rotated once, scores and the value sum are formed in the
 * rotated domain, one inverse transform per output block at the end):
 *   out[h] = sum_j softmax_j(scale * <q_h, k~_j>) v~_j
 * with query head h reading KV head h / (n_q_heads / n_kv_heads) and k~, v~
 * the tq_dequantize reconstructions of the cached units.
 *   kcfg, vcfg  formats of K and V: block-32 layout (dt = 32), fp16 norms,
 *               K at 3, 4 or 8 bits and V at 3 or 4 bits (K and V may differ;
 *               8-bit keys with 4-bit values is the asymmetric allocation of
 *               [Scratch] §4 "Finding 1" and §10 "Takeaways"), equal head_dim
 *               of 128 or 256, no flags (TQ_ERR_UNSUPPORTED otherwise)
 *   q           device, [n_q_heads][head_dim] of q_dtype, contiguous
 *   n_q_heads   a multiple of n_kv_heads (all heads of a KV head share each
 *               K and V read: up to 16 in the decode kernel, more in row
 *               groups of 128 of the multi-row kernel)
 *   k_codes, v_codes  device, 4-byte aligned, units in (kv head, token,
 *               block) order, i.e. rows of tq_quantize over
 *               [n_kv_heads][n_tokens][head_dim]
 *   k_norms, v_norms  device fp16, same unit order
 *   scale       softmax scale; <= 0 selects 1/sqrt(head_dim)
 *   out         device fp32 [n_q_heads][head_dim]
 *   ws          256-byte aligned device workspace of
 *               tq_workspace_size(TQ_OP_DECODE_ATTN, kcfg, n_q_heads,
 *               n_kv_heads, n_tokens) bytes (per-wave partial maxima, sums
 *               and value accumulators; contents are scratch)
 * Precision: scores use a two-term fp16 split of the rotated query and of the
 * K centroids (about 2^-22 relative); the value sum takes the softmax weight
 * times the V norm and the V centroids as fp16 operands (unit roundoff 2^-11)
 * with fp32 accumulation.  n_tokens = 0 leaves out untouched.
 */
tq_status tq_decode_attn(const tq_config* kcfg, const tq_config* vcfg, const void* q, tq_dtype q_dtype,
                         int n_q_heads, int n_kv_heads, int64_t n_tokens, const uint8_t* k_codes, const void* k_norms,
                         const uint8_t* v_codes, const void* v_norms, float scale, float* out, void* ws,
                         size_t ws_bytes, void* stream);

/*
 * tq_decode_attn for callers that cannot allocate: code inside HIP graph
 * capture, tight serving loops, and harnesses that forbid hipMalloc.  Same
 * arguments, kernels and results as tq_decode_attn, but no workspace: the
 * per-workgroup softmax partials go to a static scratch array of 16 MiB that
 * the library keeps on each device (resolved with hipGetSymbolAddress on the
 * first call on a device, held until the process ends).  The call allocates
 * and frees nothing.  A call whose partials need more than 16 MiB
 * (tq_workspace_size(TQ_OP_DECODE_ATTN, ...) > 16 MiB; at head_dim 256 and 16
 * query heads per KV head that is n_kv_heads * n_tokens above about 8.3 M,
 * e.g. 4 KV heads of more than 2 M tokens) returns TQ_ERR_UNSUPPORTED before
 * anything is launched.  All calls on one
 * device share that device's scratch: calls that overlap in time on one
 * device (different streams, or different threads without ordering) race and
 * give undefined results; calls ordered on one stream are safe.
 */
tq_status tq_decode_attn_noalloc(const tq_config* kcfg, const tq_config* vcfg, const void* q, tq_dtype q_dtype,
                                 int n_q_heads, int n_kv_heads, int64_t n_tokens, const uint8_t* k_codes,
                                 const void* k_norms, const uint8_t* v_codes, const void* v_norms, float scale,
                                 float* out, void* stream);

/*
 * Attention of several query tokens over the same quantized cache (the
 * [Fork] "Fused tile path" with more than one query column: a prefill chunk
 * or a batch of draft tokens).  Query token i (0 <= i < n_q) with head h:
 *   out[i][h] = sum_{j in S_i} softmax_j(scale * <q_ih, k~_j>) v~_j
 * over KV head h / (n_q_heads / n_kv_heads), where S_i is every cached token,
 * or with causal != 0 the tokens j <= n_tokens - n_q + i (the n_q queries are
 * the last n_q positions of the cache, whose K and V are already in it).
 *   kcfg, vcfg, k_codes, k_norms, v_codes, v_norms, scale: as tq_decode_attn
 *   q     device, [n_q][n_q_heads][head_dim] of q_dtype, contiguous
 *   out   device fp32 [n_q][n_q_heads][head_dim]
 *   ws    256-byte aligned device workspace of
 *         tq_workspace_size(TQ_OP_MULTI_ATTN, kcfg, n_q * n_q_heads,
 *         n_kv_heads, n_tokens) bytes (contents are scratch)
 * The (query token, head) rows of one KV head are processed in row groups
 * that share each K and V read: one group when there are at most 16 rows,
 * otherwise groups of 128 rows.  n_q = 1 without a mask is tq_decode_attn.
 * Errors: causal with n_q > n_tokens is TQ_ERR_INVALID_ARG; more than 65535
 * (KV head, row group) pairs or 2^31 rows is TQ_ERR_UNSUPPORTED; n_q = 0 or
 * n_tokens = 0 leaves out untouched.
 * Precision as tq_decode_attn.
 */
tq_status tq_multi_attn(const tq_config* kcfg, const tq_config* vcfg, const void* q, tq_dtype q_dtype, int64_t n_q,
                        int n_q_heads, int n_kv_heads, int64_t n_tokens, const uint8_t* k_codes, const void* k_norms,
                        const uint8_t* v_codes, const void* v_norms, int causal, float scale, float* out, void* ws,
                        size_t ws_bytes, void* stream);

/* Workspace bytes for op (TQ_OP_*) with sizes (a, b, c) as described per op; 0 if none. */
size_t tq_workspace_size(int op, const tq_config* cfg, int64_t a, int64_t b, int64_t c);

const char* tq_status_str(tq_status s);
const char* tq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H_ */
