/*
 * qmm.h -- C ABI of libqmm: group-wise INT4 weight quantization and the
 * quantized matmuls that consume it, for AMD Instinct MI355X (gfx950).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  * All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or retains them.  Tensors are dense row-major.
 *  * `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *    compute call only enqueues kernels on `stream` and returns; results are
 *    ready when the stream has reached that point.  Calls on one stream are
 *    ordered; calls that overlap in time must not share output buffers.
 *  * Shapes are int64_t.  The weight matrix W is [N, K]: N output channels
 *    (rows), K input features; activations are [M, K] (or [B, K]); outputs
 *    are [M, N].  Y = X W^T.
 *  * Return value: QMM_OK (0) or a negative status.  On any error nothing is
 *    launched and no output is written.  Argument errors are detected on the
 *    host before any HIP call.  Nothing throws or aborts across the ABI.
 *  * Pointers must be 16-byte aligned (QMM_EALIGN otherwise), except the
 *    per-row / per-column vectors (scales, zero-points, column maxima) which
 *    need only their element alignment; the smoothing factors passed to the
 *    INT8 quantizers are read 16 bytes at a time and must be 16-byte aligned.
 *
 * INT4 storage format (one format for every entry point):
 *  * codes  : uint8 [N, K/2], read as little-endian 32-bit words: word w of
 *             a row holds elements 8w..8w+7, element 8w+2i in bits 4i..4i+3
 *             and element 8w+2i+1 in bits 16+4i..16+4i+3 (i = 0..3).  So
 *             byte 0 holds elements 0 and 2, byte 1 elements 4 and 6, byte 2
 *             elements 1 and 3, byte 3 elements 5 and 7 (low nibble first).
 *             This order lets the kernels expand a word into four pairs of
 *             consecutive weights with one shift and one AND-OR per pair.
 *  * scales : float32 [N, G], G = K / group.
 *  * zeros  : uint8 [N, ceil(G/2)], zero-point of group 2j in the low nibble
 *             of byte j and of group 2j+1 in the high nibble (an odd G leaves
 *             the last high nibble 0).
 * Half a byte per weight plus a scale and a 4-bit zero-point per group is the
 * storage the sources count ("How quantization works", Exercises 2; "Quantization
 * Explained", slide "The Cost of Small Groups"); they do not fix a byte
 * layout, so this one is the library's own.  The scale is stored in fp32.
 */
#ifndef QMM_H_
#define QMM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { QMM_F32 = 0, QMM_F16 = 1, QMM_BF16 = 2, QMM_I32 = 3 } qmm_dtype;

enum {
  QMM_OK = 0,
  QMM_EINVAL = -1,        /* null pointer, non-positive size, K % group != 0, bad dtype value */
  QMM_EUNSUPPORTED = -2,  /* valid request this library does not implement (bits != 4, group != 128, dtype combo) */
  QMM_EALIGN = -3,        /* a tensor pointer is not 16-byte aligned */
  QMM_EWORKSPACE = -4,    /* workspace missing or smaller than the *_workspace_bytes query */
  QMM_EHIP = -5,          /* a HIP launch or device query failed */
  QMM_ERANGE = -6         /* a size exceeds what the arithmetic guarantees (e.g. int32 accumulator) */
};

/* Human-readable name of a status code (static string, never NULL). */
const char* qmm_status_string(int status);

/* ABI version: major * 10000 + minor * 100 + patch. */
int qmm_version(void);

/* Byte sizes of the INT4 format for a [N, K] weight with the given group size.
 * Any output pointer may be NULL.  QMM_EINVAL if N, K <= 0, group <= 0 or
 * K % group != 0.  Host-only. */
int qmm_w4_sizes(int64_t N, int64_t K, int group, size_t* codes_bytes, size_t* scales_bytes,
                 size_t* zeros_bytes);

/* ---------------------------------------------------------------------------
 * quantize_groupwise -- asymmetric per-group quantization of W.
 *
 * For every row n and group g (elements k in [g*group, (g+1)*group)):
 *   lo = min(0, min_k W), hi = max(0, max_k W)
 *   s  = (hi - lo) / (2^bits - 1)            (s = 1 when that is 0)
 *   z  = round(-lo / s)
 *   q  = clamp(round(W / s) + z, 0, 2^bits - 1)
 * in IEEE fp32 with correctly rounded division and round-half-to-even.
 * Sources: "Quantization Explained" (slides "Scale and Zero-Point", "Manual
 * Group-Wise Quantizer"); "How quantization works" ("The math of quantization",
 * asymmetric form); "Quantization from Scratch" ("Scale and zero-point", and
 * its round-to-nearest listing for the s = 1 rule and clip-after-zero-point).
 * Widening [min, max] to contain 0 keeps z a valid code for one-signed groups;
 * it changes nothing for groups that straddle 0.
 *
 * W      : [N, K] of w_dtype (QMM_F32, QMM_BF16 or QMM_F16).
 * codes, scales, zeros : outputs in the INT4 format above.
 * bits must be 4 and group 128 (QMM_EUNSUPPORTED otherwise).
 * ------------------------------------------------------------------------- */
int quantize_groupwise(const void* W, int w_dtype, int64_t N, int64_t K, int group, int bits,
                       uint8_t* codes, float* scales, uint8_t* zeros, void* stream);

/* ---------------------------------------------------------------------------
 * quantize_groupwise_symmetric -- symmetric per-group quantization of W into
 * the same INT4 format, so dequantize, w4a16_gemv and w4a16_gemm consume it
 * unchanged.  For every row n and group g:
 *   s    = max(max_k |W|, 1e-8) / (2^(bits-1) - 1)
 *   q    = clamp(round(W / s), -2^(bits-1), 2^(bits-1) - 1)
 *   code = q + 2^(bits-1), stored zero-point 2^(bits-1)   ((code - z) s = q s)
 * in IEEE fp32 with correctly rounded division and round-half-to-even.
 * Sources: "How quantization works" ("The math of quantization", symmetric
 * form); "Quantization from Scratch" ("Scale and zero-point": the symmetric
 * grid, 15 of the 16 levels at 4 bits, the 16th an extra negative level).
 * The 1e-8 floor of an all-zero group's absmax is the one the INT8 path uses
 * ("How quantization works", fake-quantization listing).
 * Arguments, layouts and errors as quantize_groupwise; every stored
 * zero-point nibble is 8.
 * ------------------------------------------------------------------------- */
int quantize_groupwise_symmetric(const void* W, int w_dtype, int64_t N, int64_t K, int group, int bits,
                                 uint8_t* codes, float* scales, uint8_t* zeros, void* stream);

/* ---------------------------------------------------------------------------
 * dequantize -- W_hat = (q - z) * s, one fp32 rounding, then rounded to
 * out_dtype (QMM_F32, QMM_BF16 or QMM_F16; round to nearest even).
 * Sources: "Quantization from Scratch" ("Scale and zero-point"); "Quantization
 * Explained" (slide "Uniform Affine Quantization").
 * W_hat : [N, K] output.  bits 4, group 128.
 * ------------------------------------------------------------------------- */
int dequantize(const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K,
               int group, int bits, void* W_hat, int out_dtype, void* stream);

/* ---------------------------------------------------------------------------
 * w4a16_gemv -- decode-time matmul with INT4 weights and 16-bit activations:
 *   y[b, n] = sum_k x[b, k] * W_hat[n, k],  W_hat = (q - z) * s,
 * accumulated in fp32, the weights dequantized in registers and never
 * written out.  Sources: "How quantization works" ("Inference view": unpack
 * in registers, scale, compute in 16 bits); "Quantization Explained" ("Why It
 * Is Faster"); "Quantization from Scratch" ("What it buys at decode").
 * x : [B, K] of x_dtype (QMM_BF16 or QMM_F16), 1 <= B <= 8.
 * y : [B, N] of y_dtype (x_dtype or QMM_F32).
 * group 128.  B == 1 runs on the vector ALUs only (no matrix cores);
 * 2 <= B <= 8 contracts on the matrix cores (the kernel of w4a16_gemm).
 * K <= 2^24 and N < 2^31 (QMM_ERANGE otherwise): tile offsets are 32-bit.
 * ------------------------------------------------------------------------- */
int w4a16_gemv(const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K,
               int group, const void* x, int x_dtype, int64_t B, void* y, int y_dtype, void* stream);

/* ---------------------------------------------------------------------------
 * w4a16_gemm -- the same product for a batch of M tokens (prefill / large
 * batch): Y[M, N] = X[M, K] W_hat^T, bf16 MFMA with fp32 accumulation.
 * Source: "How quantization works" ("Inference view"); "Quantization from
 * Scratch" ("What it buys at decode", growing batch).
 * X : [M, K] QMM_BF16 or QMM_F16.  Y : [M, N] of X's type or QMM_F32.
 * M >= 1, group 128, K <= 2^24, N and M < 2^31 (QMM_ERANGE otherwise).
 * A block keeps the zero points of its weight rows in
 * LDS, which bounds K for those kernels: K <= 52224 for M > 16 and
 * K <= 384000 for M <= 16; beyond that a slower kernel without the table
 * serves both activation types.
 * ------------------------------------------------------------------------- */
int w4a16_gemm(const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K,
               int group, const void* X, int x_dtype, int64_t M, void* Y, int y_dtype, void* stream);

/* ---------------------------------------------------------------------------
 * w8a16_gemv -- weight-only INT8 decode matmul:
 *   y[b, n] = w_scale[n] * sum_k x[b, k] * qW[n, k]
 * with per-output-channel INT8 weights (sq_quantize_weight with smooth NULL
 * writes them) and 16-bit activations, accumulated in fp32; each weight byte
 * is converted exactly to a 16-bit float.  B <= 2 runs on the vector ALUs
 * (dot2), 3 <= B <= 8 on bf16/fp16 matrix cores with the weights as operand.
 * Source: "How quantization works" ("Mainstream schemes at a glance": W8A16
 * halves the weight bytes of decode while computing in 16 bits).
 * qW : int8 [N, K] row-major, 16-byte aligned.  w_scale : float32 [N].
 * x  : [B, K] of x_dtype (QMM_BF16 or QMM_F16), 16-byte aligned, 1 <= B <= 8.
 * y  : [B, N] of y_dtype (x_dtype or QMM_F32).
 * K a multiple of 64 (QMM_EUNSUPPORTED otherwise), K <= 2^24 and N < 2^31
 * (QMM_ERANGE).  Errors are detected on the host before any launch.
 * ------------------------------------------------------------------------- */
int w8a16_gemv(const int8_t* qW, const float* w_scale, int64_t N, int64_t K, const void* x, int x_dtype,
               int64_t B, void* y, int y_dtype, void* stream);

/* ---------------------------------------------------------------------------
 * SmoothQuant W8A8.
 * Sources: "How quantization works" ("Activation quantization and outliers":
 * per-row INT8 weights, the smoothing factor with alpha and its 1e-5 floor);
 * "Quantization" (Engine Room ch. 15), "The Mathematics", the smoothing
 * equation Y = (X diag(s)^-1)(diag(s) W); "Quantization: Smaller Weights, Same
 * Answers (Mostly)" ("How does quantized matrix multiplication actually run
 * on the GPU?": INT8 products summed exactly in 32 bits; "Quick Reference":
 * per-token dynamic activation scales).
 * ------------------------------------------------------------------------- */

/* Calibration: x_colmax[k] = max_m |X[m,k]|, w_colmax[k] = max_n |W[n,k]| and
 *   smooth[k] = max(x_colmax,1e-5)^alpha / max(w_colmax,1e-5)^(1-alpha)
 * (alpha = 0.5 uses two correctly rounded square roots and one division, so
 * it is exact in fp32; other alpha use powf).  X [M, K], W [N, K] of
 * QMM_BF16 / QMM_F16 / QMM_F32; outputs float32 [K]. */
int sq_smooth_factors(const void* X, int x_dtype, int64_t M, const void* W, int w_dtype, int64_t N,
                      int64_t K, float alpha, float* x_colmax, float* w_colmax, float* smooth, void* stream);

/* Offline weight side: Ws = W * smooth[k] (fp32), w_scale[n] = max(max_k |Ws|, 1e-8) / 127,
 * qW = clamp(round(Ws / w_scale[n]), -128, 127).  smooth may be NULL (no smoothing).
 * qW int8 [N, K], w_scale float32 [N]. */
int sq_quantize_weight(const void* W, int w_dtype, const float* smooth, int64_t N, int64_t K, int8_t* qW,
                       float* w_scale, void* stream);

/* Online activation side (per token): Xs = X / smooth[k] (fp32),
 * x_scale[m] = max(max_k |Xs|, 1e-8) / 127, qX = clamp(round(Xs / x_scale[m]), -128, 127).
 * smooth may be NULL.  qX int8 [M, K], x_scale float32 [M]. */
int sq_quantize_activation(const void* X, int x_dtype, const float* smooth, int64_t M, int64_t K,
                           int8_t* qX, float* x_scale, void* stream);

/* Per-tensor activation quantization, the W8A8 baseline that the per-token
 * form improves on ("How quantization works", "Activation quantization and
 * outliers": one scale for the whole activation matrix, set by its largest
 * entry).  Xs = X / smooth[k] (fp32), a = max(max_{m,k} |Xs|, 1e-8) / 127,
 * qX = clamp(round(Xs / a), -128, 127); a is written to every x_scale[m], so
 * sq_int8_gemm consumes the result unchanged.  Three launches on the stream
 * (row maxima into x_scale, the tensor scale, quantization); X is read
 * twice.  Arguments and errors as sq_quantize_activation. */
int sq_quantize_activation_per_tensor(const void* X, int x_dtype, const float* smooth, int64_t M, int64_t K,
                                      int8_t* qX, float* x_scale, void* stream);

/* INT8 GEMM: acc[m,n] = sum_k qX[m,k] qW[n,k] exactly in int32 (i8 MFMA), then
 * Y = acc * x_scale[m] * w_scale[n] rounded to y_dtype (QMM_BF16 or QMM_F32), or
 * the raw int32 acc when y_dtype is QMM_I32 (x_scale / w_scale ignored, may be NULL).
 * K must be a multiple of 64 and at most 131008, the largest such K with
 * 128 * 128 * K < 2^31, so no int32 sum can overflow (QMM_ERANGE otherwise). */
int sq_int8_gemm(const int8_t* qX, const float* x_scale, const int8_t* qW, const float* w_scale, int64_t M,
                 int64_t N, int64_t K, void* Y, int y_dtype, void* stream);

/* Bytes of workspace smooth_quant_w8a8_gemm needs: M*K (qX) rounded up to 256
 * plus M*4 (x_scale).  Returns 0 for non-positive sizes.  Host-only. */
size_t sq_workspace_bytes(int64_t M, int64_t K);

/* The online W8A8 step: sq_quantize_activation into `workspace`, then
 * sq_int8_gemm.  smooth may be NULL.  qW / w_scale come from
 * sq_quantize_weight with the same smooth.  workspace: device memory of at
 * least sq_workspace_bytes(M, K), 16-byte aligned (QMM_EWORKSPACE otherwise). */
int smooth_quant_w8a8_gemm(const void* X, int x_dtype, const float* smooth, const int8_t* qW,
                           const float* w_scale, int64_t M, int64_t N, int64_t K, void* Y, int y_dtype,
                           void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H_ */
