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

/* Diagnostics: a plain streaming read of `bytes` bytes of device memory at
 * `data`, every 16-byte piece once, folded into *out (device, uint32) as the
 * XOR of all 32-bit words so that no load can be dropped.  For measuring the
 * bandwidth a plain read reaches on this GPU, the practical ceiling of the
 * HBM-bound kernels above (decode time is the weight bytes over that
 * bandwidth: "Quantization from Scratch", "What it buys at decode").  Two
 * launches on the stream (a one-thread clear of *out, then the read).
 * QMM_EINVAL for a null pointer or bytes == 0; QMM_EALIGN unless data is
 * 16-byte aligned, bytes % 16 == 0 and out 4-byte aligned. */
int qmm_stream_read(const void* data, size_t bytes, uint32_t* out, void* stream);

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
 * codes, scales, zeros : outputs in the INT4 format above (bits 4, group
 *          128); other group sizes and bit widths write the formats of
 *          quantize_groupwise_ex with fp32 scales.
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
 * W_hat : [N, K] output.  Other group sizes and bit widths: as dequantize_ex
 * with fp32 scales.
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
 * group 128 (other group sizes: as wxa16_gemv with 4 bits and fp32 scales).
 * B == 1 runs on the vector ALUs only (no matrix cores);
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
 * M >= 1, group 128 (other group sizes: as wxa16_gemm with 4 bits and fp32
 * scales), K <= 2^24, N and M < 2^31 (QMM_ERANGE otherwise).
 * A block keeps the zero points of its weight rows in
 * LDS, which bounds K for those kernels: K <= 52224 for M > 16 and
 * K <= 384000 for M <= 16; beyond that a slower kernel without the table
 * serves both activation types.
 * ------------------------------------------------------------------------- */
int w4a16_gemm(const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K,
               int group, const void* X, int x_dtype, int64_t M, void* Y, int y_dtype, void* stream);

/* ---------------------------------------------------------------------------
 * Other stored formats: group sizes, 3- and 8-bit codes, 16-bit scales.
 *
 * The same method (asymmetric s = (hi - lo) / (2^bits - 1), z = round(-lo / s),
 * or the symmetric grid with code q + 2^(bits-1)) with:
 *  * group  : 32, 64, 128, 256, 512 or 1024 consecutive weights of a row
 *             ("Quantization Explained", "Measuring Your Own Error": group sizes
 *             from 32 to 1024);
 *  * bits   : 3, 4 or 8 ("Quantization from Scratch", "Measured on two real
 *             layers": 8-, 4- and 3-bit codes with group scales);
 *  * scale_dtype : QMM_F32, or QMM_F16 for one binary16 scale per group ("How
 *             quantization works", Exercise 2; "Quantization from Scratch",
 *             "Where to put the scales").  The codes are computed with the
 *             stored value: the fp32 scale rounded to nearest even, saturating
 *             at 65504, and 1 if that is 0.
 * Storage:
 *  * codes  : 4 bits -- the code words described above; 8 bits -- one byte per
 *             weight, [N, K]; 3 bits -- [N, 3K/8] bytes, each run of 32
 *             weights e = 0..31 of a row in three little-endian 32-bit words
 *             W0..W2: e < 30 in word e / 10 at bit 3 (r / 2) + 16 (r % 2),
 *             r = e % 10, so consecutive codes sit 16 bits apart; bit t of
 *             e = 30 at bit 15 of W[t], bit t of e = 31 at bit 31 of W[t]
 *             (K % 32 == 0 follows from the group sizes).
 *  * scales : [N, G] of scale_dtype.
 *  * zeros  : [N, ceil(G/2)] nibble pairs for 3 and 4 bits (as above), [N, G]
 *             bytes for 8 bits.
 * group 128 with 4 bits and fp32 scales is the format above and runs its
 * kernels.  Errors: QMM_EUNSUPPORTED for other groups / bits / scale types,
 * otherwise as the 4-bit calls.
 * ------------------------------------------------------------------------- */

/* Byte sizes of a stored format (any output pointer may be NULL).  Host-only. */
int qmm_wq_sizes(int64_t N, int64_t K, int group, int bits, int scale_dtype, size_t* codes_bytes,
                 size_t* scales_bytes, size_t* zeros_bytes);

/* Quantize W [N, K] (QMM_F32 / QMM_BF16 / QMM_F16) into a stored format;
 * symmetric != 0 selects the symmetric grid.  codes 16-byte aligned, scales
 * aligned to their element. */
int quantize_groupwise_ex(const void* W, int w_dtype, int64_t N, int64_t K, int group, int bits, int scale_dtype,
                          int symmetric, uint8_t* codes, void* scales, uint8_t* zeros, void* stream);

/* W_hat = (q - z) s in fp32 (one rounding), then out_dtype (QMM_F32 / QMM_BF16 / QMM_F16). */
int dequantize_ex(const uint8_t* codes, const void* scales, const uint8_t* zeros, int64_t N, int64_t K, int group,
                  int bits, int scale_dtype, void* W_hat, int out_dtype, void* stream);

/* y [B, N] = x [B, K] W_hat^T for 1 <= B <= 8, x QMM_BF16 / QMM_F16, y of x's
 * type or QMM_F32, fp32 accumulation with each group's scale applied to its
 * exact partial sums.  B <= 2 on the vector ALUs, B >= 3 on the matrix cores.
 * K <= 2^24 (QMM_ERANGE). */
int wxa16_gemv(const uint8_t* codes, const void* scales, const uint8_t* zeros, int64_t N, int64_t K, int group,
               int bits, int scale_dtype, const void* x, int x_dtype, int64_t B, void* y, int y_dtype, void* stream);

/* Y [M, N] = X [M, K] W_hat^T for any M >= 1 (matrix cores from 3 tokens). */
int wxa16_gemm(const uint8_t* codes, const void* scales, const uint8_t* zeros, int64_t N, int64_t K, int group,
               int bits, int scale_dtype, const void* X, int x_dtype, int64_t M, void* Y, int y_dtype, void* stream);

/* ---------------------------------------------------------------------------
 * Repack of 4-bit codes between plain nibble order (byte j of a row holds
 * element 2j in its low nibble and 2j+1 in its high nibble) and the library's
 * code words (above), both [N, K/2] bytes; K % 8 == 0, 16-byte aligned
 * pointers.  The pages fix half a byte per weight but no order; weights
 * packed in plain order by other tools go through repack_from_plain before
 * dequantize / w4a16_gemv / w4a16_gemm.  Input and output may be the same
 * buffer (each word is read before it is written by the same thread);
 * otherwise they must not overlap.
 * ------------------------------------------------------------------------- */
int qmm_w4_repack_from_plain(const uint8_t* plain, uint8_t* codes, int64_t N, int64_t K, void* stream);
int qmm_w4_repack_to_plain(const uint8_t* codes, uint8_t* plain, int64_t N, int64_t K, void* stream);

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

/* Size of the library's own device scratch used by smooth_quant_w8a8_gemm_noalloc. */
#define QMM_SQ_STATIC_SCRATCH_BYTES ((size_t)16 * 1024 * 1024 + (size_t)64 * 1024)

/* ---------------------------------------------------------------------------
 * smooth_quant_w8a8_gemm_noalloc -- smooth_quant_w8a8_gemm for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  It computes the same result with
 * the same kernels, but qX and x_scale live in a device array inside the
 * library (QMM_SQ_STATIC_SCRATCH_BYTES per GPU, held until the process ends)
 * instead of a caller workspace; the call itself allocates and frees nothing.
 * Its device address is looked up on the first call on each device.
 * Arguments and errors as smooth_quant_w8a8_gemm, without the workspace;
 * QMM_ERANGE when sq_workspace_bytes(M, K) > QMM_SQ_STATIC_SCRATCH_BYTES
 * (e.g. M * K above about 16.7 million), QMM_EHIP if the address lookup fails.
 * All calls on one GPU share the array: calls that overlap in time on one GPU
 * (other streams, other threads) race and must be serialized by the caller.
 * ------------------------------------------------------------------------- */
int smooth_quant_w8a8_gemm_noalloc(const void* X, int x_dtype, const float* smooth, const int8_t* qW,
                                   const float* w_scale, int64_t M, int64_t N, int64_t K, void* Y, int y_dtype,
                                   void* stream);

/* ---------------------------------------------------------------------------
 * FP8 E4M3 W8A8 -- 8-bit floating-point weights and activations on the fp8
 * matrix cores.  Sources: "How quantization works" (the fake-quantization
 * listing: s = max|x| / 448, E4M3's largest value, then x / s cast to E4M3;
 * "Mainstream schemes at a glance", FP8 row: FP8 weights and activations with
 * dynamic or static scales); "Quantization: Smaller Weights, Same Answers
 * (Mostly)" ("What about FP8, MXFP4, NVFP4 and GGUF?": E4M3, 4 exponent and 3
 * mantissa bits, up to 448).
 * Codes are OCP E4M3 ("E4M3FN": exponent bias 7, no infinities, largest
 * finite 448) bytes; the conversion of the correctly rounded fp32 quotient
 * x / s rounds to nearest even and gives +-448 from 448 up.  The absmax is
 * floored at 1e-8 (as the INT8 path).
 * ------------------------------------------------------------------------- */

/* q [rows, K] = E4M3(X / s) with s = max(max|X|, 1e-8) / 448 per row
 * (per_tensor == 0: per token for activations, per output channel for
 * weights) or for the whole matrix (per_tensor != 0, the listing's form; the
 * scale is written to every scale[row]).  X QMM_F32 / QMM_BF16 / QMM_F16,
 * K % 64 == 0. */
int fp8_quantize(const void* X, int x_dtype, int64_t rows, int64_t K, int per_tensor, uint8_t* q, float* scale,
                 void* stream);

/* Y [M, N] = (sum_k E4M3(qX[m,k]) E4M3(qW[n,k])) * x_scale[m] * w_scale[n],
 * products exact, fp32 accumulation, Y QMM_BF16 or QMM_F32.  K % 64 == 0,
 * K <= 131008. */
int fp8_gemm(const uint8_t* qX, const float* x_scale, const uint8_t* qW, const float* w_scale, int64_t M, int64_t N,
             int64_t K, void* Y, int y_dtype, void* stream);

/* The online FP8 step: per-token fp8_quantize of X into `workspace` (at
 * least sq_workspace_bytes(M, K) bytes, 16-byte aligned), then fp8_gemm. */
int fp8_w8a8_gemm(const void* X, int x_dtype, const uint8_t* qW, const float* w_scale, int64_t M, int64_t N,
                  int64_t K, void* Y, int y_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* -------------------------------------------------------------------------
 * LLM.int8() -- vector-wise INT8 with the outlier feature dimensions carved
 * out and multiplied in 16-bit.  Sources: "Quantization" (Engine Room ch.
 * 15), "The Mathematics" (the vector-wise scheme, one scale per row of X and
 * per output channel, with the outlier dimensions removed from the integer
 * product and added back as a 16-bit product: C = S_out (X_q W_q) +
 * X_16 W_16) and its history of LLM.int8() (a handful of systematically
 * large dimensions; more than 99.9% of the values still multiplied in
 * 8-bit); "Quantization: Smaller Weights, Same Answers (Mostly)" ("How do
 * LLM-specific quantization schemes protect against outliers?", family 1).
 * Readings where the pages leave the rule open:
 *  - a feature (column of X) is an outlier dimension of the batch when some
 *    token's |x| in it is >= `threshold` (an argument; the tests and the
 *    benchmark use 6);
 *  - the weights are stored once, as per-output-channel INT8 (qW, w_scale
 *    from sq_quantize_weight with no smoothing); the 16-bit weights of an
 *    outlier column are q * w_scale rounded to the activations' type
 *    (binary16 saturating at 65504);
 *  - the outlier columns are zero in X_q and take no part in a token's scale.
 * At most `max_outliers` columns are carved out: the first ones in column
 * order; any further outlier columns stay in the INT8 product (their count
 * is reported, so a caller can tell).  max_outliers above K means K.
 * X QMM_BF16 or QMM_F16 [M, K] (QMM_F32: QMM_EUNSUPPORTED), K % 64 == 0,
 * K <= 131008; threshold >= 0 (+inf: no outlier; 0: every column), else
 * QMM_EINVAL.
 * ------------------------------------------------------------------------- */

/* Outlier detection alone (the first two steps of llm_int8_gemm):
 * factor [K] (caller-owned, 4-byte aligned; used as scratch first) receives
 * +inf for each carved-out column and 1 for every other, index
 * [max(1, min(max_outliers, K))] the carved-out columns in increasing order,
 * counts [2] {carved out, found}.  sq_quantize_activation(X, factor) then
 * gives the call's X_q and token scales. */
int llm_int8_outliers(const void* X, int x_dtype, int64_t M, int64_t K, float threshold, int64_t max_outliers,
                      float* factor, int32_t* index, int32_t* counts, void* stream);

/* Bytes of workspace llm_int8_gemm needs: X_q (M K bytes) and the token
 * scales, the column factors, the outlier list (4 min(max_outliers, K)
 * bytes) and its counts, each part at a 256-byte boundary; N does not enter.
 * 0 for invalid sizes. */
size_t llm_int8_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t max_outliers);

/* Y [M, N] = acc * x_scale[m] * w_scale[n] + sum over the carved-out
 * columns j of X[m, j] * W16[n, j], where acc is the exact int32 product of
 * X_q and qW [N, K]; the 16-bit products are exact and everything is summed
 * in fp32, then rounded once to Y's type (QMM_BF16 or QMM_F32).
 * `n_outliers` (device, nullable) receives the number of outlier columns
 * found.  `workspace`: at least llm_int8_workspace_bytes(M, N, K,
 * max_outliers) bytes, 16-byte aligned, no clearing needed; QMM_EWORKSPACE
 * otherwise. */
int llm_int8_gemm(const void* X, int x_dtype, const int8_t* qW, const float* w_scale, int64_t M, int64_t N,
                  int64_t K, float threshold, int64_t max_outliers, void* Y, int y_dtype, int32_t* n_outliers,
                  void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * AWQ -- activation-aware scaling search for INT4 weights ("Quantization
 * from Scratch", "AWQ: protect the channels that matter", and its awq
 * listing): channels with large activations get their weights scaled up
 * before quantization and their inputs down by the same factor,
 * W x = (W diag(s)) (diag(s)^-1 x).  For each alpha of a grid:
 *   mag_j = max(mean_t |X[t, j]|, 1e-8)            (fp64; its sum over the
 *           tokens is exact, so the same in any order, while a channel's
 *           nonzero |x| span less than 2^(42 - log2 T) in ratio)
 *   s     = mag^alpha / sqrt(max_j mag_j^alpha * min_j mag_j^alpha)
 *                                                   (fp64, stored in fp32)
 *   codes = quantize_groupwise(fl32(W diag(s)))    (INT4, groups of 128)
 *   err   = || X W^T - h16(fl32(X diag(s)^-1)) W_hat^T ||_F^2 over the T
 *           calibration tokens, in fp64 (the output error as the quantized
 *           layer computes it: the inverse scaling folded into its 16-bit
 *           input, h16 = rounding to X's type, binary16 saturating at
 *           65504; X W^T by a 16-bit product with fp32 accumulation);
 * the first alpha of the smallest error is kept.
 * W : [N, K] and X : [T, K] calibration activations, both QMM_BF16 or both
 * QMM_F16.
 * alphas : HOST array of n_alpha (1 .. 64) values in [0, 1] (the listing's
 *          grid is 0, 0.1, .., 1).
 * Outputs (device): codes / scales / zeros of W diag(s_best) in the INT4
 * group-128 format above; smooth [K] = s_best (inference divides X by it,
 * or folds it into the previous operation); err [n_alpha] fp64; best
 * (int64, the chosen index).  Nothing is copied back to the host.
 * Errors, all found before any launch: QMM_EINVAL for a null pointer, a
 * non-positive size or an alpha outside [0, 1]; QMM_EUNSUPPORTED for fp32
 * operands, W and X of different types, K % 128 != 0 or more than 64
 * alphas; QMM_ERANGE for
 * K > 2^22, N >= 2^31 or T > 2097120; QMM_EALIGN for W, X, codes not 16-byte
 * aligned, scales or smooth not 4-byte, err or best not 8-byte aligned;
 * QMM_EWORKSPACE for a workspace smaller than awq_workspace_bytes(N, K, T,
 * n_alpha) (0 for invalid sizes), QMM_EALIGN for one not 256-byte aligned.
 * The workspace is the caller's device memory, used only during the call
 * (stream-ordered); the outputs are written on the stream.
 * ------------------------------------------------------------------------- */
size_t awq_workspace_bytes(int64_t N, int64_t K, int64_t T, int64_t n_alpha);
int awq_search(const void* W, int w_dtype, const void* X, int x_dtype, int64_t N, int64_t K, int64_t T,
               const double* alphas, int64_t n_alpha, uint8_t* codes, float* scales, uint8_t* zeros, float* smooth,
               double* err, int64_t* best, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H_ */
