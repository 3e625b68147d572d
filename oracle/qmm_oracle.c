/*
 * qmm_oracle.c -- plain, slow CPU oracle for group-wise quantization and the
 * quantized matmuls.  TEST INFRASTRUCTURE ONLY: it exists to check the HIP
 * library and is called from tests, the smoke check and the benchmark's CPU
 * baseline, never from the product path.  It shares no code, header, table or
 * helper with the HIP library.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fPIC -shared (x86-64 SSE
 * scalar float, so every float expression below is one IEEE binary32 operation
 * rounded to nearest-even; no FMA contraction).  The same file built with
 * -fopenmp gives the timing-only all-cores variant: the `omp parallel for`
 * lines split the independent output rows of the dequantizer and of the
 * matmul reference across threads (each output is still computed by the same
 * sequential loop, so results are identical); the serial build ignores them.
 *
 * Sources (page title, then section / slide / equation):
 *  [HQ]  "How quantization works" (AI-infra handbook): "The math of
 *        quantization" (symmetric and asymmetric formulas, the s/2 rounding
 *        bound), "Granularity" table, the fake-quantization listing
 *        (absmax floored at 1e-8), "Activation quantization and outliers"
 *        (per-row INT8 and the SmoothQuant factors with alpha and the 1e-5
 *        floor), "Exercises" 1 and 2.
 *  [ER]  "Quantization" (Engine Room ch. 15): "The Mathematics", the
 *        symmetric quantization equation and the SmoothQuant smoothing
 *        equation Y = (X diag(s)^-1)(diag(s) W).
 *  [QS]  "Quantization from Scratch: Scale, Zero-Point, GPTQ and AWQ":
 *        "Scale and zero-point" (dequantization (q - z) s, zero exactly
 *        representable), the round-to-nearest listing (scale 0 replaced by 1,
 *        clip after adding the zero-point), the worked 8-weight example.
 *  [QE]  "Quantization Explained: INT8, INT4, GPTQ and AWQ for LLMs": slides
 *        "Uniform Affine Quantization", "Scale and Zero-Point", "Error Bound",
 *        the six-weight worked example, "Manual Group-Wise Quantizer".
 *  [SW]  "Quantization: Smaller Weights, Same Answers (Mostly)": "How does
 *        quantized matrix multiplication actually run on the GPU?" (INT8
 *        products summed exactly in a 32-bit accumulator, then rescaled).
 *
 * Readings where the pages leave a point open (each one is a choice):
 *  R1  a group's range is widened to contain 0: lo = min(min w, 0),
 *      hi = max(max w, 0).  Identical to the pages' min/max whenever the group
 *      straddles zero, and the only way the zero-point stays a valid code.
 *  R2  a group whose widened range is empty (all zeros) gets s = 1 ([QS]
 *      listing).
 *  R3  "round" is round-half-to-even (rintf in the default rounding mode).
 *  R5  codes divide by s (w / s), as the listings do; no reciprocal.
 *  R6  clamp after adding the zero-point.
 *  R7  alpha = 0.5 uses sqrtf for both powers; other alpha use powf.
 *  R8  symmetric scales floor the absmax at `floor` (1e-8 in [HQ]).
 *  R26 an input feature (column of X) is an outlier dimension of a batch when
 *      some token's |x| in it reaches the threshold tau (>=); tau is an
 *      argument.
 *  R27 the weights are stored once, as per-output-channel INT8; the 16-bit
 *      weight slice of the outlier product is that INT8 weight dequantized
 *      (q * b) and rounded to the activations' 16-bit type (binary16
 *      saturating at 65504 as in R24).
 *  R28 the outlier columns are zero in X_q and take no part in a token's
 *      absmax.
 *  R32 AWQ's error for a candidate alpha is the layer's output error as the
 *      quantized layer computes it: || X W^T - X_s W_hat^T ||_F^2, X_s the
 *      activations divided by the scales (the inverse scaling folded into
 *      the layer's 16-bit input: fp32 quotient, then rounded to the
 *      activations' own type, bf16 or binary16, binary16 saturating at
 *      65504 as in R24) and
 *      W_hat the dequantized codes of W diag(s); the sums in fp64.  (The
 *      [QS] listing evaluates the same quantity as sum((D H) * D) with
 *      D = W - W_hat / s and H from the calibration inputs.)
 *  R33 AWQ's channel magnitudes are mean |x_j| over the calibration tokens
 *      in fp64, floored at 1e-8 so that a silent channel keeps a finite
 *      scale; the scales s = mag^alpha / sqrt(max * min) are computed in
 *      fp64 and stored in fp32; the weights are quantized to INT4 in groups
 *      of 128 with fp32 scales (the format of the rest of the path).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OQ_OK 0
#define OQ_BAD_ARG (-1)
#define OQ_OVERFLOW (-2)

/* ------------------------------------------------------------------------ */
/* binary16 storage of a scale ([HQ] Exercise 2 and [QS] "Where to put the   */
/* scales" count one 16-bit scale per group).  Conversion from fp32 by the    */
/* IEEE 754 definition: round to nearest, ties to even, in the subnormal      */
/* range too; magnitudes at or above the largest finite binary16 (65504)      */
/* saturate to it (reading R24).  Input finite.                               */
/* ------------------------------------------------------------------------ */
uint16_t oq_f32_to_f16_bits(float f)
{
    const uint16_t sign = signbit(f) ? 0x8000u : 0u;
    double a = fabs((double)f);
    if (a >= 65504.0) return (uint16_t)(sign | 0x7BFFu);
    if (a < ldexp(1.0, -14)) {                       /* subnormal: units of 2^-24 */
        double r = nearbyint(a * ldexp(1.0, 24));    /* exact scaling, then RNE   */
        return (uint16_t)(sign | (uint16_t)r);       /* r == 1024 is the smallest normal */
    }
    int ex;
    frexp(a, &ex);                                   /* a = m 2^ex, m in [0.5, 1) */
    int e = ex - 1;                                  /* a in [2^e, 2^(e+1))       */
    double r = nearbyint(ldexp(a, 10 - e));          /* significand in [1024, 2048] */
    if (r == 2048.0) {
        r = 1024.0;
        e += 1;
    }
    if (e > 15) return (uint16_t)(sign | 0x7BFFu);
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(r - 1024.0));
}

float oq_f16_bits_to_f32(uint16_t h)
{
    const int e = (h >> 10) & 0x1F;
    const int m = h & 0x3FF;
    double v = (e == 0) ? ldexp((double)m, -24) : ldexp((double)(1024 + m), e - 25);
    return (float)((h & 0x8000u) ? -v : v);          /* exact: 11 significant bits */
}

/* Elementwise forms of the two conversions above (for marshalling). */
int oq_f32_to_f16_array(const float* a, int64_t n, uint16_t* out)
{
    if (!a || !out || n < 0) return OQ_BAD_ARG;
    for (int64_t i = 0; i < n; ++i) out[i] = oq_f32_to_f16_bits(a[i]);
    return OQ_OK;
}

int oq_f16_to_f32_array(const uint16_t* h, int64_t n, float* out)
{
    if (!h || !out || n < 0) return OQ_BAD_ARG;
    for (int64_t i = 0; i < n; ++i) out[i] = oq_f16_bits_to_f32(h[i]);
    return OQ_OK;
}

/* A scale kept in 16 bits: the binary16 value of s, and 1 when that is 0     */
/* (the [QS] listing's rule for an unusable scale, applied to the stored one; */
/* reading R24).                                                              */
static float f16_scale(float s)
{
    float s16 = oq_f16_bits_to_f32(oq_f32_to_f16_bits(s));
    if (s16 == 0.0f) s16 = 1.0f;
    return s16;
}

/* ------------------------------------------------------------------------ */
/* Group-wise quantization, one (scale, zero-point) per group of `group`     */
/* consecutive elements along a row, `bits` bits per code.                   */
/* Asymmetric (affine): [HQ] "The math of quantization" (asymmetric form);   */
/* [QE] "Scale and Zero-Point": s = (max - min) / (2^b - 1), z = round(-min  */
/* / s); [QE] "Uniform Affine Quantization" and "Manual Group-Wise           */
/* Quantizer": q = clamp(round(w / s) + z, 0, 2^b - 1).                      */
/* Symmetric: [HQ] "The math of quantization": s = max|w| / (2^(b-1) - 1)    */
/* (absmax floored at 1e-8, R8), q = clamp(round(w / s), -2^(b-1),           */
/* 2^(b-1) - 1), stored as the code q + 2^(b-1) with that zero-point (R22).  */
/* scale_f16: the scale is stored in binary16 and the codes are computed     */
/* with the stored value ([HQ] Exercise 2; [QS] "Where to put the scales").  */
/* group == cols gives per-channel; a single row with group == cols gives    */
/* per-tensor ([HQ] "Granularity").                                          */
/* Outputs: q[rows*cols] codes (unpacked, one per byte), scales (the stored  */
/* value, as float) and zeros [rows * (cols / group)].                       */
/* ------------------------------------------------------------------------ */
int oq_quantize_format(const float* w, int64_t rows, int64_t cols, int64_t group, int bits, int symmetric,
                       int scale_f16, uint8_t* q, float* scales, uint8_t* zeros)
{
    if (!w || !q || !scales || !zeros || rows < 0 || cols < 0 || group <= 0 || cols % group != 0 ||
        bits < 2 || bits > 8)
        return OQ_BAD_ARG;
    const int64_t groups_per_row = cols / group;
    const float qmax = (float)((1 << bits) - 1);
    const float half = (float)(1 << (bits - 1));
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t g = 0; g < groups_per_row; ++g) {
            const float* v = w + r * cols + g * group;
            float s, zf;
            if (!symmetric) {
                /* R1: the range always contains 0. */
                float lo = 0.0f, hi = 0.0f;
                for (int64_t i = 0; i < group; ++i) {
                    if (v[i] < lo) lo = v[i];
                    if (v[i] > hi) hi = v[i];
                }
                float range = hi - lo;           /* one fp32 subtraction */
                s = range / qmax;                /* one fp32 division    */
                if (s == 0.0f) s = 1.0f;         /* R2 */
                if (scale_f16) s = f16_scale(s);
                float neg_lo = -lo;
                zf = rintf(neg_lo / s);          /* R3, R5 */
                /* beyond the code range only when a 16-bit scale saturated */
                if (scale_f16 && zf > qmax) zf = qmax;
                if (zf < 0.0f || zf > qmax) return OQ_BAD_ARG;  /* impossible under R1 */
            } else {
                float amax = 0.0f;
                for (int64_t i = 0; i < group; ++i) {
                    float a = fabsf(v[i]);
                    if (a > amax) amax = a;
                }
                if (amax < 1e-8f) amax = 1e-8f;  /* R8 */
                s = amax / (half - 1.0f);
                if (scale_f16) s = f16_scale(s);
                zf = half;                       /* R22 */
            }
            int z = (int)zf;
            scales[r * groups_per_row + g] = s;
            zeros[r * groups_per_row + g] = (uint8_t)z;
            for (int64_t i = 0; i < group; ++i) {
                float t = rintf(v[i] / s) + (float)z;   /* R3, R5 */
                if (t < 0.0f) t = 0.0f;                 /* R6 */
                if (t > qmax) t = qmax;
                q[r * cols + g * group + i] = (uint8_t)t;
            }
        }
    }
    return OQ_OK;
}

/* The asymmetric quantizer with fp32 scales (the format of every workload). */
int oq_asym_quantize(const float* w, int64_t rows, int64_t cols, int64_t group, int bits,
                     uint8_t* q, float* scales, uint8_t* zeros)
{
    if (bits < 2) return OQ_BAD_ARG;
    return oq_quantize_format(w, rows, cols, group, bits, 0, 0, q, scales, zeros);
}

/* Dequantization w_hat = (q - z) * s, one fp32 rounding.  [QS] "Scale and   */
/* zero-point"; [QE] "Uniform Affine Quantization".                          */
int oq_asym_dequantize(const uint8_t* q, const float* scales, const uint8_t* zeros, int64_t rows,
                       int64_t cols, int64_t group, float* out)
{
    if (!q || !scales || !zeros || !out || group <= 0 || cols % group != 0) return OQ_BAD_ARG;
    const int64_t groups_per_row = cols / group;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            int64_t gi = r * groups_per_row + c / group;
            float d = (float)((int)q[r * cols + c] - (int)zeros[gi]);
            out[r * cols + c] = d * scales[gi];
        }
    return OQ_OK;
}

/* ------------------------------------------------------------------------ */
/* Symmetric quantization, one scale per group along a row.  [HQ] "The math  */
/* of quantization": s = max|x| / (2^(b-1) - 1), q = clamp(round(x / s),     */
/* -2^(b-1), 2^(b-1) - 1); the absmax is floored at `floor` first (R8, the   */
/* [HQ] fake-quantization listing).  [ER] writes the same map as            */
/* round(x * (2^(b-1)-1) / max|x|); the division form is used (R5).          */
/* ------------------------------------------------------------------------ */
int oq_sym_quantize(const float* x, int64_t rows, int64_t cols, int64_t group, int bits, float floor_,
                    int8_t* q, float* scales)
{
    if (!x || !q || !scales || group <= 0 || cols % group != 0 || bits < 2 || bits > 8) return OQ_BAD_ARG;
    const int64_t groups_per_row = cols / group;
    const float qpos = (float)((1 << (bits - 1)) - 1);
    const float qneg = -(float)(1 << (bits - 1));
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t g = 0; g < groups_per_row; ++g) {
            const float* v = x + r * cols + g * group;
            float amax = 0.0f;
            for (int64_t i = 0; i < group; ++i) {
                float a = fabsf(v[i]);
                if (a > amax) amax = a;
            }
            if (amax < floor_) amax = floor_;
            float s = amax / qpos;
            scales[r * groups_per_row + g] = s;
            for (int64_t i = 0; i < group; ++i) {
                float t = rintf(v[i] / s);
                if (t < qneg) t = qneg;
                if (t > qpos) t = qpos;
                q[r * cols + g * group + i] = (int8_t)t;
            }
        }
    return OQ_OK;
}

/* x_hat = q * s.  [HQ] "The math of quantization".                          */
int oq_sym_dequantize(const int8_t* q, const float* scales, int64_t rows, int64_t cols, int64_t group,
                      float* out)
{
    if (!q || !scales || !out || group <= 0 || cols % group != 0) return OQ_BAD_ARG;
    const int64_t groups_per_row = cols / group;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = (float)q[r * cols + c] * scales[r * groups_per_row + c / group];
    return OQ_OK;
}

/* ------------------------------------------------------------------------ */
/* Storage: 4-bit values packed two per byte along each row, element 2j in   */
/* the low nibble of byte j and element 2j+1 in the high nibble; an odd      */
/* count leaves the last high nibble zero.  Half a byte per weight plus the  */
/* per-group scale and zero-point is the storage the pages count ([HQ]       */
/* Exercise 2; [QE] "The Cost of Small Groups").                             */
/* ------------------------------------------------------------------------ */
int oq_pack_nibbles(const uint8_t* vals, int64_t rows, int64_t count, uint8_t* out)
{
    if (!vals || !out || rows < 0 || count < 0) return OQ_BAD_ARG;
    const int64_t bytes = (count + 1) / 2;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < bytes; ++j) {
            uint8_t lo = vals[r * count + 2 * j] & 0xF;
            uint8_t hi = (2 * j + 1 < count) ? (vals[r * count + 2 * j + 1] & 0xF) : 0;
            out[r * bytes + j] = (uint8_t)(lo | (hi << 4));
        }
    return OQ_OK;
}

/* ------------------------------------------------------------------------ */
/* Weight codes: the pages fix half a byte per weight but no order, so this  */
/* follows the library's stated layout.  Each run of 8 elements of a row is  */
/* one little-endian 32-bit word holding element 2i of the run in bits       */
/* 4i..4i+3 and element 2i+1 in bits 16+4i..16+4i+3 (i = 0..3).  count must  */
/* be a multiple of 8.                                                       */
/* ------------------------------------------------------------------------ */
int oq_pack_codes(const uint8_t* vals, int64_t rows, int64_t count, uint8_t* out)
{
    if (!vals || !out || rows < 0 || count < 0 || count % 8 != 0) return OQ_BAD_ARG;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t w = 0; w < count / 8; ++w) {
            const uint8_t* e = vals + r * count + 8 * w;
            uint32_t word = 0;
            for (int i = 0; i < 4; ++i) {
                word |= (uint32_t)(e[2 * i] & 0xF) << (4 * i);
                word |= (uint32_t)(e[2 * i + 1] & 0xF) << (16 + 4 * i);
            }
            for (int b = 0; b < 4; ++b) out[r * (count / 2) + 4 * w + b] = (uint8_t)(word >> (8 * b));
        }
    return OQ_OK;
}

/* ------------------------------------------------------------------------ */
/* 3-bit codes.  The pages count bits per weight, not an order; the stored   */
/* layout is the library's, chosen so that two consecutive codes sit 16 bits */
/* apart in one word.  Each run of 32 elements e = 0..31 of a row fills      */
/* three little-endian 32-bit words W0, W1, W2 (12 bytes):                   */
/*   e < 30: word W[e / 10]; with r = e % 10, bits 3 (r / 2) .. +2 when r is */
/*           even and 16 + 3 (r / 2) .. +2 when r is odd;                    */
/*   e = 30: bit t of its code is bit 15 of W[t] (t = 0, 1, 2);              */
/*   e = 31: bit t of its code is bit 31 of W[t].                            */
/* count must be a multiple of 32.                                           */
/* ------------------------------------------------------------------------ */
int oq_pack_codes3(const uint8_t* vals, int64_t rows, int64_t count, uint8_t* out)
{
    if (!vals || !out || rows < 0 || count < 0 || count % 32 != 0) return OQ_BAD_ARG;
    const int64_t row_bytes = count * 3 / 8;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t run = 0; run < count / 32; ++run) {
            const uint8_t* e = vals + r * count + 32 * run;
            uint32_t w[3] = {0, 0, 0};
            for (int i = 0; i < 30; ++i) {
                const int rr = i % 10;
                const int pos = 3 * (rr / 2) + 16 * (rr % 2);
                w[i / 10] |= (uint32_t)(e[i] & 7u) << pos;
            }
            for (int t = 0; t < 3; ++t) {
                w[t] |= (uint32_t)((e[30] >> t) & 1u) << 15;
                w[t] |= (uint32_t)((e[31] >> t) & 1u) << 31;
            }
            uint8_t* o = out + r * row_bytes + 12 * run;
            for (int k = 0; k < 3; ++k)
                for (int b = 0; b < 4; ++b) o[4 * k + b] = (uint8_t)(w[k] >> (8 * b));
        }
    return OQ_OK;
}

/* ------------------------------------------------------------------------ */
/* FP8 E4M3 (OCP "E4M3FN": 1 sign, 4 exponent bits with bias 7, 3 mantissa  */
/* bits, no infinities, the only NaN S.1111.111; largest finite 448, smallest */
/* normal 2^-6, subnormals m 2^-9).  [HQ] "Quantization formats" and its     */
/* fake-quantization listing (E4M3's maximum is 448); [SW] "What about FP8,  */
/* MXFP4, NVFP4 and GGUF?".  Conversion from fp32 by the definition: round   */
/* to nearest, ties to even; a magnitude at or above 448 gives 448 (reading */
/* R25: nothing above 464 rounds to a finite value, and the listing's        */
/* quotients never exceed 448 by more than an fp32 rounding).                */
/* ------------------------------------------------------------------------ */
uint8_t oq_f32_to_e4m3(float f)
{
    const uint8_t sign = signbit(f) ? 0x80u : 0u;
    double a = fabs((double)f);
    if (a >= 448.0) return (uint8_t)(sign | 0x7Eu);
    if (a < ldexp(1.0, -6)) {                       /* subnormal: units of 2^-9  */
        double r = nearbyint(a * ldexp(1.0, 9));
        return (uint8_t)(sign | (uint8_t)r);        /* r == 8 is the smallest normal */
    }
    int ex;
    frexp(a, &ex);
    int e = ex - 1;                                 /* a in [2^e, 2^(e+1))       */
    double r = nearbyint(ldexp(a, 3 - e));          /* significand in [8, 16]    */
    if (r == 16.0) {
        r = 8.0;
        e += 1;
    }
    if (e > 8) return (uint8_t)(sign | 0x7Eu);
    return (uint8_t)(sign | (uint8_t)((e + 7) << 3) | (uint8_t)(r - 8.0));
}

float oq_e4m3_to_f32(uint8_t b)
{
    const int e = (b >> 3) & 0xF;
    const int m = b & 7;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    if (e == 15 && m == 7) v = NAN;
    return (float)((b & 0x80u) ? -v : v);
}

int oq_e4m3_array(const float* a, int64_t n, uint8_t* out)
{
    if (!a || !out || n < 0) return OQ_BAD_ARG;
    for (int64_t i = 0; i < n; ++i) out[i] = oq_f32_to_e4m3(a[i]);
    return OQ_OK;
}

int oq_e4m3_decode_array(const uint8_t* b, int64_t n, float* out)
{
    if (!b || !out || n < 0) return OQ_BAD_ARG;
    for (int64_t i = 0; i < n; ++i) out[i] = oq_e4m3_to_f32(b[i]);
    return OQ_OK;
}

/* FP8 quantization, [HQ] fake_quant_fp8: s = max|x| / 448 over each group of */
/* `group` consecutive elements (a row: per token / per output channel; the  */
/* whole tensor as one row: the listing's per-tensor form), q = E4M3(x / s). */
/* The absmax is floored at 1e-8 as in the integer path (R8, R25).           */
int oq_fp8_quantize(const float* x, int64_t rows, int64_t cols, int64_t group, uint8_t* q, float* scales)
{
    if (!x || !q || !scales || group <= 0 || cols % group != 0) return OQ_BAD_ARG;
    const int64_t groups_per_row = cols / group;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t g = 0; g < groups_per_row; ++g) {
            const float* v = x + r * cols + g * group;
            float amax = 0.0f;
            for (int64_t i = 0; i < group; ++i) {
                float a = fabsf(v[i]);
                if (a > amax) amax = a;
            }
            if (amax < 1e-8f) amax = 1e-8f;
            float s = amax / 448.0f;
            scales[r * groups_per_row + g] = s;
            for (int64_t i = 0; i < group; ++i) q[r * cols + g * group + i] = oq_f32_to_e4m3(v[i] / s);
        }
    return OQ_OK;
}

/* FP8 product: acc[m][n] = sum_k e4m3(qa[m][k]) e4m3(qb[n][k]) in fp64 (each */
/* product of two 4-significant-bit values is exact).                        */
int oq_fp8_matmul_nt(const uint8_t* qa, const uint8_t* qb, int64_t m, int64_t n, int64_t k, double* acc)
{
    if (!qa || !qb || !acc || m < 0 || n < 0 || k < 0) return OQ_BAD_ARG;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            double sacc = 0.0;
            for (int64_t t = 0; t < k; ++t)
                sacc += (double)oq_e4m3_to_f32(qa[i * k + t]) * (double)oq_e4m3_to_f32(qb[j * k + t]);
            acc[i * n + j] = sacc;
        }
    return OQ_OK;
}

/* ------------------------------------------------------------------------ */
/* Reference product C[m][n] = sum_k A[m][k] * B[n][k] in fp64 (B is stored  */
/* [N, K] like a weight matrix, so C = A B^T).  For the W4A16 matmuls A is   */
/* the activations and B the dequantized weights: the plain definition of   */
/* the product the kernels compute ([HQ] "Inference view"; [QE] "Why It Is   */
/* Faster").                                                                 */
/* ------------------------------------------------------------------------ */
int oq_matmul_nt_f64(const float* a, const float* b, int64_t m, int64_t n, int64_t k, double* c)
{
    if (!a || !b || !c || m < 0 || n < 0 || k < 0) return OQ_BAD_ARG;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0;
            for (int64_t t = 0; t < k; ++t) acc += (double)a[i * k + t] * (double)b[j * k + t];
            c[i * n + j] = acc;
        }
    return OQ_OK;
}

/* Exact integer product acc[m][n] = sum_k qa[m][k] * qb[n][k], summed in    */
/* int64; returns OQ_OVERFLOW if any sum leaves the int32 range the 32-bit   */
/* accumulator of [SW] holds.                                                */
int oq_int8_matmul_nt(const int8_t* qa, const int8_t* qb, int64_t m, int64_t n, int64_t k, int32_t* acc)
{
    if (!qa || !qb || !acc || m < 0 || n < 0 || k < 0) return OQ_BAD_ARG;
    int status = OQ_OK;
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            int64_t s = 0;
            for (int64_t t = 0; t < k; ++t) s += (int64_t)qa[i * k + t] * (int64_t)qb[j * k + t];
            if (s > INT32_MAX || s < INT32_MIN) status = OQ_OVERFLOW;
            acc[i * n + j] = (int32_t)s;
        }
    return status;
}

/* Rescale of the integer product: Y[m][n] = acc[m][n] * a[m] * b[n] in fp64  */
/* (per-token activation scale a, per-output-channel weight scale b); the    */
/* S_out factor of the vector-wise scheme in [ER] "The Mathematics".         */
int oq_rescale_f64(const int32_t* acc, const float* a, const float* b, int64_t m, int64_t n, double* y)
{
    if (!acc || !a || !b || !y) return OQ_BAD_ARG;
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) y[i * n + j] = (double)acc[i * n + j] * (double)a[i] * (double)b[j];
    return OQ_OK;
}

/* ------------------------------------------------------------------------ */
/* SmoothQuant.  [HQ] "Activation quantization and outliers" and [ER]        */
/* "The Mathematics": s_j = max|X_j|^alpha / max|W_j|^(1-alpha), each max    */
/* floored at 1e-5 before the power; X <- X / s (columns), W <- W * s        */
/* (input-channel columns of the [N, K] weight).                             */
/* ------------------------------------------------------------------------ */
int oq_col_absmax(const float* a, int64_t rows, int64_t cols, float* out)
{
    if (!a || !out || rows < 0 || cols < 0) return OQ_BAD_ARG;
    for (int64_t j = 0; j < cols; ++j) {
        float m = 0.0f;
        for (int64_t i = 0; i < rows; ++i) {
            float v = fabsf(a[i * cols + j]);
            if (v > m) m = v;
        }
        out[j] = m;
    }
    return OQ_OK;
}

int oq_smooth_factors(const float* cx, const float* cw, int64_t k, float alpha, float* s)
{
    if (!cx || !cw || !s || k < 0) return OQ_BAD_ARG;
    const float fl = 1e-5f;
    for (int64_t j = 0; j < k; ++j) {
        float x = cx[j] < fl ? fl : cx[j];
        float w = cw[j] < fl ? fl : cw[j];
        float num, den;
        if (alpha == 0.5f) {             /* R7 */
            num = sqrtf(x);
            den = sqrtf(w);
        } else {
            num = powf(x, alpha);
            den = powf(w, 1.0f - alpha);
        }
        s[j] = num / den;
    }
    return OQ_OK;
}

int oq_scale_columns_mul(const float* a, const float* s, int64_t rows, int64_t cols, float* out)
{
    if (!a || !s || !out) return OQ_BAD_ARG;
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < cols; ++j) out[i * cols + j] = a[i * cols + j] * s[j];
    return OQ_OK;
}

int oq_scale_columns_div(const float* a, const float* s, int64_t rows, int64_t cols, float* out)
{
    if (!a || !s || !out) return OQ_BAD_ARG;
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < cols; ++j) out[i * cols + j] = a[i * cols + j] / s[j];
    return OQ_OK;
}

/* ------------------------------------------------------------------------ */
/* LLM.int8() mixed-precision decomposition.  [ER] "The Mathematics": the    */
/* vector-wise scheme (one scale per row of X and per column of the product, */
/* i.e. per output channel of the [N, K] weight) with the outlier feature    */
/* dimensions removed from the integer product and multiplied in 16-bit,     */
/* C = S_out (X_q W_q) + X_16 W_16; the history paragraph on LLM.int8() (a   */
/* handful of systematically large dimensions, more than 99.9% of the values */
/* still multiplied in 8-bit, half the memory).  [SW] "How do LLM-specific   */
/* quantization schemes protect against outliers?", family 1.               */
/* ------------------------------------------------------------------------ */

/* bfloat16 value of a finite float: the top 16 bits of its encoding after   */
/* rounding the 16 dropped bits to nearest, ties to even.                    */
static float bf16_round(float f)
{
    union { float f; uint32_t u; } v;
    v.f = f;
    const uint32_t dropped = v.u & 0xFFFFu;
    uint32_t top = v.u >> 16;
    if (dropped > 0x8000u || (dropped == 0x8000u && (top & 1u))) top += 1u;
    v.u = top << 16;
    return v.f;
}

/* x [m, k]: the 16-bit activations as floats (exact); qw [n, k] and b [n]:  */
/* the per-output-channel INT8 weights (R27).  In column order, the first    */
/* `cap` outlier columns (R26) are carved out; idx[0 .. counts[0]) lists     */
/* them, counts[1] is the number found (the columns past the cap stay in the */
/* integer product).  Outputs qx [m, k], a [m] (R28) and y [m, n] in fp64:   */
/* y = acc * a * b + sum over the outlier columns of x * w16.                */
int oq_llm_int8(const float* x, int64_t m, int64_t k, const int8_t* qw, const float* b, int64_t n, float tau,
                int64_t cap, int x_bf16, int32_t* idx, int64_t* counts, int8_t* qx, float* a, double* y)
{
    if (!x || !qw || !b || !idx || !counts || !qx || !a || !y || m <= 0 || n <= 0 || k <= 0 || cap < 0)
        return OQ_BAD_ARG;
    if (!(tau >= 0.0f)) return OQ_BAD_ARG;
    float* cx = (float*)malloc((size_t)k * sizeof(float));
    float* xr = (float*)malloc((size_t)(m * k) * sizeof(float));
    float* w16 = (float*)malloc((size_t)(n * (cap > 0 ? cap : 1)) * sizeof(float));
    int32_t* acc = (int32_t*)malloc((size_t)(m * n) * sizeof(int32_t));
    if (!cx || !xr || !w16 || !acc) {
        free(cx); free(xr); free(w16); free(acc);
        return OQ_BAD_ARG;
    }
    /* 1. each feature's largest magnitude over the batch's tokens */
    oq_col_absmax(x, m, k, cx);
    /* 2. the outlier dimensions, in column order (R26) */
    int64_t kept = 0, found = 0;
    for (int64_t j = 0; j < k; ++j)
        if (cx[j] >= tau) {
            if (kept < cap) idx[kept++] = (int32_t)j;
            ++found;
        }
    counts[0] = kept;
    counts[1] = found;
    /* 3. vector-wise INT8 of the remaining columns: the outlier columns are */
    /*    zeroed, so they neither set a token's scale nor enter X_q (R28)     */
    memcpy(xr, x, (size_t)(m * k) * sizeof(float));
    for (int64_t i = 0; i < m; ++i)
        for (int64_t p = 0; p < kept; ++p) xr[i * k + idx[p]] = 0.0f;
    oq_sym_quantize(xr, m, k, k, 8, 1e-8f, qx, a);
    /* 4. the integer product and its rescale by the token and channel scales */
    int status = oq_int8_matmul_nt(qx, qw, m, n, k, acc);
    oq_rescale_f64(acc, a, b, m, n, y);
    /* 5. the 16-bit weight slice of the outlier columns (R27) */
    for (int64_t j = 0; j < n; ++j)
        for (int64_t p = 0; p < kept; ++p) {
            const float w = (float)qw[j * k + idx[p]] * b[j];
            w16[j * cap + p] = x_bf16 ? bf16_round(w) : oq_f16_bits_to_f32(oq_f32_to_f16_bits(w));
        }
    /* 6. the outlier product X_16 W_16, added to the rescaled integer part */
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            double s = 0.0;
            for (int64_t p = 0; p < kept; ++p) s += (double)x[i * k + idx[p]] * (double)w16[j * cap + p];
            y[i * n + j] += s;
        }
    free(cx); free(xr); free(w16); free(acc);
    return status;
}

/* ------------------------------------------------------------------------ */
/* AWQ's activation-aware scaling search.  [QS] "AWQ: protect the channels   */
/* that matter" (W x = (W diag(s)) (diag(s)^-1 x), exact in full precision;  */
/* s_j = mean|x_j|^alpha, one alpha per layer chosen on calibration data) and */
/* the awq listing after it (s normalized by sqrt(max s * min s), the weights */
/* W diag(s) quantized group-wise, the candidate of the smallest calibration  */
/* output error kept).  Readings R32, R33.                                   */
/* w [n, k] and x [t, k] hold the 16-bit values as floats; alphas[n_alpha].  */
/* Outputs: err[n_alpha]; *best, the first alpha of the smallest error;      */
/* s_best[k]; q (unpacked codes), scales, zeros of W diag(s_best).           */
/* ------------------------------------------------------------------------ */
/* The factors of every alpha: s_all[a * k + j] (R33). */
int oq_awq_factors(const float* x, int64_t k, int64_t t, const double* alphas, int64_t n_alpha, float* s_all)
{
    if (!x || !alphas || !s_all || k <= 0 || t <= 0 || n_alpha <= 0) return OQ_BAD_ARG;
    double* mag = malloc((size_t)k * sizeof(double));
    double* p = malloc((size_t)k * sizeof(double));
    if (!mag || !p) {
        free(mag); free(p);
        return OQ_BAD_ARG;
    }
    /* channel magnitudes: mean |x_j| over the tokens */
    for (int64_t j = 0; j < k; ++j) {
        double acc = 0.0;
        for (int64_t r = 0; r < t; ++r) acc += fabs((double)x[r * k + j]);
        const double m = acc / (double)t;
        mag[j] = m < 1e-8 ? 1e-8 : m;
    }
    for (int64_t a = 0; a < n_alpha; ++a) {
        double mx = 0.0, mn = INFINITY;
        for (int64_t j = 0; j < k; ++j) {
            p[j] = pow(mag[j], alphas[a]);
            if (p[j] > mx) mx = p[j];
            if (p[j] < mn) mn = p[j];
        }
        const double norm = sqrt(mx * mn);
        for (int64_t j = 0; j < k; ++j) s_all[a * k + j] = (float)(p[j] / norm);
    }
    free(mag); free(p);
    return OQ_OK;
}

int oq_awq_search(const float* w, const float* x, int64_t n, int64_t k, int64_t t, const double* alphas,
                  int64_t n_alpha, double* err, int64_t* best, float* s_best, uint8_t* q, float* scales,
                  uint8_t* zeros, int x_f16)
{
    if (!w || !x || !alphas || !err || !best || !s_best || !q || !scales || !zeros) return OQ_BAD_ARG;
    if (n <= 0 || k <= 0 || t <= 0 || n_alpha <= 0 || k % 128 != 0) return OQ_BAD_ARG;
    const int64_t g = k / 128;
    float* s_all = malloc((size_t)(n_alpha * k) * sizeof(float));
    float* ws = malloc((size_t)(n * k) * sizeof(float));
    float* what = malloc((size_t)(n * k) * sizeof(float));
    float* xs = malloc((size_t)(t * k) * sizeof(float));
    double* yref = malloc((size_t)(t * n) * sizeof(double));
    double* yq = malloc((size_t)(t * n) * sizeof(double));
    uint8_t* qa = malloc((size_t)(n * k));
    float* sa = malloc((size_t)(n * g) * sizeof(float));
    uint8_t* za = malloc((size_t)(n * g));
    int status = OQ_OK;
    if (!s_all || !ws || !what || !xs || !yref || !yq || !qa || !sa || !za) {
        status = OQ_BAD_ARG;
        goto done;
    }
    oq_awq_factors(x, k, t, alphas, n_alpha, s_all);
    oq_matmul_nt_f64(x, w, t, n, k, yref);          /* the full-precision output X W^T */
    int64_t bi = 0;
    for (int64_t a = 0; a < n_alpha; ++a) {
        const float* s = s_all + a * k;
        oq_scale_columns_mul(w, s, n, k, ws);       /* W diag(s) */
        oq_asym_quantize(ws, n, k, 128, 4, qa, sa, za);
        oq_asym_dequantize(qa, sa, za, n, k, 128, what);
        oq_scale_columns_div(x, s, t, k, xs);       /* diag(s)^-1 folded into the 16-bit input (R32) */
        for (int64_t i = 0; i < t * k; ++i)
            xs[i] = x_f16 ? oq_f16_bits_to_f32(oq_f32_to_f16_bits(xs[i])) : bf16_round(xs[i]);
        oq_matmul_nt_f64(xs, what, t, n, k, yq);
        double e = 0.0;
        for (int64_t i = 0; i < t * n; ++i) {
            const double d = yref[i] - yq[i];
            e += d * d;
        }
        err[a] = e;
        if (a == 0 || e < err[bi]) {
            bi = a;
            memcpy(s_best, s, (size_t)k * sizeof(float));
            memcpy(q, qa, (size_t)(n * k));
            memcpy(scales, sa, (size_t)(n * g) * sizeof(float));
            memcpy(zeros, za, (size_t)(n * g));
        }
    }
    *best = bi;
done:
    free(s_all); free(ws); free(what); free(xs); free(yref); free(yq);
    free(qa); free(sa); free(za);
    return status;
}

/* Threads the row loops above use: 1 in the serial build. */
int oq_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
