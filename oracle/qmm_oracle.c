/*
 * qmm_oracle.c -- plain, slow CPU oracle for group-wise quantization and the
 * quantized matmuls.  TEST INFRASTRUCTURE ONLY: it exists to check the HIP
 * library and is called from tests, the smoke check and the benchmark's CPU
 * baseline, never from the product path.  It shares no code, header, table or
 * helper with the HIP library.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fPIC -shared (x86-64 SSE
 * scalar float, so every float expression below is one IEEE binary32 operation
 * rounded to nearest-even; no FMA contraction).
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
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#define OQ_OK 0
#define OQ_BAD_ARG (-1)
#define OQ_OVERFLOW (-2)

/* ------------------------------------------------------------------------ */
/* Asymmetric (affine) quantization, one (scale, zero-point) per group of    */
/* `group` consecutive elements along a row.  [HQ] "The math of              */
/* quantization" (asymmetric form); [QE] "Scale and Zero-Point": s = (max -  */
/* min) / (2^b - 1), z = round(-min / s); [QE] "Uniform Affine               */
/* Quantization" and "Manual Group-Wise Quantizer": q = clamp(round(w / s) + */
/* z, 0, 2^b - 1).  group == cols gives per-channel; a single row with       */
/* group == cols gives per-tensor ([HQ] "Granularity").                      */
/* Outputs: q[rows*cols] codes (unpacked, one per byte), scales and zeros    */
/* [rows * (cols / group)].                                                  */
/* ------------------------------------------------------------------------ */
int oq_asym_quantize(const float* w, int64_t rows, int64_t cols, int64_t group, int bits,
                     uint8_t* q, float* scales, uint8_t* zeros)
{
    if (!w || !q || !scales || !zeros || rows < 0 || cols < 0 || group <= 0 || cols % group != 0 ||
        bits < 1 || bits > 8)
        return OQ_BAD_ARG;
    const int64_t groups_per_row = cols / group;
    const float qmax = (float)((1 << bits) - 1);
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t g = 0; g < groups_per_row; ++g) {
            const float* v = w + r * cols + g * group;
            /* R1: the range always contains 0. */
            float lo = 0.0f, hi = 0.0f;
            for (int64_t i = 0; i < group; ++i) {
                if (v[i] < lo) lo = v[i];
                if (v[i] > hi) hi = v[i];
            }
            float range = hi - lo;           /* one fp32 subtraction */
            float s = range / qmax;          /* one fp32 division    */
            if (s == 0.0f) s = 1.0f;         /* R2 */
            float neg_lo = -lo;
            float zf = rintf(neg_lo / s);    /* R3, R5 */
            if (zf < 0.0f || zf > qmax) return OQ_BAD_ARG;  /* impossible under R1 */
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

/* Dequantization w_hat = (q - z) * s, one fp32 rounding.  [QS] "Scale and   */
/* zero-point"; [QE] "Uniform Affine Quantization".                          */
int oq_asym_dequantize(const uint8_t* q, const float* scales, const uint8_t* zeros, int64_t rows,
                       int64_t cols, int64_t group, float* out)
{
    if (!q || !scales || !zeros || !out || group <= 0 || cols % group != 0) return OQ_BAD_ARG;
    const int64_t groups_per_row = cols / group;
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
/* Reference product C[m][n] = sum_k A[m][k] * B[n][k] in fp64 (B is stored  */
/* [N, K] like a weight matrix, so C = A B^T).  For the W4A16 matmuls A is   */
/* the activations and B the dequantized weights: the plain definition of   */
/* the product the kernels compute ([HQ] "Inference view"; [QE] "Why It Is   */
/* Faster").                                                                 */
/* ------------------------------------------------------------------------ */
int oq_matmul_nt_f64(const float* a, const float* b, int64_t m, int64_t n, int64_t k, double* c)
{
    if (!a || !b || !c || m < 0 || n < 0 || k < 0) return OQ_BAD_ARG;
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
