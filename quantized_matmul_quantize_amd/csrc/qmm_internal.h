// qmm_internal.h -- host-side helpers shared by the libqmm entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmm.h"

namespace qmm {

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Status of the launches just made on this thread.
inline int launch_status() { return hipGetLastError() == hipSuccess ? QMM_OK : QMM_EHIP; }

// Compute units of the current device (cached per device ordinal).
int device_cus();

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The stored formats other than 4-bit codes with fp32 scales per 128 weights
// (formats.hip); the 4-bit / group-128 entry points hand other formats here.
int quantize_fmt(const void* W, int w_dtype, int64_t N, int64_t K, int group, int bits, int scale_dtype,
                 int symmetric, uint8_t* codes, void* scales, uint8_t* zeros, void* stream);
int dequantize_fmt(const uint8_t* codes, const void* scales, const uint8_t* zeros, int64_t N, int64_t K, int group,
                   int bits, int scale_dtype, void* W_hat, int out_dtype, void* stream);
int matmul_fmt(const uint8_t* codes, const void* scales, const uint8_t* zeros, int64_t N, int64_t K, int group,
               int bits, int scale_dtype, const void* x, int x_dtype, int64_t M, void* y, int y_dtype, void* stream);

// Group-128 asymmetric INT4 of fl32(W[n, k] * colscale[k]) for 16-bit W
// (w_dtype QMM_BF16 or QMM_F16; quantize.hip, the quantizer kernels with a
// per-column factor), into the format of quantize_groupwise.  K % 128 == 0;
// W, colscale, codes 16-byte aligned.  No argument checks: the caller's.
void launch_quantize_colscaled(const uint16_t* W, int w_dtype, const float* colscale, int64_t N, int64_t K,
                               uint8_t* codes, float* scales, uint8_t* zeros, hipStream_t s);

// Plain product Y[M, N] = A[M, K] B[N, K]^T of 16-bit operands (dtype
// QMM_BF16 or QMM_F16) in fp32 (w8a8.hip, the INT8 GEMM's tiles on 16-bit
// matrix instructions).  K % 32 == 0, rows 16-byte aligned, 256 * 2K < 2^31.
void launch_h16_gemm(const uint16_t* A, const uint16_t* B, int dtype, int64_t M, int64_t N, int64_t K, float* Y,
                     hipStream_t s);

// The W4A16 product of w4a16_gemm into fp32 Y with the caller's column sums
// xsum [M][K / 128] (the per-group sums of X's rows, exactly as X holds them;
// w4a16.hip): where w4a16_gemm would run its shared-tile kernel that kernel
// reads them instead of recomputing them, elsewhere this is w4a16_gemm.
// Arguments as w4a16_gemm (group 128, x_dtype QMM_BF16 or QMM_F16), xsum
// 16-byte aligned; returns its status.
int w4a16_gemm_colsums(const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K,
                       const uint16_t* X, const float* xsum, int x_dtype, int64_t M, float* Y, hipStream_t s);

}  // namespace qmm
