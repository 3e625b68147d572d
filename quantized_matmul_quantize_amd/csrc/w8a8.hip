// w8a8.hip -- SmoothQuant W8A8: smoothing factors, symmetric INT8 quantizers and
// the INT8 GEMM with int32 accumulation and a fused rescale.
//
// Sources: "How quantization works" (AI-infra handbook), "Activation
// quantization and outliers": per-row INT8 weights (absmax / 127), the
// smoothing factor s_j = max|X_j|^alpha / max|W_j|^(1-alpha) with each maximum
// floored at 1e-5, X <- X / s and W <- W * s; its fake-quantization listing
// floors the absmax at 1e-8.  "Quantization" (Engine Room ch. 15), "The
// Mathematics": the smoothing equation and the symmetric quantizer.
// "Quantization: Smaller Weights, Same Answers (Mostly)": INT8 x INT8
// products summed exactly in a 32-bit accumulator ("How does quantized matrix
// multiplication actually run on the GPU?") and per-token dynamic activation
// scales ("Quick Reference").
//
// All fp32 steps (X / s, W * s, absmax / 127, value / scale) are single IEEE
// operations with correctly rounded division, and codes use round-half-to-
// even, so the INT8 codes and scales are reproducible bit for bit.

#include <atomic>
#include <mutex>

#include "qmm_device.h"

namespace qmm {
namespace {

constexpr float kQ8 = 127.0f;
constexpr float kAbsFloor = 1e-8f;
constexpr float kSmoothFloor = 1e-5f;
constexpr float kFp8Max = 448.0f;   // largest finite E4M3
// Largest K (a multiple of 64) with 128 * 128 * K < 2^31: no int32 sum can overflow.
constexpr int64_t kMaxK = 131008;

// ----------------------------------------------------------------------------
// Column absolute maxima (calibration statistics).  Block = 512 columns x a
// band of 64 rows: lane l of wavefront w takes columns 8 l .. +8 of rows
// 16 w .. +16 of the band, eight rows per batch of loads (each row read is 1
// KiB contiguous per wavefront); the four wavefronts' maxima are combined in
// LDS and each column gets one atomicMax per block, on the float's bit
// pattern (non-negative floats order like unsigned integers).  (64-row bands:
// a 2048 x 4096 activation matrix alone makes 256 blocks, one per CU.)
// ----------------------------------------------------------------------------
constexpr int kCmCols = 512;
constexpr int64_t kCmBand = 64;

// Zeroes two arrays of n words in one launch (the column maxima targets).
__global__ __launch_bounds__(256) void fill_zero2_kernel(uint32_t* __restrict__ p, uint32_t* __restrict__ q,
                                                         int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    p[i] = 0u;
    q[i] = 0u;
  }
}

template <int DT>
__device__ __forceinline__ void colmax_band(const uint8_t* __restrict__ a, int64_t cols, int64_t col8, int64_t r0,
                                            int64_t r1, float m[8]) {
  constexpr int kElem = DT == QMM_F32 ? 4 : 2;
  constexpr int kRows = 8;   // rows loaded together, so their latencies overlap
  for (int64_t rb = r0; rb < r1; rb += kRows) {
    float v[kRows][8];
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
      const int64_t r = (rb + j < r1) ? rb + j : r1 - 1;   // repeats the last row: max unchanged
      Vec8<DT>::load(a + (r * cols + col8) * kElem, v[j]);
    }
#pragma unroll
    for (int j = 0; j < kRows; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) m[i] = fmaxf(m[i], fabsf(v[j][i]));
  }
}

// grid.x: column blocks of 512; grid.y: row bands of the two matrices (the
// first `bands_x` bands belong to X, the rest to W).
template <int XDT, int WDT>
__global__ __launch_bounds__(256) void colmax2_kernel(const uint8_t* __restrict__ X, int64_t M,
                                                      const uint8_t* __restrict__ W, int64_t N, int64_t K,
                                                      int64_t bands_x, uint32_t* __restrict__ cx,
                                                      uint32_t* __restrict__ cw) {
  __shared__ float red[4][kCmCols];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kCmCols;
  const int64_t col8 = c0 + lane * 8;
  const int64_t yb = blockIdx.y;
  const bool isx = yb < bands_x;
  const int64_t rows = isx ? M : N;
  const int64_t band0 = (isx ? yb : yb - bands_x) * kCmBand;
  const int64_t r0 = band0 + wave * (kCmBand / 4);
  const int64_t r1e = r0 + kCmBand / 4;
  const int64_t r1 = r1e < rows ? r1e : rows;
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (col8 < K && r0 < r1) {
    if (isx) colmax_band<XDT>(X, K, col8, r0, r1, m);
    else colmax_band<WDT>(W, K, col8, r0, r1, m);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[wave][lane * 8 + i] = m[i];
  __syncthreads();
  uint32_t* out = isx ? cx : cw;
  for (int c = threadIdx.x; c < kCmCols; c += 256) {
    if (c0 + c >= K) break;
    const float v = fmaxf(fmaxf(red[0][c], red[1][c]), fmaxf(red[2][c], red[3][c]));
    atomicMax(out + c0 + c, __float_as_uint(v));
  }
}

__global__ __launch_bounds__(256) void smooth_finalize_kernel(const float* __restrict__ cx,
                                                              const float* __restrict__ cw, int64_t K, float alpha,
                                                              float* __restrict__ smooth) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (j >= K) return;
  const float x = fmaxf(cx[j], kSmoothFloor);
  const float w = fmaxf(cw[j], kSmoothFloor);
  float num, den;
  if (alpha == 0.5f) {
    num = sqrtf(x);   // correctly rounded
    den = sqrtf(w);
  } else {
    num = powf(x, alpha);
    den = powf(w, 1.0f - alpha);
  }
  smooth[j] = num / den;
}

// ----------------------------------------------------------------------------
// Per-row symmetric INT8 quantization with column smoothing.  One wavefront
// per row; MODE 0 multiplies by the smoothing factor (weights), MODE 1
// divides (activations, a correctly rounded division per element); SM false
// skips the smoothing.  The row is read in batches of kRqChunks 8-element
// chunks per lane (4096 elements), every load of a batch issued before any is
// used.  Pass 1 finds the absmax of the smoothed row; pass 2 quantizes the
// values kept in registers (rows of up to 4096) or re-reads the batch.
// ----------------------------------------------------------------------------
constexpr int kRqChunks = 8;
constexpr int64_t kRqBatch = static_cast<int64_t>(kWave) * 8 * kRqChunks;   // 4096

// clamp(rint(fl32(v / s)), -128, 127) for 8 values, bit-identical to the
// correctly rounded division, from y = RN(1/s) (one division per row, by the
// caller): q0 = RN(v y), exact residual r = v - q0 s (fma), q1 = RN(q0 + r y)
// = RN(v / s) by Markstein's theorem (no overflow or underflow for scales in
// [2^-100, 2^100] and quotients of magnitude at least 1/4; smaller ones round
// to 0 either way).  Rows with a scale outside that range divide exactly.
__device__ __forceinline__ void quant8_int8(const float v[8], float s, float y, uint32_t* lo, uint32_t* hi) {
  const bool scale_ok = (s >= 0x1p-100f) && (s <= 0x1p100f);
  float k[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float q0 = v[i] * y;
    const float r = fmaf(-q0, s, v[i]);
    k[i] = rintf(fmaf(r, y, q0));
  }
  if (!scale_ok) {   // uniform: one scale per row
#pragma unroll
    for (int i = 0; i < 8; ++i) k[i] = rintf(v[i] / s);
  }
  uint32_t l = 0, h = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float c = __builtin_amdgcn_fmed3f(k[i], -128.0f, kQ8);
    const uint32_t byte = static_cast<uint32_t>(static_cast<int32_t>(c)) & 0xFFu;
    if (i < 4) l |= byte << (8 * i);
    else h |= byte << (8 * (i - 4));
  }
  *lo = l;
  *hi = h;
}

// FP8 E4M3 ("E4M3FN": bias 7, 3 mantissa bits, largest finite 448) code of
// t, round to nearest even, magnitudes from 448 up giving 448 (reading R25).
__device__ __forceinline__ uint32_t e4m3_code(float t) {
  const uint32_t u = __float_as_uint(t);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x43E00000u) {                       // |t| >= 448
    code = 0x7Eu;
  } else if (a < 0x3C800000u) {                 // |t| < 2^-6: multiples of 2^-9, rounded to nearest even
    code = static_cast<uint32_t>(rintf(__uint_as_float(a) * 512.0f));
  } else {                                      // keep 3 of the 23 mantissa bits, nearest even
    const uint32_t keep = a >> 20;
    const uint32_t rest = a & 0xFFFFFu;
    const uint32_t up = (rest > 0x80000u) || (rest == 0x80000u && (keep & 1u));
    code = keep + up - (120u << 3);             // exponent bias 127 -> 7; a carry moves into the exponent
  }
  return sign | code;
}

// E4M3 codes of 8 values with scale s: e4m3(fl32(v / s)), correctly rounded
// division (the quotient itself is rounded, not only its integer part).
__device__ __forceinline__ void quant8_fp8(const float v[8], float s, uint32_t* lo, uint32_t* hi) {
  uint32_t l = 0, h = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t byte = e4m3_code(v[i] / s);
    if (i < 4) l |= byte << (8 * i);
    else h |= byte << (8 * (i - 4));
  }
  *lo = l;
  *hi = h;
}

// Loads chunk c of the batch starting at `base` for every lane (zeros past K)
// and applies the smoothing; all loads are issued before any arithmetic.
template <int DT, int MODE, bool SM>
__device__ __forceinline__ void rq_load_batch(const uint8_t* arow, const float* smooth, int64_t K, int64_t base,
                                              int lane, float v[kRqChunks][8]) {
  constexpr int kElem = DT == QMM_F32 ? 4 : 2;
  float4 sm[kRqChunks][2];
#pragma unroll
  for (int c = 0; c < kRqChunks; ++c) {
    const int64_t k = base + static_cast<int64_t>(c) * (kWave * 8) + lane * 8;
    const int64_t kc = k < K ? k : K - 8;   // in bounds; the values are discarded below
    Vec8<DT>::load(arow + kc * kElem, v[c]);
    if constexpr (SM) {
      sm[c][0] = *reinterpret_cast<const float4*>(smooth + kc);
      sm[c][1] = *reinterpret_cast<const float4*>(smooth + kc + 4);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c < kRqChunks; ++c) {
    const int64_t k = base + static_cast<int64_t>(c) * (kWave * 8) + lane * 8;
    if constexpr (SM) {
      const float f[8] = {sm[c][0].x, sm[c][0].y, sm[c][0].z, sm[c][0].w,
                          sm[c][1].x, sm[c][1].y, sm[c][1].z, sm[c][1].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) v[c][i] = MODE == 0 ? v[c][i] * f[i] : v[c][i] / f[i];
    }
    if (k >= K) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[c][i] = 0.0f;
    }
  }
}

// PHASE 0: one pass per row (per-row scale).  For one scale over the whole
// tensor: PHASE 1 writes each row's absmax to scale[row]; tensor_scale_kernel
// turns them into the tensor's scale, stored for every row; PHASE 2 then
// quantizes each row with scale[row].
// FMT 1: FP8 E4M3 codes with s = max|x| / 448 ("How quantization works",
// fake-quantization listing) instead of INT8 with max|x| / 127.
// Four wavefronts per SIMD for 16-bit inputs (128 VGPRs, a few bytes of the
// smoothing factors' registers spilled): 4096 rows then run as one round of
// wavefronts on 256 compute units instead of one and a third (13.7 against
// ~15 us for a 4096 x 4096 weight matrix).
template <int DT, int MODE, bool SM, int PHASE, int FMT = 0>
__global__ __launch_bounds__(256, DT == QMM_F32 ? 1 : 4) void rowquant8_kernel(const uint8_t* __restrict__ a, const float* __restrict__ smooth,
                                                        int64_t rows, int64_t K, int8_t* __restrict__ q,
                                                        float* __restrict__ scale) {
  constexpr float kLevels = FMT == 1 ? kFp8Max : kQ8;
  constexpr int kElem = DT == QMM_F32 ? 4 : 2;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (row >= rows) return;
  const uint8_t* arow = a + row * K * kElem;
  const bool resident = K <= kRqBatch;

  float v[kRqChunks][8];
  float s;
  if constexpr (PHASE == 2) {
    s = scale[row];
  } else {
    float amax = 0.0f;
    for (int64_t base = 0; base < K; base += kRqBatch) {
      rq_load_batch<DT, MODE, SM>(arow, smooth, K, base, lane, v);
#pragma unroll
      for (int c = 0; c < kRqChunks; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[c][i]));
    }
    amax = wave_max(amax);
    if constexpr (PHASE == 1) {
      if (lane == 0) scale[row] = amax;
      return;
    }
    s = fmaxf(amax, kAbsFloor) / kLevels;
    if (lane == 0) scale[row] = s;
  }
  const float r = 1.0f / s;   // correctly rounded reciprocal

  for (int64_t base = 0; base < K; base += kRqBatch) {
    if (PHASE == 2 || !resident) rq_load_batch<DT, MODE, SM>(arow, smooth, K, base, lane, v);
#pragma unroll
    for (int c = 0; c < kRqChunks; ++c) {
      const int64_t k = base + static_cast<int64_t>(c) * (kWave * 8) + lane * 8;
      if (k < K) {
        uint32_t lo, hi;
        if constexpr (FMT == 1) quant8_fp8(v[c], s, &lo, &hi);
        else quant8_int8(v[c], s, r, &lo, &hi);
        *reinterpret_cast<uint2*>(q + row * K + k) = make_uint2(lo, hi);
      }
    }
  }
}

// The tensor's scale from the rows' absmax values in scale[0..rows): a =
// fl32(max(max_m absmax_m, 1e-8) / 127), then written to every scale[m].  One
// block; the maximum is exact, so the order of the reduction does not matter.
template <int FMT = 0>
__global__ __launch_bounds__(256) void tensor_scale_kernel(float* __restrict__ scale, int64_t rows) {
  __shared__ float part[256 / kWave];
  float m = 0.0f;
  for (int64_t i = threadIdx.x; i < rows; i += blockDim.x) m = fmaxf(m, scale[i]);
  m = wave_max(m);
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = m;
  __syncthreads();
  float a = part[0];
  for (int w = 1; w < static_cast<int>(blockDim.x / kWave); ++w) a = fmaxf(a, part[w]);
  a = fmaxf(a, kAbsFloor) / (FMT == 1 ? kFp8Max : kQ8);
  for (int64_t i = threadIdx.x; i < rows; i += blockDim.x) scale[i] = a;
}

// ----------------------------------------------------------------------------
// INT8 GEMM on v_mfma_i32_16x16x64_i8: C[m, n] = sum_k A[m, k] B[n, k], exact
// in int32.  Operand layout (16x16x64): lane l supplies row l%16 of A (row
// l%16 of B, i.e. column l%16 of C) and k = 16*(l/16) .. +16; D lane l holds
// rows 4*(l/16) .. +4 of column l%16.
//
// Block tile 256 x 128, k-step 128 (two 64-wide chunks), eight wavefronts:
// wavefront w = 4 wn + wm owns rows 64 wm .. + 64 and columns 64 wn .. + 64
// (4 x 4 instructions per chunk).  Two wavefronts share each SIMD, so one's
// MFMAs run while the other waits on LDS or on the barrier (measured 36.4 us
// against 41.8 us for four wavefronts of 64 x 128 at 2048 x 4096 x 4096).
//
// Global -> LDS: buffer loads that write LDS directly (16 bytes per lane,
// lane l of an instruction lands at byte 16 l of its destination), so no
// registers stage the operands.  Eight consecutive lanes fetch the eight
// 16-byte chunks of one row's 128-byte k-step (a whole cache line), in an
// order chosen so that the LDS image is XOR-swizzled: within each 16-row
// slice (2 KiB) row r, chunk c sits at 16-byte slot 8 r + (c ^ g(r)) with
// g(r) = (r >> 1) & 7 (the two rows sharing a 256-byte bank line use its two
// halves).  Fragment reads (16 rows, one 16-byte part each per 16 lanes) are
// then free of bank conflicts: measured 1.8% conflict cycles on gfx950, where
// g(r) = (r & 7) ^ (r >> 3) measured 48%.
//
// Pipeline, three LDS stages of A and B (48 KiB each) and one barrier per
// k-step t, placed between its two chunks:
//   chunk 0: MFMAs on fragments (t, 0) | read fragments (t, 1) | issue the
//            loads of step t+2 into the stage step t-1 used;
//   wait for this wave's loads of step t+1, barrier;
//   chunk 1: MFMAs on fragments (t, 1) | read fragments (t+1, 0).
// Every load is issued on every step (clamped past the end, never read), so
// the explicit wait count is exact.  Rows past M / N lie beyond the buffer
// resource and read as zero; when K % 128 == 64 the second chunk of the last
// step (A and B) is likewise fetched out of range, so its MFMAs add zero.  Tiles
// are ordered so that the blocks sharing an XCD (block id mod 8) cover a
// compact 4 x 8 patch of the output and share A and B rows in that XCD's L2.
//
// Epilogue: Y = acc * a[m] * b[n] in fp32 (or the raw int32 accumulator),
// staged through LDS per wavefront so that global stores are whole 16-byte
// row segments.
// ----------------------------------------------------------------------------
constexpr int kBM = 256, kBN = 128, kBK = 128;
constexpr int kSlice = 16 * kBK;               // one 16-row slice of a stage: 2 KiB
constexpr int kStageA = kBM * kBK;             // 32 KiB
constexpr int kStage = (kBM + kBN) * kBK;      // A then B: 48 KiB
constexpr size_t kGemmLds = 3 * kStage;        // 144 KiB
constexpr int kXcds = 8;
constexpr int kOutOfRange = 0x40000000;        // added to a lane offset: reads zero

__device__ __forceinline__ void xcd_tile(int64_t b, int64_t tm, int64_t tn, int64_t* m_tile, int64_t* n_tile,
                                         bool* valid) {
  const int64_t T = tm * tn;
  const int64_t per = (T + kXcds - 1) / kXcds;
  const int64_t t = (b % kXcds) * per + b / kXcds;
  *valid = t < T;
  const int64_t gm_band = 4;
  const int64_t band = t / (gm_band * tn);
  const int64_t gm = (tm - band * gm_band < gm_band) ? tm - band * gm_band : gm_band;
  const int64_t r = t - band * gm_band * tn;
  *m_tile = band * gm_band + (gm > 0 ? r % gm : 0);
  *n_tile = gm > 0 ? r / gm : 0;
}

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }


constexpr int kLoadsA8 = kBM * kBK / 1024 / 8;  // 1 KiB load instructions per wavefront per step: 4
constexpr int kLoadsB8 = kBN * kBK / 1024 / 8;  // 2
constexpr int kP2 = 144;                        // epilogue row pitch, 64 x 2-byte outputs
constexpr int kP4 = 272;                        // 64 x 4-byte outputs
constexpr int kEpiWave = 64 * kP4;              // per-wavefront epilogue region (64 rows)
static_assert(64 * kP2 <= kEpiWave && 8 * kEpiWave <= static_cast<int>(kGemmLds), "epilogue must fit");

// FP8: the same tiles, LDS layout and loads with E4M3 operands, but one
// v_mfma_scale_f32_16x16x128_f8f6f4 per tile and k-step (block scales all
// 1.0, E8M0 0x7F): a lane passes its 16-byte fragments of both 64-wide
// chunks as the instruction's 32 bytes.  A and B lanes are filled the same
// way, so each k of the step meets its partner whatever order the
// instruction gives the 32 bytes.  (The 16x16x32 fp8 form runs at the bf16
// rate on gfx950: half the throughput per k.)
template <bool FP8>
struct GemmAcc {
  typedef i32x4 type;
};
template <>
struct GemmAcc<true> {
  typedef f32x4 type;
};

__device__ __forceinline__ void mfma_frag(const i32x4& b, const i32x4& a, i32x4& acc) {
  acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(b, a, acc, 0, 0, 0);
}

// H16 = QMM_BF16 or QMM_F16: the same 16-byte fragments of a 64-byte chunk
// hold 8 16-bit values (32 k per chunk across the four lane groups), one
// v_mfma_f32_16x16x32_{bf16,f16} per chunk -- the kernel's tiles, loads and
// LDS layout are byte-based, so a 16-bit operand of K elements is a K * 2
// byte row.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

template <int H16>
__device__ __forceinline__ void mfma_frag16(const i32x4& b, const i32x4& a, f32x4& acc) {
  if constexpr (H16 == QMM_F16)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, b), __builtin_bit_cast(f16x8_t, a), acc,
                                                 0, 0, 0);
  else
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, b), __builtin_bit_cast(bf16x8_t, a),
                                                  acc, 0, 0, 0);
}

// One chunk's product: INT8 (int32 accumulators) or 16-bit operands (fp32).
template <int H16, class Acc>
__device__ __forceinline__ void mfma_chunk(const i32x4& b, const i32x4& a, Acc& acc) {
  if constexpr (H16 != 0) mfma_frag16<H16>(b, a, acc);
  else mfma_frag(b, a, acc);
}

typedef int i32x8 __attribute__((ext_vector_type(8)));
constexpr int kUnitScales = 0x7F7F7F7F;   // E8M0 1.0 in every byte

// D += B^T-side x A over the 128 k of one step: fragments (b0, b1) and (a0,
// a1) of the step's two chunks.
__device__ __forceinline__ void mfma_fp8_step(const i32x4& b0, const i32x4& b1, const i32x4& a0, const i32x4& a1,
                                              f32x4& acc) {
  const i32x8 bv = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
  const i32x8 av = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bv, av, acc, 0, 0, 0, kUnitScales, 0, kUnitScales);
}

// OUTL: LLM.int8()'s 16-bit outlier product is added in the epilogue before
// the output is rounded.  *count outlier columns idx[0 ..); for column j the
// activations X[m, j] (16-bit, x_f16 selects fp16 over bf16) and the 16-bit
// weights, B[n, j] * bscale[n] rounded to X's type.  The first kOutlLds of
// them are fetched at the start of the kernel (their latency hidden behind the
// main loop) and kept in LDS past the stages; any further ones are read from
// global memory in the epilogue.
struct Outliers {
  const int32_t* count;
  const int32_t* idx;
  const uint16_t* X;
  int x_f16;
};
constexpr int kOutlLds = 8;
constexpr size_t kOutlLdsBytes = static_cast<size_t>(kOutlLds) * (kBM + kBN) * 4;   // 12 KiB
static_assert(kGemmLds + kOutlLdsBytes <= 160 * 1024, "outlier operands fit beside the stages");

// The value of v in X's 16-bit type (nearest even; binary16 saturates at its
// largest finite value).
__device__ __forceinline__ float round16(float v, int x_f16) {
  return x_f16 ? f16lo_to_f32(f32_to_f16_bits(__builtin_amdgcn_fmed3f(v, -65504.0f, 65504.0f)))
               : bf16lo_to_f32(f32_to_bf16_bits(v));
}
__device__ __forceinline__ float x16_value(uint32_t u, int x_f16) {
  return x_f16 ? f16lo_to_f32(u) : bf16lo_to_f32(u);
}

template <int YDT, bool FP8 = false, bool OUTL = false, int H16 = 0>
__global__ __launch_bounds__(512) void i8_gemm_kernel(const int8_t* __restrict__ A, const float* __restrict__ ascale,
                                                       const int8_t* __restrict__ B, const float* __restrict__ bscale,
                                                       int64_t M, int64_t N, int64_t K, void* __restrict__ Y,
                                                       Outliers outl) {
  static_assert(H16 == 0 || ((H16 == QMM_BF16 || H16 == QMM_F16) && !FP8 && !OUTL),
                "16-bit operands: the plain product");
  using Acc = typename GemmAcc<FP8 || H16 != 0>::type;
  extern __shared__ __attribute__((aligned(16))) int8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave & 3;
  const int wn = wave >> 2;
  int64_t mt, nt;
  bool valid;
  xcd_tile(blockIdx.x, (M + kBM - 1) / kBM, (N + kBN - 1) / kBN, &mt, &nt, &valid);
  if (!valid) return;
  const int64_t m0 = mt * kBM;
  const int64_t n0 = nt * kBN;
  const int kk = static_cast<int>(K);

  const int64_t arows = (M - m0 < kBM) ? M - m0 : kBM;
  const int64_t brows = (N - n0 < kBN) ? N - n0 : kBN;
  const __amdgpu_buffer_rsrc_t arsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(A + m0 * K), 0, static_cast<int>(arows * K), kBufferWord3);
  const __amdgpu_buffer_rsrc_t brsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(B + n0 * K), 0, static_cast<int>(brows * K), kBufferWord3);

  // Load q of this wavefront fills half-slice I = loads * wave + q of A (4
  // per wavefront) or of B (2); lane l writes slot 64 (I & 1) + l of slice
  // I / 2, i.e. row r = 8 (I & 1) + l / 8 of that slice, chunk (l % 8) ^ g(r).
  // When K % 128 == 64 the second chunk of the last step lies past the end
  // of each row (the next row's first bytes): both operands fetch it out of
  // the buffer's range (zeros), so no value from another row enters a
  // product -- an fp8 NaN code there would otherwise survive a zero partner.
  int aoff[kLoadsA8], az[kLoadsA8], boff[kLoadsB8], bz[kLoadsB8];
#pragma unroll
  for (int q = 0; q < kLoadsA8; ++q) {
    const int I = kLoadsA8 * wave + q;
    const int r = 8 * (I & 1) + (lane >> 3);
    const int row = 16 * (I >> 1) + r;
    const int c = (lane & 7) ^ swz(r);
    aoff[q] = row * kk + c * 16;
    az[q] = (c >= 4) ? kOutOfRange : 0;
  }
#pragma unroll
  for (int q = 0; q < kLoadsB8; ++q) {
    const int I = kLoadsB8 * wave + q;
    const int r = 8 * (I & 1) + (lane >> 3);
    const int row = 16 * (I >> 1) + r;
    const int c = (lane & 7) ^ swz(r);
    boff[q] = row * kk + c * 16;
    bz[q] = (c >= 4) ? kOutOfRange : 0;
  }
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  const int nsteps = (kk + kBK - 1) / kBK;
  auto issue = [&](int step, int stage) {
    const int st = min(step, nsteps - 1);
    const int k0 = st * kBK;
    const bool tail = k0 + 64 >= kk;
    const uint32_t sbase = lds_base + static_cast<uint32_t>(stage * kStage);
#pragma unroll
    for (int q = 0; q < kLoadsA8; ++q) {
      const int I = kLoadsA8 * wave + q;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc, (lds_ptr_t)(uintptr_t)(sbase + (I >> 1) * kSlice + (I & 1) * 1024),
                                               16, aoff[q] + (tail ? az[q] : 0), k0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < kLoadsB8; ++q) {
      const int I = kLoadsB8 * wave + q;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          brsrc, (lds_ptr_t)(uintptr_t)(sbase + kStageA + (I >> 1) * kSlice + (I & 1) * 1024), 16,
          boff[q] + (tail ? bz[q] : 0), k0, 0, 0);
    }
  };

  const int fr = lane & 15;
  const int rd0 = (8 * fr + ((lane >> 4) ^ swz(fr))) * 16;
  const int rd1 = (8 * fr + ((4 + (lane >> 4)) ^ swz(fr))) * 16;
  i32x4 fa0[4], fb0[4], fa1[4], fb1[4];
  auto read_chunk = [&](i32x4 (&fa)[4], i32x4 (&fb)[4], int stage, int rd) {
    const int8_t* sa = lds + stage * kStage + (4 * wm) * kSlice + rd;
    const int8_t* sb = lds + stage * kStage + kStageA + (4 * wn) * kSlice + rd;
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = *reinterpret_cast<const i32x4*>(sa + i * kSlice);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = *reinterpret_cast<const i32x4*>(sb + j * kSlice);
  };
  auto barrier = [&]() {
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  };

  Acc acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = Acc{0, 0, 0, 0};

  // The epilogue's scales, fetched now so that their latency hides behind
  // the main loop: tile (i, j) register r of lane l is row 16 i + l % 16 and
  // column 16 j + 4 (l / 16) + r of the wavefront's 64 x 64 (the MFMAs take
  // B as their first operand, so D is the transposed tile).
  const int64_t mw = m0 + 64 * wm;
  const int64_t nw = n0 + 64 * wn;
  float as[4], bs[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = mw + 16 * i + (lane & 15);
    as[i] = (YDT == QMM_I32 || H16 != 0) ? 1.0f : ascale[m < M ? m : M - 1];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t n = nw + 16 * j + 4 * (lane >> 4) + r;
      bs[j][r] = (YDT == QMM_I32 || H16 != 0) ? 1.0f : bscale[n < N ? n : N - 1];
    }

  // Outlier operands of this tile (the first kOutlLds columns): thread t
  // fetches X rows (t + 512 q) % 256 of outlier (t + 512 q) / 256 and weight
  // columns (t + 512 q) % 128 of outlier (t + 512 q) / 128; they wait in
  // registers until the stages are free.
  int okept = 0;
  uint32_t ox[4];
  int32_t ow[2];
  float os[2];
  if constexpr (OUTL) {
    okept = *outl.count;
    const int nk = okept < kOutlLds ? okept : kOutlLds;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int slot = tid + 512 * q;
      const int p = slot / kBM;
      const int64_t m = m0 + slot % kBM;
      ox[q] = (p < nk) ? outl.X[(m < M ? m : M - 1) * K + outl.idx[p]] : 0u;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int slot = tid + 512 * q;
      const int p = slot / kBN;
      const int64_t n = n0 + slot % kBN;
      const int64_t nc = n < N ? n : N - 1;
      ow[q] = (p < nk) ? B[nc * K + outl.idx[p]] : 0;
      os[q] = (p < nk) ? bscale[nc] : 0.0f;
    }
  }

  issue(0, 0);
  issue(1, 1);
  wait_vm<kLoadsA8 + kLoadsB8>();
  barrier();
  read_chunk(fa0, fb0, 0, rd0);

  if constexpr (FP8) {
    // Per step: issue the loads of step t+2, the 16 MFMAs of step t (their
    // fragments were read in the previous iteration), then wait for step
    // t+1's loads, the barrier, and read step t+1's fragments while the
    // MFMAs run.
    read_chunk(fa1, fb1, 0, rd1);
    i32x4 na0[4], nb0[4], na1[4], nb1[4];
    int s0 = 0;
    for (int t = 0; t < nsteps; ++t) {
      const int s1 = (s0 == 2) ? 0 : s0 + 1;
      const int s2 = (s1 == 2) ? 0 : s1 + 1;
      issue(t + 2, s2);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mfma_fp8_step(fb0[j], fb1[j], fa0[i], fa1[i], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
      wait_vm<kLoadsA8 + kLoadsB8>();
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      barrier();
      read_chunk(na0, nb0, s1, rd0);
      read_chunk(na1, nb1, s1, rd1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fa0[i] = na0[i];
        fb0[i] = nb0[i];
        fa1[i] = na1[i];
        fb1[i] = nb1[i];
      }
      s0 = s1;
    }
  } else {
  int s0 = 0;
  for (int t = 0; t < nsteps; ++t) {
    const int s1 = (s0 == 2) ? 0 : s0 + 1;
    const int s2 = (s1 == 2) ? 0 : s1 + 1;
    read_chunk(fa1, fb1, s0, rd1);
    issue(t + 2, s2);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) mfma_chunk<H16>(fb0[j], fa0[i], acc[i][j]);
#pragma unroll
    for (int g = 0; g < 6; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<kLoadsA8 + kLoadsB8>();
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    barrier();
    read_chunk(fa0, fb0, s1, rd0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) mfma_chunk<H16>(fb1[j], fa1[i], acc[i][j]);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
    }
    s0 = s1;
  }
  }
  wait_vm<0>();
  __syncthreads();   // the epilogue reuses the LDS
  float* olds = reinterpret_cast<float*>(lds + kGemmLds);   // [outlier][256 rows], then [outlier][128 columns]
  if constexpr (OUTL) {
    const int nk = okept < kOutlLds ? okept : kOutlLds;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int slot = tid + 512 * q;
      if (slot / kBM < nk) olds[slot] = x16_value(ox[q], outl.x_f16);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int slot = tid + 512 * q;
      if (slot / kBN < nk) olds[kOutlLds * kBM + slot] = round16(static_cast<float>(ow[q]) * os[q], outl.x_f16);
    }
    __syncthreads();
  }

  // Epilogue: Y = acc * a[m] * b[n] (+ the outlier product), four
  // consecutive columns per lane and tile, staged through LDS so that global
  // stores are whole 16-byte row segments.
  int8_t* region = lds + wave * kEpiWave;
  f32x4 fv[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) fv[i][j][r] = static_cast<float>(acc[i][j][r]) * as[i] * bs[j][r];
  if constexpr (OUTL) {
    // the block-local rows and columns of this lane's outputs
    const int nk = okept < kOutlLds ? okept : kOutlLds;
    for (int p = 0; p < nk; ++p) {
      float xv[4];
      f32x4 wv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) xv[i] = olds[p * kBM + 64 * wm + 16 * i + (lane & 15)];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        wv[j] = *reinterpret_cast<const f32x4*>(olds + kOutlLds * kBM + p * kBN + 64 * wn + 16 * j + 4 * (lane >> 4));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) fv[i][j][r] = fmaf(xv[i], wv[j][r], fv[i][j][r]);
    }
    // outliers past the LDS copy: straight from X and the weights (rows and
    // columns clamped; values past M or N are never stored)
    for (int p = nk; p < okept; ++p) {
      const int64_t j = outl.idx[p];
      float xv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = mw + 16 * i + (lane & 15);
        xv[i] = x16_value(outl.X[(m < M ? m : M - 1) * K + j], outl.x_f16);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float wv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t n = nw + 16 * jj + 4 * (lane >> 4) + r;
          const int64_t nc = n < N ? n : N - 1;
          wv[r] = round16(static_cast<float>(B[nc * K + j]) * bscale[nc], outl.x_f16);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) fv[i][jj][r] = fmaf(xv[i], wv[r], fv[i][jj][r]);
      }
    }
  }
  if constexpr (YDT == QMM_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 f = fv[i][j];
        // Round to nearest even, two values per conversion.
        const bf16x2_t lo = __builtin_convertvector(f.xy, bf16x2_t);
        const bf16x2_t hi = __builtin_convertvector(f.zw, bf16x2_t);
        const uint2 v = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
        *reinterpret_cast<uint2*>(region + (16 * i + (lane & 15)) * kP2 + (16 * j + 4 * (lane >> 4)) * 2) = v;
      }
    __syncthreads();
    const bool vec = (N % 8 == 0) && ((reinterpret_cast<uintptr_t>(Y) & 15) == 0);
#pragma unroll 4
    for (int it = 0; it < 8; ++it) {
      const int lr = 8 * it + (lane >> 3);
      const int64_t m = mw + lr;
      const int64_t n = nw + (lane & 7) * 8;
      if (m >= M || n >= N) continue;
      const u32x4 v = *reinterpret_cast<const u32x4*>(region + lr * kP2 + (lane & 7) * 16);
      uint16_t* dst = static_cast<uint16_t*>(Y) + m * N + n;
      if (vec && n + 8 <= N) {
        *reinterpret_cast<u32x4*>(dst) = v;
      } else {
        for (int e = 0; e < 8 && n + e < N; ++e) dst[e] = static_cast<uint16_t>(v[e >> 1] >> (16 * (e & 1)));
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (YDT == QMM_I32) v[r] = static_cast<uint32_t>(acc[i][j][r]);
          else v[r] = __float_as_uint(fv[i][j][r]);
        }
        *reinterpret_cast<u32x4*>(region + (16 * i + (lane & 15)) * kP4 + (16 * j + 4 * (lane >> 4)) * 4) = v;
      }
    __syncthreads();
    const bool vec = (N % 4 == 0) && ((reinterpret_cast<uintptr_t>(Y) & 15) == 0);
#pragma unroll 4
    for (int it = 0; it < 16; ++it) {
      const int lr = 4 * it + (lane >> 4);
      const int64_t m = mw + lr;
      const int64_t n = nw + (lane & 15) * 4;
      if (m < M && n < N) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(region + lr * kP4 + (lane & 15) * 16);
        uint32_t* dst = static_cast<uint32_t*>(Y) + m * N + n;
        if (vec && n + 4 <= N) {
          *reinterpret_cast<u32x4*>(dst) = v;
        } else {
          for (int e = 0; e < 4 && n + e < N; ++e) dst[e] = v[e];
        }
      }
    }
  }
}

bool float_dtype(int dt) { return dt == QMM_F32 || dt == QMM_BF16 || dt == QMM_F16; }

template <int MODE, int PHASE = 0, int FMT = 0>
int launch_rowquant(const void* a, int dt, const float* smooth, int64_t rows, int64_t K, int8_t* q, float* scale,
                    hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(ceil_div(rows, 4)));
  const dim3 block(256);
  const uint8_t* p = static_cast<const uint8_t*>(a);
  if (smooth) {
    switch (dt) {
      case QMM_BF16: rowquant8_kernel<QMM_BF16, MODE, true, PHASE, FMT><<<grid, block, 0, s>>>(p, smooth, rows, K, q, scale); break;
      case QMM_F16: rowquant8_kernel<QMM_F16, MODE, true, PHASE, FMT><<<grid, block, 0, s>>>(p, smooth, rows, K, q, scale); break;
      default: rowquant8_kernel<QMM_F32, MODE, true, PHASE, FMT><<<grid, block, 0, s>>>(p, smooth, rows, K, q, scale); break;
    }
  } else {
    switch (dt) {
      case QMM_BF16: rowquant8_kernel<QMM_BF16, MODE, false, PHASE, FMT><<<grid, block, 0, s>>>(p, smooth, rows, K, q, scale); break;
      case QMM_F16: rowquant8_kernel<QMM_F16, MODE, false, PHASE, FMT><<<grid, block, 0, s>>>(p, smooth, rows, K, q, scale); break;
      default: rowquant8_kernel<QMM_F32, MODE, false, PHASE, FMT><<<grid, block, 0, s>>>(p, smooth, rows, K, q, scale); break;
    }
  }
  return launch_status();
}

int check_rowquant(const void* a, int dt, const float* smooth, int64_t rows, int64_t K, const int8_t* q,
                   const float* scale) {
  if (!a || !q || !scale) return QMM_EINVAL;
  if (rows <= 0 || K <= 0) return QMM_EINVAL;
  if (!float_dtype(dt)) return dt == QMM_I32 ? QMM_EUNSUPPORTED : QMM_EINVAL;
  if (K % 64 != 0) return QMM_EUNSUPPORTED;
  if (!aligned(a, 16) || !aligned(q, 16) || !aligned(scale, 4) || (smooth && !aligned(smooth, 16)))
    return QMM_EALIGN;
  return QMM_OK;
}

int check_gemm(const int8_t* qX, const float* xs, const int8_t* qW, const float* ws, int64_t M, int64_t N,
               int64_t K, const void* Y, int ydt) {
  if (!qX || !qW || !Y) return QMM_EINVAL;
  if (M <= 0 || N <= 0 || K <= 0) return QMM_EINVAL;
  if (ydt != QMM_BF16 && ydt != QMM_F32 && ydt != QMM_I32) return ydt == QMM_F16 ? QMM_EUNSUPPORTED : QMM_EINVAL;
  if (ydt != QMM_I32 && (!xs || !ws)) return QMM_EINVAL;
  if (K % 64 != 0) return QMM_EUNSUPPORTED;
  if (K > kMaxK) return QMM_ERANGE;
  if (!aligned(qX, 16) || !aligned(qW, 16) || !aligned(Y, 4) || (xs && !aligned(xs, 4)) || (ws && !aligned(ws, 4)))
    return QMM_EALIGN;
  return QMM_OK;
}

template <int YDT, bool FP8 = false, bool OUTL = false, int H16 = 0>
void launch_gemm_t(const int8_t* qX, const float* xs, const int8_t* qW, const float* ws, int64_t M, int64_t N,
                   int64_t K, void* Y, hipStream_t s, Outliers outl = Outliers{nullptr, nullptr, nullptr, 0}) {
  // 144 KiB of dynamic LDS (+12 KiB of outlier operands); the attribute is
  // cheap to set and idempotent, so it is set on every launch (no per-device
  // bookkeeping).
  constexpr size_t lds = kGemmLds + (OUTL ? kOutlLdsBytes : 0);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&i8_gemm_kernel<YDT, FP8, OUTL, H16>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  const int64_t tiles = ceil_div(M, kBM) * ceil_div(N, kBN);
  const dim3 grid(static_cast<unsigned>(ceil_div(tiles, kXcds) * kXcds));
  i8_gemm_kernel<YDT, FP8, OUTL, H16><<<grid, dim3(512), lds, s>>>(qX, xs, qW, ws, M, N, K, Y, outl);
}

void launch_gemm(const int8_t* qX, const float* xs, const int8_t* qW, const float* ws, int64_t M, int64_t N,
                 int64_t K, void* Y, int ydt, hipStream_t s) {
  switch (ydt) {
    case QMM_I32: launch_gemm_t<QMM_I32>(qX, xs, qW, ws, M, N, K, Y, s); break;
    case QMM_F32: launch_gemm_t<QMM_F32>(qX, xs, qW, ws, M, N, K, Y, s); break;
    default: launch_gemm_t<QMM_BF16>(qX, xs, qW, ws, M, N, K, Y, s); break;
  }
}

void launch_gemm_fp8(const uint8_t* qX, const float* xs, const uint8_t* qW, const float* ws, int64_t M, int64_t N,
                     int64_t K, void* Y, int ydt, hipStream_t s) {
  const int8_t* a = reinterpret_cast<const int8_t*>(qX);
  const int8_t* b = reinterpret_cast<const int8_t*>(qW);
  if (ydt == QMM_F32) launch_gemm_t<QMM_F32, true>(a, xs, b, ws, M, N, K, Y, s);
  else launch_gemm_t<QMM_BF16, true>(a, xs, b, ws, M, N, K, Y, s);
}

}  // namespace

void launch_h16_gemm(const uint16_t* A, const uint16_t* B, int dtype, int64_t M, int64_t N, int64_t K, float* Y,
                     hipStream_t s) {
  if (dtype == QMM_F16)
    launch_gemm_t<QMM_F32, false, false, QMM_F16>(reinterpret_cast<const int8_t*>(A), nullptr,
                                                  reinterpret_cast<const int8_t*>(B), nullptr, M, N, 2 * K, Y, s);
  else
    launch_gemm_t<QMM_F32, false, false, QMM_BF16>(reinterpret_cast<const int8_t*>(A), nullptr,
                                                   reinterpret_cast<const int8_t*>(B), nullptr, M, N, 2 * K, Y, s);
}
}  // namespace qmm

using namespace qmm;

extern "C" int sq_smooth_factors(const void* X, int x_dtype, int64_t M, const void* W, int w_dtype, int64_t N,
                                 int64_t K, float alpha, float* x_colmax, float* w_colmax, float* smooth,
                                 void* stream) {
  if (!X || !W || !x_colmax || !w_colmax || !smooth) return QMM_EINVAL;
  if (M <= 0 || N <= 0 || K <= 0) return QMM_EINVAL;
  if (!float_dtype(x_dtype) || !float_dtype(w_dtype)) return QMM_EINVAL;
  if (!(alpha >= 0.0f && alpha <= 1.0f)) return QMM_EINVAL;
  if (K % 8 != 0) return QMM_EUNSUPPORTED;
  if (!aligned(X, 16) || !aligned(W, 16) || !aligned(x_colmax, 4) || !aligned(w_colmax, 4) || !aligned(smooth, 4))
    return QMM_EALIGN;
  hipStream_t s = as_stream(stream);
  uint32_t* cx = reinterpret_cast<uint32_t*>(x_colmax);
  uint32_t* cw = reinterpret_cast<uint32_t*>(w_colmax);
  const unsigned fill_blocks = static_cast<unsigned>(ceil_div(K, 256));
  fill_zero2_kernel<<<fill_blocks, 256, 0, s>>>(cx, cw, K);
  const int64_t bands_x = ceil_div(M, kCmBand);
  const int64_t bands_w = ceil_div(N, kCmBand);
  const dim3 grid(static_cast<unsigned>(ceil_div(K, kCmCols)), static_cast<unsigned>(bands_x + bands_w));
  const uint8_t* xp = static_cast<const uint8_t*>(X);
  const uint8_t* wp = static_cast<const uint8_t*>(W);
#define QMM_COLMAX(XD, WD) colmax2_kernel<XD, WD><<<grid, 256, 0, s>>>(xp, M, wp, N, K, bands_x, cx, cw)
  if (x_dtype == QMM_BF16 && w_dtype == QMM_BF16) QMM_COLMAX(QMM_BF16, QMM_BF16);
  else if (x_dtype == QMM_F16 && w_dtype == QMM_F16) QMM_COLMAX(QMM_F16, QMM_F16);
  else if (x_dtype == QMM_F32 && w_dtype == QMM_F32) QMM_COLMAX(QMM_F32, QMM_F32);
  else if (x_dtype == QMM_BF16 && w_dtype == QMM_F32) QMM_COLMAX(QMM_BF16, QMM_F32);
  else if (x_dtype == QMM_F16 && w_dtype == QMM_F32) QMM_COLMAX(QMM_F16, QMM_F32);
  else if (x_dtype == QMM_F32 && w_dtype == QMM_BF16) QMM_COLMAX(QMM_F32, QMM_BF16);
  else if (x_dtype == QMM_F32 && w_dtype == QMM_F16) QMM_COLMAX(QMM_F32, QMM_F16);
  else if (x_dtype == QMM_BF16 && w_dtype == QMM_F16) QMM_COLMAX(QMM_BF16, QMM_F16);
  else QMM_COLMAX(QMM_F16, QMM_BF16);
#undef QMM_COLMAX
  smooth_finalize_kernel<<<fill_blocks, 256, 0, s>>>(x_colmax, w_colmax, K, alpha, smooth);
  return launch_status();
}

extern "C" int sq_quantize_weight(const void* W, int w_dtype, const float* smooth, int64_t N, int64_t K, int8_t* qW,
                                  float* w_scale, void* stream) {
  int st = check_rowquant(W, w_dtype, smooth, N, K, qW, w_scale);
  if (st != QMM_OK) return st;
  return launch_rowquant<0>(W, w_dtype, smooth, N, K, qW, w_scale, as_stream(stream));
}

extern "C" int sq_quantize_activation(const void* X, int x_dtype, const float* smooth, int64_t M, int64_t K,
                                      int8_t* qX, float* x_scale, void* stream) {
  int st = check_rowquant(X, x_dtype, smooth, M, K, qX, x_scale);
  if (st != QMM_OK) return st;
  return launch_rowquant<1>(X, x_dtype, smooth, M, K, qX, x_scale, as_stream(stream));
}

extern "C" int sq_quantize_activation_per_tensor(const void* X, int x_dtype, const float* smooth, int64_t M,
                                                 int64_t K, int8_t* qX, float* x_scale, void* stream) {
  int st = check_rowquant(X, x_dtype, smooth, M, K, qX, x_scale);
  if (st != QMM_OK) return st;
  hipStream_t s = as_stream(stream);
  st = launch_rowquant<1, 1>(X, x_dtype, smooth, M, K, qX, x_scale, s);
  if (st != QMM_OK) return st;
  tensor_scale_kernel<0><<<1, 256, 0, s>>>(x_scale, M);
  st = launch_status();
  if (st != QMM_OK) return st;
  return launch_rowquant<1, 2>(X, x_dtype, smooth, M, K, qX, x_scale, s);
}

extern "C" int sq_int8_gemm(const int8_t* qX, const float* x_scale, const int8_t* qW, const float* w_scale, int64_t M,
                            int64_t N, int64_t K, void* Y, int y_dtype, void* stream) {
  int st = check_gemm(qX, x_scale, qW, w_scale, M, N, K, Y, y_dtype);
  if (st != QMM_OK) return st;
  launch_gemm(qX, x_scale, qW, w_scale, M, N, K, Y, y_dtype, as_stream(stream));
  return launch_status();
}

extern "C" size_t sq_workspace_bytes(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0) return 0;
  const size_t q = static_cast<size_t>(M) * static_cast<size_t>(K);
  return (q + 255u) / 256u * 256u + static_cast<size_t>(M) * 4u;
}

namespace qmm {
namespace {

// Arguments of the online W8A8 call other than its workspace.
int check_online(const void* X, int x_dtype, const float* smooth, const int8_t* qW, const float* w_scale, int64_t M,
                 int64_t N, int64_t K, void* Y, int y_dtype) {
  if (!X || !qW || !w_scale || !Y) return QMM_EINVAL;
  if (M <= 0 || N <= 0 || K <= 0) return QMM_EINVAL;
  if (!float_dtype(x_dtype)) return x_dtype == QMM_I32 ? QMM_EUNSUPPORTED : QMM_EINVAL;
  if (y_dtype != QMM_BF16 && y_dtype != QMM_F32 && y_dtype != QMM_I32)
    return y_dtype == QMM_F16 ? QMM_EUNSUPPORTED : QMM_EINVAL;
  if (K % 64 != 0) return QMM_EUNSUPPORTED;
  if (K > kMaxK) return QMM_ERANGE;
  if (!aligned(X, 16) || !aligned(qW, 16) || !aligned(w_scale, 4) || !aligned(Y, 4) ||
      (smooth && !aligned(smooth, 16)))
    return QMM_EALIGN;
  return QMM_OK;
}

// Per-token smoothing + INT8 quantization of X into the workspace (qX, then
// x_scale at the next 256-byte boundary), then the INT8 GEMM.  Every byte of
// qX and x_scale is written before it is read, so the workspace needs no
// clearing.
int online_launch(const void* X, int x_dtype, const float* smooth, const int8_t* qW, const float* w_scale, int64_t M,
                  int64_t N, int64_t K, void* Y, int y_dtype, uint8_t* workspace, hipStream_t s) {
  int8_t* qX = reinterpret_cast<int8_t*>(workspace);
  float* xs = reinterpret_cast<float*>(workspace +
                                       (static_cast<size_t>(M) * static_cast<size_t>(K) + 255u) / 256u * 256u);
  int st = launch_rowquant<1>(X, x_dtype, smooth, M, K, qX, xs, s);
  if (st != QMM_OK) return st;
  launch_gemm(qX, xs, qW, w_scale, M, N, K, Y, y_dtype, s);
  return launch_status();
}

}  // namespace
}  // namespace qmm

extern "C" int smooth_quant_w8a8_gemm(const void* X, int x_dtype, const float* smooth, const int8_t* qW,
                                      const float* w_scale, int64_t M, int64_t N, int64_t K, void* Y, int y_dtype,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_online(X, x_dtype, smooth, qW, w_scale, M, N, K, Y, y_dtype);
  if (st != QMM_OK) return st;
  if (!workspace || workspace_bytes < sq_workspace_bytes(M, K) || !aligned(workspace, 16)) return QMM_EWORKSPACE;
  return online_launch(X, x_dtype, smooth, qW, w_scale, M, N, K, Y, y_dtype, static_cast<uint8_t*>(workspace),
                       as_stream(stream));
}

// ----------------------------------------------------------------------------
// Allocation-free variant: the workspace is this file-scope device array, one
// copy per GPU, resident until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol):
// its device address is looked up once per device with hipGetSymbolAddress,
// with that device current, and that address is what the kernels receive.
// Calls on one GPU share the array, so calls that overlap in time on one GPU
// (different streams, or threads) race on it.
static __device__ __align__(256) uint8_t scratch[QMM_SQ_STATIC_SCRATCH_BYTES];

namespace qmm {
namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
std::atomic<uint8_t*> scratch_addr[kMaxDevices];

// Device address of `scratch` on the device that `stream` belongs to (the
// current device for the null stream), looked up on the first call on that
// device.  QMM_EHIP if a HIP query fails.
int scratch_for(hipStream_t stream, uint8_t** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return QMM_EHIP;
  int dev = cur;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return QMM_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return QMM_EHIP;
  uint8_t* p = scratch_addr[dev].load(std::memory_order_acquire);
  if (p) {
    *out = p;
    return QMM_OK;
  }
  std::lock_guard<std::mutex> lock(scratch_mu);
  p = scratch_addr[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return QMM_EHIP;
    void* addr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return QMM_EHIP;
    if (e != hipSuccess || !addr) return QMM_EHIP;
    p = static_cast<uint8_t*>(addr);
    scratch_addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return QMM_OK;
}

}  // namespace
}  // namespace qmm

extern "C" int smooth_quant_w8a8_gemm_noalloc(const void* X, int x_dtype, const float* smooth, const int8_t* qW,
                                              const float* w_scale, int64_t M, int64_t N, int64_t K, void* Y,
                                              int y_dtype, void* stream) {
  int st = check_online(X, x_dtype, smooth, qW, w_scale, M, N, K, Y, y_dtype);
  if (st != QMM_OK) return st;
  if (sq_workspace_bytes(M, K) > QMM_SQ_STATIC_SCRATCH_BYTES) return QMM_ERANGE;
  hipStream_t s = as_stream(stream);
  uint8_t* ws = nullptr;
  st = scratch_for(s, &ws);
  if (st != QMM_OK) return st;
  return online_launch(X, x_dtype, smooth, qW, w_scale, M, N, K, Y, y_dtype, ws, s);
}

// ----------------------------------------------------------------------------
// FP8 E4M3 W8A8 ("How quantization works", the fake-quantization listing:
// s = max|x| / 448, q = E4M3(x / s); "Mainstream schemes at a glance": FP8
// weights and activations with dynamic or static scales).  The row quantizer
// and the GEMM tiles above with E4M3 codes and fp8 matrix instructions.
// ----------------------------------------------------------------------------
namespace qmm {
namespace {

int check_fp8_gemm(const uint8_t* qX, const float* xs, const uint8_t* qW, const float* ws, int64_t M, int64_t N,
                   int64_t K, const void* Y, int ydt) {
  if (!qX || !qW || !Y || !xs || !ws) return QMM_EINVAL;
  if (M <= 0 || N <= 0 || K <= 0) return QMM_EINVAL;
  if (ydt != QMM_BF16 && ydt != QMM_F32) return (ydt == QMM_F16 || ydt == QMM_I32) ? QMM_EUNSUPPORTED : QMM_EINVAL;
  if (K % 64 != 0) return QMM_EUNSUPPORTED;
  if (K > kMaxK) return QMM_ERANGE;
  if (!aligned(qX, 16) || !aligned(qW, 16) || !aligned(Y, 4) || !aligned(xs, 4) || !aligned(ws, 4))
    return QMM_EALIGN;
  return QMM_OK;
}

}  // namespace
}  // namespace qmm

extern "C" int fp8_quantize(const void* X, int x_dtype, int64_t rows, int64_t K, int per_tensor, uint8_t* q,
                            float* scale, void* stream) {
  int8_t* qq = reinterpret_cast<int8_t*>(q);
  int st = check_rowquant(X, x_dtype, nullptr, rows, K, qq, scale);
  if (st != QMM_OK) return st;
  hipStream_t s = as_stream(stream);
  if (!per_tensor) return launch_rowquant<1, 0, 1>(X, x_dtype, nullptr, rows, K, qq, scale, s);
  st = launch_rowquant<1, 1, 1>(X, x_dtype, nullptr, rows, K, qq, scale, s);
  if (st != QMM_OK) return st;
  tensor_scale_kernel<1><<<1, 256, 0, s>>>(scale, rows);
  st = launch_status();
  if (st != QMM_OK) return st;
  return launch_rowquant<1, 2, 1>(X, x_dtype, nullptr, rows, K, qq, scale, s);
}

extern "C" int fp8_gemm(const uint8_t* qX, const float* x_scale, const uint8_t* qW, const float* w_scale, int64_t M,
                        int64_t N, int64_t K, void* Y, int y_dtype, void* stream) {
  int st = check_fp8_gemm(qX, x_scale, qW, w_scale, M, N, K, Y, y_dtype);
  if (st != QMM_OK) return st;
  launch_gemm_fp8(qX, x_scale, qW, w_scale, M, N, K, Y, y_dtype, as_stream(stream));
  return launch_status();
}

extern "C" int fp8_w8a8_gemm(const void* X, int x_dtype, const uint8_t* qW, const float* w_scale, int64_t M, int64_t N,
                             int64_t K, void* Y, int y_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!X || !qW || !w_scale || !Y) return QMM_EINVAL;
  if (M <= 0 || N <= 0 || K <= 0) return QMM_EINVAL;
  if (!float_dtype(x_dtype)) return x_dtype == QMM_I32 ? QMM_EUNSUPPORTED : QMM_EINVAL;
  if (y_dtype != QMM_BF16 && y_dtype != QMM_F32)
    return (y_dtype == QMM_F16 || y_dtype == QMM_I32) ? QMM_EUNSUPPORTED : QMM_EINVAL;
  if (K % 64 != 0) return QMM_EUNSUPPORTED;
  if (K > kMaxK) return QMM_ERANGE;
  if (!aligned(X, 16) || !aligned(qW, 16) || !aligned(w_scale, 4) || !aligned(Y, 4)) return QMM_EALIGN;
  if (!workspace || workspace_bytes < sq_workspace_bytes(M, K) || !aligned(workspace, 16)) return QMM_EWORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int8_t* qX = reinterpret_cast<int8_t*>(ws);
  float* xs = reinterpret_cast<float*>(ws + (static_cast<size_t>(M) * static_cast<size_t>(K) + 255u) / 256u * 256u);
  hipStream_t s = as_stream(stream);
  int st = launch_rowquant<1, 0, 1>(X, x_dtype, nullptr, M, K, qX, xs, s);
  if (st != QMM_OK) return st;
  launch_gemm_fp8(reinterpret_cast<const uint8_t*>(qX), xs, qW, w_scale, M, N, K, Y, y_dtype, s);
  return launch_status();
}

// ----------------------------------------------------------------------------
// LLM.int8() mixed-precision decomposition ("Quantization" (Engine Room ch.
// 15), "The Mathematics": the vector-wise INT8 product with the outlier
// feature dimensions removed and multiplied in 16-bit, C = S_out (X_q W_q) +
// X_16 W_16; "Quantization: Smaller Weights, Same Answers (Mostly)", the
// first outlier family).  Steps, all on the caller's stream:
//  1. column maxima of |X| (the calibration kernel above, X alone);
//  2. one block walks the columns in order: a column whose maximum reaches
//     the threshold is an outlier dimension; the first `cap` of them get an
//     index and the factor +inf, every other column the factor 1 (written
//     over the maxima);
//  3. the per-token INT8 quantizer with those factors as its smoothing
//     divisors: x / inf = 0, so the outlier columns are zero in X_q and take
//     no part in a token's absmax, while x / 1 = x leaves the rest unchanged;
//  4. the INT8 GEMM: each block fetches its rows' outlier activations and its
//     columns' 16-bit outlier weights (the INT8 weight times its channel
//     scale, rounded to the activations' type) at its start, and its epilogue
//     adds the outlier product before rounding.
// ----------------------------------------------------------------------------
namespace qmm {
namespace {

constexpr int kSelThreads = 1024;

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

// One block.  Chunk of 1024 columns: a ballot per wavefront ranks the
// outliers inside it, the wavefront counts in LDS give each wavefront's
// offset, and `base` carries the count of the chunks before.  The maxima of
// four chunks are loaded together (one memory round trip per 4096 columns).
__global__ __launch_bounds__(kSelThreads) void outlier_select_kernel(float* __restrict__ cx_factor, int64_t K,
                                                                     float tau, int64_t cap,
                                                                     int32_t* __restrict__ idx,
                                                                     int32_t* __restrict__ counts,
                                                                     int32_t* __restrict__ found_out) {
  constexpr int kWaves = kSelThreads / kWave;
  constexpr int kBatch = 4;
  __shared__ int wsum[kWaves];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  int64_t base = 0;
  for (int64_t b0 = 0; b0 < K; b0 += kBatch * kSelThreads) {
    float v[kBatch];
#pragma unroll
    for (int c = 0; c < kBatch; ++c) {
      const int64_t j = b0 + c * kSelThreads + threadIdx.x;
      v[c] = j < K ? cx_factor[j] : 0.0f;
    }
#pragma unroll
    for (int c = 0; c < kBatch; ++c) {
      const int64_t j = b0 + c * kSelThreads + threadIdx.x;
      const bool in = j < K;
      const bool flag = in && v[c] >= tau;
      const uint64_t mask = __ballot(flag);
      const int below = __popcll(mask & ((1ull << lane) - 1ull));
      if (lane == 0) wsum[wave] = __popcll(mask);
      __syncthreads();
      int before = 0, total = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const int cnt = wsum[w];
        total += cnt;
        before += (w < wave) ? cnt : 0;
      }
      const int64_t rank = base + before + below;
      const bool keep = flag && rank < cap;
      if (keep) idx[rank] = static_cast<int32_t>(j);
      if (in) cx_factor[j] = keep ? __builtin_inff() : 1.0f;
      base += total;
      __syncthreads();   // wsum is rewritten by the next chunk
    }
  }
  if (threadIdx.x == 0) {
    counts[0] = static_cast<int32_t>(base < cap ? base : cap);
    counts[1] = static_cast<int32_t>(base);
    if (found_out) *found_out = static_cast<int32_t>(base);
  }
}

// Workspace of the LLM.int8() call, every part at a 256-byte boundary.
struct LlmLayout {
  size_t qx, xs, factor, idx, counts, total;
};

LlmLayout llm_layout(int64_t M, int64_t K, int64_t cap) {
  auto up = [](size_t b) { return (b + 255u) / 256u * 256u; };
  const size_t m = static_cast<size_t>(M), k = static_cast<size_t>(K), c = static_cast<size_t>(cap);
  LlmLayout L;
  size_t off = 0;
  L.qx = off;     off += up(m * k);
  L.xs = off;     off += up(m * 4u);
  L.factor = off; off += up(k * 4u);
  L.idx = off;    off += up((c > 0 ? c : 1u) * 4u);
  L.counts = off; off += 256u;
  L.total = off;
  return L;
}

int check_llm(const void* X, int x_dtype, int64_t M, int64_t K, float tau, int64_t cap) {
  if (!X) return QMM_EINVAL;
  if (M <= 0 || K <= 0 || cap < 0) return QMM_EINVAL;
  if (x_dtype != QMM_BF16 && x_dtype != QMM_F16) return x_dtype == QMM_F32 ? QMM_EUNSUPPORTED : QMM_EINVAL;
  if (!(tau >= 0.0f)) return QMM_EINVAL;
  if (K % 64 != 0) return QMM_EUNSUPPORTED;
  if (K > kMaxK) return QMM_ERANGE;
  if (!aligned(X, 16)) return QMM_EALIGN;
  return QMM_OK;
}

// Steps 1 and 2: factor [K] (1 or +inf), idx [cap], counts {kept, found}.
int llm_select(const void* X, int x_dtype, int64_t M, int64_t K, float tau, int64_t cap, float* factor,
               int32_t* idx, int32_t* counts, int32_t* found_out, hipStream_t s) {
  uint32_t* cx = reinterpret_cast<uint32_t*>(factor);
  fill_zero_kernel<<<static_cast<unsigned>(ceil_div(K, 256)), 256, 0, s>>>(cx, K);
  const int64_t bands = ceil_div(M, kCmBand);
  const dim3 grid(static_cast<unsigned>(ceil_div(K, kCmCols)), static_cast<unsigned>(bands));
  const uint8_t* xp = static_cast<const uint8_t*>(X);
  if (x_dtype == QMM_BF16) colmax2_kernel<QMM_BF16, QMM_BF16><<<grid, 256, 0, s>>>(xp, M, xp, 0, K, bands, cx, cx);
  else colmax2_kernel<QMM_F16, QMM_F16><<<grid, 256, 0, s>>>(xp, M, xp, 0, K, bands, cx, cx);
  outlier_select_kernel<<<1, kSelThreads, 0, s>>>(factor, K, tau, cap, idx, counts, found_out);
  return launch_status();
}

}  // namespace
}  // namespace qmm

extern "C" int llm_int8_outliers(const void* X, int x_dtype, int64_t M, int64_t K, float threshold,
                                 int64_t max_outliers, float* factor, int32_t* index, int32_t* counts,
                                 void* stream) {
  int st = check_llm(X, x_dtype, M, K, threshold, max_outliers);
  if (st != QMM_OK) return st;
  if (!factor || !index || !counts) return QMM_EINVAL;
  if (!aligned(factor, 4) || !aligned(index, 4) || !aligned(counts, 4)) return QMM_EALIGN;
  const int64_t cap = max_outliers < K ? max_outliers : K;
  return llm_select(X, x_dtype, M, K, threshold, cap, factor, index, counts, nullptr, as_stream(stream));
}

extern "C" size_t llm_int8_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t max_outliers) {
  if (M <= 0 || N <= 0 || K <= 0 || max_outliers < 0) return 0;
  return llm_layout(M, K, max_outliers < K ? max_outliers : K).total;
}

extern "C" int llm_int8_gemm(const void* X, int x_dtype, const int8_t* qW, const float* w_scale, int64_t M, int64_t N,
                             int64_t K, float threshold, int64_t max_outliers, void* Y, int y_dtype,
                             int32_t* n_outliers, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_llm(X, x_dtype, M, K, threshold, max_outliers);
  if (st != QMM_OK) return st;
  if (!qW || !w_scale || !Y || N <= 0) return QMM_EINVAL;
  if (y_dtype != QMM_BF16 && y_dtype != QMM_F32)
    return (y_dtype == QMM_F16 || y_dtype == QMM_I32) ? QMM_EUNSUPPORTED : QMM_EINVAL;
  if (!aligned(qW, 16) || !aligned(w_scale, 4) || !aligned(Y, 4) || (n_outliers && !aligned(n_outliers, 4)))
    return QMM_EALIGN;
  const int64_t cap = max_outliers < K ? max_outliers : K;
  const LlmLayout L = llm_layout(M, K, cap);
  if (!workspace || workspace_bytes < L.total || !aligned(workspace, 16)) return QMM_EWORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int8_t* qX = reinterpret_cast<int8_t*>(ws + L.qx);
  float* xs = reinterpret_cast<float*>(ws + L.xs);
  float* factor = reinterpret_cast<float*>(ws + L.factor);
  int32_t* idx = reinterpret_cast<int32_t*>(ws + L.idx);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  hipStream_t s = as_stream(stream);
  st = llm_select(X, x_dtype, M, K, threshold, cap, factor, idx, counts, n_outliers, s);
  if (st != QMM_OK) return st;
  st = launch_rowquant<1>(X, x_dtype, factor, M, K, qX, xs, s);
  if (st != QMM_OK) return st;
  const Outliers outl{counts, idx, static_cast<const uint16_t*>(X), x_dtype == QMM_F16 ? 1 : 0};
  if (y_dtype == QMM_F32) launch_gemm_t<QMM_F32, false, true>(qX, xs, qW, w_scale, M, N, K, Y, s, outl);
  else launch_gemm_t<QMM_BF16, false, true>(qX, xs, qW, w_scale, M, N, K, Y, s, outl);
  return launch_status();
}
