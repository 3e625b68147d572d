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

#include "qmm_device.h"

namespace qmm {
namespace {

constexpr float kQ8 = 127.0f;
constexpr float kAbsFloor = 1e-8f;
constexpr float kSmoothFloor = 1e-5f;
// Largest K (a multiple of 64) with 128 * 128 * K < 2^31: no int32 sum can overflow.
constexpr int64_t kMaxK = 131008;

// ----------------------------------------------------------------------------
// Column absolute maxima (calibration statistics).  Thread = 8 consecutive
// columns of a band of rows; one atomicMax per column per thread on the
// float's bit pattern (non-negative floats order like unsigned integers).
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

template <int DT>
__device__ __forceinline__ void colmax_band(const uint8_t* __restrict__ a, int64_t rows, int64_t cols, int64_t col8,
                                            int64_t r0, int64_t r1, uint32_t* __restrict__ out) {
  constexpr int kElem = DT == QMM_F32 ? 4 : 2;
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int64_t r = r0; r < r1; ++r) {
    float v[8];
    Vec8<DT>::load(a + (r * cols + col8) * kElem, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) m[i] = fmaxf(m[i], fabsf(v[i]));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) atomicMax(out + col8 + i, __float_as_uint(m[i]));
}

// grid.x: column blocks of 2048; grid.y: row bands of the two matrices
// (first `bands_x` bands belong to X, the rest to W).
template <int XDT, int WDT>
__global__ __launch_bounds__(256) void colmax2_kernel(const uint8_t* __restrict__ X, int64_t M,
                                                      const uint8_t* __restrict__ W, int64_t N, int64_t K,
                                                      int64_t band, int64_t bands_x, uint32_t* __restrict__ cx,
                                                      uint32_t* __restrict__ cw) {
  const int64_t col8 = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 8;
  if (col8 >= K) return;
  const int64_t yb = blockIdx.y;
  if (yb < bands_x) {
    const int64_t r0 = yb * band, r1 = (r0 + band < M) ? r0 + band : M;
    colmax_band<XDT>(X, M, K, col8, r0, r1, cx);
  } else {
    const int64_t r0 = (yb - bands_x) * band, r1 = (r0 + band < N) ? r0 + band : N;
    colmax_band<WDT>(W, N, K, col8, r0, r1, cw);
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
// divides (activations); smooth == nullptr skips the smoothing.  The row is
// processed in 8-element slices, twice: pass 1 finds the absmax of the
// smoothed row, pass 2 recomputes the same smoothed values and quantizes.
// CH slices per lane are kept in registers between the passes when the row
// fits (K <= 512 * CH), otherwise pass 2 re-reads the row.
// ----------------------------------------------------------------------------
template <int MODE>
__device__ __forceinline__ float smooth_op(float v, const float* smooth, int64_t k) {
  if (smooth == nullptr) return v;
  const float sj = smooth[k];
  return MODE == 0 ? v * sj : v / sj;
}

template <int DT, int MODE, int CH>
__global__ __launch_bounds__(256) void rowquant8_kernel(const uint8_t* __restrict__ a, const float* __restrict__ smooth,
                                                        int64_t rows, int64_t K, int8_t* __restrict__ q,
                                                        float* __restrict__ scale) {
  constexpr int kElem = DT == QMM_F32 ? 4 : 2;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (row >= rows) return;
  const uint8_t* arow = a + row * K * kElem;
  const bool resident = K <= static_cast<int64_t>(kWave) * 8 * CH;

  float keep[CH][8];
  float amax = 0.0f;
  int ch = 0;
  for (int64_t k = static_cast<int64_t>(lane) * 8; k < K; k += kWave * 8, ++ch) {
    float v[8];
    Vec8<DT>::load(arow + k * kElem, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = smooth_op<MODE>(v[i], smooth, k + i);
      amax = fmaxf(amax, fabsf(v[i]));
    }
    if (resident) {
#pragma unroll
      for (int c = 0; c < CH; ++c)
        if (c == ch) {
#pragma unroll
          for (int i = 0; i < 8; ++i) keep[c][i] = v[i];
        }
    }
  }
  amax = wave_max(amax);
  const float s = fmaxf(amax, kAbsFloor) / kQ8;
  if (lane == 0) scale[row] = s;

  ch = 0;
  for (int64_t k = static_cast<int64_t>(lane) * 8; k < K; k += kWave * 8, ++ch) {
    float v[8];
    if (resident) {
#pragma unroll
      for (int c = 0; c < CH; ++c)
        if (c == ch) {
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = keep[c][i];
        }
    } else {
      Vec8<DT>::load(arow + k * kElem, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = smooth_op<MODE>(v[i], smooth, k + i);
    }
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float t = __builtin_amdgcn_fmed3f(rintf(v[i] / s), -128.0f, kQ8);
      const uint32_t b = static_cast<uint32_t>(static_cast<int32_t>(t)) & 0xFFu;
      if (i < 4) lo |= b << (8 * i);
      else hi |= b << (8 * (i - 4));
    }
    *reinterpret_cast<uint2*>(q + row * K + k) = make_uint2(lo, hi);
  }
}

// ----------------------------------------------------------------------------
// INT8 GEMM on v_mfma_i32_16x16x64_i8: C[m, n] = sum_k A[m, k] B[n, k], exact
// in int32.  Block tile 256 x 128, k-step 128 (two 64-wide MFMA chunks), four
// wavefronts of 128 x 64 (8 x 4 instructions per chunk; 128 int32
// accumulators per lane).  Operand layout (16x16x64): lane l supplies row
// l%16 of A (column l%16 of B) and k = 16*(l/16) .. +16; D lane l holds rows
// 4*(l/16) .. +4 of column l%16.
//
// LDS layout: for each 64-wide chunk, each 16-row slice is stored
// fragment-major, [k-part (4)][row (16)][16 bytes], so the 16-byte fragment of
// lane l sits at slice_base + 16*l.  The cooperative global->LDS copy uses the
// same order (copy vector v lands at byte 16*v), so LDS stores and fragment
// reads are lane-linear and free of bank conflicts, while each copy
// instruction still reads 16 rows x 64 contiguous bytes of global memory.
//
// Pipeline: two k-steps of LDS and two register sets.  During step t the
// MFMAs read LDS buffer t%2 while the global loads of step t+2 are in flight;
// the registers of step t+1 (issued one step earlier) are then written to the
// other LDS buffer, so every load has two k-steps of MFMA work to arrive.
// Tiles are ordered so that the blocks sharing an XCD (block id mod 8) cover a
// compact 4 x 8 patch of the output and reuse A and B rows in that XCD's L2.
// Epilogue: Y = acc * a[m] * b[n] in fp32 (or the raw int32 accumulator).
// ----------------------------------------------------------------------------
constexpr int kBM = 256, kBN = 128, kBK = 128;
constexpr int kAVec = kBM * kBK / 16 / 256;   // 16-byte copy vectors per thread per step: 8
constexpr int kBVec = kBN * kBK / 16 / 256;   // 4
constexpr int kStageA = kBM * kBK;             // bytes per LDS stage
constexpr int kStageB = kBN * kBK;
constexpr size_t kGemmLds = 2 * (kStageA + kStageB);   // 96 KiB
constexpr int kXcds = 8;

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

// Copy vector v of a k-step over R rows: 64-wide chunk h = v / (4R), slice
// (v % 4R) / 64, row slice*16 + v%16, 16-byte part (v/16)%4.  Returns the
// global offset from the tile's first row at k = 0 without the chunk's 64*h
// (added at load time, where h is a compile-time constant).
__device__ __forceinline__ uint32_t copy_offset(int v, int vecs_per_chunk, int rmax, int kk) {
  const int rem = v % vecs_per_chunk;
  const int row = min((rem >> 6) * 16 + (rem & 15), rmax);
  return static_cast<uint32_t>(row * kk + ((rem >> 4) & 3) * 16);
}

template <int YDT>
__global__ __launch_bounds__(256) void i8_gemm_kernel(const int8_t* __restrict__ A, const float* __restrict__ ascale,
                                                      const int8_t* __restrict__ B, const float* __restrict__ bscale,
                                                      int64_t M, int64_t N, int64_t K, void* __restrict__ Y) {
  extern __shared__ __attribute__((aligned(16))) int8_t lds[];
  // LDS: A stages at [0, 2*kStageA), B stages after them.
  int8_t* const sb0 = lds + 2 * kStageA;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = (wave & 1) * 128;   // wavefront sub-tile origin
  const int wn = (wave >> 1) * 64;
  int64_t mt, nt;
  bool valid;
  xcd_tile(blockIdx.x, (M + kBM - 1) / kBM, (N + kBN - 1) / kBN, &mt, &nt, &valid);
  if (!valid) return;
  const int64_t m0 = mt * kBM;
  const int64_t n0 = nt * kBN;
  const int kk = static_cast<int>(K);

  // Rows past M / N re-read the last valid row (their results are never stored).
  const int8_t* abase = A + m0 * K;
  const int8_t* bbase = B + n0 * K;
  const int amax = static_cast<int>((M - 1 - m0 < kBM - 1) ? M - 1 - m0 : kBM - 1);
  const int bmax = static_cast<int>((N - 1 - n0 < kBN - 1) ? N - 1 - n0 : kBN - 1);
  uint32_t aoff[kAVec], boff[kBVec];
#pragma unroll
  for (int j = 0; j < kAVec; ++j) aoff[j] = copy_offset(tid + 256 * j, kBM * 4, amax, kk);
#pragma unroll
  for (int j = 0; j < kBVec; ++j) boff[j] = copy_offset(tid + 256 * j, kBN * 4, bmax, kk);

  i32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

  u32x4 ra[2][kAVec], rb[2][kBVec];
  // When K % 128 == 64 the second chunk of the last step lies past K: it
  // re-reads the first chunk (in bounds) and its MFMAs are skipped.
  auto gload = [&](int set, int step) {
    const uint32_t k0 = static_cast<uint32_t>(step * kBK);
    const uint32_t k1 = (k0 + 64 < static_cast<uint32_t>(kk)) ? k0 + 64 : k0;
#pragma unroll
    for (int j = 0; j < kAVec; ++j) ra[set][j] = ld16(abase + aoff[j] + (j < kAVec / 2 ? k0 : k1));
#pragma unroll
    for (int j = 0; j < kBVec; ++j) rb[set][j] = ld16(bbase + boff[j] + (j < kBVec / 2 ? k0 : k1));
  };
  auto lstore = [&](int set, int buf) {
#pragma unroll
    for (int j = 0; j < kAVec; ++j) *reinterpret_cast<u32x4*>(lds + buf * kStageA + (tid + 256 * j) * 16) = ra[set][j];
#pragma unroll
    for (int j = 0; j < kBVec; ++j) *reinterpret_cast<u32x4*>(sb0 + buf * kStageB + (tid + 256 * j) * 16) = rb[set][j];
  };

  const int nsteps = (kk + kBK - 1) / kBK;
  const int last_chunks = (kk % kBK) ? 1 : 2;
  gload(0, 0);
  gload(1, min(1, nsteps - 1));
  lstore(0, 0);
  __syncthreads();

  // One k-step on LDS buffer / register set `cur`; called with a literal so
  // the register-set index is a compile-time constant after inlining.
  auto kstep = [&](const int cur, const int t) {
    // Set `cur` held step t, already in LDS.  Loads and stores are issued on
    // every step (past the end they repeat the last step, in bounds, and are
    // never read) so that the number of loads in flight is the same at every
    // wait and the compiler's wait counts stay exact.
    gload(cur, min(t + 2, nsteps - 1));
    const int chunks = (t + 1 < nsteps) ? 2 : last_chunks;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h >= chunks) break;
      const int8_t* a_h = lds + cur * kStageA + h * (kBM * 64);
      const int8_t* b_h = sb0 + cur * kStageB + h * (kBN * 64);
      i32x4 fa[8], fb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[j] = *reinterpret_cast<const i32x4*>(b_h + ((wn >> 4) + j) * 1024 + lane * 16);
#pragma unroll
      for (int i = 0; i < 8; ++i) fa[i] = *reinterpret_cast<const i32x4*>(a_h + ((wm >> 4) + i) * 1024 + lane * 16);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    lstore(cur ^ 1, cur ^ 1);   // step t+1 (loaded during step t-1)
    __syncthreads();
  };
  // Pairs of steps, then an odd last step outside the loop: no path leaves
  // the loop body half way, so every iteration starts with the same loads in
  // flight.
  int t = 0;
  for (; t + 1 < nsteps; t += 2) {
    kstep(0, t);
    kstep(1, t + 1);
  }
  if (t < nsteps) kstep(0, t);

  // D tile (i, j): rows m0 + wm + 16i + 4*(lane/16) + r, column n0 + wn + 16j + lane%16.
  const int l16 = lane & 15;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = n0 + wn + 16 * j + l16;
    if (n >= N) continue;
    float bs = 1.0f;
    if constexpr (YDT != QMM_I32) bs = bscale[n];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm + 16 * i + 4 * (lane >> 4) + r;
        if (m >= M) continue;
        const int32_t v = acc[i][j][r];
        if constexpr (YDT == QMM_I32) {
          static_cast<int32_t*>(Y)[m * N + n] = v;
        } else {
          const float f = static_cast<float>(v) * ascale[m] * bs;
          if constexpr (YDT == QMM_F32) static_cast<float*>(Y)[m * N + n] = f;
          else static_cast<uint16_t*>(Y)[m * N + n] = static_cast<uint16_t>(f32_to_bf16_bits(f));
        }
      }
    }
  }
}

bool float_dtype(int dt) { return dt == QMM_F32 || dt == QMM_BF16 || dt == QMM_F16; }

template <int MODE>
int launch_rowquant(const void* a, int dt, const float* smooth, int64_t rows, int64_t K, int8_t* q, float* scale,
                    hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(ceil_div(rows, 4)));
  const dim3 block(256);
  const uint8_t* p = static_cast<const uint8_t*>(a);
  switch (dt) {
    case QMM_BF16: rowquant8_kernel<QMM_BF16, MODE, 8><<<grid, block, 0, s>>>(p, smooth, rows, K, q, scale); break;
    case QMM_F16: rowquant8_kernel<QMM_F16, MODE, 8><<<grid, block, 0, s>>>(p, smooth, rows, K, q, scale); break;
    default: rowquant8_kernel<QMM_F32, MODE, 8><<<grid, block, 0, s>>>(p, smooth, rows, K, q, scale); break;
  }
  return launch_status();
}

int check_rowquant(const void* a, int dt, const float* smooth, int64_t rows, int64_t K, const int8_t* q,
                   const float* scale) {
  if (!a || !q || !scale) return QMM_EINVAL;
  if (rows <= 0 || K <= 0) return QMM_EINVAL;
  if (!float_dtype(dt)) return dt == QMM_I32 ? QMM_EUNSUPPORTED : QMM_EINVAL;
  if (K % 64 != 0) return QMM_EUNSUPPORTED;
  if (!aligned(a, 16) || !aligned(q, 16) || !aligned(scale, 4) || (smooth && !aligned(smooth, 4)))
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

template <int YDT>
void launch_gemm_t(const int8_t* qX, const float* xs, const int8_t* qW, const float* ws, int64_t M, int64_t N,
                   int64_t K, void* Y, hipStream_t s) {
  // 96 KiB of dynamic LDS; the attribute is cheap to set and idempotent, so it
  // is set on every launch (no per-device bookkeeping).
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&i8_gemm_kernel<YDT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kGemmLds));
  const int64_t tiles = ceil_div(M, kBM) * ceil_div(N, kBN);
  const dim3 grid(static_cast<unsigned>(ceil_div(tiles, kXcds) * kXcds));
  i8_gemm_kernel<YDT><<<grid, dim3(256), kGemmLds, s>>>(qX, xs, qW, ws, M, N, K, Y);
}

void launch_gemm(const int8_t* qX, const float* xs, const int8_t* qW, const float* ws, int64_t M, int64_t N,
                 int64_t K, void* Y, int ydt, hipStream_t s) {
  switch (ydt) {
    case QMM_I32: launch_gemm_t<QMM_I32>(qX, xs, qW, ws, M, N, K, Y, s); break;
    case QMM_F32: launch_gemm_t<QMM_F32>(qX, xs, qW, ws, M, N, K, Y, s); break;
    default: launch_gemm_t<QMM_BF16>(qX, xs, qW, ws, M, N, K, Y, s); break;
  }
}

}  // namespace
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
  fill_zero_kernel<<<fill_blocks, 256, 0, s>>>(cx, K);
  fill_zero_kernel<<<fill_blocks, 256, 0, s>>>(cw, K);
  const int64_t band = 32;
  const int64_t bands_x = ceil_div(M, band);
  const int64_t bands_w = ceil_div(N, band);
  const dim3 grid(static_cast<unsigned>(ceil_div(K, 2048)), static_cast<unsigned>(bands_x + bands_w));
  const uint8_t* xp = static_cast<const uint8_t*>(X);
  const uint8_t* wp = static_cast<const uint8_t*>(W);
#define QMM_COLMAX(XD, WD) colmax2_kernel<XD, WD><<<grid, 256, 0, s>>>(xp, M, wp, N, K, band, bands_x, cx, cw)
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

extern "C" int smooth_quant_w8a8_gemm(const void* X, int x_dtype, const float* smooth, const int8_t* qW,
                                      const float* w_scale, int64_t M, int64_t N, int64_t K, void* Y, int y_dtype,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!X || !qW || !w_scale || !Y) return QMM_EINVAL;
  if (M <= 0 || N <= 0 || K <= 0) return QMM_EINVAL;
  if (!float_dtype(x_dtype)) return x_dtype == QMM_I32 ? QMM_EUNSUPPORTED : QMM_EINVAL;
  if (y_dtype != QMM_BF16 && y_dtype != QMM_F32 && y_dtype != QMM_I32)
    return y_dtype == QMM_F16 ? QMM_EUNSUPPORTED : QMM_EINVAL;
  if (K % 64 != 0) return QMM_EUNSUPPORTED;
  if (K > kMaxK) return QMM_ERANGE;
  if (!workspace || workspace_bytes < sq_workspace_bytes(M, K) || !aligned(workspace, 16)) return QMM_EWORKSPACE;
  if (!aligned(X, 16) || !aligned(qW, 16) || !aligned(w_scale, 4) || !aligned(Y, 4) ||
      (smooth && !aligned(smooth, 4)))
    return QMM_EALIGN;
  int8_t* qX = static_cast<int8_t*>(workspace);
  float* xs = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                       (static_cast<size_t>(M) * static_cast<size_t>(K) + 255u) / 256u * 256u);
  hipStream_t s = as_stream(stream);
  int st = launch_rowquant<1>(X, x_dtype, smooth, M, K, qX, xs, s);
  if (st != QMM_OK) return st;
  launch_gemm(qX, xs, qW, w_scale, M, N, K, Y, y_dtype, s);
  return launch_status();
}
