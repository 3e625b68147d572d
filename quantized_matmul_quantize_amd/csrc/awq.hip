// awq.hip -- AWQ's activation-aware scaling search on the GPU.
//
// Source: "Quantization from Scratch: Scale, Zero-Point, GPTQ and AWQ", "AWQ:
// protect the channels that matter" and the awq listing after it: a few input
// channels carry much larger activations, so the weights they multiply are
// scaled up before quantization and the inputs down by the same factor,
// W x = (W diag(s)) (diag(s)^-1 x); s_j = mean|x_j|^alpha, normalized by
// sqrt(max s * min s), with one alpha per layer kept from a grid by the
// calibration output error.
//
// For every alpha of the grid (the loop runs on the host, the choice on the
// device, so nothing waits for the host):
//   s      = mag^alpha / sqrt(max * min), fp64, stored in fp32 (all alphas
//            at once, before the loop);
//   codes  = group-128 INT4 of fl32(W diag(s)), the product formed inside
//            the quantizer (no fp32 copy of the scaled weights);
//   X_s    = fl32(X / s) rounded to X's 16-bit type, bf16 or binary16
//            (the inverse scaling folded into the input);
//   Y_q    = w4a16_gemm(X_s, codes);
//   err    = sum (X W^T - Y_q)^2 in fp64, X W^T once by the 16-bit product;
// then the first alpha of the smallest error is selected, and W diag(s_best)
// quantized into the caller's format buffers.  mag_j = max(mean_t |x_j|,
// 1e-8) in fp64: the sum of |x| over the tokens is taken over slices of 32
// rows and the slices in order; it is exact (so equal to any other order's)
// while each channel's nonzero |x| span less than 2^(42 - log2 T) in ratio
// (16-bit values carry at most 11 significant bits, fp64 53), true of any
// activations with an ordinary dynamic range.

#include "qmm_device.h"

namespace qmm {
namespace {

constexpr int kMagRows = 32;       // rows per partial sum of the channel magnitudes
constexpr int kErrBlocks = 1024;   // partial sums of one squared error
constexpr int kMaxAlphas = 64;

// The alpha grid, passed by value (a kernel argument of 512 bytes).
struct AlphaGrid {
  double a[kMaxAlphas];
};

// The two 16-bit halves of a word as fp32 (XDT: QMM_BF16 or QMM_F16).
template <int XDT>
__device__ __forceinline__ float h16_lo(uint32_t w) {
  if constexpr (XDT == QMM_F16) return f16lo_to_f32(w);
  else return bf16lo_to_f32(w);
}
template <int XDT>
__device__ __forceinline__ float h16_hi(uint32_t w) {
  if constexpr (XDT == QMM_F16) return f16hi_to_f32(w);
  else return bf16hi_to_f32(w);
}

// fl32 v rounded to the 16-bit type (nearest even; binary16 saturating at its
// largest finite value), as bits in the low half.
template <int XDT>
__device__ __forceinline__ uint32_t h16_bits(float v) {
  if constexpr (XDT == QMM_F16) return f32_to_f16_bits(__builtin_amdgcn_fmed3f(v, -65504.0f, 65504.0f));
  else return f32_to_bf16_bits(v);
}

// Partial sums of |x| over rows [kMagRows b, +kMagRows) of each column,
// fp64; a thread takes 8 consecutive columns (one 16-byte load per row).
template <int XDT>
__global__ __launch_bounds__(256) void awq_mag_partial_kernel(const uint16_t* __restrict__ x, int64_t T, int64_t K,
                                                              double* __restrict__ part) {
  const int64_t j0 = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 8;
  if (j0 >= K) return;
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * kMagRows;
  const int64_t r1 = (r0 + kMagRows < T) ? r0 + kMagRows : T;
  double acc[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  for (int64_t r = r0; r < r1; r += 8) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = (r + u < r1) ? ld16(x + (r + u) * K + j0) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        acc[2 * h] += static_cast<double>(fabsf(h16_lo<XDT>(w[h])));
        acc[2 * h + 1] += static_cast<double>(fabsf(h16_hi<XDT>(w[h])));
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) part[blockIdx.y * K + j0 + c] = acc[c];
}

// mag_j = max(sum of the partial sums in order / T, 1e-8).
__global__ __launch_bounds__(256) void awq_mag_kernel(const double* __restrict__ part, int64_t slices, int64_t T,
                                                      int64_t K, double* __restrict__ mag) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (j >= K) return;
  double acc = 0.0;
  for (int64_t b = 0; b < slices; b += 8) {   // eight loads in flight, then their sums in order
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = (b + u < slices) ? part[(b + u) * K + j] : 0.0;
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  const double m = acc / static_cast<double>(T);
  mag[j] = m < 1e-8 ? 1e-8 : m;
}

// Block (b, a): p_j = mag_j^alpha_a for its 256 columns, and the block's max
// and min of p.
__global__ __launch_bounds__(256) void awq_pow_kernel(const double* __restrict__ mag, int64_t K, AlphaGrid alphas,
                                                      double* __restrict__ pbuf, double* __restrict__ bmax,
                                                      double* __restrict__ bmin) {
  __shared__ double smax[256], smin[256];
  const int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  double mx = 0.0, mn = INFINITY;
  if (j < K) {
    const double pj = pow(mag[j], alphas.a[blockIdx.y]);
    pbuf[blockIdx.y * K + j] = pj;
    mx = pj;
    mn = pj;
  }
  smax[threadIdx.x] = mx;
  smin[threadIdx.x] = mn;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {   // max and min are exact in any order
    if (static_cast<int>(threadIdx.x) < o) {
      smax[threadIdx.x] = fmax(smax[threadIdx.x], smax[threadIdx.x + o]);
      smin[threadIdx.x] = fmin(smin[threadIdx.x], smin[threadIdx.x + o]);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    bmax[blockIdx.y * gridDim.x + blockIdx.x] = smax[0];
    bmin[blockIdx.y * gridDim.x + blockIdx.x] = smin[0];
  }
}

// One block per alpha: norm = sqrt(max p * min p) over the blocks' extremes.
__global__ __launch_bounds__(256) void awq_norm_kernel(const double* __restrict__ bmax, const double* __restrict__ bmin,
                                                       int64_t nb, double* __restrict__ norm) {
  __shared__ double smax[256], smin[256];
  double mx = 0.0, mn = INFINITY;
  for (int64_t b = threadIdx.x; b < nb; b += blockDim.x) {
    mx = fmax(mx, bmax[blockIdx.x * nb + b]);
    mn = fmin(mn, bmin[blockIdx.x * nb + b]);
  }
  smax[threadIdx.x] = mx;
  smin[threadIdx.x] = mn;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (static_cast<int>(threadIdx.x) < o) {
      smax[threadIdx.x] = fmax(smax[threadIdx.x], smax[threadIdx.x + o]);
      smin[threadIdx.x] = fmin(smin[threadIdx.x], smin[threadIdx.x + o]);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) norm[blockIdx.x] = sqrt(smax[0] * smin[0]);
}

// s[a, j] = fl32(p[a, j] / norm[a]).
__global__ __launch_bounds__(256) void awq_factor_kernel(const double* __restrict__ pbuf,
                                                         const double* __restrict__ norm, int64_t K,
                                                         float* __restrict__ s_all) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (j < K) s_all[blockIdx.y * K + j] = static_cast<float>(pbuf[blockIdx.y * K + j] / norm[blockIdx.y]);
}

// X_s = h16(fl32(X / s)) in X's own 16-bit type, correctly rounded division,
// eight values per thread.  Also the per-group sums of the rounded outputs, xsum[t][g] (fp32), for
// the products' zero-point term: the 16 lanes of a group (consecutive
// threads, 8 values each) add their sums by a fixed butterfly.  The thread
// count and the grid stride are multiples of 16 and K of 128, so a group's
// lanes are always active together.
template <int XDT>
__global__ __launch_bounds__(256) void awq_scale_x_kernel(const uint16_t* __restrict__ x, const float* __restrict__ s,
                                                          int64_t total8, int64_t K, uint16_t* __restrict__ out,
                                                          float* __restrict__ xsum) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total8;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t e = i * 8;
    const int64_t j = e % K;
    const u32x4 v = ld16(x + e);
    const uint32_t a[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
    float sum = 0.0f;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float lo = h16_lo<XDT>(a[h]) / s[j + 2 * h];
      const float hi = h16_hi<XDT>(a[h]) / s[j + 2 * h + 1];
      o[h] = h16_bits<XDT>(lo) | (h16_bits<XDT>(hi) << 16);
      sum += h16_lo<XDT>(o[h]);
      sum += h16_hi<XDT>(o[h]);
    }
    *reinterpret_cast<u32x4*>(out + e) = u32x4{o[0], o[1], o[2], o[3]};
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) sum += __shfl_xor(sum, m, kWave);
    if ((i & 15) == 0) xsum[e / kGroup] = sum;   // [t][g] = element e / 128 of the row-major sums
  }
}

// Partial sums of (a - b)^2 in fp64: block b takes a fixed contiguous range
// (a multiple of 4 elements long, so 16-byte aligned), each thread four
// consecutive elements at a fixed stride within it, and the block tree is
// fixed, so the result does not depend on scheduling.
__global__ __launch_bounds__(256) void awq_sqerr_kernel(const float* __restrict__ a, const float* __restrict__ b,
                                                        int64_t n, double* __restrict__ part) {
  __shared__ double red[256];
  const int64_t per = (n + 4 * gridDim.x - 1) / (4 * gridDim.x) * 4;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t i1 = (i0 + per < n) ? i0 + per : n;
  double acc = 0.0;
  for (int64_t i = i0 + 4 * threadIdx.x; i < i1; i += 4 * blockDim.x) {
    if (i + 4 <= i1) {
      const f32x4 va = *reinterpret_cast<const f32x4*>(a + i);
      const f32x4 vb = *reinterpret_cast<const f32x4*>(b + i);
      const double d0 = static_cast<double>(va.x) - static_cast<double>(vb.x);
      const double d1 = static_cast<double>(va.y) - static_cast<double>(vb.y);
      const double d2 = static_cast<double>(va.z) - static_cast<double>(vb.z);
      const double d3 = static_cast<double>(va.w) - static_cast<double>(vb.w);
      acc += d0 * d0;
      acc += d1 * d1;
      acc += d2 * d2;
      acc += d3 * d3;
    } else {
      for (int64_t e = i; e < i1; ++e) {
        const double d = static_cast<double>(a[e]) - static_cast<double>(b[e]);
        acc += d * d;
      }
    }
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (static_cast<int>(threadIdx.x) < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

// err[a] = the partial sums of alpha a by one fixed order: wavefront w
// takes alphas w, w + 16, ..; its lane l sums partials l, l + 64, .. in turn,
// then the 64 lane sums are added by a fixed butterfly.  best = the first
// alpha of the smallest error; s_best = its factors, into the caller's buffer
// and the workspace copy the final quantization reads.
__global__ __launch_bounds__(kErrBlocks) void awq_select_kernel(const double* __restrict__ part, int n_alpha,
                                                                const float* __restrict__ s_all, int64_t K,
                                                                double* __restrict__ err, int64_t* __restrict__ best,
                                                                float* __restrict__ s_best,
                                                                float* __restrict__ s_copy) {
  __shared__ double e_s[kMaxAlphas];
  __shared__ int b_s;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  constexpr int kWaves = kErrBlocks / kWave;
  for (int a = wave; a < n_alpha; a += kWaves) {
    double v = 0.0;
    for (int b = lane; b < kErrBlocks; b += kWave) v += part[a * kErrBlocks + b];
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);   // every lane ends with the same sum
    if (lane == 0) {
      e_s[a] = v;
      err[a] = v;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int bi = 0;
    for (int a = 1; a < n_alpha; ++a)
      if (e_s[a] < e_s[bi]) bi = a;
    b_s = bi;
    *best = bi;
  }
  __syncthreads();
  for (int64_t j = threadIdx.x; j < K; j += blockDim.x) {
    const float v = s_all[b_s * K + j];
    s_best[j] = v;
    s_copy[j] = v;
  }
}

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// Workspace regions, in order.
struct AwqLayout {
  size_t part, mag, pbuf, bmax, bmin, norm, s_all, s_best, xs, xsum, codes, scales, zeros, yref, yq, err, total;
};

AwqLayout awq_layout(int64_t N, int64_t K, int64_t T, int64_t n_alpha) {
  AwqLayout l;
  const int64_t G = K / kGroup;
  const int64_t nb = ceil_div(K, 256);
  size_t o = 0;
  l.part = o; o += align256(static_cast<size_t>(ceil_div(T, kMagRows) * K) * sizeof(double));
  l.mag = o; o += align256(static_cast<size_t>(K) * sizeof(double));
  l.pbuf = o; o += align256(static_cast<size_t>(n_alpha * K) * sizeof(double));
  l.bmax = o; o += align256(static_cast<size_t>(n_alpha * nb) * sizeof(double));
  l.bmin = o; o += align256(static_cast<size_t>(n_alpha * nb) * sizeof(double));
  l.norm = o; o += align256(static_cast<size_t>(n_alpha) * sizeof(double));
  l.s_all = o; o += align256(static_cast<size_t>(n_alpha * K) * sizeof(float));
  l.s_best = o; o += align256(static_cast<size_t>(K) * sizeof(float));
  l.xs = o; o += align256(static_cast<size_t>(T * K) * 2);
  l.xsum = o; o += align256(static_cast<size_t>(T * G) * sizeof(float));
  l.codes = o; o += align256(static_cast<size_t>(N * K / 2));
  l.scales = o; o += align256(static_cast<size_t>(N * G) * sizeof(float));
  l.zeros = o; o += align256(static_cast<size_t>(N * ((G + 1) / 2)));
  l.yref = o; o += align256(static_cast<size_t>(T * N) * sizeof(float));
  l.yq = o; o += align256(static_cast<size_t>(T * N) * sizeof(float));
  l.err = o; o += align256(static_cast<size_t>(n_alpha * kErrBlocks) * sizeof(double));
  l.total = o;
  return l;
}

unsigned grid_for(int64_t items) {
  const int64_t blocks = ceil_div(items, 256);
  const int64_t cap = static_cast<int64_t>(device_cus()) * 8;
  return static_cast<unsigned>(blocks < cap ? blocks : cap);
}

}  // namespace
}  // namespace qmm

using namespace qmm;

extern "C" size_t awq_workspace_bytes(int64_t N, int64_t K, int64_t T, int64_t n_alpha) {
  if (N <= 0 || K <= 0 || T <= 0 || n_alpha <= 0 || n_alpha > kMaxAlphas || K % kGroup != 0) return 0;
  return awq_layout(N, K, T, n_alpha).total;
}

extern "C" int awq_search(const void* W, int w_dtype, const void* X, int x_dtype, int64_t N, int64_t K, int64_t T,
                          const double* alphas, int64_t n_alpha, uint8_t* codes, float* scales, uint8_t* zeros,
                          float* smooth, double* err, int64_t* best, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (!W || !X || !alphas || !codes || !scales || !zeros || !smooth || !err || !best) return QMM_EINVAL;
  if (N <= 0 || K <= 0 || T <= 0 || n_alpha <= 0) return QMM_EINVAL;
  if (K % kGroup != 0) return QMM_EUNSUPPORTED;
  const bool h16w = w_dtype == QMM_BF16 || w_dtype == QMM_F16;
  const bool h16x = x_dtype == QMM_BF16 || x_dtype == QMM_F16;
  if (!(h16w || w_dtype == QMM_F32) || !(h16x || x_dtype == QMM_F32)) return QMM_EINVAL;
  if (!h16w || !h16x || w_dtype != x_dtype) return QMM_EUNSUPPORTED;   // fp32, or two 16-bit types
  if (n_alpha > kMaxAlphas) return QMM_EUNSUPPORTED;
  for (int64_t a = 0; a < n_alpha; ++a)
    if (!(alphas[a] >= 0.0 && alphas[a] <= 1.0)) return QMM_EINVAL;
  // the 16-bit product's 32-bit offsets (256 rows of 2K bytes), the W4A16
  // product's, and the magnitude slices' grid rows (at most 65535 slices)
  if (K > (int64_t(1) << 22) || N > INT32_MAX || T > int64_t{65535} * kMagRows) return QMM_ERANGE;
  if (!aligned(W, 16) || !aligned(X, 16) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(smooth, 4) ||
      !aligned(err, 8) || !aligned(best, 8))
    return QMM_EALIGN;
  if (!workspace || workspace_bytes < awq_layout(N, K, T, n_alpha).total) return QMM_EWORKSPACE;
  if (!aligned(workspace, 256)) return QMM_EALIGN;
  const AwqLayout L = awq_layout(N, K, T, n_alpha);
  uint8_t* base = static_cast<uint8_t*>(workspace);
  double* mpart = reinterpret_cast<double*>(base + L.part);
  double* mag = reinterpret_cast<double*>(base + L.mag);
  double* pbuf = reinterpret_cast<double*>(base + L.pbuf);
  double* bmax = reinterpret_cast<double*>(base + L.bmax);
  double* bmin = reinterpret_cast<double*>(base + L.bmin);
  double* norm = reinterpret_cast<double*>(base + L.norm);
  float* s_all = reinterpret_cast<float*>(base + L.s_all);
  float* s_copy = reinterpret_cast<float*>(base + L.s_best);
  uint16_t* xs = reinterpret_cast<uint16_t*>(base + L.xs);
  float* xsum = reinterpret_cast<float*>(base + L.xsum);
  uint8_t* qc = base + L.codes;
  float* qs = reinterpret_cast<float*>(base + L.scales);
  uint8_t* qz = base + L.zeros;
  float* yref = reinterpret_cast<float*>(base + L.yref);
  float* yq = reinterpret_cast<float*>(base + L.yq);
  double* epart = reinterpret_cast<double*>(base + L.err);
  hipStream_t s = as_stream(stream);
  const uint16_t* w = static_cast<const uint16_t*>(W);
  const uint16_t* x = static_cast<const uint16_t*>(X);

  // channel magnitudes and every alpha's factors
  const int64_t slices = ceil_div(T, kMagRows);
  const unsigned nb = static_cast<unsigned>(ceil_div(K, 256));
  const dim3 mgrid(static_cast<unsigned>(ceil_div(K, 2048)), static_cast<unsigned>(slices));
  if (x_dtype == QMM_F16) awq_mag_partial_kernel<QMM_F16><<<mgrid, 256, 0, s>>>(x, T, K, mpart);
  else awq_mag_partial_kernel<QMM_BF16><<<mgrid, 256, 0, s>>>(x, T, K, mpart);
  awq_mag_kernel<<<nb, 256, 0, s>>>(mpart, slices, T, K, mag);
  AlphaGrid grid{};
  for (int64_t a = 0; a < n_alpha; ++a) grid.a[a] = alphas[a];
  awq_pow_kernel<<<dim3(nb, static_cast<unsigned>(n_alpha)), 256, 0, s>>>(mag, K, grid, pbuf, bmax, bmin);
  awq_norm_kernel<<<static_cast<unsigned>(n_alpha), 256, 0, s>>>(bmax, bmin, nb, norm);
  awq_factor_kernel<<<dim3(nb, static_cast<unsigned>(n_alpha)), 256, 0, s>>>(pbuf, norm, K, s_all);
  int st = launch_status();
  if (st != QMM_OK) return st;
  // the full-precision output X W^T
  launch_h16_gemm(x, w, x_dtype, T, N, K, yref, s);
  st = launch_status();
  if (st != QMM_OK) return st;

  const int64_t xn8 = T * K / 8;
  for (int64_t a = 0; a < n_alpha; ++a) {
    const float* sa = s_all + a * K;
    launch_quantize_colscaled(w, w_dtype, sa, N, K, qc, qs, qz, s);
    if (x_dtype == QMM_F16) awq_scale_x_kernel<QMM_F16><<<grid_for(xn8), 256, 0, s>>>(x, sa, xn8, K, xs, xsum);
    else awq_scale_x_kernel<QMM_BF16><<<grid_for(xn8), 256, 0, s>>>(x, sa, xn8, K, xs, xsum);
    st = launch_status();
    if (st != QMM_OK) return st;
    st = w4a16_gemm_colsums(qc, qs, qz, N, K, xs, xsum, x_dtype, T, yq, s);
    if (st != QMM_OK) return st;
    awq_sqerr_kernel<<<kErrBlocks, 256, 0, s>>>(yref, yq, T * N, epart + a * kErrBlocks);
    st = launch_status();
    if (st != QMM_OK) return st;
  }
  awq_select_kernel<<<1, kErrBlocks, 0, s>>>(epart, static_cast<int>(n_alpha), s_all, K, err, best, smooth, s_copy);
  st = launch_status();
  if (st != QMM_OK) return st;
  // the chosen alpha's weights in the caller's format
  launch_quantize_colscaled(w, w_dtype, s_copy, N, K, codes, scales, zeros, s);
  return launch_status();
}
