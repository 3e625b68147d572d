// w4a16.hip -- matmuls with INT4 group-quantized weights and 16-bit activations:
//   y[t, n] = sum_k x[t, k] * W_hat[n, k],  W_hat[n, k] = (q[n, k] - z[n, g]) * s[n, g].
//
// Sources: "How quantization works" (AI-infra handbook), "Inference view":
// the packed weights are expanded in registers, scaled and consumed by the
// 16-bit arithmetic, so only the packed bytes cross HBM; "Quantization from
// Scratch", "What it buys at decode": a decode step reads every weight once,
// so its time is the weight bytes over the bandwidth until the batch is large.
//
// Arithmetic used by every kernel here.  A code word's nibbles are turned into
// 16-bit floats 128 + q (bf16) or 16 + q (fp16) with a shift and an AND-OR
// (Int4Magic::unpack), so per group g of 128 weights
//   sum_k (q - z) x = sum_k (off + q) x - (off + z) * X_g,   X_g = sum_{k in g} x,
//   y += s * (that),
// with the products exact and the sums in fp32.
//
// Kernels
//  * gemv_valu_kernel: B <= 8 tokens on the vector ALUs (v_dot2_f32_{bf16,f16}),
//    no matrix cores: a lane streams 16 bytes (32 weights) per row per step,
//    R rows at a time so R x 16 bytes are in flight, with the activation slice
//    held in registers across those rows.  Used for B == 1 (decode).
//  * w4_mfma_skinny_kernel: up to 16*MT tokens per block on
//    v_mfma_f32_16x16x32_{bf16,f16}; the weights are the A operand (16 rows x
//    32 k per instruction, one code word per lane) and never touch LDS; the
//    wavefronts of a block split K and are summed through LDS at the end.

#include "qmm_device.h"

namespace qmm {
namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

template <int YDT>
__device__ __forceinline__ void store_y(void* y, int64_t idx, float v) {
  if constexpr (YDT == QMM_F32) {
    static_cast<float*>(y)[idx] = v;
  } else if constexpr (YDT == QMM_BF16) {
    static_cast<uint16_t*>(y)[idx] = static_cast<uint16_t>(f32_to_bf16_bits(v));
  } else {
    static_cast<uint16_t*>(y)[idx] = static_cast<uint16_t>(f32_to_f16_bits(v));
  }
}

// ----------------------------------------------------------------------------
// Vector-ALU GEMV.
// ----------------------------------------------------------------------------
constexpr int kValuWaves = 4;
constexpr int kLaneK = 32;                                   // weights per lane per row per step
constexpr int64_t kValuStepK = kValuWaves * kWave * kLaneK;  // 8192

template <int XDT, int YDT, int B, int R>
__global__ __launch_bounds__(256) void gemv_valu_kernel(const uint8_t* __restrict__ codes,
                                                        const float* __restrict__ scales,
                                                        const uint8_t* __restrict__ zeros, int64_t N, int64_t K,
                                                        const uint16_t* __restrict__ x, void* __restrict__ y) {
  using Mg = Int4Magic<XDT>;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * R;
  const int64_t G = K / kGroup;
  const int64_t zrow = (G + 1) / 2;
  const int64_t row_bytes = K / 2;

  int64_t rows[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rows[r] = (row0 + r < N) ? row0 + r : N - 1;

  float acc[R][B];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;

  for (int64_t k0 = 0; k0 < K; k0 += kValuStepK) {
    const int64_t kb = k0 + static_cast<int64_t>(wave) * (kWave * kLaneK) + lane * kLaneK;
    if (kb < K) {
      u32x4 cw[R];
#pragma unroll
      for (int r = 0; r < R; ++r) cw[r] = ld16_nt(codes + rows[r] * row_bytes + kb / 2);
      const int64_t g = kb >> 7;
      float sc[R], zo[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        sc[r] = scales[rows[r] * G + g];
        zo[r] = Mg::offset + static_cast<float>(zero_nibble(zeros + rows[r] * zrow, g));
      }
      uint32_t xp[B][16];
      float xs[B];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const uint16_t* xv = x + b * K + kb;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const u32x4 a = ld16(xv + 8 * c);
          const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
          permute_pairs(aw, &xp[b][4 * c]);
        }
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
          s0 = dot2<XDT>(xp[b][j], Mg::one_pair, s0);
          s1 = dot2<XDT>(xp[b][j + 1], Mg::one_pair, s1);
        }
        xs[b] = s0 + s1;
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t words[4] = {cw[r].x, cw[r].y, cw[r].z, cw[r].w};
        float a0[B], a1[B];
#pragma unroll
        for (int b = 0; b < B; ++b) a0[b] = a1[b] = 0.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          uint32_t p[4];
          Mg::unpack(words[c], p);
#pragma unroll
          for (int b = 0; b < B; ++b) {
            a0[b] = dot2<XDT>(p[0], xp[b][4 * c + 0], a0[b]);
            a1[b] = dot2<XDT>(p[1], xp[b][4 * c + 1], a1[b]);
            a0[b] = dot2<XDT>(p[2], xp[b][4 * c + 2], a0[b]);
            a1[b] = dot2<XDT>(p[3], xp[b][4 * c + 3], a1[b]);
          }
        }
#pragma unroll
        for (int b = 0; b < B; ++b) acc[r][b] = fmaf(sc[r], fmaf(-zo[r], xs[b], a0[b] + a1[b]), acc[r][b]);
      }
    }
  }

  __shared__ float red[kValuWaves][R * B];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float v = wave_sum(acc[r][b]);
      if (lane == 0) red[wave][r * B + b] = v;
    }
  __syncthreads();
  if (threadIdx.x < R * B) {
    const int r = threadIdx.x / B;
    const int b = threadIdx.x % B;
    const int64_t row = row0 + r;
    if (row < N) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < kValuWaves; ++w) v += red[w][threadIdx.x];
      store_y<YDT>(y, static_cast<int64_t>(b) * N + row, v);
    }
  }
}

// ----------------------------------------------------------------------------
// MFMA kernel for a small number of tokens.
// ----------------------------------------------------------------------------
template <int XDT>
__device__ __forceinline__ f32x4 mfma16x16x32(const uint32_t a[4], const uint32_t b[4], f32x4 c) {
  const u32x4 av = {a[0], a[1], a[2], a[3]};
  const u32x4 bv = {b[0], b[1], b[2], b[3]};
  if constexpr (XDT == QMM_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bv),
                                                   c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, av), __builtin_bit_cast(f16x8_t, bv), c,
                                                  0, 0, 0);
  }
}

// Block: NW = blockDim.x / 64 wavefronts sharing rows [row0, row0 + 16*RT)
// and tokens [t0, t0 + 16*MT); wavefront w owns a contiguous range of groups.
// MFMA operand layout (16x16x32): lane l supplies A row l%16 and B column
// l%16, k = 8*(l/16) .. +8 of the instruction; D lane l holds rows
// 4*(l/16) .. +4 of column l%16.  Here each lane loads one 16-byte code
// vector = k-chunks 4*(l/16) .. +4 of a group, so instruction j of the group
// takes chunk 4*(l/16) + j; the activation operand is loaded the same way.
template <int XDT, int YDT, int RT, int MT>
__global__ __launch_bounds__(1024) void w4_mfma_skinny_kernel(const uint8_t* __restrict__ codes,
                                                              const float* __restrict__ scales,
                                                              const uint8_t* __restrict__ zeros, int64_t N,
                                                              int64_t K, const uint16_t* __restrict__ x, int64_t M,
                                                              void* __restrict__ y) {
  using Mg = Int4Magic<XDT>;
  extern __shared__ float red[];   // [NW][RT*MT*4][64]
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  const int l16 = lane & 15;
  const int quad = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * 16 * RT;
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * 16 * MT;
  const int64_t G = K / kGroup;
  const int64_t zrow = (G + 1) / 2;
  const int64_t row_bytes = K / 2;
  const int64_t gper = (G + nw - 1) / nw;
  const int64_t gbeg = wave * gper;
  const int64_t gend = (gbeg + gper < G) ? gbeg + gper : G;

  int64_t arow[RT];      // A-operand row of this lane
  int64_t drow[RT][4];   // D rows of this lane
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int64_t ra = row0 + 16 * rt + l16;
    arow[rt] = ra < N ? ra : N - 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t rd = row0 + 16 * rt + 4 * quad + i;
      drow[rt][i] = rd < N ? rd : N - 1;
    }
  }
  bool tvalid[MT];
  int64_t tok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    tok[mt] = t0 + 16 * mt + l16;
    tvalid[mt] = tok[mt] < M;
  }

  f32x4 acc[RT][MT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  for (int64_t g = gbeg; g < gend; ++g) {
    u32x4 cw[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) cw[rt] = ld16_nt(codes + arow[rt] * row_bytes + g * 64 + quad * 16);
    float sc[RT][4], zo[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc[rt][i] = scales[drow[rt][i] * G + g];
        zo[rt][i] = Mg::offset + static_cast<float>(zero_nibble(zeros + drow[rt][i] * zrow, g));
      }
    uint32_t wa[RT][16];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const uint32_t words[4] = {cw[rt].x, cw[rt].y, cw[rt].z, cw[rt].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) Mg::unpack(words[j], &wa[rt][4 * j]);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      uint32_t xb[16];
      if (tvalid[mt]) {
        const uint16_t* xv = x + tok[mt] * K + g * kGroup + quad * 32;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const u32x4 a = ld16(xv + 8 * c);
          const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
          permute_pairs(aw, &xb[4 * c]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) xb[j] = 0u;
      }
      float xs0 = 0.0f, xs1 = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; j += 2) {
        xs0 = dot2<XDT>(xb[j], Mg::one_pair, xs0);
        xs1 = dot2<XDT>(xb[j + 1], Mg::one_pair, xs1);
      }
      float xg = xs0 + xs1;
      xg += __shfl_xor(xg, 16, kWave);
      xg += __shfl_xor(xg, 32, kWave);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        f32x4 p = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int j = 0; j < 4; ++j) p = mfma16x16x32<XDT>(&wa[rt][4 * j], &xb[4 * j], p);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[rt][mt][i] = fmaf(sc[rt][i], fmaf(-zo[rt][i], xg, p[i]), acc[rt][mt][i]);
      }
    }
  }

  constexpr int kOut = RT * MT * 4;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[(wave * kOut + (rt * MT + mt) * 4 + i) * kWave + lane] = acc[rt][mt][i];
  __syncthreads();
  for (int o = threadIdx.x; o < kOut * kWave; o += blockDim.x) {
    float v = 0.0f;
    for (int w = 0; w < nw; ++w) v += red[w * kOut * kWave + o];
    const int l = o % kWave;
    const int slot = o / kWave;
    const int i = slot % 4;
    const int mt = (slot / 4) % MT;
    const int rt = slot / (4 * MT);
    const int64_t row = row0 + 16 * rt + 4 * (l >> 4) + i;
    const int64_t t = t0 + 16 * mt + (l & 15);
    if (row < N && t < M) store_y<YDT>(y, t * N + row, v);
  }
}

// ----------------------------------------------------------------------------
// Host side.
// ----------------------------------------------------------------------------
int check_common(const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K, int group,
                 const void* x, int x_dtype, int64_t M, const void* y, int y_dtype) {
  if (!codes || !scales || !zeros || !x || !y) return QMM_EINVAL;
  if (N <= 0 || K <= 0 || M <= 0 || group <= 0 || K % group != 0) return QMM_EINVAL;
  if ((x_dtype != QMM_BF16 && x_dtype != QMM_F16 && x_dtype != QMM_F32 && x_dtype != QMM_I32) ||
      (y_dtype != QMM_BF16 && y_dtype != QMM_F16 && y_dtype != QMM_F32 && y_dtype != QMM_I32))
    return QMM_EINVAL;
  if (group != kGroup) return QMM_EUNSUPPORTED;
  if (x_dtype != QMM_BF16 && x_dtype != QMM_F16) return QMM_EUNSUPPORTED;
  if (y_dtype != x_dtype && y_dtype != QMM_F32) return QMM_EUNSUPPORTED;
  if (!aligned(codes, 16) || !aligned(x, 16) || !aligned(scales, 4) || !aligned(y, y_dtype == QMM_F32 ? 4 : 2))
    return QMM_EALIGN;
  return QMM_OK;
}

template <int XDT, int YDT, int B>
void launch_valu(const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K,
                 const uint16_t* x, void* y, hipStream_t s) {
  constexpr int R = B == 1 ? 8 : (B <= 4 ? 4 : 2);
  const dim3 grid(static_cast<unsigned>(ceil_div(N, R)));
  gemv_valu_kernel<XDT, YDT, B, R><<<grid, dim3(kValuWaves * kWave), 0, s>>>(codes, scales, zeros, N, K, x, y);
}

template <int XDT, int YDT>
void launch_valu_b(int64_t B, const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K,
                   const uint16_t* x, void* y, hipStream_t s) {
  switch (B) {
    case 1: launch_valu<XDT, YDT, 1>(codes, scales, zeros, N, K, x, y, s); break;
    case 2: launch_valu<XDT, YDT, 2>(codes, scales, zeros, N, K, x, y, s); break;
    case 3: launch_valu<XDT, YDT, 3>(codes, scales, zeros, N, K, x, y, s); break;
    case 4: launch_valu<XDT, YDT, 4>(codes, scales, zeros, N, K, x, y, s); break;
    case 5: launch_valu<XDT, YDT, 5>(codes, scales, zeros, N, K, x, y, s); break;
    case 6: launch_valu<XDT, YDT, 6>(codes, scales, zeros, N, K, x, y, s); break;
    case 7: launch_valu<XDT, YDT, 7>(codes, scales, zeros, N, K, x, y, s); break;
    default: launch_valu<XDT, YDT, 8>(codes, scales, zeros, N, K, x, y, s); break;
  }
}

// Wavefronts per block for the skinny MFMA kernel: split K further when the
// grid alone would leave compute units short of wavefronts.
// The per-block reduction buffer (nw * out_per_wave floats) stays within 64 KiB.
int skinny_waves(int64_t blocks, int64_t G, int64_t out_per_wave) {
  const int64_t target = static_cast<int64_t>(device_cus()) * 16;   // wavefronts wanted in flight
  int nw = 4;
  while (nw < 16 && blocks * nw < target && G >= 2 * nw * 2 &&
         2 * nw * out_per_wave * static_cast<int64_t>(sizeof(float)) <= 65536)
    nw *= 2;
  return nw;
}

template <int XDT, int YDT, int RT, int MT>
void launch_skinny(const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K,
                   const uint16_t* x, int64_t M, void* y, hipStream_t s) {
  const int64_t bx = ceil_div(N, 16 * RT);
  const int64_t by = ceil_div(M, 16 * MT);
  const int nw = skinny_waves(bx * by, K / kGroup, static_cast<int64_t>(RT) * MT * 4 * kWave);
  const size_t lds = static_cast<size_t>(nw) * RT * MT * 4 * kWave * sizeof(float);
  w4_mfma_skinny_kernel<XDT, YDT, RT, MT>
      <<<dim3(static_cast<unsigned>(bx), static_cast<unsigned>(by)), dim3(nw * kWave), lds, s>>>(codes, scales, zeros,
                                                                                                 N, K, x, M, y);
}

template <int XDT, int YDT>
void launch_skinny_m(int64_t M, const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N,
                     int64_t K, const uint16_t* x, void* y, hipStream_t s) {
  if (M <= 16)
    launch_skinny<XDT, YDT, 2, 1>(codes, scales, zeros, N, K, x, M, y, s);
  else
    launch_skinny<XDT, YDT, 2, 4>(codes, scales, zeros, N, K, x, M, y, s);
}

}  // namespace
}  // namespace qmm

using namespace qmm;

extern "C" int w4a16_gemv(const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K,
                          int group, const void* x, int x_dtype, int64_t B, void* y, int y_dtype, void* stream) {
  int st = check_common(codes, scales, zeros, N, K, group, x, x_dtype, B, y, y_dtype);
  if (st != QMM_OK) return st;
  if (B > 8) return QMM_EUNSUPPORTED;
  hipStream_t s = as_stream(stream);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  if (B == 1 || x_dtype == QMM_F16) {
    if (x_dtype == QMM_BF16) {
      if (y_dtype == QMM_F32) launch_valu_b<QMM_BF16, QMM_F32>(B, codes, scales, zeros, N, K, xp, y, s);
      else launch_valu_b<QMM_BF16, QMM_BF16>(B, codes, scales, zeros, N, K, xp, y, s);
    } else {
      if (y_dtype == QMM_F32) launch_valu_b<QMM_F16, QMM_F32>(B, codes, scales, zeros, N, K, xp, y, s);
      else launch_valu_b<QMM_F16, QMM_F16>(B, codes, scales, zeros, N, K, xp, y, s);
    }
  } else {
    if (y_dtype == QMM_F32) launch_skinny<QMM_BF16, QMM_F32, 2, 1>(codes, scales, zeros, N, K, xp, B, y, s);
    else launch_skinny<QMM_BF16, QMM_BF16, 2, 1>(codes, scales, zeros, N, K, xp, B, y, s);
  }
  return launch_status();
}

extern "C" int w4a16_gemm(const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K,
                          int group, const void* X, int x_dtype, int64_t M, void* Y, int y_dtype, void* stream) {
  int st = check_common(codes, scales, zeros, N, K, group, X, x_dtype, M, Y, y_dtype);
  if (st != QMM_OK) return st;
  if (x_dtype != QMM_BF16) return QMM_EUNSUPPORTED;
  hipStream_t s = as_stream(stream);
  const uint16_t* xp = static_cast<const uint16_t*>(X);
  if (y_dtype == QMM_F32) launch_skinny_m<QMM_BF16, QMM_F32>(M, codes, scales, zeros, N, K, xp, Y, s);
  else launch_skinny_m<QMM_BF16, QMM_BF16>(M, codes, scales, zeros, N, K, xp, Y, s);
  return launch_status();
}
