// quantize.hip -- group-wise asymmetric INT4 quantization and dequantization.
//
// Method: "Quantization Explained: INT8, INT4, GPTQ and AWQ for LLMs", slides
// "Scale and Zero-Point" and "Manual Group-Wise Quantizer" (per-group min/max,
// s = (max - min) / 15, z = round(-min / s), q = clamp(round(w / s) + z, 0, 15));
// "Quantization from Scratch: Scale, Zero-Point, GPTQ and AWQ", section "Scale
// and zero-point" (w_hat = (q - z) s) and its round-to-nearest listing (a zero
// scale becomes 1; clip after adding the zero-point).  The range is widened to
// contain 0 so the zero-point is always a valid 4-bit code.
//
// Mapping: one wavefront quantizes a "chunk" of four consecutive groups of one
// row (512 elements).  Each group is one DPP row of 16 lanes; a lane owns 8
// consecutive elements, loads them with one 16-byte (bf16/fp16) or two
// 16-byte (fp32) loads and stores their 8 codes as one 32-bit word, so a
// wavefront reads 1 KiB (2 KiB) and writes 256 B, both contiguous.

#include "qmm_device.h"

namespace qmm {
namespace {

constexpr float kLevels = 15.0f;                 // 2^4 - 1
constexpr float kSymLevels = 7.0f;               // 2^(4-1) - 1
constexpr float kSymFloor = 1e-8f;               // absmax floor of the symmetric grid
constexpr float kSymZero = 8.0f;                 // stored zero-point of symmetric codes

// Codes of 8 elements of a group with scale s, y = RN(1/s) (one correctly
// rounded division per group, by the caller) and zero-point zf (an
// integer-valued float): clamp(rint(fl32(v / s)) + z, 0, 15), bit-identical to
// dividing each element, without dividing each element.  q0 = RN(v y) is
// within one ulp of v / s, the residual r = v - q0 s is exact through fma, and
// q1 = RN(q0 + r y) is then exactly RN(v / s) (Markstein's theorem for
// division by a correctly rounded reciprocal; it needs no overflow or
// underflow, which the scale range [2^-100, 2^100] guarantees for every
// element whose quotient reaches 1/4 in magnitude -- smaller quotients round
// to 0 either way).  Groups with a scale outside that range divide exactly.
// (16-bit weights put about 2 quotients in 1000 exactly on a half-integer,
// where only the exact quotient rounds correctly, half to even.)
__device__ __forceinline__ uint32_t quantize8(const float v[8], float s, float y, float zf) {
  const bool scale_ok = (s >= 0x1p-100f) && (s <= 0x1p100f);
  float k[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float q0 = v[i] * y;
    const float r = fmaf(-q0, s, v[i]);
    k[i] = rintf(fmaf(r, y, q0)) + zf;
  }
  if (__builtin_amdgcn_ballot_w64(!scale_ok)) {   // wavefront-uniform, practically never taken
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float e = rintf(v[i] / s) + zf;
      if (!scale_ok) k[i] = e;
    }
  }
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float c = __builtin_amdgcn_fmed3f(k[i], 0.0f, kLevels);
    word |= static_cast<uint32_t>(c) << (4 * code_nibble(i));
  }
  return word;
}

// Scale and zero-point of a group from its range, lo = min(min w, 0) and
// hi = max(max w, 0).  Asymmetric ("Quantization from Scratch", "Scale and
// zero-point"; "How quantization works", "The math of quantization"):
// s = fl32((hi - lo) / 15), 1 for an all-zero group, z = rint(fl32(-lo / s)).
// Symmetric (the same sections' symmetric grid): s = fl32(max|w| / 7) with
// max|w| floored at 1e-8, q = clamp(rint(fl32(w / s)), -8, 7), stored as the
// code q + 8 with the zero-point 8, so the dequantizer and the matmuls read
// it unchanged ((code - 8) s = q s).
template <bool SYM>
__device__ __forceinline__ void group_params(float lo, float hi, float* s, float* zf) {
  if constexpr (SYM) {
    *s = fmaxf(fmaxf(hi, -lo), kSymFloor) / kSymLevels;   // correctly rounded fp32 division
    *zf = kSymZero;
  } else {
    float sc = (hi - lo) / kLevels;                         // correctly rounded fp32 division
    if (sc == 0.0f) sc = 1.0f;
    *s = sc;
    *zf = rintf(-lo / sc);                                  // in [0, 15] because lo <= 0 <= hi
  }
}

// Flat variant for an even number of groups per row: the matrix is then one
// array of N*G groups whose codes, scales and zero-point bytes are all
// consecutive, so a wavefront takes 16 consecutive groups: 4 lanes per group,
// 32 elements (64 bytes of bf16/fp16) per lane, 4 16-byte loads and one
// 16-byte code store per lane.  Four lanes share a group's min/max (two DPP
// steps) and its s and z, so the per-group division costs are spread over 32
// elements per lane instead of 8.
template <int DT, bool SYM>
__global__ __launch_bounds__(256) void quantize_g128_flat_kernel(const uint8_t* __restrict__ w, int64_t total_groups,
                                                                 uint8_t* __restrict__ codes,
                                                                 float* __restrict__ scales,
                                                                 uint8_t* __restrict__ zeros) {
  constexpr int kElemBytes = DT == QMM_F32 ? 4 : 2;
  const int lane = threadIdx.x & (kWave - 1);
  const int part = lane & 3;
  const int64_t waves_per_block = blockDim.x / kWave;
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * waves_per_block;
  const int64_t nchunks = (total_groups + 15) / 16;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * waves_per_block + (threadIdx.x / kWave); c < nchunks;
       c += nwaves) {
    const int64_t gi = c * 16 + (lane >> 2);
    const bool active = gi < total_groups;
    const int64_t gl = active ? gi : total_groups - 1;     // in-bounds address for idle lanes
    const uint8_t* src = w + (gl * kGroup + part * 32) * kElemBytes;
    float v[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) Vec8<DT>::load(src + q * 8 * kElemBytes, &v[8 * q]);
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      lo = fminf(lo, v[i]);
      hi = fmaxf(hi, v[i]);
    }
    lo = fminf(lo, dpp_f<kDppXor1>(lo));
    hi = fmaxf(hi, dpp_f<kDppXor1>(hi));
    lo = fminf(lo, dpp_f<kDppXor2>(lo));
    hi = fmaxf(hi, dpp_f<kDppXor2>(hi));
    float s, zf;
    group_params<SYM>(lo, hi, &s, &zf);
    const float y = 1.0f / s;           // correctly rounded reciprocal
    uint32_t out[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) out[q] = quantize8(&v[8 * q], s, y, zf);
    const float z_next = __shfl_down(zf, 4, kWave);   // zero-point of the next (odd) group
    if (active) {
      st16_nt(codes + gi * 64 + part * 16, u32x4{out[0], out[1], out[2], out[3]});
      if (part == 0) {
        scales[gi] = s;
        if ((lane & 7) == 0) {
          const uint32_t zo = (gi + 1 < total_groups) ? static_cast<uint32_t>(z_next) : 0u;
          zeros[gi >> 1] = static_cast<uint8_t>(static_cast<uint32_t>(zf) | (zo << 4));
        }
      }
    }
  }
}

// 16-bit weights, even number of groups per row: the flat mapping above
// (lane l quantizes 32 elements of group l/4), but each wavefront's chunk of
// 16 groups (4 KiB) reaches LDS by four buffer loads that each cover 1 KiB
// contiguously, instead of every lane loading its own 64 bytes (a 4 KiB span
// per instruction), which left the kernel at its memory skeleton's ~150 us
// per 70B matrix against ~103 us with contiguous loads.  Chunks are double
// buffered: the next chunk's loads are issued before the current one is read.
// A 16-byte piece P of the chunk (lane l reads pieces 4l .. 4l+3) sits in LDS
// slot 64 (P / 64) + 4 m + ((j + m / 4) & 3), m = (P / 4) % 16, j = P % 4, so
// the four reads of each lane are free of bank conflicts.
constexpr int kQChunkBytes = 16 * kGroup * 2;   // 4 KiB of 16-bit weights

//
// CS = true quantizes fl32(w * colscale[column]) instead of w (one fp32
// product per weight, the factors read through the cache; G = groups per
// row locates a group's columns): AWQ's scaled weights without a stored
// fp32 copy of them.
template <int DT, bool SYM, bool CS = false>
__global__ __launch_bounds__(256) void quantize_g128_lds_kernel(const uint8_t* __restrict__ w, int64_t total_groups,
                                                                uint8_t* __restrict__ codes,
                                                                float* __restrict__ scales,
                                                                uint8_t* __restrict__ zeros,
                                                                const float* __restrict__ colscale = nullptr,
                                                                int64_t G = 0) {
  static_assert(DT != QMM_F32, "16-bit weights only");
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * 2 * kQChunkBytes];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int part = lane & 3;
  const int64_t waves_per_block = blockDim.x / kWave;
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * waves_per_block;
  const int64_t nchunks = (total_groups + 15) / 16;
  const uint32_t wbase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)) + wave * 2 * kQChunkBytes;

  // Load lane l of instruction q fetches piece 64 q + 4 m + ((l % 4 - m / 4) & 3),
  // m = l / 4, and writes slot 64 q + l.
  const int lm = lane >> 2;
  const int fetch = (4 * lm + (((lane & 3) - (lm >> 2)) & 3)) * 16;
  auto issue = [&](int64_t c, int buf) {
    const int64_t left = (total_groups - c * 16) * (kGroup * 2);
    const int bytes = static_cast<int>(left < kQChunkBytes ? left : kQChunkBytes);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(w + c * kQChunkBytes), 0, bytes, kBufferWord3);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (lds_ptr_t)(uintptr_t)(wbase + buf * kQChunkBytes + q * 1024), 16, fetch + q * 1024, 0, 0, 0);
  };
  // Reader: lane l's pieces 4l + j are in instruction l / 16, m = l % 16.
  const int rm = lane & 15;
  int rd[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) rd[j] = (lane >> 4) * 1024 + (4 * rm + ((j + (rm >> 2)) & 3)) * 16;

  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * waves_per_block + wave;
  int buf = 0;
  if (c0 < nchunks) issue(c0, 0);
  for (int64_t c = c0; c < nchunks; c += nwaves, buf ^= 1) {
    const bool next = c + nwaves < nchunks;   // uniform
    // CS: this chunk's column factors are requested before the next chunk's
    // loads, so the wait below covers them too (loads complete in order).
    f32x4 fcs[CS ? 8 : 1];
    if constexpr (CS) {
      const float* cs = colscale + ((c * 16 + (lane >> 2)) % G) * kGroup + part * 32;   // in [0, K), idle lanes too
#pragma unroll
      for (int q = 0; q < 8; ++q) fcs[q] = *reinterpret_cast<const f32x4*>(cs + 4 * q);
    }
    if (next) {
      issue(c + nwaves, buf ^ 1);
      wait_vm<4>();
    } else {
      wait_vm<0>();
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint8_t* cb = lds + wave * 2 * kQChunkBytes + buf * kQChunkBytes;
    float v[32];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 u = *reinterpret_cast<const u32x4*>(cb + rd[j]);
      const uint32_t a[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if constexpr (DT == QMM_BF16) {
          v[8 * j + 2 * h] = bf16lo_to_f32(a[h]);
          v[8 * j + 2 * h + 1] = bf16hi_to_f32(a[h]);
        } else {
          v[8 * j + 2 * h] = f16lo_to_f32(a[h]);
          v[8 * j + 2 * h + 1] = f16hi_to_f32(a[h]);
        }
      }
    }
    const int64_t gi = c * 16 + (lane >> 2);
    const bool active = gi < total_groups;
    if constexpr (CS) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const f32x4 f = fcs[q];
        v[4 * q] = v[4 * q] * f.x;
        v[4 * q + 1] = v[4 * q + 1] * f.y;
        v[4 * q + 2] = v[4 * q + 2] * f.z;
        v[4 * q + 3] = v[4 * q + 3] * f.w;
      }
    }
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      lo = fminf(lo, v[i]);
      hi = fmaxf(hi, v[i]);
    }
    lo = fminf(lo, dpp_f<kDppXor1>(lo));
    hi = fmaxf(hi, dpp_f<kDppXor1>(hi));
    lo = fminf(lo, dpp_f<kDppXor2>(lo));
    hi = fmaxf(hi, dpp_f<kDppXor2>(hi));
    float sc, zf;
    group_params<SYM>(lo, hi, &sc, &zf);
    const float y = 1.0f / sc;          // correctly rounded reciprocal
    uint32_t out[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) out[q] = quantize8(&v[8 * q], sc, y, zf);
    const float z_next = __shfl_down(zf, 4, kWave);   // zero-point of the next (odd) group
    if (active) {
      st16_nt(codes + gi * 64 + part * 16, u32x4{out[0], out[1], out[2], out[3]});
      if (part == 0) {
        scales[gi] = sc;
        if ((lane & 7) == 0) {
          const uint32_t zo = (gi + 1 < total_groups) ? static_cast<uint32_t>(z_next) : 0u;
          zeros[gi >> 1] = static_cast<uint8_t>(static_cast<uint32_t>(zf) | (zo << 4));
        }
      }
    }
  }
}

template <int DT, bool SYM, bool CS = false>
__global__ __launch_bounds__(256) void quantize_g128_kernel(const uint8_t* __restrict__ w, int64_t K, int64_t G,
                                                            int64_t chunks_per_row, int64_t total_chunks,
                                                            uint32_t* __restrict__ codes,
                                                            float* __restrict__ scales,
                                                            uint8_t* __restrict__ zeros, int64_t zeros_row_bytes,
                                                            const float* __restrict__ colscale = nullptr) {
  constexpr int kElemBytes = DT == QMM_F32 ? 4 : 2;
  const int lane = threadIdx.x & (kWave - 1);
  const int gl = lane >> 4;     // group of the chunk handled by this DPP row
  const int part = lane & 15;   // 8-element slice of the group
  const int64_t waves_per_block = blockDim.x / kWave;
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * waves_per_block;

  for (int64_t c = static_cast<int64_t>(blockIdx.x) * waves_per_block + (threadIdx.x / kWave); c < total_chunks;
       c += nwaves) {
    const int64_t n = c / chunks_per_row;
    const int64_t g = (c - n * chunks_per_row) * 4 + gl;
    const bool active = g < G;
    const int64_t e = n * K + g * kGroup + part * 8;   // first element of this lane

    float v[8];
    // Unconditional load (idle lanes re-read this row's first group) so the
    // load is not split by a branch; idle lanes store nothing.
    Vec8<DT>::load(w + (active ? e : n * K + part * 8) * kElemBytes, v);
    if constexpr (CS) {   // fl32(w * colscale[column]), as the LDS kernel
      const float* cs = colscale + (active ? g : 0) * kGroup + part * 8;
      const f32x4 f0 = *reinterpret_cast<const f32x4*>(cs);
      const f32x4 f1 = *reinterpret_cast<const f32x4*>(cs + 4);
      const float f[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = v[i] * f[i];
    }
    // Group range, widened to contain 0.
    float lo = fminf(fminf(fminf(0.0f, v[0]), fminf(v[1], v[2])), fminf(fminf(v[3], v[4]), fminf(v[5], v[6])));
    float hi = fmaxf(fmaxf(fmaxf(0.0f, v[0]), fmaxf(v[1], v[2])), fmaxf(fmaxf(v[3], v[4]), fmaxf(v[5], v[6])));
    lo = fminf(lo, v[7]);
    hi = fmaxf(hi, v[7]);
    lo = row16_min(lo);
    hi = row16_max(hi);

    float s, zf;
    group_params<SYM>(lo, hi, &s, &zf);
    const float y = 1.0f / s;           // correctly rounded reciprocal

    const uint32_t word = quantize8(v, s, y, zf);
    // Zero-point of the odd group of each pair, fetched from the next DPP row.
    const float z_next = __shfl_down(zf, 16, kWave);
    if (active) {
      codes[e >> 3] = word;
      if (part == 0) {
        scales[n * G + g] = s;
        if ((gl & 1) == 0) {
          const uint32_t zo = (g + 1 < G) ? static_cast<uint32_t>(z_next) : 0u;
          zeros[n * zeros_row_bytes + (g >> 1)] = static_cast<uint8_t>(static_cast<uint32_t>(zf) | (zo << 4));
        }
      }
    }
  }
}

template <int DT>
__global__ __launch_bounds__(256) void dequantize_g128_kernel(const uint32_t* __restrict__ codes,
                                                              const float* __restrict__ scales,
                                                              const uint8_t* __restrict__ zeros, int64_t K,
                                                              int64_t G, int64_t chunks_per_row,
                                                              int64_t total_chunks, int64_t zeros_row_bytes,
                                                              uint8_t* __restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int gl = lane >> 4;
  const int part = lane & 15;
  const int64_t waves_per_block = blockDim.x / kWave;
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * waves_per_block;

  for (int64_t c = static_cast<int64_t>(blockIdx.x) * waves_per_block + (threadIdx.x / kWave); c < total_chunks;
       c += nwaves) {
    const int64_t n = c / chunks_per_row;
    const int64_t g = (c - n * chunks_per_row) * 4 + gl;
    if (g >= G) continue;
    const int64_t e = n * K + g * kGroup + part * 8;
    const uint32_t word = __builtin_nontemporal_load(codes + (e >> 3));
    const float s = scales[n * G + g];
    const int z = static_cast<int>(zero_nibble(zeros + n * zeros_row_bytes, g));
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = static_cast<int>((word >> (4 * code_nibble(i))) & 0xFu);
      v[i] = static_cast<float>(q - z) * s;   // one fp32 rounding
    }
    if constexpr (DT == QMM_F32) {
      uint8_t* o = out + e * 4;
      st16_nt(o, u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
      st16_nt(o + 16, u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])});
    } else {
      st16_nt(out + e * 2, u32x4{pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3]), pack2<DT>(v[4], v[5]),
                                 pack2<DT>(v[6], v[7])});
    }
  }
}

// Persistent grid: enough 256-thread blocks to fill every CU several times,
// each wavefront striding over chunks.
int64_t chunk_grid(int64_t total_chunks) {
  const int64_t blocks = ceil_div(total_chunks, 4);
  const int64_t cap = static_cast<int64_t>(device_cus()) * 8;
  return blocks < cap ? blocks : cap;
}

int check_w4_args(const void* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K, int group,
                  int bits) {
  if (!codes || !scales || !zeros) return QMM_EINVAL;
  if (N <= 0 || K <= 0 || group <= 0 || K % group != 0) return QMM_EINVAL;
  if (bits != 4 || group != kGroup) return QMM_EUNSUPPORTED;
  if (!aligned(codes, 16) || !aligned(scales, 4)) return QMM_EALIGN;
  return QMM_OK;
}

}  // namespace
}  // namespace qmm

using namespace qmm;

namespace qmm {
namespace {

template <bool SYM>
int quantize_launch(const void* W, int w_dtype, int64_t N, int64_t K, int group, int bits, uint8_t* codes,
                    float* scales, uint8_t* zeros, void* stream) {
  if (!W) return QMM_EINVAL;
  if (w_dtype != QMM_F32 && w_dtype != QMM_BF16 && w_dtype != QMM_F16)
    return w_dtype == QMM_I32 ? QMM_EUNSUPPORTED : QMM_EINVAL;
  // other group sizes and bit widths: the stored formats with fp32 scales
  if (group != kGroup || bits != 4)
    return quantize_fmt(W, w_dtype, N, K, group, bits, QMM_F32, SYM ? 1 : 0, codes, scales, zeros, stream);
  int st = check_w4_args(codes, scales, zeros, N, K, group, bits);
  if (st != QMM_OK) return st;
  if (!aligned(W, 16)) return QMM_EALIGN;

  const int64_t G = K / kGroup;
  hipStream_t s = as_stream(stream);
  const uint8_t* w = static_cast<const uint8_t*>(W);
  const dim3 block(256);
  if (G % 2 == 0) {
    const int64_t T = N * G;
    const int64_t chunks = ceil_div(T, 16);
    int64_t blocks = ceil_div(chunks, 4);
    const int64_t cap = static_cast<int64_t>(device_cus()) * 16;
    if (blocks > cap) blocks = cap;
    const dim3 grid(static_cast<unsigned>(blocks));
    switch (w_dtype) {
      case QMM_BF16: quantize_g128_lds_kernel<QMM_BF16, SYM><<<grid, block, 0, s>>>(w, T, codes, scales, zeros); break;
      case QMM_F16: quantize_g128_lds_kernel<QMM_F16, SYM><<<grid, block, 0, s>>>(w, T, codes, scales, zeros); break;
      default: quantize_g128_flat_kernel<QMM_F32, SYM><<<grid, block, 0, s>>>(w, T, codes, scales, zeros); break;
    }
    return launch_status();
  }
  const int64_t chunks_per_row = ceil_div(G, 4);
  const int64_t total = N * chunks_per_row;
  const int64_t zrow = ceil_div(G, 2);
  const dim3 grid(static_cast<unsigned>(chunk_grid(total)));
  uint32_t* cw = reinterpret_cast<uint32_t*>(codes);
  switch (w_dtype) {
    case QMM_BF16:
      quantize_g128_kernel<QMM_BF16, SYM><<<grid, block, 0, s>>>(w, K, G, chunks_per_row, total, cw, scales, zeros, zrow);
      break;
    case QMM_F16:
      quantize_g128_kernel<QMM_F16, SYM><<<grid, block, 0, s>>>(w, K, G, chunks_per_row, total, cw, scales, zeros, zrow);
      break;
    default:
      quantize_g128_kernel<QMM_F32, SYM><<<grid, block, 0, s>>>(w, K, G, chunks_per_row, total, cw, scales, zeros, zrow);
      break;
  }
  return launch_status();
}

}  // namespace

namespace {

template <int DT>
void launch_colscaled_t(const uint8_t* w, const float* colscale, int64_t N, int64_t K, uint8_t* codes, float* scales,
                        uint8_t* zeros, hipStream_t s) {
  const int64_t G = K / kGroup;
  const dim3 block(256);
  if (G % 2 == 0) {
    const int64_t T = N * G;
    int64_t blocks = ceil_div(ceil_div(T, 16), 4);
    const int64_t cap = static_cast<int64_t>(device_cus()) * 16;
    if (blocks > cap) blocks = cap;
    quantize_g128_lds_kernel<DT, false, true><<<dim3(static_cast<unsigned>(blocks)), block, 0, s>>>(
        w, T, codes, scales, zeros, colscale, G);
    return;
  }
  const int64_t chunks_per_row = ceil_div(G, 4);
  const int64_t total = N * chunks_per_row;
  quantize_g128_kernel<DT, false, true><<<dim3(static_cast<unsigned>(chunk_grid(total))), block, 0, s>>>(
      w, K, G, chunks_per_row, total, reinterpret_cast<uint32_t*>(codes), scales, zeros, ceil_div(G, 2), colscale);
}

}  // namespace

void launch_quantize_colscaled(const uint16_t* W, int w_dtype, const float* colscale, int64_t N, int64_t K,
                               uint8_t* codes, float* scales, uint8_t* zeros, hipStream_t s) {
  const uint8_t* w = reinterpret_cast<const uint8_t*>(W);
  if (w_dtype == QMM_F16) launch_colscaled_t<QMM_F16>(w, colscale, N, K, codes, scales, zeros, s);
  else launch_colscaled_t<QMM_BF16>(w, colscale, N, K, codes, scales, zeros, s);
}

}  // namespace qmm

extern "C" int quantize_groupwise(const void* W, int w_dtype, int64_t N, int64_t K, int group, int bits,
                                  uint8_t* codes, float* scales, uint8_t* zeros, void* stream) {
  return quantize_launch<false>(W, w_dtype, N, K, group, bits, codes, scales, zeros, stream);
}

extern "C" int quantize_groupwise_symmetric(const void* W, int w_dtype, int64_t N, int64_t K, int group, int bits,
                                            uint8_t* codes, float* scales, uint8_t* zeros, void* stream) {
  return quantize_launch<true>(W, w_dtype, N, K, group, bits, codes, scales, zeros, stream);
}

extern "C" int dequantize(const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K,
                          int group, int bits, void* W_hat, int out_dtype, void* stream) {
  if (!W_hat) return QMM_EINVAL;
  if (out_dtype != QMM_F32 && out_dtype != QMM_BF16 && out_dtype != QMM_F16)
    return out_dtype == QMM_I32 ? QMM_EUNSUPPORTED : QMM_EINVAL;
  if (group != kGroup || bits != 4)
    return dequantize_fmt(codes, scales, zeros, N, K, group, bits, QMM_F32, W_hat, out_dtype, stream);
  int st = check_w4_args(codes, scales, zeros, N, K, group, bits);
  if (st != QMM_OK) return st;
  if (!aligned(W_hat, 16)) return QMM_EALIGN;

  const int64_t G = K / kGroup;
  const int64_t chunks_per_row = ceil_div(G, 4);
  const int64_t total = N * chunks_per_row;
  const int64_t zrow = ceil_div(G, 2);
  const dim3 grid(static_cast<unsigned>(chunk_grid(total)));
  const dim3 block(256);
  hipStream_t s = as_stream(stream);
  const uint32_t* cw = reinterpret_cast<const uint32_t*>(codes);
  uint8_t* o = static_cast<uint8_t*>(W_hat);
  switch (out_dtype) {
    case QMM_BF16:
      dequantize_g128_kernel<QMM_BF16><<<grid, block, 0, s>>>(cw, scales, zeros, K, G, chunks_per_row, total, zrow, o);
      break;
    case QMM_F16:
      dequantize_g128_kernel<QMM_F16><<<grid, block, 0, s>>>(cw, scales, zeros, K, G, chunks_per_row, total, zrow, o);
      break;
    default:
      dequantize_g128_kernel<QMM_F32><<<grid, block, 0, s>>>(cw, scales, zeros, K, G, chunks_per_row, total, zrow, o);
      break;
  }
  return launch_status();
}
