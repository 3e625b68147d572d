// formats.hip -- the stored weight formats beyond 4-bit codes with fp32
// scales per 128 weights: group sizes 32 .. 1024, 3-, 4- and 8-bit codes,
// binary16 scales, asymmetric or symmetric grids; their quantizer,
// dequantizer and matmuls; and the repack between plain nibble order and the
// library's 4-bit code words.
//
// Sources: "How quantization works" ("The math of quantization", the
// asymmetric and symmetric grids; Exercise 2, one 16-bit scale and a 4-bit
// zero-point per group of 128); "Quantization from Scratch" ("Where to put the
// scales": a 16-bit scale per group; "Measured on two real layers": 8-, 4- and
// 3-bit codes with group scales); "Quantization Explained" ("Measuring Your
// Own Error": group sizes from 32 to 1024; "The Cost of Small Groups").
//
// Stored format (fixed by include/qmm.h):
//  * codes: 4 bits -- the library's code words (element 8w+2i of a row at bits
//    4i of little-endian word w, element 8w+2i+1 at bits 16+4i); 8 bits -- one
//    byte per weight; 3 bits -- each run of 32 weights e = 0..31 of a row in
//    three little-endian words W0..W2: e < 30 in word e / 10 at bit
//    3 (r / 2) + 16 (r % 2), r = e % 10 (so consecutive codes 2m, 2m+1 sit 16
//    bits apart, like the 4-bit pairs); bit t of e = 30 at bit 15 of W[t],
//    bit t of e = 31 at bit 31 of W[t].
//  * scales: [N, G] fp32 or binary16.  The codes are computed with the stored
//    value: a binary16 scale is the fp32 scale rounded to nearest even
//    (saturating at 65504), and 1 if that is 0.
//  * zeros: [N, ceil(G/2)] nibble pairs up to 4 bits, [N, G] bytes at 8 bits.
//
// Every kernel maps a lane to 32 consecutive weights of a row (a group of G
// weights is G/32 lanes), so per-group min/max, scale and zero-point need at
// most a 32-lane reduction, and a lane's weights lie in one group.

#include <algorithm>

#include "qmm_device.h"

namespace qmm {
namespace {

typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

constexpr int kChunk = 2048;                 // weights of a row per wavefront pass (64 lanes x 32)
constexpr float kScaleMax16 = 65504.0f;      // largest finite binary16

// ---- stored scale and zero-point ---------------------------------------------
// The value a scale takes when stored (the codes are computed with it).
__device__ __forceinline__ float stored_scale(float s, bool s16) {
  if (!s16) return s;
  const _Float16 h = static_cast<_Float16>(s >= kScaleMax16 ? kScaleMax16 : s);   // round to nearest even
  const float v = static_cast<float>(h);
  return v == 0.0f ? 1.0f : v;
}

__device__ __forceinline__ float load_scale(const void* scales, int64_t idx, bool s16) {
  return s16 ? static_cast<float>(static_cast<const _Float16*>(scales)[idx]) : static_cast<const float*>(scales)[idx];
}

template <int BITS>
__device__ __forceinline__ uint32_t load_zero(const uint8_t* zrow, int64_t g) {
  if constexpr (BITS == 8) {
    return zrow[g];
  } else {
    const uint32_t b = zrow[g >> 1];
    return (g & 1) ? (b >> 4) : (b & 0xFu);
  }
}

__host__ __device__ constexpr int64_t zero_row_bytes(int64_t G, int bits) { return bits <= 4 ? (G + 1) / 2 : G; }
__host__ __device__ constexpr int64_t code_row_bytes(int64_t K, int bits) { return K * bits / 8; }

// ---- codes of 32 weights -------------------------------------------------------
// Stored words of a lane's 32 codes (4 bits: 4 words, 8 bits: 8, 3 bits: 3).
template <int BITS>
struct Lane32 {
  static constexpr int kWords = BITS * 32 / 32;
  uint32_t w[kWords];
};

template <int BITS>
__device__ __forceinline__ void pack32(const float c[32], Lane32<BITS>& out) {
  if constexpr (BITS == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) word |= static_cast<uint32_t>(c[8 * j + i]) << (4 * code_nibble(i));
      out.w[j] = word;
    }
  } else if constexpr (BITS == 8) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) word |= static_cast<uint32_t>(c[4 * j + i]) << (8 * i);
      out.w[j] = word;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      uint32_t word = 0;
#pragma unroll
      for (int r = 0; r < 10; ++r) word |= static_cast<uint32_t>(c[10 * j + r]) << (3 * (r >> 1) + 16 * (r & 1));
      const uint32_t v30 = static_cast<uint32_t>(c[30]), v31 = static_cast<uint32_t>(c[31]);
      word |= ((v30 >> j) & 1u) << 15;
      word |= ((v31 >> j) & 1u) << 31;
      out.w[j] = word;
    }
  }
}

// Code i (0..31) of a lane's stored words.
template <int BITS>
__device__ __forceinline__ int code_at(const Lane32<BITS>& l, int i) {
  if constexpr (BITS == 4) {
    return static_cast<int>((l.w[i >> 3] >> (4 * code_nibble(i & 7))) & 0xFu);
  } else if constexpr (BITS == 8) {
    return static_cast<int>((l.w[i >> 2] >> (8 * (i & 3))) & 0xFFu);
  } else {
    if (i < 30) {
      const int r = i % 10;
      return static_cast<int>((l.w[i / 10] >> (3 * (r >> 1) + 16 * (r & 1))) & 7u);
    }
    const int b = i == 30 ? 15 : 31;
    return static_cast<int>(((l.w[0] >> b) & 1u) | (((l.w[1] >> b) & 1u) << 1) | (((l.w[2] >> b) & 1u) << 2));
  }
}

template <int BITS>
__device__ __forceinline__ void load32(const uint8_t* p, Lane32<BITS>& l) {
  if constexpr (BITS == 4) {
    const u32x4 a = ld16_nt(p);
    l.w[0] = a.x; l.w[1] = a.y; l.w[2] = a.z; l.w[3] = a.w;
  } else if constexpr (BITS == 8) {
    const u32x4 a = ld16_nt(p);
    const u32x4 b = ld16_nt(p + 16);
    l.w[0] = a.x; l.w[1] = a.y; l.w[2] = a.z; l.w[3] = a.w;
    l.w[4] = b.x; l.w[5] = b.y; l.w[6] = b.z; l.w[7] = b.w;
  } else {   // one 12-byte access for the 96-bit slice
    const u32x3 a = __builtin_nontemporal_load(reinterpret_cast<const u32x3*>(p));
    l.w[0] = a.x; l.w[1] = a.y; l.w[2] = a.z;
  }
}

template <int BITS>
__device__ __forceinline__ void store32(uint8_t* p, const Lane32<BITS>& l) {
  if constexpr (BITS == 4) {
    st16_nt(p, u32x4{l.w[0], l.w[1], l.w[2], l.w[3]});
  } else if constexpr (BITS == 8) {
    st16_nt(p, u32x4{l.w[0], l.w[1], l.w[2], l.w[3]});
    st16_nt(p + 16, u32x4{l.w[4], l.w[5], l.w[6], l.w[7]});
  } else {
    __builtin_nontemporal_store(u32x3{l.w[0], l.w[1], l.w[2]}, reinterpret_cast<u32x3*>(p));
  }
}

// Reduction over the L lanes of a group (L a power of two up to 32).
__device__ __forceinline__ float group_min(float v, int L) {
  for (int o = 1; o < L; o <<= 1) v = fminf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float group_max(float v, int L) {
  for (int o = 1; o < L; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// ----------------------------------------------------------------------------
// Quantizer.  A wavefront takes 2048 weights of one row per pass (lane l:
// weights 32 l .. +32 of the pass), so a group of G weights is G / 32
// consecutive lanes and every pair of groups (2j, 2j+1) sharing a zero-point
// byte sits in one pass.  Codes are clamp(rint(fl32(w / s)) + z, 0, 2^b - 1)
// bit for bit, through a correctly rounded reciprocal and one fma correction
// (the correction of the 4-bit quantizer), exact division outside
// [2^-100, 2^100].
// ----------------------------------------------------------------------------
// The arithmetic of one lane's 32 weights v (weights kl .. kl + 31 of row n;
// `active` false for lanes past K, which compute but store nothing).
template <int BITS, bool SYM>
__device__ __forceinline__ void quantize_fmt_lane(const float v[32], int lane, int L, int lg, int s16, bool active,
                                                  int64_t n, int64_t kl, int64_t K, int64_t G, int64_t zrb,
                                                  uint8_t* __restrict__ codes, void* __restrict__ scales,
                                                  uint8_t* __restrict__ zeros) {
  constexpr float kQmax = static_cast<float>((1 << BITS) - 1);
  constexpr float kHalf = static_cast<float>(1 << (BITS - 1));
  float s, zf;
  if constexpr (SYM) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = group_max(amax, L);
    s = stored_scale(fmaxf(amax, 1e-8f) / (kHalf - 1.0f), s16 != 0);
    zf = kHalf;
  } else {
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      lo = fminf(lo, v[i]);
      hi = fmaxf(hi, v[i]);
    }
    lo = group_min(lo, L);
    hi = group_max(hi, L);
    float sc = (hi - lo) / kQmax;                    // correctly rounded fp32 division
    if (sc == 0.0f) sc = 1.0f;
    s = stored_scale(sc, s16 != 0);
    zf = fminf(rintf(-lo / s), kQmax);               // beyond kQmax only for a saturated 16-bit scale
  }
  const float y = 1.0f / s;
  const bool scale_ok = (s >= 0x1p-100f) && (s <= 0x1p100f);
  float cq[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float q0 = v[i] * y;
    const float r = fmaf(-q0, s, v[i]);
    cq[i] = rintf(fmaf(r, y, q0)) + zf;
  }
  if (__builtin_amdgcn_ballot_w64(!scale_ok)) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float e = rintf(v[i] / s) + zf;
      if (!scale_ok) cq[i] = e;
    }
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) cq[i] = __builtin_amdgcn_fmed3f(cq[i], 0.0f, kQmax);
  Lane32<BITS> out;
  pack32<BITS>(cq, out);
  const float z_next = __shfl_down(zf, L, kWave);      // zero-point of the next group
  if (active) {
    store32<BITS>(codes + n * code_row_bytes(K, BITS) + kl * BITS / 8, out);
    const int64_t g = kl >> lg;
    if ((lane & (L - 1)) == 0) {
      if (s16) {
        static_cast<uint16_t*>(scales)[n * G + g] = static_cast<uint16_t>(f32_to_f16_bits(s));
      } else {
        static_cast<float*>(scales)[n * G + g] = s;
      }
      if constexpr (BITS == 8) {
        zeros[n * zrb + g] = static_cast<uint8_t>(zf);
      } else if ((g & 1) == 0) {
        const uint32_t zo = (g + 1 < G) ? static_cast<uint32_t>(z_next) : 0u;
        zeros[n * zrb + (g >> 1)] = static_cast<uint8_t>(static_cast<uint32_t>(zf) | (zo << 4));
      }
    }
  }
}

template <int DT, int BITS, bool SYM>
__global__ __launch_bounds__(256) void quantize_fmt_kernel(const uint8_t* __restrict__ w, int64_t N, int64_t K,
                                                           int lg, int s16, uint8_t* __restrict__ codes,
                                                           void* __restrict__ scales, uint8_t* __restrict__ zeros) {
  constexpr int kElem = DT == QMM_F32 ? 4 : 2;
  const int lane = threadIdx.x & (kWave - 1);
  const int L = 1 << (lg - 5);
  const int64_t G = K >> lg;
  const int64_t cpr = (K + kChunk - 1) / kChunk;
  const int64_t total = N * cpr;
  const int64_t zrb = zero_row_bytes(G, BITS);
  const int64_t waves_per_block = blockDim.x / kWave;
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * waves_per_block;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * waves_per_block + (threadIdx.x / kWave); c < total;
       c += nwaves) {
    const int64_t n = c / cpr;
    const int64_t k = (c - n * cpr) * kChunk + static_cast<int64_t>(lane) * 32;
    const bool active = k < K;
    const int64_t kl = active ? k : 0;                  // idle lanes read their row's first weights
    const uint8_t* src = w + (n * K + kl) * kElem;
    float v[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) Vec8<DT>::load(src + q * 8 * kElem, &v[8 * q]);
    quantize_fmt_lane<BITS, SYM>(v, lane, L, lg, s16, active, n, kl, K, G, zrb, codes, scales, zeros);
  }
}

// 16-bit weights: each wavefront's 2048-weight chunk (4 KiB, contiguous in
// its row) reaches LDS by four buffer loads that each cover 1 KiB
// contiguously -- every lane loading its own 64 bytes spans 4 KiB per
// instruction -- double buffered (the next chunk's loads issued before the
// current one is read).  LDS slots as in the 4-bit quantizer of 16-bit
// weights: 16-byte piece P (lane l reads pieces 4l .. 4l+3) at slot
// 64 (P / 64) + 4 m + ((j + m / 4) & 3), m = (P / 4) % 16, j = P % 4, so the
// four reads of each lane are free of bank conflicts.  Bytes of a chunk past
// the end of its row read zero.
constexpr int kFmtChunkBytes = kChunk * 2;

template <int DT, int BITS, bool SYM>
__global__ __launch_bounds__(256) void quantize_fmt_lds_kernel(const uint8_t* __restrict__ w, int64_t N, int64_t K,
                                                               int lg, int s16, uint8_t* __restrict__ codes,
                                                               void* __restrict__ scales,
                                                               uint8_t* __restrict__ zeros) {
  static_assert(DT != QMM_F32, "16-bit weights only");
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * 2 * kFmtChunkBytes];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int L = 1 << (lg - 5);
  const int64_t G = K >> lg;
  const int64_t cpr = (K + kChunk - 1) / kChunk;
  const int64_t total = N * cpr;
  const int64_t zrb = zero_row_bytes(G, BITS);
  const int64_t waves_per_block = blockDim.x / kWave;
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * waves_per_block;
  const uint32_t wbase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)) + wave * 2 * kFmtChunkBytes;

  // Load lane l of instruction q fetches piece 64 q + 4 m + ((l % 4 - m / 4) & 3),
  // m = l / 4, and writes slot 64 q + l.
  const int lm = lane >> 2;
  const int fetch = (4 * lm + (((lane & 3) - (lm >> 2)) & 3)) * 16;
  auto issue = [&](int64_t c, int buf) {
    const int64_t n = c / cpr;
    const int64_t k0 = (c - n * cpr) * kChunk;
    const int64_t left = (K - k0) * 2;
    const int bytes = static_cast<int>(left < kFmtChunkBytes ? left : kFmtChunkBytes);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(w + (n * K + k0) * 2), 0, bytes, kBufferWord3);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t dst = wbase + buf * kFmtChunkBytes + q * 1024;
      int off = fetch + q * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(uintptr_t)dst, 16, off, 0, 0, 0);
    }
  };
  // Reader: lane l's pieces 4l + j are in instruction l / 16, m = l % 16.
  const int rm = lane & 15;
  int rd[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) rd[j] = (lane >> 4) * 1024 + (4 * rm + ((j + (rm >> 2)) & 3)) * 16;

  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * waves_per_block + wave;
  int buf = 0;
  if (c0 < total) issue(c0, 0);
  for (int64_t c = c0; c < total; c += nwaves, buf ^= 1) {
    const bool next = c + nwaves < total;   // uniform
    if (next) {
      issue(c + nwaves, buf ^ 1);
      wait_vm<4>();
    } else {
      wait_vm<0>();
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint8_t* cb = lds + wave * 2 * kFmtChunkBytes + buf * kFmtChunkBytes;
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
    const int64_t n = c / cpr;
    const int64_t k = (c - n * cpr) * kChunk + static_cast<int64_t>(lane) * 32;
    const bool active = k < K;
    quantize_fmt_lane<BITS, SYM>(v, lane, L, lg, s16, active, n, active ? k : 0, K, G, zrb, codes, scales, zeros);
    // the LDS reads of this chunk are done before the next iteration's
    // loads overwrite its buffer (they feed the arithmetic above)
  }
}

// ----------------------------------------------------------------------------
// Dequantizer: w_hat = (q - z) s, one fp32 rounding, 32 weights per lane.
// ----------------------------------------------------------------------------
template <int ODT, int BITS>
__global__ __launch_bounds__(256) void dequantize_fmt_kernel(const uint8_t* __restrict__ codes,
                                                             const void* __restrict__ scales,
                                                             const uint8_t* __restrict__ zeros, int64_t N, int64_t K,
                                                             int lg, int s16, uint8_t* __restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t G = K >> lg;
  const int64_t cpr = (K + kChunk - 1) / kChunk;
  const int64_t total = N * cpr;
  const int64_t zrb = zero_row_bytes(G, BITS);
  const int64_t waves_per_block = blockDim.x / kWave;
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * waves_per_block;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * waves_per_block + (threadIdx.x / kWave); c < total;
       c += nwaves) {
    const int64_t n = c / cpr;
    const int64_t k = (c - n * cpr) * kChunk + static_cast<int64_t>(lane) * 32;
    if (k >= K) continue;
    Lane32<BITS> l;
    load32<BITS>(codes + n * code_row_bytes(K, BITS) + k * BITS / 8, l);
    const int64_t g = k >> lg;
    const float s = load_scale(scales, n * G + g, s16 != 0);
    const int z = static_cast<int>(load_zero<BITS>(zeros + n * zrb, g));
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = static_cast<float>(code_at<BITS>(l, i) - z) * s;
    const int64_t e = n * K + k;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (ODT == QMM_F32) {
        uint8_t* o = out + (e + 8 * q) * 4;
        st16_nt(o, u32x4{__float_as_uint(v[8 * q]), __float_as_uint(v[8 * q + 1]), __float_as_uint(v[8 * q + 2]),
                         __float_as_uint(v[8 * q + 3])});
        st16_nt(o + 16, u32x4{__float_as_uint(v[8 * q + 4]), __float_as_uint(v[8 * q + 5]),
                              __float_as_uint(v[8 * q + 6]), __float_as_uint(v[8 * q + 7])});
      } else {
        st16_nt(out + (e + 8 * q) * 2, u32x4{pack2<ODT>(v[8 * q], v[8 * q + 1]), pack2<ODT>(v[8 * q + 2], v[8 * q + 3]),
                                             pack2<ODT>(v[8 * q + 4], v[8 * q + 5]),
                                             pack2<ODT>(v[8 * q + 6], v[8 * q + 7])});
      }
    }
  }
}

// ----------------------------------------------------------------------------
// 16-bit float pairs of consecutive codes, exact, for dot2 / MFMA against the
// activations as loaded.  Each pair is (off + q_2j, off + q_2j+1):
//  * 4 bits: the nibble magic of the 4-bit kernels (off 128 bf16, 16 fp16);
//  * 3 bits: a 6-bit field holds a pair, each code placed one step lower in
//    the mantissa (off 8, Int3Magic);
//  * 8 bits: byte -> fp32 (exact), then the pair packed (off 0; an integer up
//    to 255 has 8 significant bits, exact in bf16 and fp16).
// ----------------------------------------------------------------------------
// 3-bit codes sit one step lower in the mantissa than the 4-bit nibbles, at
// offset 8 instead of 128 (bf16) / 16 (fp16): 8.0 = 0x4100 (bf16, one code
// step at mantissa bit 4) or 0x4800 (fp16, bit 7); a smaller offset cancels
// less in the fold.
template <int XDT>
struct Int3Magic;
template <>
struct Int3Magic<QMM_BF16> {
  static constexpr float offset = 8.0f;
  static constexpr uint32_t kMagic = 0x41004100u;
};
template <>
struct Int3Magic<QMM_F16> {
  static constexpr float offset = 8.0f;
  static constexpr uint32_t kMagic = 0x48004800u;
};

template <int XDT, int BITS>
struct PairOff {
  static constexpr float value = BITS == 8 ? 0.0f : (BITS == 3 ? Int3Magic<XDT>::offset : Int4Magic<XDT>::offset);
  static constexpr uint32_t magic = BITS == 3 ? Int3Magic<XDT>::kMagic : Int4Magic<XDT>::kMagic;
};

// Pair i (0..4) of a 3-bit code word -- the codes at bits 3i and 16 + 3i --
// moved to the magic's mantissa position with one shift and one AND-OR.
template <int XDT>
__device__ __forceinline__ uint32_t pair3_at(uint32_t w, int i, uint32_t magic) {
  constexpr int kPos = XDT == QMM_BF16 ? 4 : 7;
  constexpr uint32_t kMask = 0x00070007u << kPos;
  const int sh = kPos - 3 * i;
  return ((sh >= 0 ? w << sh : w >> -sh) & kMask) | magic;
}

// The run's last pair (codes 30 and 31), one bit from each word's bits 15 and 31.
template <int XDT>
__device__ __forceinline__ uint32_t pair3_last(const uint32_t w[3], uint32_t magic) {
  constexpr int kPos = XDT == QMM_BF16 ? 4 : 7;
  uint32_t p = ((w[0] >> (15 - kPos)) & (0x00010001u << kPos)) | magic;
  p |= (w[1] >> (14 - kPos)) & (0x00020002u << kPos);
  p |= (w[2] >> (13 - kPos)) & (0x00040004u << kPos);
  return p;
}

template <int XDT>
__device__ __forceinline__ uint32_t pair_from_bytes(uint32_t w, int b0) {
  // bytes b0 and b0 + 1 of w
  const float f0 = static_cast<float>((w >> (8 * b0)) & 0xFFu);
  const float f1 = static_cast<float>((w >> (8 * b0 + 8)) & 0xFFu);
  if constexpr (XDT == QMM_BF16) {
    return __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  } else {
    return f32_to_f16_bits(f0) | (f32_to_f16_bits(f1) << 16);
  }
}

template <int YDT>
__device__ __forceinline__ void store_out(void* y, int64_t idx, float v) {
  if constexpr (YDT == QMM_F32) {
    static_cast<float*>(y)[idx] = v;
  } else if constexpr (YDT == QMM_BF16) {
    static_cast<uint16_t*>(y)[idx] = static_cast<uint16_t>(f32_to_bf16_bits(v));
  } else {
    static_cast<uint16_t*>(y)[idx] = static_cast<uint16_t>(f32_to_f16_bits(v));
  }
}

// ----------------------------------------------------------------------------
// Vector-ALU GEMV for one or two tokens: a block of 4 wavefronts owns 8
// weight rows; per step a lane takes a slice of each row -- 32 weights of 3-
// or 4-bit codes (12 or 16 bytes), 16 weights of 8-bit codes (16 bytes) --
// inside one group (one scale and zero-point per row), converts it to pairs
// and multiplies with v_dot2 against the activations as loaded; per lane and
// row the group fold s (sum (off + q) x - (off + z) sum x) is exact in the
// products.  The scale type is a template parameter, so every load of a step
// is issued before any arithmetic.
// ----------------------------------------------------------------------------
constexpr int kFmtWaves = 4;
constexpr int kFmtRows = 8;

template <int BITS>
struct Slice {
  static constexpr int kWeights = BITS == 8 ? 16 : 32;   // weights of a row per lane per step
  static constexpr int kWords = BITS == 3 ? 3 : 4;       // code words per lane per row
  static constexpr int kPairs = kWeights / 2;
  static constexpr int kXVec = kWeights / 8;             // 16-byte activation loads per token
  uint32_t w[kWords];
};

template <int BITS>
__device__ __forceinline__ void load_slice(const uint8_t* p, Slice<BITS>& sl) {
  if constexpr (BITS == 3) {   // one 12-byte load (dwordx3) for the 96-bit slice
    const u32x3 a = __builtin_nontemporal_load(reinterpret_cast<const u32x3*>(p));
    sl.w[0] = a.x; sl.w[1] = a.y; sl.w[2] = a.z;
  } else {
    const u32x4 a = ld16_nt(p);
    sl.w[0] = a.x; sl.w[1] = a.y; sl.w[2] = a.z; sl.w[3] = a.w;
  }
}


template <int XDT, int BITS>
__device__ __forceinline__ void slice_pairs(const Slice<BITS>& sl, uint32_t magic, uint32_t p[Slice<BITS>::kPairs]) {
  if constexpr (BITS == 4) {
#pragma unroll
    for (int c = 0; c < 4; ++c) Int4Magic<XDT>::unpack(sl.w[c], magic, &p[4 * c]);
  } else if constexpr (BITS == 8) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      p[2 * c] = pair_from_bytes<XDT>(sl.w[c], 0);
      p[2 * c + 1] = pair_from_bytes<XDT>(sl.w[c], 2);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
      for (int i = 0; i < 5; ++i) p[5 * j + i] = pair3_at<XDT>(sl.w[j], i, magic);
    p[15] = pair3_last<XDT>(sl.w, magic);
  }
}

template <bool S16>
__device__ __forceinline__ float scale_at(const void* scales, int64_t idx) {
  if constexpr (S16) {
    return static_cast<float>(static_cast<const _Float16*>(scales)[idx]);
  } else {
    return static_cast<const float*>(scales)[idx];
  }
}

template <int XDT, int YDT, int B, int BITS, bool S16>
__global__ __launch_bounds__(256) void gemv_fmt_kernel(const uint8_t* __restrict__ codes,
                                                       const void* __restrict__ scales,
                                                       const uint8_t* __restrict__ zeros, int64_t N, int64_t K, int lg,
                                                       const uint16_t* __restrict__ x, void* __restrict__ y) {
  constexpr int R = kFmtRows;
  using Sl = Slice<BITS>;
  constexpr int LW = Sl::kWeights;
  constexpr int64_t kStep = kFmtWaves * kWave * LW;
  using Mg = Int4Magic<XDT>;
  constexpr float kOff = PairOff<XDT, BITS>::value;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * R;
  const uint32_t magic = vgpr_const(PairOff<XDT, BITS>::magic);
  const int64_t G = K >> lg;
  const int64_t zrb = zero_row_bytes(G, BITS);
  const int64_t crb = code_row_bytes(K, BITS);
  int64_t rows[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rows[r] = (row0 + r < N) ? row0 + r : N - 1;
  float acc[R][B];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;

  for (int64_t k0 = 0; k0 < K; k0 += kStep) {
    if (k0 + wave * (kWave * LW) >= K) break;
    const int64_t kb_raw = k0 + wave * (kWave * LW) + lane * LW;
    const bool inside = kb_raw < K;
    const int64_t kb = inside ? kb_raw : K - LW;
    u32x4 xraw[B][Sl::kXVec];
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int c = 0; c < Sl::kXVec; ++c) xraw[b][c] = ld16(x + b * K + kb + 8 * c);
    const int64_t g = kb >> lg;
    float sc[R];
    uint32_t zb[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      sc[r] = scale_at<S16>(scales, rows[r] * G + g);
      zb[r] = load_zero<BITS>(zeros + rows[r] * zrb, g);
    }
    Sl cw[R];
#pragma unroll
    for (int r = 0; r < R; ++r) load_slice<BITS>(codes + rows[r] * crb + kb * BITS / 8, cw[r]);
    __builtin_amdgcn_sched_barrier(0);
    if (!inside) {
#pragma unroll
      for (int b = 0; b < B; ++b)
#pragma unroll
        for (int c = 0; c < Sl::kXVec; ++c) xraw[b][c] = u32x4{0u, 0u, 0u, 0u};
    }
    uint32_t xp[B][Sl::kPairs];
    float xs[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
#pragma unroll
      for (int c = 0; c < Sl::kXVec; ++c) {
        xp[b][4 * c] = xraw[b][c].x;
        xp[b][4 * c + 1] = xraw[b][c].y;
        xp[b][4 * c + 2] = xraw[b][c].z;
        xp[b][4 * c + 3] = xraw[b][c].w;
      }
      float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
      for (int j = 0; j < Sl::kPairs; j += 2) {
        s0 = dot2<XDT>(xp[b][j], Mg::one_pair, s0);
        s1 = dot2<XDT>(xp[b][j + 1], Mg::one_pair, s1);
      }
      xs[b] = s0 + s1;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      uint32_t p[Sl::kPairs];
      slice_pairs<XDT, BITS>(cw[r], magic, p);
      const float zo = kOff + static_cast<float>(zb[r]);
#pragma unroll
      for (int b = 0; b < B; ++b) {
        float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
        for (int j = 0; j < Sl::kPairs; j += 2) {
          a0 = dot2<XDT>(p[j], xp[b][j], a0);
          a1 = dot2<XDT>(p[j + 1], xp[b][j + 1], a1);
        }
        acc[r][b] = fmaf(sc[r], fmaf(-zo, xs[b], a0 + a1), acc[r][b]);
      }
    }
  }

  __shared__ float red[kFmtWaves][R * B];
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
      for (int w = 0; w < kFmtWaves; ++w) v += red[w][threadIdx.x];
      store_out<YDT>(y, static_cast<int64_t>(b) * N + row, v);
    }
  }
}

// ----------------------------------------------------------------------------
// MFMA kernel for 3 or more tokens: block = 4 wavefronts, output tile 16
// tokens x 64 weight rows; the wavefronts split K into contiguous ranges of
// 32-weight chunks and their partial tiles are summed through LDS at the end.
// v_mfma_f32_16x16x32_{bf16,f16}: the weights are the A operand straight from
// registers (lane l: row l % 16 of a 16-row slice, weights 8 (l / 16) .. +8 of
// the chunk), the activations the B operand as loaded (lane l: token l % 16);
// one more MFMA against a ones operand gives the chunk's activation sums.
// Products of a group accumulate in P and are folded every 128 weights, at
// the group's end and at the end of the wavefront's range, as
// acc += s (P - (off + z) X) (linear in the pieces); D lane l
// holds rows 4 (l / 16) .. +4 of token l % 16, whose scales and zero-points
// are loaded one per lane and broadcast within each quad.
// ----------------------------------------------------------------------------
template <int XDT>
__device__ __forceinline__ f32x4 mfma_k32(const uint32_t a[4], const uint32_t b[4], f32x4 c) {
  const u32x4 av = {a[0], a[1], a[2], a[3]};
  const u32x4 bv = {b[0], b[1], b[2], b[3]};
  if constexpr (XDT == QMM_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bv),
                                                   c, 0, 0, 0);
  } else {
    typedef _Float16 f16x8_v __attribute__((ext_vector_type(8)));
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_v, av), __builtin_bit_cast(f16x8_v, bv), c,
                                                  0, 0, 0);
  }
}

constexpr int kMfmaRT = 4;   // 16-row slices per block

// Eight codes of a row at weight k (a multiple of 8) as four pairs.
template <int XDT, int BITS>
__device__ __forceinline__ void load_pairs8(const uint8_t* crow, int64_t k, uint32_t magic, uint32_t p[4]) {
  if constexpr (BITS == 4) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(crow + (k >> 1));
    Int4Magic<XDT>::unpack(w, magic, p);
  } else if constexpr (BITS == 8) {
    const uint2 w = *reinterpret_cast<const uint2*>(crow + k);
    p[0] = pair_from_bytes<XDT>(w.x, 0);
    p[1] = pair_from_bytes<XDT>(w.x, 2);
    p[2] = pair_from_bytes<XDT>(w.y, 0);
    p[3] = pair_from_bytes<XDT>(w.y, 2);
  } else {
    // pairs 4q .. 4q + 3 of the run's 16 (q = (k % 32) / 8)
    const uint32_t* wc = reinterpret_cast<const uint32_t*>(crow + (k >> 5) * 12);
    const int q = static_cast<int>((k >> 3) & 3);
    const uint32_t w[3] = {wc[0], wc[1], wc[2]};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = 4 * q + j;
      p[j] = m == 15 ? pair3_last<XDT>(w, magic) : pair3_at<XDT>(m < 5 ? w[0] : m < 10 ? w[1] : w[2], m % 5, magic);
    }
  }
}

template <int XDT, int YDT, int BITS, bool S16>
__global__ __launch_bounds__(256) void wq_mfma_kernel(const uint8_t* __restrict__ codes,
                                                      const void* __restrict__ scales,
                                                      const uint8_t* __restrict__ zeros, int64_t N, int64_t K, int lg,
                                                      const uint16_t* __restrict__ x, int64_t M,
                                                      void* __restrict__ y) {
  using Mg = Int4Magic<XDT>;
  constexpr int RT = kMfmaRT;
  constexpr float kOff = PairOff<XDT, BITS>::value;
  __shared__ float red[kFmtWaves][RT * 4][kWave];
  const uint32_t magic = vgpr_const(PairOff<XDT, BITS>::magic);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int l16 = lane & 15;
  const int quad = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * 16 * RT;
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * 16;
  const int64_t G = K >> lg;
  const int64_t zrb = zero_row_bytes(G, BITS);
  const int64_t crb = code_row_bytes(K, BITS);
  const int64_t nch = K >> 5;
  const int64_t per = (nch + kFmtWaves - 1) / kFmtWaves;
  const int64_t cbeg = wave * per;
  const int64_t cend = (cbeg + per < nch) ? cbeg + per : nch;

  const uint8_t* arow[RT];
  int64_t srow[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int64_t ra = row0 + 16 * rt + l16;
    const int64_t rs = row0 + 16 * rt + 4 * quad + (lane & 3);
    arow[rt] = codes + ((ra < N) ? ra : N - 1) * crb;
    srow[rt] = (rs < N) ? rs : N - 1;
  }
  const int64_t tok = (t0 + l16 < M) ? t0 + l16 : M - 1;
  const uint16_t* xrow = x + tok * K + 8 * quad;
  const uint32_t ones[4] = {Mg::one_pair, Mg::one_pair, Mg::one_pair, Mg::one_pair};

  f32x4 acc[RT], pacc[RT];
  f32x4 xsum = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) acc[rt] = pacc[rt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  for (int64_t c = cbeg; c < cend; ++c) {
    const int64_t k0 = c << 5;
    const int64_t g = k0 >> lg;
    uint32_t a[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) load_pairs8<XDT, BITS>(arow[rt], k0 + 8 * quad, magic, a[rt]);
    const u32x4 xv = ld16(xrow + k0);
    const uint32_t b[4] = {xv.x, xv.y, xv.z, xv.w};
    // fold at the group's end, and at least every 128 weights, so the sums
    // that cancel against (off + z) X stay short
    const bool fold = (c + 1 == cend) || ((c + 1) & 3) == 0 || (((c + 1) << 5) >> lg) != g;
    float sv[RT], zv[RT];
    if (fold) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        sv[rt] = scale_at<S16>(scales, srow[rt] * G + g);
        zv[rt] = kOff + static_cast<float>(load_zero<BITS>(zeros + srow[rt] * zrb, g));
      }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) pacc[rt] = mfma_k32<XDT>(a[rt], b, pacc[rt]);
    xsum = mfma_k32<XDT>(ones, b, xsum);
    if (fold) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float s4[4] = {dpp_f<0x00>(sv[rt]), dpp_f<0x55>(sv[rt]), dpp_f<0xAA>(sv[rt]), dpp_f<0xFF>(sv[rt])};
        const float z4[4] = {dpp_f<0x00>(zv[rt]), dpp_f<0x55>(zv[rt]), dpp_f<0xAA>(zv[rt]), dpp_f<0xFF>(zv[rt])};
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[rt][i] = fmaf(s4[i], fmaf(-z4[i], xsum[i], pacc[rt][i]), acc[rt][i]);
        pacc[rt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
      xsum = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }

#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][rt * 4 + i][lane] = acc[rt][i];
  __syncthreads();
  for (int o = threadIdx.x; o < RT * 4 * kWave; o += blockDim.x) {
    const int slot = o / kWave;
    const int l = o % kWave;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kFmtWaves; ++w) v += red[w][slot][l];
    const int rt = slot / 4;
    const int i = slot % 4;
    const int64_t row = row0 + 16 * rt + 4 * (l >> 4) + i;
    const int64_t t = t0 + (l & 15);
    if (row < N && t < M) store_out<YDT>(y, t * N + row, v);
  }
}

// ----------------------------------------------------------------------------
// Repack between plain nibble order (element 2j in the low nibble of byte j,
// 2j+1 in the high nibble: element e of an 8-element word at bits 4e) and the
// library's code words (element 2i at bits 4i, 2i+1 at bits 16+4i).
// ----------------------------------------------------------------------------
__device__ __forceinline__ uint32_t plain_to_words(uint32_t p) {
  uint32_t even = 0, odd = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    even |= ((p >> (8 * i)) & 0xFu) << (4 * i);
    odd |= ((p >> (8 * i + 4)) & 0xFu) << (4 * i);
  }
  return even | (odd << 16);
}
__device__ __forceinline__ uint32_t words_to_plain(uint32_t w) {
  uint32_t p = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p |= ((w >> (4 * i)) & 0xFu) << (8 * i);
    p |= ((w >> (16 + 4 * i)) & 0xFu) << (8 * i + 4);
  }
  return p;
}

template <bool TO_WORDS>
__global__ __launch_bounds__(256) void repack_kernel(const uint32_t* in, uint32_t* out,
                                                     int64_t nwords) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t nvec = nwords / 4;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < nvec; i += stride) {
    const u32x4 v = ld16_nt(in + 4 * i);
    const u32x4 r = TO_WORDS ? u32x4{plain_to_words(v.x), plain_to_words(v.y), plain_to_words(v.z), plain_to_words(v.w)}
                             : u32x4{words_to_plain(v.x), words_to_plain(v.y), words_to_plain(v.z), words_to_plain(v.w)};
    st16_nt(out + 4 * i, r);
  }
  const int64_t tail = nvec * 4 + static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (tail < nwords) out[tail] = TO_WORDS ? plain_to_words(in[tail]) : words_to_plain(in[tail]);
}

// ---- host side -----------------------------------------------------------------
int log2_group(int group) {
  for (int lg = 5; lg <= 10; ++lg)
    if (group == (1 << lg)) return lg;
  return -1;
}

// Arguments shared by every format entry point.
int check_fmt(const void* codes, const void* scales, const uint8_t* zeros, int64_t N, int64_t K, int group, int bits,
              int scale_dtype) {
  if (!codes || !scales || !zeros) return QMM_EINVAL;
  if (N <= 0 || K <= 0 || group <= 0 || K % group != 0) return QMM_EINVAL;
  if (scale_dtype != QMM_F32 && scale_dtype != QMM_F16) return scale_dtype == QMM_BF16 ? QMM_EUNSUPPORTED : QMM_EINVAL;
  if ((bits != 3 && bits != 4 && bits != 8) || log2_group(group) < 0) return QMM_EUNSUPPORTED;
  if (!aligned(codes, 16) || !aligned(scales, scale_dtype == QMM_F32 ? 4 : 2)) return QMM_EALIGN;
  return QMM_OK;
}

int64_t fmt_grid(int64_t N, int64_t K) {
  const int64_t blocks = ceil_div(N * ceil_div(K, kChunk), 4);
  const int64_t cap = static_cast<int64_t>(device_cus()) * 16;
  return blocks < cap ? blocks : cap;
}

template <int BITS, bool SYM>
void launch_quant_fmt(const uint8_t* w, int dt, int64_t N, int64_t K, int lg, int s16, uint8_t* codes, void* scales,
                      uint8_t* zeros, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(fmt_grid(N, K)));
  switch (dt) {
    case QMM_BF16:
      quantize_fmt_lds_kernel<QMM_BF16, BITS, SYM><<<grid, 256, 0, s>>>(w, N, K, lg, s16, codes, scales, zeros);
      break;
    case QMM_F16:
      quantize_fmt_lds_kernel<QMM_F16, BITS, SYM><<<grid, 256, 0, s>>>(w, N, K, lg, s16, codes, scales, zeros);
      break;
    default:
      quantize_fmt_kernel<QMM_F32, BITS, SYM><<<grid, 256, 0, s>>>(w, N, K, lg, s16, codes, scales, zeros);
      break;
  }
}

template <int BITS>
void launch_deq_fmt(const uint8_t* codes, const void* scales, const uint8_t* zeros, int64_t N, int64_t K, int lg,
                    int s16, uint8_t* out, int odt, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(fmt_grid(N, K)));
  switch (odt) {
    case QMM_BF16:
      dequantize_fmt_kernel<QMM_BF16, BITS><<<grid, 256, 0, s>>>(codes, scales, zeros, N, K, lg, s16, out);
      break;
    case QMM_F16:
      dequantize_fmt_kernel<QMM_F16, BITS><<<grid, 256, 0, s>>>(codes, scales, zeros, N, K, lg, s16, out);
      break;
    default:
      dequantize_fmt_kernel<QMM_F32, BITS><<<grid, 256, 0, s>>>(codes, scales, zeros, N, K, lg, s16, out);
      break;
  }
}

template <int XDT, int YDT, int BITS, bool S16>
void launch_mm_fmt_s(const uint8_t* codes, const void* scales, const uint8_t* zeros, int64_t N, int64_t K, int lg,
                     const uint16_t* x, int64_t M, void* y, hipStream_t s) {
  if (M == 1) {
    gemv_fmt_kernel<XDT, YDT, 1, BITS, S16><<<dim3(static_cast<unsigned>(ceil_div(N, kFmtRows))), 256, 0, s>>>(
        codes, scales, zeros, N, K, lg, x, y);
  } else if (M == 2) {
    gemv_fmt_kernel<XDT, YDT, 2, BITS, S16><<<dim3(static_cast<unsigned>(ceil_div(N, kFmtRows))), 256, 0, s>>>(
        codes, scales, zeros, N, K, lg, x, y);
  } else {
    const dim3 grid(static_cast<unsigned>(ceil_div(N, 16 * kMfmaRT)), static_cast<unsigned>(ceil_div(M, 16)));
    wq_mfma_kernel<XDT, YDT, BITS, S16><<<grid, 256, 0, s>>>(codes, scales, zeros, N, K, lg, x, M, y);
  }
}

template <int XDT, int YDT, int BITS>
void launch_mm_fmt_t(const uint8_t* codes, const void* scales, const uint8_t* zeros, int64_t N, int64_t K, int lg,
                     int s16, const uint16_t* x, int64_t M, void* y, hipStream_t s) {
  if (s16) launch_mm_fmt_s<XDT, YDT, BITS, true>(codes, scales, zeros, N, K, lg, x, M, y, s);
  else launch_mm_fmt_s<XDT, YDT, BITS, false>(codes, scales, zeros, N, K, lg, x, M, y, s);
}

template <int BITS>
void launch_mm_fmt(int xdt, int ydt, const uint8_t* codes, const void* scales, const uint8_t* zeros, int64_t N,
                   int64_t K, int lg, int s16, const uint16_t* x, int64_t M, void* y, hipStream_t s) {
  if (xdt == QMM_BF16) {
    if (ydt == QMM_F32) launch_mm_fmt_t<QMM_BF16, QMM_F32, BITS>(codes, scales, zeros, N, K, lg, s16, x, M, y, s);
    else launch_mm_fmt_t<QMM_BF16, QMM_BF16, BITS>(codes, scales, zeros, N, K, lg, s16, x, M, y, s);
  } else {
    if (ydt == QMM_F32) launch_mm_fmt_t<QMM_F16, QMM_F32, BITS>(codes, scales, zeros, N, K, lg, s16, x, M, y, s);
    else launch_mm_fmt_t<QMM_F16, QMM_F16, BITS>(codes, scales, zeros, N, K, lg, s16, x, M, y, s);
  }
}

}  // namespace

// ---- internal entry points (used by the public calls below and by the
// 4-bit / group-128 entry points for other formats) ----------------------------
bool fmt_is_default(int group, int bits, int scale_dtype) {
  return group == kGroup && bits == 4 && scale_dtype == QMM_F32;
}

int quantize_fmt(const void* W, int w_dtype, int64_t N, int64_t K, int group, int bits, int scale_dtype,
                 int symmetric, uint8_t* codes, void* scales, uint8_t* zeros, void* stream) {
  if (!W) return QMM_EINVAL;
  if (w_dtype != QMM_F32 && w_dtype != QMM_BF16 && w_dtype != QMM_F16)
    return w_dtype == QMM_I32 ? QMM_EUNSUPPORTED : QMM_EINVAL;
  int st = check_fmt(codes, scales, zeros, N, K, group, bits, scale_dtype);
  if (st != QMM_OK) return st;
  if (!aligned(W, 16)) return QMM_EALIGN;
  const int lg = log2_group(group);
  const int s16 = scale_dtype == QMM_F16;
  const uint8_t* w = static_cast<const uint8_t*>(W);
  hipStream_t s = as_stream(stream);
  if (symmetric) {
    switch (bits) {
      case 3: launch_quant_fmt<3, true>(w, w_dtype, N, K, lg, s16, codes, scales, zeros, s); break;
      case 4: launch_quant_fmt<4, true>(w, w_dtype, N, K, lg, s16, codes, scales, zeros, s); break;
      default: launch_quant_fmt<8, true>(w, w_dtype, N, K, lg, s16, codes, scales, zeros, s); break;
    }
  } else {
    switch (bits) {
      case 3: launch_quant_fmt<3, false>(w, w_dtype, N, K, lg, s16, codes, scales, zeros, s); break;
      case 4: launch_quant_fmt<4, false>(w, w_dtype, N, K, lg, s16, codes, scales, zeros, s); break;
      default: launch_quant_fmt<8, false>(w, w_dtype, N, K, lg, s16, codes, scales, zeros, s); break;
    }
  }
  return launch_status();
}

int dequantize_fmt(const uint8_t* codes, const void* scales, const uint8_t* zeros, int64_t N, int64_t K, int group,
                   int bits, int scale_dtype, void* W_hat, int out_dtype, void* stream) {
  if (!W_hat) return QMM_EINVAL;
  if (out_dtype != QMM_F32 && out_dtype != QMM_BF16 && out_dtype != QMM_F16)
    return out_dtype == QMM_I32 ? QMM_EUNSUPPORTED : QMM_EINVAL;
  int st = check_fmt(codes, scales, zeros, N, K, group, bits, scale_dtype);
  if (st != QMM_OK) return st;
  if (!aligned(W_hat, 16)) return QMM_EALIGN;
  const int lg = log2_group(group);
  const int s16 = scale_dtype == QMM_F16;
  uint8_t* o = static_cast<uint8_t*>(W_hat);
  hipStream_t s = as_stream(stream);
  switch (bits) {
    case 3: launch_deq_fmt<3>(codes, scales, zeros, N, K, lg, s16, o, out_dtype, s); break;
    case 4: launch_deq_fmt<4>(codes, scales, zeros, N, K, lg, s16, o, out_dtype, s); break;
    default: launch_deq_fmt<8>(codes, scales, zeros, N, K, lg, s16, o, out_dtype, s); break;
  }
  return launch_status();
}

int matmul_fmt(const uint8_t* codes, const void* scales, const uint8_t* zeros, int64_t N, int64_t K, int group,
               int bits, int scale_dtype, const void* x, int x_dtype, int64_t M, void* y, int y_dtype, void* stream) {
  if (!x || !y) return QMM_EINVAL;
  int st = check_fmt(codes, scales, zeros, N, K, group, bits, scale_dtype);
  if (st != QMM_OK) return st;
  if (M <= 0) return QMM_EINVAL;
  if (x_dtype != QMM_BF16 && x_dtype != QMM_F16) return x_dtype == QMM_F32 ? QMM_EUNSUPPORTED : QMM_EINVAL;
  if (y_dtype != x_dtype && y_dtype != QMM_F32) return QMM_EUNSUPPORTED;
  if (K > (int64_t(1) << 24) || N >= (int64_t(1) << 31) || M >= (int64_t(1) << 31)) return QMM_ERANGE;
  if (!aligned(x, 16) || !aligned(y, 4)) return QMM_EALIGN;
  const int lg = log2_group(group);
  const int s16 = scale_dtype == QMM_F16;
  const uint16_t* xx = static_cast<const uint16_t*>(x);
  hipStream_t s = as_stream(stream);
  switch (bits) {
    case 3: launch_mm_fmt<3>(x_dtype, y_dtype, codes, scales, zeros, N, K, lg, s16, xx, M, y, s); break;
    case 4: launch_mm_fmt<4>(x_dtype, y_dtype, codes, scales, zeros, N, K, lg, s16, xx, M, y, s); break;
    default: launch_mm_fmt<8>(x_dtype, y_dtype, codes, scales, zeros, N, K, lg, s16, xx, M, y, s); break;
  }
  return launch_status();
}

}  // namespace qmm

using namespace qmm;

extern "C" int qmm_wq_sizes(int64_t N, int64_t K, int group, int bits, int scale_dtype, size_t* codes_bytes,
                            size_t* scales_bytes, size_t* zeros_bytes) {
  if (N <= 0 || K <= 0 || group <= 0 || K % group != 0) return QMM_EINVAL;
  if (scale_dtype != QMM_F32 && scale_dtype != QMM_F16) return scale_dtype == QMM_BF16 ? QMM_EUNSUPPORTED : QMM_EINVAL;
  if ((bits != 3 && bits != 4 && bits != 8) || log2_group(group) < 0) return QMM_EUNSUPPORTED;
  const int64_t G = K / group;
  if (codes_bytes) *codes_bytes = static_cast<size_t>(N) * static_cast<size_t>(code_row_bytes(K, bits));
  if (scales_bytes) *scales_bytes = static_cast<size_t>(N * G) * (scale_dtype == QMM_F32 ? 4u : 2u);
  if (zeros_bytes) *zeros_bytes = static_cast<size_t>(N) * static_cast<size_t>(zero_row_bytes(G, bits));
  return QMM_OK;
}

extern "C" int quantize_groupwise_ex(const void* W, int w_dtype, int64_t N, int64_t K, int group, int bits,
                                     int scale_dtype, int symmetric, uint8_t* codes, void* scales, uint8_t* zeros,
                                     void* stream) {
  if (fmt_is_default(group, bits, scale_dtype)) {
    return symmetric ? quantize_groupwise_symmetric(W, w_dtype, N, K, group, bits, codes, static_cast<float*>(scales),
                                                    zeros, stream)
                     : quantize_groupwise(W, w_dtype, N, K, group, bits, codes, static_cast<float*>(scales), zeros,
                                          stream);
  }
  return quantize_fmt(W, w_dtype, N, K, group, bits, scale_dtype, symmetric, codes, scales, zeros, stream);
}

extern "C" int dequantize_ex(const uint8_t* codes, const void* scales, const uint8_t* zeros, int64_t N, int64_t K,
                             int group, int bits, int scale_dtype, void* W_hat, int out_dtype, void* stream) {
  if (fmt_is_default(group, bits, scale_dtype))
    return dequantize(codes, static_cast<const float*>(scales), zeros, N, K, group, bits, W_hat, out_dtype, stream);
  return dequantize_fmt(codes, scales, zeros, N, K, group, bits, scale_dtype, W_hat, out_dtype, stream);
}

extern "C" int wxa16_gemv(const uint8_t* codes, const void* scales, const uint8_t* zeros, int64_t N, int64_t K,
                          int group, int bits, int scale_dtype, const void* x, int x_dtype, int64_t B, void* y,
                          int y_dtype, void* stream) {
  if (fmt_is_default(group, bits, scale_dtype))
    return w4a16_gemv(codes, static_cast<const float*>(scales), zeros, N, K, group, x, x_dtype, B, y, y_dtype, stream);
  if (B > 8) return QMM_EUNSUPPORTED;
  return matmul_fmt(codes, scales, zeros, N, K, group, bits, scale_dtype, x, x_dtype, B, y, y_dtype, stream);
}

extern "C" int wxa16_gemm(const uint8_t* codes, const void* scales, const uint8_t* zeros, int64_t N, int64_t K,
                          int group, int bits, int scale_dtype, const void* X, int x_dtype, int64_t M, void* Y,
                          int y_dtype, void* stream) {
  if (fmt_is_default(group, bits, scale_dtype))
    return w4a16_gemm(codes, static_cast<const float*>(scales), zeros, N, K, group, X, x_dtype, M, Y, y_dtype, stream);
  return matmul_fmt(codes, scales, zeros, N, K, group, bits, scale_dtype, X, x_dtype, M, Y, y_dtype, stream);
}

extern "C" int qmm_w4_repack_from_plain(const uint8_t* plain, uint8_t* codes, int64_t N, int64_t K, void* stream) {
  if (!plain || !codes) return QMM_EINVAL;
  if (N <= 0 || K <= 0 || K % 8 != 0) return QMM_EINVAL;
  if (!aligned(plain, 16) || !aligned(codes, 16)) return QMM_EALIGN;
  const int64_t nwords = N * K / 8;
  const int64_t blocks = std::min<int64_t>(ceil_div(ceil_div(nwords, 4), 256), static_cast<int64_t>(device_cus()) * 8);
  repack_kernel<true><<<dim3(static_cast<unsigned>(blocks > 0 ? blocks : 1)), 256, 0, as_stream(stream)>>>(
      reinterpret_cast<const uint32_t*>(plain), reinterpret_cast<uint32_t*>(codes), nwords);
  return launch_status();
}

extern "C" int qmm_w4_repack_to_plain(const uint8_t* codes, uint8_t* plain, int64_t N, int64_t K, void* stream) {
  if (!plain || !codes) return QMM_EINVAL;
  if (N <= 0 || K <= 0 || K % 8 != 0) return QMM_EINVAL;
  if (!aligned(plain, 16) || !aligned(codes, 16)) return QMM_EALIGN;
  const int64_t nwords = N * K / 8;
  const int64_t blocks = std::min<int64_t>(ceil_div(ceil_div(nwords, 4), 256), static_cast<int64_t>(device_cus()) * 8);
  repack_kernel<false><<<dim3(static_cast<unsigned>(blocks > 0 ? blocks : 1)), 256, 0, as_stream(stream)>>>(
      reinterpret_cast<const uint32_t*>(codes), reinterpret_cast<uint32_t*>(plain), nwords);
  return launch_status();
}
