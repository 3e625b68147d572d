// qmm_device.h -- device-side helpers shared by the gfx950 kernels of libqmm.
//
// Storage formats (fixed by the C-ABI in include/qmm.h):
//  * INT4 codes: row-major [N, K/2] bytes; little-endian 32-bit word w of a
//    row holds elements 8w..8w+7, element 8w+2i in bits 4i..4i+3 and element
//    8w+2i+1 in bits 16+4i..16+4i+3 (see code_nibble).
//  * scales: fp32 [N, K/128]; zero-points: nibble-packed [N, ceil(G/2)] bytes,
//    group 2j in the low nibble of byte j, group 2j+1 in the high nibble.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmm_internal.h"

namespace qmm {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kGroup = 128;

// ---- buffer loads straight into LDS ------------------------------------------
// Word 3 of a raw buffer resource (32-bit data format); offsets at or past the
// resource's byte count read as zero, which the kernels use for ragged tiles.
constexpr int kBufferWord3 = 0x00020000;
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt with only the vector-memory counter limited (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ---- 16-byte global memory access ------------------------------------------
// Streaming loads/stores use the nontemporal hint (data touched once).
__device__ __forceinline__ u32x4 ld16_nt(const void* p) { return __builtin_nontemporal_load((const u32x4*)p); }
__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }
__device__ __forceinline__ void st16_nt(void* p, u32x4 v) { __builtin_nontemporal_store(v, (u32x4*)p); }

// ---- 16-bit float <-> fp32 ------------------------------------------------
__device__ __forceinline__ float bf16lo_to_f32(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }
__device__ __forceinline__ float f16lo_to_f32(uint32_t u) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xFFFFu));
}
__device__ __forceinline__ float f16hi_to_f32(uint32_t u) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
// fp32 -> fp16 bits (hardware conversion, round to nearest even).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b);
template <>
__device__ __forceinline__ uint32_t pack2<QMM_BF16>(float a, float b) {
  return f32_to_bf16_bits(a) | (f32_to_bf16_bits(b) << 16);
}
template <>
__device__ __forceinline__ uint32_t pack2<QMM_F16>(float a, float b) {
  return f32_to_f16_bits(a) | (f32_to_f16_bits(b) << 16);
}

// Eight consecutive elements of a 16/32-bit float row as fp32.
template <int DT>
struct Vec8;
template <>
struct Vec8<QMM_BF16> {
  static __device__ __forceinline__ void load(const void* p, float v[8]) {
    const u32x4 u = ld16_nt(p);
    v[0] = bf16lo_to_f32(u.x); v[1] = bf16hi_to_f32(u.x);
    v[2] = bf16lo_to_f32(u.y); v[3] = bf16hi_to_f32(u.y);
    v[4] = bf16lo_to_f32(u.z); v[5] = bf16hi_to_f32(u.z);
    v[6] = bf16lo_to_f32(u.w); v[7] = bf16hi_to_f32(u.w);
  }
};
template <>
struct Vec8<QMM_F16> {
  static __device__ __forceinline__ void load(const void* p, float v[8]) {
    const u32x4 u = ld16_nt(p);
    v[0] = f16lo_to_f32(u.x); v[1] = f16hi_to_f32(u.x);
    v[2] = f16lo_to_f32(u.y); v[3] = f16hi_to_f32(u.y);
    v[4] = f16lo_to_f32(u.z); v[5] = f16hi_to_f32(u.z);
    v[6] = f16lo_to_f32(u.w); v[7] = f16hi_to_f32(u.w);
  }
};
template <>
struct Vec8<QMM_F32> {
  static __device__ __forceinline__ void load(const void* p, float v[8]) {
    const u32x4 a = ld16_nt(p);
    const u32x4 b = ld16_nt(static_cast<const uint8_t*>(p) + 16);
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y); v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  }
};

// ---- cross-lane reductions inside a row of 16 lanes (DPP) -------------------
// quad_perm [1,0,3,2] = xor 1; [2,3,0,1] = xor 2; row_half_mirror pairs the
// two quads of each half-row; row_mirror pairs the two halves of the row.
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float row16_min(float v) {
  v = fminf(v, dpp_f<kDppXor1>(v));
  v = fminf(v, dpp_f<kDppXor2>(v));
  v = fminf(v, dpp_f<kDppHalfMirror>(v));
  v = fminf(v, dpp_f<kDppMirror>(v));
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  return v;
}

// Sums eight per-lane values across the wavefront at once (recursive halving):
// on return lane l holds the 64-lane sum of v[l >> 3].  v_permlane32_swap
// exchanges lanes 32-63 of its first operand with lanes 0-31 of its second,
// v_permlane16_swap the odd 16-lane rows of the first with the even rows of
// the second, so each swap + add halves the lanes per value and packs two
// values into one register; the last 16 -> 1 steps use DPP mirrors and
// quad permutes.  18 instructions instead of 8 separate 64-lane sums.
__device__ __forceinline__ float wave_sum8(const float v[8]) {
  float u[4], w[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 4]), false, false);
    u[i] = __uint_as_float(s[0]) + __uint_as_float(s[1]);   // lanes 0-31: v[i], lanes 32-63: v[i+4]
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(u[i]), __float_as_uint(u[i + 2]), false, false);
    w[i] = __uint_as_float(s[0]) + __uint_as_float(s[1]);   // 16-lane rows: v[i], v[i+2], v[i+4], v[i+6]
  }
  const float t0 = w[0] + dpp_f<kDppMirror>(w[0]);
  const float t1 = w[1] + dpp_f<kDppMirror>(w[1]);
  float c = (threadIdx.x & 8) ? t1 : t0;                    // 8-lane group g holds v[g]
  c += dpp_f<kDppHalfMirror>(c);
  c += dpp_f<kDppXor2>(c);
  c += dpp_f<kDppXor1>(c);
  return c;
}

// Keeps a constant in a VGPR.  gfx9 VOP3 encodings take no 32-bit literal and
// read at most one SGPR, so a three-operand op such as v_and_or_b32 with two
// non-inline constants needs one of them in a VGPR; otherwise the compiler
// splits it into v_and_b32 + v_or_b32.
__device__ __forceinline__ uint32_t vgpr_const(uint32_t c) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(c), 0xE4, 0xF, 0xF, false));
}

// Full-wave sum, result valid in every lane.
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  v += __shfl_xor(v, 16, kWave);
  v += __shfl_xor(v, 32, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  v = fmaxf(v, __shfl_xor(v, 16, kWave));
  v = fmaxf(v, __shfl_xor(v, 32, kWave));
  return v;
}

// ---- INT4 code layout and unpack --------------------------------------------
// A 32-bit code word holds 8 consecutive elements e0..e7 of a row, element i
// in nibble code_nibble(i): the even elements in nibbles 0-3, the odd ones in
// nibbles 4-7, so nibbles j and j + 4 hold the consecutive pair (e_2j, e_2j+1).
// Each pair is built with a shift and one AND-OR that drop both nibbles into
// the mantissas of a 16-bit float pair whose exponent makes one code step
// worth 1:
//   bf16: nibble at mantissa bits 0-3 of 0x4300 (128.0)  -> 128 + q exactly;
//   fp16: nibble at mantissa bits 6-9 of 0x4C00 (16.0)   ->  16 + q exactly,
// ready for dot / MFMA instructions against the activations as loaded.  The
// constant offset is removed per group as offset * sum(x).  (A smaller offset
// means less cancellation in that subtraction; bf16's 7-bit mantissa has no
// room to place the nibble higher without an extra shift.)
__host__ __device__ constexpr int code_nibble(int i) { return (i >> 1) | ((i & 1) << 2); }

template <int DT>
struct Int4Magic;
// `magic` is the kMagic constant held in a VGPR (vgpr_const), so each pair
// costs one shift and one v_and_or_b32.
template <>
struct Int4Magic<QMM_BF16> {
  static constexpr float offset = 128.0f;
  static constexpr uint32_t one_pair = 0x3F803F80u;  // (1.0, 1.0)
  static constexpr uint32_t kMagic = 0x43004300u;
  static __device__ __forceinline__ void unpack(uint32_t w, uint32_t magic, uint32_t p[4]) {
    constexpr uint32_t kMask = 0x000F000Fu;
    p[0] = (w & kMask) | magic;
    p[1] = ((w >> 4) & kMask) | magic;
    p[2] = ((w >> 8) & kMask) | magic;
    p[3] = ((w >> 12) & kMask) | magic;
  }
};
template <>
struct Int4Magic<QMM_F16> {
  static constexpr float offset = 16.0f;
  static constexpr uint32_t one_pair = 0x3C003C00u;
  static constexpr uint32_t kMagic = 0x4C004C00u;
  static __device__ __forceinline__ void unpack(uint32_t w, uint32_t magic, uint32_t p[4]) {
    constexpr uint32_t kMask = 0x03C003C0u;
    p[0] = ((w << 6) & kMask) | magic;
    p[1] = ((w << 2) & kMask) | magic;
    p[2] = ((w >> 2) & kMask) | magic;
    p[3] = ((w >> 6) & kMask) | magic;
  }
};

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
}

template <int DT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c);
template <>
__device__ __forceinline__ float dot2<QMM_BF16>(uint32_t a, uint32_t b, float c) { return dot2_bf16(a, b, c); }
template <>
__device__ __forceinline__ float dot2<QMM_F16>(uint32_t a, uint32_t b, float c) { return dot2_f16(a, b, c); }

__device__ __forceinline__ uint32_t zero_nibble(const uint8_t* zeros_row, int64_t g) {
  uint32_t b = zeros_row[g >> 1];
  return (g & 1) ? (b >> 4) : (b & 0xFu);
}

}  // namespace qmm
