// w8a16.hip -- weight-only INT8 decode matmul (W8A16):
//   y[b, n] = w_scale[n] * sum_k x[b, k] * qW[n, k]
// with the per-channel INT8 weights that sq_quantize_weight writes (no
// smoothing) and 16-bit activations.  Weight-only INT8 halves the bytes of a
// 16-bit weight read while the arithmetic stays in 16-bit floats ("How
// quantization works", "Mainstream schemes at a glance": the W8A16 / W4A16
// row, which speeds up weight reads at small batch).
//
// Kernel (vector ALUs only; decode is a stream of weight bytes, not a dense
// contraction):
//  * w8_gemv_kernel: a block of four wavefronts takes R = 8 weight rows; per
//    step a lane loads 16 bytes (16 weights) of each row, so 8 x 16 bytes are
//    in flight per lane, and the matching 16 activations per token.  A weight
//    byte becomes an fp32 integer in one instruction (sign-extending byte
//    select), two of them one 16-bit pair (exact: |q| <= 128 has at most 8
//    significant bits), and v_dot2_f32_{bf16,f16} multiplies that pair with
//    the activation pair as loaded.  The per-channel scale multiplies the
//    row's total once.  Used for B <= 2.
//  * w8_mfma_kernel: 3..8 tokens, where the dot products of the kernel above
//    (one per weight pair and token) outrun the weight stream.  The weights
//    are the A operand of v_mfma_f32_16x16x32_{bf16,f16} straight from
//    registers (converted as above), the activations the B operand as loaded;
//    a block of four wavefronts owns 16 rows, each wavefront a contiguous
//    quarter of K, summed through LDS at the end.  Used when K is not a
//    multiple of 256.
//  * w8_lds_kernel: the same operands and block shape for K a multiple of
//    256, with each wavefront's weights brought into a private LDS ring in
//    runs of 256 contiguous bytes per row (the register kernel's loads cover
//    16 rows x 64 bytes per instruction, a pattern that streams from HBM
//    well below the contiguous one).

#include "qmm_device.h"

namespace qmm {
namespace {

constexpr int kW8Waves = 4;
constexpr int kW8LaneK = 16;                                  // weights per lane per row per step
constexpr int64_t kW8StepK = kW8Waves * kWave * kW8LaneK;     // 4096
constexpr int kW8Rows = 8;                                    // rows per block
constexpr int64_t kW8MaxK = int64_t(1) << 24;                 // lane offsets stay 32-bit

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

// Bytes 2i and 2i+1 of w (signed) as one pair of 16-bit floats of type DT,
// element 2i in the low half.  Both conversions are exact.
template <int DT, int I>
__device__ __forceinline__ uint32_t i8_pair(uint32_t w) {
  const float lo = static_cast<float>(static_cast<int8_t>(w >> (16 * I)));
  const float hi = static_cast<float>(static_cast<int8_t>(w >> (16 * I + 8)));
  if constexpr (DT == QMM_BF16) {
    // An integer of at most 8 significant bits has zero low 16 bits in fp32:
    // its bfloat16 is the high half.
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
  }
}

template <int XDT, int YDT, int B, int R>
__global__ __launch_bounds__(256) void w8_gemv_kernel(const int8_t* __restrict__ qW,
                                                      const float* __restrict__ w_scale, int64_t N, int64_t K,
                                                      const uint16_t* __restrict__ x, void* __restrict__ y) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * R;
  const int kk = static_cast<int>(K);

  const int8_t* wrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = (row0 + r < N) ? row0 + r : N - 1;
    wrow[r] = qW + row * K;
  }

  float acc[R][B];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;

  for (uint32_t k0 = 0; k0 < static_cast<uint32_t>(kk); k0 += static_cast<uint32_t>(kW8StepK)) {
    // A wavefront with no lane inside K leaves the loop; in a partly covered
    // step the lanes past K load the last 16 weights of the row (in bounds)
    // and take zero activations.
    if (k0 + static_cast<uint32_t>(wave * (kWave * kW8LaneK)) >= static_cast<uint32_t>(kk)) break;
    const uint32_t kb_raw = k0 + static_cast<uint32_t>(wave * (kWave * kW8LaneK) + lane * kW8LaneK);
    const bool inside = kb_raw < static_cast<uint32_t>(kk);
    const uint32_t kb = inside ? kb_raw : static_cast<uint32_t>(kk - kW8LaneK);

    // All loads of the step before any use: activations, then the rows in
    // the order they are consumed.
    u32x4 xraw[B][2];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      xraw[b][0] = ld16(x + b * K + kb);
      xraw[b][1] = ld16(x + b * K + kb + 8);
    }
    u32x4 cw[R];
#pragma unroll
    for (int r = 0; r < R; ++r) cw[r] = ld16_nt(wrow[r] + kb);
    __builtin_amdgcn_sched_barrier(0);
    if (!inside) {
#pragma unroll
      for (int b = 0; b < B; ++b) xraw[b][0] = xraw[b][1] = u32x4{0u, 0u, 0u, 0u};
    }
    // Activation word j holds elements kb + 2j (low half) and kb + 2j + 1.
    uint32_t xp[B][8];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      xp[b][0] = xraw[b][0].x;
      xp[b][1] = xraw[b][0].y;
      xp[b][2] = xraw[b][0].z;
      xp[b][3] = xraw[b][0].w;
      xp[b][4] = xraw[b][1].x;
      xp[b][5] = xraw[b][1].y;
      xp[b][6] = xraw[b][1].z;
      xp[b][7] = xraw[b][1].w;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      // Weight word c holds elements kb + 4c .. kb + 4c + 3 (byte i = element 4c + i).
      const uint32_t words[4] = {cw[r].x, cw[r].y, cw[r].z, cw[r].w};
      float a0[B], a1[B];
#pragma unroll
      for (int b = 0; b < B; ++b) a0[b] = a1[b] = 0.0f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t p0 = i8_pair<XDT, 0>(words[c]);
        const uint32_t p1 = i8_pair<XDT, 1>(words[c]);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          a0[b] = dot2<XDT>(p0, xp[b][2 * c], a0[b]);
          a1[b] = dot2<XDT>(p1, xp[b][2 * c + 1], a1[b]);
        }
      }
#pragma unroll
      for (int b = 0; b < B; ++b) acc[r][b] += a0[b] + a1[b];
    }
  }

  __shared__ float red[kW8Waves][R * B];
  static_assert((R * B) % 8 == 0, "rows x tokens must be a multiple of 8");
#pragma unroll
  for (int h = 0; h < R * B / 8; ++h) {
    float v8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v8[i] = acc[(8 * h + i) / B][(8 * h + i) % B];
    const float v = wave_sum8(v8);   // lane l holds the sum of value l >> 3
    if ((lane & 7) == 0) red[wave][8 * h + (lane >> 3)] = v;
  }
  __syncthreads();
  if (threadIdx.x < R * B) {
    const int r = threadIdx.x / B;
    const int b = threadIdx.x % B;
    const int64_t row = row0 + r;
    if (row < N) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < kW8Waves; ++w) v += red[w][threadIdx.x];
      store_out<YDT>(y, static_cast<int64_t>(b) * N + row, v * w_scale[row]);
    }
  }
}

// MFMA kernel.  Operand layout of v_mfma_f32_16x16x32: lane l supplies A row
// l%16 and B column l%16 with k = 8*(l/16) .. +8 of the instruction; D lane l
// holds rows 4*(l/16) .. +4 of column l%16.  Chunk j of a wavefront's step is
// 64 k; lane l loads 16 weight bytes of row l%16 at k = 16*(l/16) within it
// and feeds bytes 0..7 to one instruction and 8..15 to the next, with the
// activations of token l%16 at the same k (16 bytes each), so both operands
// cover the same k in the same order.
constexpr int kW8MfmaU = 8;   // 64-k chunks per step: 8 x 16 weight bytes in flight per lane

template <int XDT>
__device__ __forceinline__ f32x4 mfma16x16x32_w8(const uint32_t a[4], u32x4 b, f32x4 c) {
  const u32x4 av = {a[0], a[1], a[2], a[3]};
  if constexpr (XDT == QMM_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  } else {
    typedef _Float16 f16x8_w8 __attribute__((ext_vector_type(8)));
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_w8, av), __builtin_bit_cast(f16x8_w8, b), c,
                                                  0, 0, 0);
  }
}

template <int XDT, int YDT, int NW>
__global__ __launch_bounds__(NW * 64) void w8_mfma_kernel(const int8_t* __restrict__ qW, const float* __restrict__ w_scale,
                                                      int64_t N, int64_t K, const uint16_t* __restrict__ x, int64_t B,
                                                      void* __restrict__ y) {
  __shared__ float red[NW][4][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int l16 = lane & 15;
  const int quad = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int64_t ra = (row0 + l16 < N) ? row0 + l16 : N - 1;        // rows past N read the last row
  const int64_t ta = (l16 < B) ? l16 : B - 1;                      // tokens past B repeat the last token
  const int nchunks = static_cast<int>(K / 64);
  const int cper = (nchunks + NW - 1) / NW;
  const int cbeg = wave * cper;
  const int cend = (cbeg + cper < nchunks) ? cbeg + cper : nchunks;
  const int8_t* wp = qW + ra * K + 16 * quad;
  const uint16_t* xp = x + ta * K + 16 * quad;

  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int c0 = cbeg; c0 < cend; c0 += kW8MfmaU) {
    u32x4 wv[kW8MfmaU], xv[kW8MfmaU][2];
#pragma unroll
    for (int u = 0; u < kW8MfmaU; ++u) {
      if (c0 + u < cend) {   // wavefront-uniform
        const int64_t k = static_cast<int64_t>(c0 + u) * 64;
        xv[u][0] = ld16(xp + k);
        xv[u][1] = ld16(xp + k + 8);
        wv[u] = ld16_nt(wp + k);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kW8MfmaU; ++u) {
      if (c0 + u < cend) {
        const uint32_t a0[4] = {i8_pair<XDT, 0>(wv[u].x), i8_pair<XDT, 1>(wv[u].x), i8_pair<XDT, 0>(wv[u].y),
                                i8_pair<XDT, 1>(wv[u].y)};
        const uint32_t a1[4] = {i8_pair<XDT, 0>(wv[u].z), i8_pair<XDT, 1>(wv[u].z), i8_pair<XDT, 0>(wv[u].w),
                                i8_pair<XDT, 1>(wv[u].w)};
        acc = mfma16x16x32_w8<XDT>(a0, xv[u][0], acc);
        acc = mfma16x16x32_w8<XDT>(a1, xv[u][1], acc);
      }
    }
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][i][lane] = acc[i];
  __syncthreads();
  if (threadIdx.x < 4 * kWave) {
    const int i = threadIdx.x >> 6;          // 256 threads: one D value each
    const int l = threadIdx.x & (kWave - 1);
    const int64_t row = row0 + 4 * (l >> 4) + i;
    const int64_t t = l & 15;
    if (row < N && t < B) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) v += red[w][i][l];
      store_out<YDT>(y, t * N + row, v * w_scale[row]);
    }
  }
}

// Staged MFMA kernel for K a multiple of 256.  Same operands and block shape
// as w8_mfma_kernel (16 rows, four wavefronts over contiguous quarters of
// K), but a wavefront brings each 256-k step of its 16 rows into a private
// LDS ring by direct buffer loads of 4 rows x 256 contiguous bytes each
// (1 KiB per instruction) instead of loading 16 rows x 64 bytes per
// instruction into registers: the second pattern streams from HBM at well
// under the first's rate.  Chunk d (16 bytes) of row r sits at
// position d ^ lds_row_swz(r) of the row's 256 bytes; lane l then reads row
// l%16, chunk 4(l/16) + c for c = 0..3, a read the swizzle keeps free of
// bank conflicts.  Weights (two-slot ring) and activations (the B operand,
// two register sets) are requested one step ahead; lanes of token columns
// past B load nothing (zeros from past the buffer resource), so at B = 8
// half the activation loads move no data.
__host__ __device__ constexpr int lds_row_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
constexpr int kW8StageBytes = 16 * 256;   // 16 rows x 256 k of int8 weights

template <int XDT, int YDT>
__global__ __launch_bounds__(256) void w8_lds_kernel(const int8_t* __restrict__ qW, const float* __restrict__ w_scale,
                                                     int64_t N, int64_t K, const uint16_t* __restrict__ x, int64_t B,
                                                     void* __restrict__ y) {
  // 32 KiB per block, so five blocks share a compute unit; the reduction at
  // the end reuses the ring.
  __shared__ __attribute__((aligned(16))) uint8_t ring[kW8Waves][2][kW8StageBytes];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int l16 = lane & 15;
  const int quad = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int nrows = static_cast<int>((N - row0 < 16) ? N - row0 : 16);
  const int64_t ta = (l16 < B) ? l16 : B - 1;   // an in-range row; columns past B read zeros (load_x)
  const int kk = static_cast<int>(K);           // K <= 2^24 (checked on the host)
  const int nsteps = kk / 256;
  const int sper = (nsteps + kW8Waves - 1) / kW8Waves;
  const int sbeg = wave * sper;
  const int send = (sbeg + sper < nsteps) ? sbeg + sper : nsteps;
  const int ns = send > sbeg ? send - sbeg : 0;   // this wavefront's steps

  // Rows past N lie past the resource's byte count and read as zero.
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(qW + row0 * K), 0, nrows * kk, kBufferWord3);
  // Load j of a step: lane L writes LDS bytes [16 L, 16 L + 16) of the
  // step's kilobyte j, i.e. row 4 j + L/16 at position L%16, which holds
  // chunk (L%16) ^ lds_row_swz(row).
  int woff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * j + (lane >> 4);
    woff[j] = r * kk + 16 * ((lane & 15) ^ lds_row_swz(r));
  }
  const uint32_t rbase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&ring[wave][0][0]));
  auto issue = [&](int i) {   // step sbeg + i of this wavefront, clamped to its last (a reload, never read)
    const int st = sbeg + (i < ns ? i : ns - 1);
    const uint32_t dst = rbase + (i & 1) * kW8StageBytes;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)(uintptr_t)(dst + j * 1024), 16, woff[j], st * 256, 0,
                                               0);
  };
  // Activations through a buffer resource over the B token rows, so that a
  // step past this wavefront's range, or a token column past B (offset past
  // the resource), reads zeros.
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x), 0, static_cast<int>(B) * kk * 2, kBufferWord3);
  const int xoff = static_cast<int>(ta * K + 16 * (4 * quad)) * 2;
  constexpr int kPastX = 1 << 30;   // beyond B * K * 2 <= 2^28 bytes
  auto load_x = [&](int i, u32x4 (&xv)[4][2]) {   // activations of step i, zeros past the range
    const int vo = (i < ns && l16 < B) ? xoff + (sbeg + i) * 512 : kPastX;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      xv[c][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, vo + 32 * c, 0, 0));
      xv[c][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, vo + 32 * c + 16, 0, 0));
    }
  };
  const int rd = l16 * 256;

  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  auto compute = [&](int slot, const u32x4 (&xv)[4][2]) {
    const uint8_t* stg = &ring[wave][0][0] + slot * kW8StageBytes;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(stg + rd + 16 * ((4 * quad + c) ^ lds_row_swz(l16)));
      const uint32_t a0[4] = {i8_pair<XDT, 0>(w.x), i8_pair<XDT, 1>(w.x), i8_pair<XDT, 0>(w.y), i8_pair<XDT, 1>(w.y)};
      const uint32_t a1[4] = {i8_pair<XDT, 0>(w.z), i8_pair<XDT, 1>(w.z), i8_pair<XDT, 0>(w.w), i8_pair<XDT, 1>(w.w)};
      acc = mfma16x16x32_w8<XDT>(a0, xv[c][0], acc);
      acc = mfma16x16x32_w8<XDT>(a1, xv[c][1], acc);
    }
  };
  // Steps go in pairs, step i in ring slot i & 1 with activation set i & 1;
  // each is requested one step ahead, so before step i is computed only step
  // i + 1's twelve loads (eight activation, four weight) may be in flight.
  // The second step of a pair is computed even past the range, with zero
  // activations (its weights: a reload of the last step), so both halves run
  // unconditionally and their loads stay where they are issued.
  u32x4 xa[4][2], xb[4][2];
  if (ns > 0) {
    load_x(0, xa);
    issue(0);
  }
  for (int i = 0; i < ns; i += 2) {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): ring slot 1 has been read
    load_x(i + 1, xb);
    issue(i + 1);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<12>();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    compute(0, xa);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // ring slot 0 has been read
    load_x(i + 2, xa);
    issue(i + 2);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<12>();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    compute(1, xb);
  }
  wait_vm<0>();
  __syncthreads();   // every wavefront is done with its ring

  float (*red)[4][kWave] = reinterpret_cast<float (*)[4][kWave]>(&ring[0][0][0]);
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][i][lane] = acc[i];
  __syncthreads();
  {
    const int i = threadIdx.x >> 6;          // 256 threads: one D value each
    const int l = threadIdx.x & (kWave - 1);
    const int64_t row = row0 + 4 * (l >> 4) + i;
    const int64_t t = l & 15;
    if (row < N && t < B) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < kW8Waves; ++w) v += red[w][i][l];
      store_out<YDT>(y, t * N + row, v * w_scale[row]);
    }
  }
}

template <int XDT, int YDT, int B>
void launch_w8_b(const int8_t* qW, const float* ws, int64_t N, int64_t K, const uint16_t* x, void* y,
                 hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(ceil_div(N, kW8Rows)));
  w8_gemv_kernel<XDT, YDT, B, kW8Rows><<<grid, dim3(kW8Waves * kWave), 0, s>>>(qW, ws, N, K, x, y);
}

template <int XDT, int YDT>
void launch_w8(int64_t B, const int8_t* qW, const float* ws, int64_t N, int64_t K, const uint16_t* x, void* y,
               hipStream_t s) {
  // One or two tokens stream fastest on the vector ALUs; from three on the
  // dot products would outrun the weight stream, so the MFMA kernel takes over.
  if (B == 1) {
    launch_w8_b<XDT, YDT, 1>(qW, ws, N, K, x, y, s);
  } else if (B == 2) {
    launch_w8_b<XDT, YDT, 2>(qW, ws, N, K, x, y, s);
  } else {
    // Four wavefronts per block (eight measured no faster on 8192 x 28672);
    // whole 256-k steps go through the LDS-staged kernel.
    const dim3 grid(static_cast<unsigned>(ceil_div(N, 16)));
    if (K % 256 == 0)
      w8_lds_kernel<XDT, YDT><<<grid, dim3(4 * kWave), 0, s>>>(qW, ws, N, K, x, B, y);
    else
      w8_mfma_kernel<XDT, YDT, 4><<<grid, dim3(4 * kWave), 0, s>>>(qW, ws, N, K, x, B, y);
  }
}

}  // namespace
}  // namespace qmm

using namespace qmm;

extern "C" int w8a16_gemv(const int8_t* qW, const float* w_scale, int64_t N, int64_t K, const void* x, int x_dtype,
                          int64_t B, void* y, int y_dtype, void* stream) {
  if (!qW || !w_scale || !x || !y) return QMM_EINVAL;
  if (N <= 0 || K <= 0 || B <= 0) return QMM_EINVAL;
  if ((x_dtype != QMM_BF16 && x_dtype != QMM_F16 && x_dtype != QMM_F32 && x_dtype != QMM_I32) ||
      (y_dtype != QMM_BF16 && y_dtype != QMM_F16 && y_dtype != QMM_F32 && y_dtype != QMM_I32))
    return QMM_EINVAL;
  if (x_dtype != QMM_BF16 && x_dtype != QMM_F16) return QMM_EUNSUPPORTED;
  if (y_dtype != x_dtype && y_dtype != QMM_F32) return QMM_EUNSUPPORTED;
  if (B > 8 || K % 64 != 0) return QMM_EUNSUPPORTED;
  if (K > kW8MaxK || N > INT32_MAX) return QMM_ERANGE;
  if (!aligned(qW, 16) || !aligned(x, 16) || !aligned(w_scale, 4) || !aligned(y, y_dtype == QMM_F32 ? 4 : 2))
    return QMM_EALIGN;
  hipStream_t s = as_stream(stream);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  if (x_dtype == QMM_BF16) {
    if (y_dtype == QMM_F32) launch_w8<QMM_BF16, QMM_F32>(B, qW, w_scale, N, K, xp, y, s);
    else launch_w8<QMM_BF16, QMM_BF16>(B, qW, w_scale, N, K, xp, y, s);
  } else {
    if (y_dtype == QMM_F32) launch_w8<QMM_F16, QMM_F32>(B, qW, w_scale, N, K, xp, y, s);
    else launch_w8<QMM_F16, QMM_F16>(B, qW, w_scale, N, K, xp, y, s);
  }
  return launch_status();
}
