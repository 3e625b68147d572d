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
//    held in registers across those rows.  Used for B <= 2 (decode).
//  * w4_rows_kernel: 2..64 tokens in 16-, 32- or 64-token tiles when the
//    weight rows give most compute units a block (64 rows) or two (32 rows)
//    on v_mfma_f32_16x16x32_{bf16,f16}; the block loads each step's codes in
//    runs of 256 or 128 contiguous bytes per row, its wavefronts split K.
//  * w4_lds_kernel: 2..32 tokens where the rows kernel would leave compute
//    units idle (and larger batches whose 64 x 128 tiles would not fill the
//    chip); a block takes 16 or 32 tokens x 32 or 64 weight rows, its four
//    wavefronts split K, each with its own LDS rings filled by direct-to-LDS
//    buffer loads.
//  * w4_tile_kernel: larger batches; 64 x 128 tiles whose activation tile is
//    shared by the four wavefronts through LDS, one barrier per group.
//  * w4_mfma_skinny_kernel: fallback when K is too large for the LDS
//    zero-point table of the kernels above; the weights are the A operand and
//    never touch LDS.

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

// Row pitch of a block's zero-point table in LDS: the zb bytes of a row
// rounded up to an odd number of dwords, so that the 16 rows of a fragment
// read fall in 16 different banks (with zb a multiple of 32 bytes, rows r and
// r + 8 would share one).
__host__ __device__ constexpr int zero_pitch(int zb) { return 4 * (((zb + 3) / 4) | 1); }

// The block's zero-point bytes (rows x zb, contiguous in memory) into LDS at
// row pitch zp; rows from `valid` on read 0.  Each pass issues all of a
// thread's loads before any store (one memory round trip per pass, not per
// byte); indexes are clamped into the valid range, so every load is in bounds.
template <int NTHREADS>
__device__ __forceinline__ void copy_zeros_to_lds(uint8_t* dst, const uint8_t* __restrict__ src, int rows, int zb,
                                                  int zp, int valid, int tid) {
  constexpr int kPer = 8;
  const int total = rows * zb;
  const int lim = valid * zb;
  for (int base = 0; base < total; base += kPer * NTHREADS) {
    uint8_t v[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (base + j * NTHREADS < total) v[j] = src[min(base + j * NTHREADS + tid, lim - 1)];   // uniform test
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int idx = base + j * NTHREADS + tid;
      if (idx < total) {
        const int r = idx / zb;
        dst[r * zp + (idx - r * zb)] = (idx < lim) ? v[j] : uint8_t(0);
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Vector-ALU GEMV.
// ----------------------------------------------------------------------------
constexpr int kValuWaves = 4;
constexpr int kLaneK = 32;   // weights per lane per row per step

// KW of the four wavefronts split K (a block step covers KW x 2048 weights of
// a row); the other 4 / KW take further sets of R rows, so that a short K
// (4096: KW = 2) still gives every wavefront work.
template <int XDT, int YDT, int B, int R, int KW>
__global__ __launch_bounds__(256) void gemv_valu_kernel(const uint8_t* __restrict__ codes,
                                                        const float* __restrict__ scales,
                                                        const uint8_t* __restrict__ zeros, int64_t N, int64_t K,
                                                        const uint16_t* __restrict__ x, void* __restrict__ y) {
  static_assert(KW == 1 || KW == 2 || KW == 4, "K split");
  constexpr int kSets = kValuWaves / KW;   // row sets per block
  constexpr uint32_t kStepK = KW * kWave * kLaneK;
  using Mg = Int4Magic<XDT>;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int kslot = wave % KW;
  const int rset = wave / KW;
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * kSets + rset) * R;
  const uint32_t magic = vgpr_const(Mg::kMagic);
  const int64_t G = K / kGroup;
  const int64_t zrow = (G + 1) / 2;
  const int kk = static_cast<int>(K);   // K <= 2^24 (checked on the host): lane offsets fit 32 bits

  // Row bases are wavefront-uniform (scalar registers); lanes add 32-bit offsets.
  const uint8_t* crow[R];
  const float* srow[R];
  const uint8_t* zrowp[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = (row0 + r < N) ? row0 + r : N - 1;
    crow[r] = codes + row * (K / 2);
    srow[r] = scales + row * G;
    zrowp[r] = zeros + row * zrow;
  }

  float acc[R][B];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;

  for (uint32_t k0 = 0; k0 < static_cast<uint32_t>(kk); k0 += kStepK) {
    // A wavefront with no lane inside K skips the step; in a partly covered
    // step the lanes past K load the last 32 weights (in bounds) and take
    // zero activations, so the step runs without a divergent branch.
    if (k0 + static_cast<uint32_t>(kslot * (kWave * kLaneK)) >= static_cast<uint32_t>(kk)) break;
    const uint32_t kb_raw = k0 + static_cast<uint32_t>(kslot * (kWave * kLaneK) + lane * kLaneK);
    const bool inside = kb_raw < static_cast<uint32_t>(kk);
    const uint32_t kb = inside ? kb_raw : static_cast<uint32_t>(kk - kLaneK);
    {
      // Every load of the step is issued before any result is consumed, in
      // the order they are needed (activations, scales and zero points, then
      // the codes row by row), so row r is computed as soon as its codes
      // arrive while the later rows are still in flight.
      u32x4 xraw[B][4];
#pragma unroll
      for (int b = 0; b < B; ++b)
#pragma unroll
        for (int c = 0; c < 4; ++c) xraw[b][c] = ld16(x + b * K + kb + 8 * c);
      const uint32_t g = kb >> 7;
      const uint32_t zshift = (g & 1u) * 4u;
      float sc[R];
      uint32_t zb[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        sc[r] = srow[r][g];
        zb[r] = zrowp[r][g >> 1];
      }
      u32x4 cw[R];
#pragma unroll
      for (int r = 0; r < R; ++r) cw[r] = ld16_nt(crow[r] + (kb >> 1));
      __builtin_amdgcn_sched_barrier(0);
      if (!inside) {
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
          for (int c = 0; c < 4; ++c) xraw[b][c] = u32x4{0u, 0u, 0u, 0u};
      }
      float zo[R];
#pragma unroll
      for (int r = 0; r < R; ++r) zo[r] = Mg::offset + static_cast<float>((zb[r] >> zshift) & 0xFu);
      uint32_t xp[B][16];
      float xs[B];
#pragma unroll
      for (int b = 0; b < B; ++b) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const u32x4 a = xraw[b][c];
          xp[b][4 * c] = a.x;
          xp[b][4 * c + 1] = a.y;
          xp[b][4 * c + 2] = a.z;
          xp[b][4 * c + 3] = a.w;
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
          Mg::unpack(words[c], magic, p);
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
  if constexpr ((R * B) % 8 == 0) {
    // Eight sums per wave_sum8: lane l ends up with the sum of value l >> 3.
#pragma unroll
    for (int h = 0; h < R * B / 8; ++h) {
      float v8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v8[i] = acc[(8 * h + i) / B][(8 * h + i) % B];
      const float v = wave_sum8(v8);
      if ((lane & 7) == 0) red[wave][8 * h + (lane >> 3)] = v;
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const float v = wave_sum(acc[r][b]);
        if (lane == 0) red[wave][r * B + b] = v;
      }
  }
  __syncthreads();
  if (threadIdx.x < kSets * R * B) {
    const int set = threadIdx.x / (R * B);
    const int i = threadIdx.x % (R * B);
    const int r = i / B;
    const int b = i % B;
    const int64_t row = (static_cast<int64_t>(blockIdx.x) * kSets + set) * R + r;
    if (row < N) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < KW; ++w) v += red[set * KW + w][i];
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
// and tokens [t0, t0 + 16); wavefront w owns a contiguous range of groups.
// MFMA operand layout (16x16x32): lane l supplies A row l%16 and B column
// l%16, k = 8*(l/16) .. +8 of the instruction; D lane l holds rows
// 4*(l/16) .. +4 of column l%16.  Here each lane loads one 16-byte code
// vector = k-chunks 4*(l/16) .. +4 of a group, so instruction j of the group
// takes chunk 4*(l/16) + j; the activation operand is loaded the same way.
// Scale and zero-point: lane l loads those of D row 4*(l/16) + l%4 and the
// four rows a lane needs are then broadcast inside its quad with DPP.
// Token columns past M read the last valid token (in bounds) and are never
// stored.  All addresses are uniform tile bases plus 32-bit lane offsets.
template <int CTRL>
__device__ __forceinline__ float quad_bcast(float v) { return dpp_f<CTRL>(v); }

// Group pairs: a wavefront works on two consecutive groups at a time, so each
// row's 128-byte line of codes (and the zero-point byte, and an 8-byte pair
// of scales) is consumed in one step instead of being half-read and evicted
// before the next group comes round.
template <int RT>
struct SkinnyLoad {
  u32x4 cw[RT][2];
  float sv[RT][2];
  uint32_t zv[RT];
  u32x4 xr[2][4];
};

// EVEN: G is even, so a pair never runs past the row and the pair of scales
// is one aligned 8-byte load.  Otherwise the last pair's second group reads
// the first one again (in bounds) with a zero scale.
template <int RT, bool EVEN>
__device__ __forceinline__ void skinny_load(SkinnyLoad<RT>& b, int gp, int G, const uint8_t* cbase,
                                            const uint32_t* coff, const float* sbase, const uint32_t* soff,
                                            const uint8_t* zbase, const uint32_t* zoff, const uint16_t* xbase,
                                            uint32_t xoff) {
  const int g = 2 * gp;
  const bool second = EVEN || g + 1 < G;
  const int g1 = second ? g + 1 : g;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    b.cw[rt][0] = ld16_nt(cbase + coff[rt] + g * 64);
    b.cw[rt][1] = ld16_nt(cbase + coff[rt] + g1 * 64);
    if constexpr (EVEN) {
      const float2 sp = *reinterpret_cast<const float2*>(sbase + soff[rt] + g);
      b.sv[rt][0] = sp.x;
      b.sv[rt][1] = sp.y;
    } else {
      b.sv[rt][0] = sbase[soff[rt] + g];
      b.sv[rt][1] = second ? sbase[soff[rt] + g1] : 0.0f;
    }
    b.zv[rt] = zbase[zoff[rt] + gp];
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) b.xr[0][c] = ld16(xbase + xoff + g * kGroup + 8 * c);
#pragma unroll
  for (int c = 0; c < 4; ++c) b.xr[1][c] = ld16(xbase + xoff + g1 * kGroup + 8 * c);
}

template <int XDT, int RT>
__device__ __forceinline__ void skinny_compute(const SkinnyLoad<RT>& b, uint32_t magic, f32x4* acc) {
  using Mg = Int4Magic<XDT>;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t xb[16];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      xb[4 * c] = b.xr[h][c].x;
      xb[4 * c + 1] = b.xr[h][c].y;
      xb[4 * c + 2] = b.xr[h][c].z;
      xb[4 * c + 3] = b.xr[h][c].w;
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
      uint32_t wa[16];
      const uint32_t words[4] = {b.cw[rt][h].x, b.cw[rt][h].y, b.cw[rt][h].z, b.cw[rt][h].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) Mg::unpack(words[j], magic, &wa[4 * j]);
      f32x4 p = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < 4; ++j) p = mfma16x16x32<XDT>(&wa[4 * j], &xb[4 * j], p);
      const float zo_own = Mg::offset + static_cast<float>((b.zv[rt] >> (4 * h)) & 0xFu);
      const float sv = b.sv[rt][h];
      const float s4[4] = {quad_bcast<0x00>(sv), quad_bcast<0x55>(sv), quad_bcast<0xAA>(sv), quad_bcast<0xFF>(sv)};
      const float z4[4] = {quad_bcast<0x00>(zo_own), quad_bcast<0x55>(zo_own), quad_bcast<0xAA>(zo_own),
                           quad_bcast<0xFF>(zo_own)};
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[rt][i] = fmaf(s4[i], fmaf(-z4[i], xg, p[i]), acc[rt][i]);
    }
  }
}

template <int XDT, int YDT, int RT, bool EVEN>
__global__ __launch_bounds__(512) void w4_mfma_skinny_kernel(const uint8_t* __restrict__ codes,
                                                             const float* __restrict__ scales,
                                                             const uint8_t* __restrict__ zeros, int64_t N,
                                                             int64_t K, const uint16_t* __restrict__ x, int64_t M,
                                                             void* __restrict__ y) {
  using Mg = Int4Magic<XDT>;
  extern __shared__ float red[];   // [NW][RT*4][64]
  const uint32_t magic = vgpr_const(Mg::kMagic);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  const int l16 = lane & 15;
  const int quad = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * 16 * RT;
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * 16;
  const int G = static_cast<int>(K / kGroup);
  const int GP = (G + 1) / 2;
  const int zrow = (G + 1) / 2;
  const int rb = static_cast<int>(K / 2);
  const int pper = (GP + nw - 1) / nw;
  const int pbeg = wave * pper;
  const int pend = (pbeg + pper < GP) ? pbeg + pper : GP;

  // Uniform bases; lane offsets clamp rows past N (and tokens past M) in bounds.
  const int rmax = static_cast<int>((N - 1 - row0 < 16 * RT - 1) ? N - 1 - row0 : 16 * RT - 1);
  const uint8_t* cbase = codes + row0 * rb;
  const float* sbase = scales + row0 * G;
  const uint8_t* zbase = zeros + row0 * zrow;
  uint32_t coff[RT], soff[RT], zoff[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int ra = min(16 * rt + l16, rmax);                  // A-operand row
    const int rs = min(16 * rt + 4 * quad + (lane & 3), rmax); // scale row loaded by this lane
    coff[rt] = static_cast<uint32_t>(ra * rb + quad * 16);
    soff[rt] = static_cast<uint32_t>(rs * G);
    zoff[rt] = static_cast<uint32_t>(rs * zrow);
  }
  const int tmax = static_cast<int>((M - 1 - t0 < 15) ? M - 1 - t0 : 15);
  const uint16_t* xbase = x + t0 * K;
  const uint32_t xoff = static_cast<uint32_t>(min(l16, tmax) * static_cast<int>(K) + quad * 32);

  f32x4 acc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  for (int gp = pbeg; gp < pend; ++gp) {
    SkinnyLoad<RT> b;
    skinny_load<RT, EVEN>(b, gp, G, cbase, coff, sbase, soff, zbase, zoff, xbase, xoff);
    __builtin_amdgcn_sched_barrier(0);
    skinny_compute<XDT, RT>(b, magic, acc);
  }

  constexpr int kOut = RT * 4;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * kOut + rt * 4 + i) * kWave + lane] = acc[rt][i];
  __syncthreads();
  for (int o = threadIdx.x; o < kOut * kWave; o += blockDim.x) {
    float v = 0.0f;
    for (int w = 0; w < nw; ++w) v += red[w * kOut * kWave + o];
    const int l = o % kWave;
    const int slot = o / kWave;
    const int i = slot % 4;
    const int rt = slot / 4;
    const int64_t row = row0 + 16 * rt + 4 * (l >> 4) + i;
    const int64_t t = t0 + (l & 15);
    if (row < N && t < M) store_y<YDT>(y, t * N + row, v);
  }
}

// ----------------------------------------------------------------------------
// LDS-tiled MFMA kernel for 2 <= tokens (batched decode and prefill).
//
// Block: 4 wavefronts, output tile MT tokens x 64 weight rows.  The
// wavefronts split K by quantization group (wavefront w takes groups w, w+4,
// ...), so every activation and weight byte of the tile is read from LDS by
// exactly one wavefront, and the four partial tiles are summed through LDS at
// the end in a fixed order.
//
// Operands reach LDS by buffer loads that write LDS directly, each wavefront
// into rings of its own, D groups ahead (no block barrier in the main loop):
//  * activations, one group = MT rows x 256 bytes: sixteen lanes fetch one
//    row's 256 bytes; 16-byte chunk j of row r sits at position j ^ row_swz(r);
//  * codes, one group = 16 NT rows x 64 bytes (NT = 2 or 4 slices of 16
//    weight rows per block): four lanes fetch one row's 64 bytes; 16-byte part p of row r (of a 16-row slice) sits at slot
//    4 r + (p ^ code_swz(r));
//  * scales, one group = 16 NT floats (one 4-byte load per lane; lanes past
//    the block's rows fall outside the buffer and read 0);
// and the block's zero-point bytes are copied to LDS once.  Both swizzles make
// the fragment reads below free of bank conflicts.
//
// MFMA v_mfma_f32_16x16x32_{bf16,f16}: activations are the A operand (lane l:
// token l%16), codes the B operand (lane l: weight row l%16); lane group
// p = l/16 of chunk c in 0..3 covers k = 32 p + 8 c .. +8 of the group, in
// natural order on both sides (the code layout makes Int4Magic::unpack yield
// consecutive pairs, so activations go to the MFMA exactly as loaded).
// The group's column sums X_g come from one more MFMA against a ones operand,
// and each group is folded as  acc += s * (P - (off + z) * X_g).
// ----------------------------------------------------------------------------
constexpr int kLdsWaves = 4;
constexpr int kLdsRows = 64;                  // weight rows per block (NT = 4 slices of 16)
constexpr size_t kLdsBytesMax = 160 * 1024;
constexpr int kScaleGroupBytes = 64 * 4;      // one scale load: 64 lanes x 4 bytes

template <int MT, int NT>
struct LdsCfg {
  static constexpr int kRows = 16 * NT;                    // weight rows per block
  static constexpr int kCodeGroupBytes = kRows * kGroup / 2;
  // Groups loaded ahead per wavefront (ring depth D + 1 for activations,
  // codes and scales alike).  D = 1 for 16 tokens keeps a block at ~66 KiB of
  // LDS, so two blocks share a compute unit.
  static constexpr int kD = MT <= 16 ? 1 : 2;
  static constexpr int kRing = kD + 1;
  static constexpr int kXBytes = MT * kGroup * 2;        // one activation group
  static constexpr int kWaveBytes = kRing * (kXBytes + kCodeGroupBytes + kScaleGroupBytes);
  static constexpr int kXLoads = MT / 4;                 // 1 KiB load instructions per activation group
  static constexpr int kLoadsPerGroup = kXLoads + NT + 1;
  static constexpr int kPartPitch = kRows + 4;           // floats per row of a partial tile
  static_assert(kLdsWaves * MT * kPartPitch * 4 <= kLdsWaves * kWaveBytes, "partial tiles fit the rings");
};

// LDS swizzles.  A ds_read_b128 is served in passes over groups of lanes
// that are not simply 16 consecutive lanes: measured on gfx950 (bank-conflict
// counter), the layout "chunk j of row r at j ^ (r & 15)" still costs two
// passes per read where these cost one.  row_swz: 16-byte chunk j of a
// 256-byte row r sits at j ^ row_swz(r) (the two low bits of r move to the
// high bits of the position).  code_swz: 16-byte part p of a 64-byte row r of
// a 16-row slice sits at slot 4 r + (p ^ code_swz(r)).
__host__ __device__ constexpr int row_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__host__ __device__ constexpr int code_swz(int r) { return ((r >> 2) ^ ((r >> 1) & 2)) & 3; }

// Host and device: it is called from lambdas, which HIP compiles for both sides.
__host__ __device__ inline lds_ptr_t lds_at(uint32_t byte) { return (lds_ptr_t)(uintptr_t)byte; }

template <int XDT, int YDT, int MT, int NT>
__global__ __launch_bounds__(256) void w4_lds_kernel(const uint8_t* __restrict__ codes,
                                                     const float* __restrict__ scales,
                                                     const uint8_t* __restrict__ zeros, int64_t N, int64_t K,
                                                     const uint16_t* __restrict__ x, int64_t M,
                                                     void* __restrict__ y) {
  using Cfg = LdsCfg<MT, NT>;
  constexpr int kRows = Cfg::kRows;
  constexpr int kCodeGroupBytes = Cfg::kCodeGroupBytes;
  using Mg = Int4Magic<XDT>;
  constexpr int RG = Cfg::kRing;
  constexpr int D = Cfg::kD;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // Wave-uniform by construction; readfirstlane makes it a scalar so every
  // buffer-load offset and LDS destination derived from it stays scalar.
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int G = static_cast<int>(K / kGroup);
  const int zb = (G + 1) / 2;

  // Tile order: the blocks of one XCD (block id mod 8) take consecutive tiles,
  // token tiles fastest, so the token tiles of one weight slice run together
  // on one XCD and the slice's codes come from HBM once.
  const int64_t mtiles = (M + MT - 1) / MT;
  const int64_t ntiles = (N + kRows - 1) / kRows;
  const int64_t T = mtiles * ntiles;
  const int64_t per = (T + 7) / 8;
  const int64_t t = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (t >= T) return;
  const int64_t n0 = (t / mtiles) * kRows;
  const int64_t m0 = (t % mtiles) * MT;
  const int64_t nrows = (N - n0 < kRows) ? N - n0 : kRows;
  const int64_t mrows = (M - m0 < MT) ? M - m0 : MT;

  // LDS: per-wavefront rings, then the zero-point table [kRows][zb].
  const uint32_t lbase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  const uint32_t wbase = lbase + wave * Cfg::kWaveBytes;
  const uint32_t xring = wbase;
  const uint32_t cring = wbase + RG * Cfg::kXBytes;
  const uint32_t sring = cring + RG * kCodeGroupBytes;
  uint8_t* const ztab = lds + kLdsWaves * Cfg::kWaveBytes;

  // Buffer resources sized to the tile's valid rows: rows past M / N read 0.
  const int kb2 = static_cast<int>(K) * 2;   // activation row bytes
  const int kh = static_cast<int>(K / 2);    // code row bytes
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x + m0 * K), 0, static_cast<int>(mrows) * kb2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(codes + n0 * (K / 2)), 0, static_cast<int>(nrows) * kh, kBufferWord3);
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(scales + n0 * G), 0, static_cast<int>(nrows) * G * 4, kBufferWord3);

  // Fixed-size offset arrays: HIP drops the host stub of this kernel when an
  // element of a template-dependent-size array is passed to the buffer-load
  // builtin inside a lambda.
  static_assert(Cfg::kXLoads <= 8, "activation loads per group");
  int xoff[8], coff[4];
#pragma unroll
  for (int q = 0; q < Cfg::kXLoads; ++q) {
    const int r = 4 * q + (lane >> 4);
    xoff[q] = r * kb2 + (((lane & 15) ^ row_swz(r & 15)) * 16);
  }
#pragma unroll
  for (int q = 0; q < NT; ++q) {
    const int r = lane >> 2;
    coff[q] = (16 * q + r) * kh + (((lane & 3) ^ code_swz(r)) * 16);
  }
  const int soff = lane * G * 4;

  const int ng = (G > wave) ? (G - wave + kLdsWaves - 1) / kLdsWaves : 0;   // this wave's groups
  auto grp = [&](int i) { return wave + kLdsWaves * min(i, max(ng - 1, 0)); };   // clamped, in range
  auto issue_x = [&](int i) {
    const int g = min(grp(i), G - 1);
    const uint32_t dst = xring + (i % RG) * Cfg::kXBytes;
#pragma unroll
    for (int q = 0; q < Cfg::kXLoads; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, lds_at(dst + q * 1024), 16, xoff[q], g * 256, 0, 0);
  };
  auto issue_w = [&](int i) {
    const int g = min(grp(i), G - 1);
    const uint32_t dst = cring + (i % RG) * kCodeGroupBytes;
#pragma unroll
    for (int q = 0; q < NT; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(cr, lds_at(dst + q * 1024), 16, coff[q], g * 64, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, lds_at(sring + (i % RG) * kScaleGroupBytes), 4, soff, g * 4, 0, 0);
  };

  // Iteration i issues the loads of group i + D into the ring position group
  // i - 1 used; the prologue issues groups 0 .. D-1.  Before group i is
  // computed only the loads of the last D iterations may be in flight.
  for (int i = 0; i < D; ++i) {
    issue_x(i);
    issue_w(i);
  }
  const int zp = zero_pitch(zb);
  copy_zeros_to_lds<256>(ztab, zeros + n0 * zb, kRows, zb, zp, static_cast<int>(nrows), tid);
  __syncthreads();   // zero-point table

  f32x4 acc[MT / 16][NT];
#pragma unroll
  for (int mt = 0; mt < MT / 16; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const uint32_t magic = vgpr_const(Mg::kMagic);
  const uint32_t ones[4] = {Mg::one_pair, Mg::one_pair, Mg::one_pair, Mg::one_pair};
  const int fr = lane & 15;
  const int fp = lane >> 4;
  const int crd = (4 * fr + (fp ^ code_swz(fr))) * 16;   // code fragment slot (per 16-row slice)

  for (int i = 0; i < ng; ++i) {
    issue_x(i + D);
    issue_w(i + D);
    wait_vm<D * Cfg::kLoadsPerGroup>();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int g = wave + kLdsWaves * i;
    const uint8_t* xg = lds + (xring - lbase) + (i % RG) * Cfg::kXBytes;
    const uint8_t* cg = lds + (cring - lbase) + (i % RG) * kCodeGroupBytes;
    const float* sg = reinterpret_cast<const float*>(lds + (sring - lbase) + (i % RG) * kScaleGroupBytes);
    u32x4 cw[NT];
    float sv[NT], zo[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      cw[nt] = *reinterpret_cast<const u32x4*>(cg + nt * 1024 + crd);
      sv[nt] = sg[16 * nt + fr];
      const uint32_t zbyte = ztab[(16 * nt + fr) * zp + (g >> 1)];
      zo[nt] = Mg::offset + static_cast<float>((g & 1) ? (zbyte >> 4) : (zbyte & 15u));
    }
    f32x4 part[MT / 16][NT], xs[MT / 16];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint32_t xa[MT / 16][4];
#pragma unroll
      for (int mt = 0; mt < MT / 16; ++mt) {
        const int r = 16 * mt + fr;
        const u32x4 v = *reinterpret_cast<const u32x4*>(xg + r * 256 + (((4 * fp + c) ^ row_swz(fr)) * 16));
        xa[mt][0] = v.x;
        xa[mt][1] = v.y;
        xa[mt][2] = v.z;
        xa[mt][3] = v.w;
      }
#pragma unroll
      for (int mt = 0; mt < MT / 16; ++mt)
        xs[mt] = mfma16x16x32<XDT>(xa[mt], ones, c == 0 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : xs[mt]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        uint32_t wb[4];
        Mg::unpack(cw[nt][c], magic, wb);
#pragma unroll
        for (int mt = 0; mt < MT / 16; ++mt)
          part[mt][nt] = mfma16x16x32<XDT>(xa[mt], wb, c == 0 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : part[mt][nt]);
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT / 16; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[mt][nt][e] = fmaf(sv[nt], fmaf(-zo[nt], xs[mt][e], part[mt][nt][e]), acc[mt][nt][e]);
  }
  wait_vm<0>();
  __syncthreads();   // every ring is drained; the LDS now holds the partial tiles

  // Partial tile of wavefront w: [MT][kPartPitch] floats; D lane l holds
  // tokens 16 mt + 4 (l/16) + e, weight row 16 nt + l%16.
  float* parts = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int mt = 0; mt < MT / 16; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        parts[(wave * MT + 16 * mt + 4 * fp + e) * Cfg::kPartPitch + 16 * nt + fr] = acc[mt][nt][e];
  __syncthreads();
  // Sum the four partials (wavefront order 0..3) and store: a thread takes 8
  // consecutive weight rows of one token row.
  constexpr int kOct = kRows / 8;
  for (int o = tid; o < MT * kOct; o += 256) {
    const int r = o / kOct;
    const int c0 = (o % kOct) * 8;
    const int64_t m = m0 + r;
    if (m >= M) continue;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float a = parts[(0 * MT + r) * Cfg::kPartPitch + c0 + j];
      a += parts[(1 * MT + r) * Cfg::kPartPitch + c0 + j];
      a += parts[(2 * MT + r) * Cfg::kPartPitch + c0 + j];
      a += parts[(3 * MT + r) * Cfg::kPartPitch + c0 + j];
      v[j] = a;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t n = n0 + c0 + j;
      if (n < N) store_y<YDT>(y, m * N + n, v[j]);
    }
  }
}

// ----------------------------------------------------------------------------
// MFMA kernel for up to 64 tokens when the weight rows give every compute
// unit a block.  Block tile: 16 TT H tokens x 16 NT weight rows, NW = 4 or 8
// wavefronts.  K advances KS = 4 / H groups per step; wavefront w takes group
// KS step + (w % 4) % KS for token slice (w % 4) / KS (TT tiles of 16) and,
// with eight wavefronts, row half w / 4.  So the KS wavefronts of one token
// slice split K, and each code slice is expanded once per TT token tiles
// (TT = 2 halves the unpack work per output against 16-token tiles, and a
// 64-token block reads every code byte from HBM once instead of four times).
//   tokens <= 16: TT = 1, H = 1 (KS = 4);  <= 32: TT = 2, H = 1 (KS = 4);
//   <= 64: TT = 2, H = 2 (KS = 2, so a stage holds 64 tokens x 256 k).
// The block loads each step's tiles cooperatively, every buffer load writing
// 1 KiB of LDS directly: codes as 16 / KS rows x KS 64 contiguous bytes,
// activations as 4 / KS token rows x KS 256 bytes, scales as 16 rows x KS
// groups per wavefront.  Swizzles (16-byte pieces): code piece p of row r at
// p ^ cswz(r) (cswz = r & 15 for 256-byte rows, (r >> 1) & 7 for 128-byte
// rows, so the 16 rows of a fragment read hit 16 different bank groups);
// activation piece p of token t at p ^ row_swz(t & 15); scales transposed,
// [group][row], so the 16 rows of a read are consecutive words.
// S LDS stages (loads S - 1 steps ahead), one barrier per step.  Each block
// starts its walk over K at its own step (its row tile index mod the step
// count), so blocks in flight do not all request the same activation lines.
// ----------------------------------------------------------------------------
template <int NT, int S, int TT, int H, int NW>
struct RowsCfg {
  static constexpr int KS = 4 / H;                         // groups per step
  static constexpr int RS = NW / 4;                        // row splits (wavefronts per K slot and token slice)
  static constexpr int RT = NT / RS;                       // 16-row tiles per wavefront
  static constexpr int kRows = 16 * NT;
  static constexpr int kTokens = 16 * TT * H;
  static constexpr int kRowBytes = KS * 64;                // a code row's bytes per step
  static constexpr int kTokBytes = KS * 256;               // a token row's bytes per step
  static constexpr int kCodeBytes = kRows * kRowBytes;
  static constexpr int kXBytes = kTokens * kTokBytes;
  static constexpr int kScaleBytes = NW * 256;             // per wavefront 16 rows x KS groups (+ pad)
  static constexpr int kStageBytes = kCodeBytes + kXBytes + kScaleBytes;
  static constexpr int kCodeLoads = kCodeBytes / (1024 * NW);   // 1 KiB loads per wavefront per step
  static constexpr int kXLoads = kXBytes / (1024 * NW);
  static constexpr int kLoads = kCodeLoads + kXLoads + 1;
  static constexpr int kPartPitch = kRows + 4;
  static_assert(KS * H == 4 && (KS == 4 || KS == 2), "K slots");
  static_assert((NW == 4 || NW == 8) && RT * RS == NT, "row split");
  static_assert(kCodeBytes % (1024 * NW) == 0 && kXBytes % (1024 * NW) == 0 && kCodeLoads > 0 && kXLoads > 0,
                "whole loads per wavefront");
  static_assert(KS * kTokens * kPartPitch * 4 <= S * kStageBytes, "partial tiles fit the stages");
  static_assert((S - 2) * kLoads < 64, "vmcnt range");
};

__device__ __forceinline__ int code_swz_rows(int r, int ks) { return ks == 4 ? (r & 15) : ((r >> 1) & 7); }

// Loop step st of a block whose walk over K starts at step rot.
__device__ __forceinline__ int rot_step(int st, int rot, int nsteps) {
  const int d = st + rot;
  return d >= nsteps ? d - nsteps : d;
}

// The step-st loads of w4_rows_kernel (all direct to LDS): codes, activations, scales.
template <class Cfg, int S>
__device__ __forceinline__ void rows_issue(int st, int nsteps, int rot, uint32_t lbase, int wave,
                                           __amdgpu_buffer_rsrc_t cr,
                                           __amdgpu_buffer_rsrc_t xr, __amdgpu_buffer_rsrc_t sr, const int* coff,
                                           const int* xoff, int soff) {
  // data step of loop step st (the block's rotation of K); past the end: a
  // reload of the last one, never read
  const int sc = rot_step(min(st, nsteps - 1), rot, nsteps);
  const uint32_t stage = lbase + (st % S) * Cfg::kStageBytes;
  // The scalar offsets go through plain (non-const) ints: a value-dependent
  // expression in that argument makes clang's host pass reject the builtin
  // call, which silently drops the kernel's host-side stub.
  int cso = sc * Cfg::kRowBytes;
  int xso = sc * Cfg::kTokBytes;
  int sso = sc * Cfg::KS * 4;
#pragma unroll
  for (int q = 0; q < Cfg::kCodeLoads; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(cr, (lds_ptr_t)(uintptr_t)(stage + (Cfg::kCodeLoads * wave + q) * 1024),
                                             16, coff[q], cso, 0, 0);
#pragma unroll
  for (int q = 0; q < Cfg::kXLoads; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        xr, (lds_ptr_t)(uintptr_t)(stage + Cfg::kCodeBytes + (Cfg::kXLoads * wave + q) * 1024), 16, xoff[q], xso, 0,
        0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      sr, (lds_ptr_t)(uintptr_t)(stage + Cfg::kCodeBytes + Cfg::kXBytes + wave * 256), 4, soff, sso, 0, 0);
}

template <int XDT, int YDT, int NT, int S, int TT, int H, int NW>
__global__ __launch_bounds__(NW * 64) void w4_rows_kernel(const uint8_t* __restrict__ codes,
                                                      const float* __restrict__ scales,
                                                      const uint8_t* __restrict__ zeros, int64_t N, int64_t K,
                                                      const uint16_t* __restrict__ x, int64_t M,
                                                      void* __restrict__ y) {
  using Cfg = RowsCfg<NT, S, TT, H, NW>;
  constexpr int KS = Cfg::KS;
  constexpr int RT = Cfg::RT;
  constexpr int D = S - 1;
  using Mg = Int4Magic<XDT>;
  constexpr int kRows = Cfg::kRows;
  constexpr int kTokens = Cfg::kTokens;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int ks = (wave & 3) % KS;
  const int hs = (wave & 3) / KS;
  const int rs = wave >> 2;           // this wavefront's row tiles: RT rs .. + RT
  const int G = static_cast<int>(K / kGroup);
  const int zb = (G + 1) / 2;
  const int nsteps = (G + KS - 1) / KS;

  const int64_t mtiles = (M + kTokens - 1) / kTokens;
  const int64_t ntiles = (N + kRows - 1) / kRows;
  const int64_t T = mtiles * ntiles;
  const int64_t per = (T + 7) / 8;
  const int64_t t = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (t >= T) return;
  const int64_t n0 = (t / mtiles) * kRows;
  const int64_t m0 = (t % mtiles) * kTokens;
  const int64_t nrows = (N - n0 < kRows) ? N - n0 : kRows;
  const int64_t mrows = (M - m0 < kTokens) ? M - m0 : kTokens;
  // Blocks start their walk over K at different steps, so that the blocks
  // in flight read different activation lines at any one time (the same
  // lines requested by every compute unit at once queue on a few L2
  // channels).  The sum over K is the same for any start.
  const int rot = static_cast<int>((t / mtiles) % nsteps);

  const uint32_t lbase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  uint8_t* const ztab = lds + S * Cfg::kStageBytes;

  const int kb2 = static_cast<int>(K) * 2;
  const int kh = static_cast<int>(K / 2);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x + m0 * K), 0, static_cast<int>(mrows) * kb2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(codes + n0 * (K / 2)), 0, static_cast<int>(nrows) * kh, kBufferWord3);
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(scales + n0 * G), 0, static_cast<int>(nrows) * G * 4, kBufferWord3);

  // Load offsets (lane l writes LDS byte 16 l of its load's kilobyte, or 4 l
  // for the scales).  Codes: 4 KS lanes per row, slot s = l % (4 KS) takes
  // source piece s ^ cswz(row).  Activations: 16 KS lanes per token row, slot
  // s takes piece s ^ row_swz(token).  Scales: lane l is row 16 w + l % 16,
  // group slot (l / 16) mod KS (for KS = 2 lanes 32..63 repeat 0..31 into the
  // upper half of the region, never read).
  int coff[Cfg::kCodeLoads], xoff[Cfg::kXLoads];
#pragma unroll
  for (int q = 0; q < Cfg::kCodeLoads; ++q) {
    const int r = (Cfg::kCodeLoads * wave + q) * (16 / KS) + lane / (4 * KS);
    const int s = lane % (4 * KS);
    coff[q] = r * kh + ((s ^ code_swz_rows(r, KS)) * 16);
  }
#pragma unroll
  for (int q = 0; q < Cfg::kXLoads; ++q) {
    const int tr = (Cfg::kXLoads * wave + q) * (4 / KS) + lane / (16 * KS);
    const int s = lane % (16 * KS);
    xoff[q] = tr * kb2 + ((s ^ row_swz(tr & 15)) * 16);
  }
  const int soff = (16 * (wave & 3) + (lane & 15)) * G * 4 + ((lane >> 4) & (KS - 1)) * 4;


  for (int st = 0; st < D; ++st) rows_issue<Cfg, S>(st, nsteps, rot, lbase, wave, cr, xr, sr, coff, xoff, soff);
  const int zp = zero_pitch(zb);
  copy_zeros_to_lds<NW * 64>(ztab, zeros + n0 * zb, kRows, zb, zp, static_cast<int>(nrows), tid);

  f32x4 acc[TT][RT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int j = 0; j < RT; ++j) acc[tt][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const uint32_t magic = vgpr_const(Mg::kMagic);
  const uint32_t ones[4] = {Mg::one_pair, Mg::one_pair, Mg::one_pair, Mg::one_pair};
  const int fr = lane & 15;
  const int fp = lane >> 4;

  for (int st = 0; st < nsteps; ++st) {
    // This wavefront's loads of step st have landed (only those of the next
    // D - 1 steps may be in flight); after the barrier every wavefront's
    // have, and all are done with the stage of step st - 1, which step
    // st + D now fills (past the end: a reload that is never read).
    wait_vm<(D - 1) * Cfg::kLoads>();
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    rows_issue<Cfg, S>(st + D, nsteps, rot, lbase, wave, cr, xr, sr, coff, xoff, soff);
    const int g = KS * rot_step(st, rot, nsteps) + ks;
    if (g < G) {
      const uint8_t* cg = lds + (st % S) * Cfg::kStageBytes;
      const uint8_t* xg = cg + Cfg::kCodeBytes;
      const float* sg = reinterpret_cast<const float*>(xg + Cfg::kXBytes);   // [row tile][group slot][row]
      u32x4 cw[RT];
      float sv[RT], zo[RT];
#pragma unroll
      for (int j = 0; j < RT; ++j) {
        const int nt = RT * rs + j;
        const int r = 16 * nt + fr;
        cw[j] = *reinterpret_cast<const u32x4*>(cg + r * Cfg::kRowBytes +
                                                (((4 * ks + fp) ^ code_swz_rows(r, KS)) * 16));
        sv[j] = sg[64 * nt + 16 * ks + fr];
        const uint32_t zbyte = ztab[r * zp + (g >> 1)];
        zo[j] = Mg::offset + static_cast<float>((g & 1) ? (zbyte >> 4) : (zbyte & 15u));
      }
      f32x4 part[TT][RT], xs[TT];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t wb[RT][4];
#pragma unroll
        for (int j = 0; j < RT; ++j) Mg::unpack(cw[j][c], magic, wb[j]);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          const int tr = 16 * (TT * hs + tt) + fr;                       // token row of the block
          const int xp = 16 * ks + 4 * fp + c;                           // piece of the token row
          const u32x4 v = *reinterpret_cast<const u32x4*>(xg + tr * Cfg::kTokBytes + ((xp ^ row_swz(fr)) * 16));
          const uint32_t xa[4] = {v.x, v.y, v.z, v.w};
          xs[tt] = mfma16x16x32<XDT>(xa, ones, c == 0 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : xs[tt]);
#pragma unroll
          for (int j = 0; j < RT; ++j)
            part[tt][j] = mfma16x16x32<XDT>(xa, wb[j], c == 0 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : part[tt][j]);
        }
      }
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int j = 0; j < RT; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[tt][j][e] = fmaf(sv[j], fmaf(-zo[j], xs[tt][e], part[tt][j][e]), acc[tt][j][e]);
    }
  }
  wait_vm<0>();
  __syncthreads();   // every stage is idle; the LDS now holds the partial tiles

  // Partial tiles [K slot][token][row], summed over the K slots in order.
  float* parts = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int j = 0; j < RT; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        parts[(ks * kTokens + 16 * (TT * hs + tt) + 4 * fp + e) * Cfg::kPartPitch + 16 * (RT * rs + j) + fr] =
            acc[tt][j][e];
  __syncthreads();
  constexpr int kOct = kRows / 8;
  for (int o = tid; o < kTokens * kOct; o += NW * 64) {
    const int r = o / kOct;
    const int c0 = (o % kOct) * 8;
    const int64_t m = m0 + r;
    if (m >= M) continue;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float a = parts[r * Cfg::kPartPitch + c0 + j];
#pragma unroll
      for (int q = 1; q < KS; ++q) a += parts[(q * kTokens + r) * Cfg::kPartPitch + c0 + j];
      v[j] = a;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t n = n0 + c0 + j;
      if (n < N) store_y<YDT>(y, m * N + n, v[j]);
    }
  }
}

// ----------------------------------------------------------------------------
// MFMA kernel for larger token counts: a block computes a BM x 128 tile of Y
// (BM = 64 tokens), its four wavefronts each BM tokens x 32 weight
// rows, walking K one group at a time in lock step.  The activation tile of a
// group is loaded to LDS once per block and shared by the four wavefronts;
// each wavefront loads the codes and scales of its own 32 rows.  Groups are
// staged kTileD ahead in kTileD + 1 slots, with one block barrier per group.
// LDS layout of a slot (same swizzles as the kernel above):
//  * activations, BM rows x 256 bytes, chunk j of row r at position j ^ row_swz(r);
//  * codes, 8 slices of 16 rows x 64 bytes, part p of row r at 4 r + (p ^ code_swz(r));
//  * scales, 256 bytes per wavefront: its 32 rows, loaded twice over.
// Two slots (one group ahead): three blocks of BM = 64 fit a compute unit
// (about 51 KiB each at K = 4096), so each SIMD interleaves the ALU work of
// one wavefront with the matrix work of two others; three slots (75 KiB, two
// blocks per unit) measured slower (AWQ's M = 2048 products by ~7%).  XS: the caller supplies the column sums X_g ([M][G] fp32, the
// sums of the activations exactly as the kernel reads them); each slot then
// also holds the tile's BM sums of its group, loaded like the scales, and
// the wavefronts skip the 4 MT matrix instructions per group that would
// otherwise recompute them (each of the four wavefronts the same ones).
// ----------------------------------------------------------------------------
constexpr int kTileN = 128;
constexpr int kTileD = 1;
constexpr int kTileSlots = kTileD + 1;

template <int BM, bool XS = false>
struct TileCfg {
  static constexpr int kXBytes = BM * kGroup * 2;
  static constexpr int kCodeBytes = kTileN * kGroup / 2;          // 8 KiB
  static constexpr int kScaleBytes = kLdsWaves * 256;
  static constexpr int kSumBytes = XS ? BM * 4 : 0;               // the tile's column sums of the group
  static constexpr int kSlotBytes = kXBytes + kCodeBytes + kScaleBytes + kSumBytes;
  static constexpr int kXLoads = BM / 16;                          // per wavefront per group
  static constexpr int kLoads = kXLoads + 2 + 1 + (XS ? 1 : 0);
  static_assert(!XS || BM == kWave, "one 4-byte load per lane holds the tile's sums");
  static constexpr int kPartPitch = kTileN + 4;
  static_assert(BM * kPartPitch * 4 <= kTileSlots * kSlotBytes, "output tile fits the slots");
};

// Loads of group i (clamped to the last group: past the end it reloads a
// group that is never read) into slot i % kTileSlots, kLoads instructions.
// (The LDS destinations are cast in place: in the host pass a function
// template that calls lds_at is dropped from overload resolution.)
template <int BM, bool XS>
__device__ __forceinline__ void tile_issue(int i, int G, int wave, uint32_t lbase, __amdgpu_buffer_rsrc_t xr,
                                           __amdgpu_buffer_rsrc_t cr, __amdgpu_buffer_rsrc_t sr,
                                           __amdgpu_buffer_rsrc_t qr, const int* xoff, const int* coff, int soff,
                                           int qoff) {
  using Cfg = TileCfg<BM, XS>;
  const int g = min(i, G - 1);
  const uint32_t slot = lbase + (i % kTileSlots) * Cfg::kSlotBytes;
#pragma unroll
  for (int q = 0; q < Cfg::kXLoads; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(uintptr_t)(slot + (wave * Cfg::kXLoads + q) * 1024), 16,
                                             xoff[q], g * 256, 0, 0);
#pragma unroll
  for (int q = 0; q < 2; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(cr, (lds_ptr_t)(uintptr_t)(slot + Cfg::kXBytes + (2 * wave + q) * 1024),
                                             16, coff[q], g * 64, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      sr, (lds_ptr_t)(uintptr_t)(slot + Cfg::kXBytes + Cfg::kCodeBytes + wave * 256), 4, soff, g * 4, 0, 0);
  // Every wavefront writes the same BM sums (lane l: token l), so each one's
  // own wait covers them.
  if constexpr (XS)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        qr, (lds_ptr_t)(uintptr_t)(slot + Cfg::kXBytes + Cfg::kCodeBytes + Cfg::kScaleBytes), 4, qoff, g * 4, 0, 0);
}

template <int XDT, int YDT, int BM, bool XS = false>
__global__ __launch_bounds__(256) void w4_tile_kernel(const uint8_t* __restrict__ codes,
                                                      const float* __restrict__ scales,
                                                      const uint8_t* __restrict__ zeros, int64_t N, int64_t K,
                                                      const uint16_t* __restrict__ x, int64_t M,
                                                      void* __restrict__ y, const float* __restrict__ xsum = nullptr) {
  using Cfg = TileCfg<BM, XS>;
  using Mg = Int4Magic<XDT>;
  constexpr int MT = BM / 16;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int G = static_cast<int>(K / kGroup);
  const int zb = (G + 1) / 2;

  // Tile order: consecutive tiles per XCD, in bands of gm token tiles whose
  // activations (gm x BM x K x 2 bytes) fit in about 2 MiB of the XCD's L2;
  // within a band the token tiles run fastest, so the blocks sharing a weight
  // slice run together and the band's activations are fetched from memory
  // once rather than once per weight slice.  (With every token tile in one
  // band this is token tiles fastest over the whole matrix.)
  const int64_t mtiles = (M + BM - 1) / BM;
  const int64_t ntiles = (N + kTileN - 1) / kTileN;
  const int64_t T = mtiles * ntiles;
  const int64_t per = (T + 7) / 8;
  const int64_t t = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (t >= T) return;
  const int64_t band_cap = (int64_t{2} << 20) / (int64_t{BM} * K * 2);
  const int64_t gm_max = band_cap > 1 ? band_cap : 1;
  const int64_t band = t / (gm_max * ntiles);
  const int64_t m_first = band * gm_max;
  const int64_t gm = (mtiles - m_first < gm_max) ? mtiles - m_first : gm_max;
  const int64_t r = t - band * gm_max * ntiles;
  const int64_t n0 = (r / gm) * kTileN;
  const int64_t m0 = (m_first + r % gm) * BM;
  const int64_t nrows = (N - n0 < kTileN) ? N - n0 : kTileN;
  const int64_t mrows = (M - m0 < BM) ? M - m0 : BM;

  const uint32_t lbase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  uint8_t* const ztab = lds + kTileSlots * Cfg::kSlotBytes;

  // Buffer resources sized to the tile's valid rows: rows past M / N read 0.
  const int kb2 = static_cast<int>(K) * 2;
  const int kh = static_cast<int>(K / 2);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x + m0 * K), 0, static_cast<int>(mrows) * kb2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(codes + n0 * (K / 2)), 0, static_cast<int>(nrows) * kh, kBufferWord3);
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(scales + n0 * G), 0, static_cast<int>(nrows) * G * 4, kBufferWord3);
  // Column sums, rows m0 .. m0 + mrows of [M][G] (tokens past M read 0).
  const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(XS ? xsum + m0 * G : scales), 0, XS ? static_cast<int>(mrows) * G * 4 : 0, kBufferWord3);
  const int qoff = lane * G * 4;

  // Load q of this wavefront: activation rows 4 (wave MT + q) .. +4, code
  // slice 2 wave + q, and its 32 scale rows (lane l: row 32 wave + l % 32).
  int xoff[4], coff[2];
  static_assert(Cfg::kXLoads <= 4, "activation loads per group");
#pragma unroll
  for (int q = 0; q < Cfg::kXLoads; ++q) {
    const int r = 4 * (wave * Cfg::kXLoads + q) + (lane >> 4);
    xoff[q] = r * kb2 + (((lane & 15) ^ row_swz(r & 15)) * 16);
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = lane >> 2;
    coff[q] = (16 * (2 * wave + q) + r) * kh + (((lane & 3) ^ code_swz(r)) * 16);
  }
  const int soff = (32 * wave + (lane & 31)) * G * 4;


  for (int i = 0; i < kTileD; ++i) tile_issue<BM, XS>(i, G, wave, lbase, xr, cr, sr, qr, xoff, coff, soff, qoff);
  const int zp = zero_pitch(zb);
  copy_zeros_to_lds<256>(ztab, zeros + n0 * zb, kTileN, zb, zp, static_cast<int>(nrows), tid);

  f32x4 acc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const uint32_t magic = vgpr_const(Mg::kMagic);
  const uint32_t ones[4] = {Mg::one_pair, Mg::one_pair, Mg::one_pair, Mg::one_pair};
  const int fr = lane & 15;
  const int fp = lane >> 4;
  const int crd = (4 * fr + (fp ^ code_swz(fr))) * 16;

  for (int i = 0; i < G; ++i) {
    // Group i has landed for this wavefront (only group i + 1's loads may be
    // outstanding); after the barrier it has landed for every wavefront, and
    // every wavefront is done with the slot of group i - 1, which group
    // i + kTileD now refills.
    wait_vm<(kTileD - 1) * Cfg::kLoads>();
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    tile_issue<BM, XS>(i + kTileD, G, wave, lbase, xr, cr, sr, qr, xoff, coff, soff, qoff);
    const uint8_t* xg = lds + (i % kTileSlots) * Cfg::kSlotBytes;
    const uint8_t* cg = xg + Cfg::kXBytes;
    const float* sg = reinterpret_cast<const float*>(cg + Cfg::kCodeBytes + wave * 256);
    u32x4 cw[2];
    float sv[2], zo[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      cw[nt] = *reinterpret_cast<const u32x4*>(cg + (2 * wave + nt) * 1024 + crd);
      sv[nt] = sg[16 * nt + fr];
      const uint32_t zbyte = ztab[(32 * wave + 16 * nt + fr) * zp + (i >> 1)];
      zo[nt] = Mg::offset + static_cast<float>((i & 1) ? (zbyte >> 4) : (zbyte & 15u));
    }
    f32x4 part[MT][2], xs[MT];
    if constexpr (XS) {
      // D lane l of token tile mt needs the sums of tokens 16 mt + 4 (l / 16) .. + 4
      const float* qg = reinterpret_cast<const float*>(cg + Cfg::kCodeBytes + Cfg::kScaleBytes);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) xs[mt] = *reinterpret_cast<const f32x4*>(qg + 16 * mt + 4 * fp);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint32_t xa[MT][4];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(xg + (16 * mt + fr) * 256 + (((4 * fp + c) ^ row_swz(fr)) * 16));
        xa[mt][0] = v.x;
        xa[mt][1] = v.y;
        xa[mt][2] = v.z;
        xa[mt][3] = v.w;
      }
      if constexpr (!XS) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          xs[mt] = mfma16x16x32<XDT>(xa[mt], ones, c == 0 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : xs[mt]);
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        uint32_t wb[4];
        Mg::unpack(cw[nt][c], magic, wb);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          part[mt][nt] = mfma16x16x32<XDT>(xa[mt], wb, c == 0 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : part[mt][nt]);
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[mt][nt][e] = fmaf(sv[nt], fmaf(-zo[nt], xs[mt][e], part[mt][nt][e]), acc[mt][nt][e]);
  }
  wait_vm<0>();
  __syncthreads();   // every slot is drained; the LDS now holds the output tile

  // Output tile [BM][kPartPitch] floats: D lane l of (mt, nt) holds tokens
  // 16 mt + 4 (l / 16) + e, weight row 32 wave + 16 nt + l % 16.
  float* tile = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        tile[(16 * mt + 4 * fp + e) * Cfg::kPartPitch + 32 * wave + 16 * nt + fr] = acc[mt][nt][e];
  __syncthreads();
  // A thread stores 8 consecutive weight rows of one token row.
  for (int o = tid; o < BM * (kTileN / 8); o += 256) {
    const int r = o / (kTileN / 8);
    const int c0 = (o % (kTileN / 8)) * 8;
    const int64_t m = m0 + r;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t n = n0 + c0 + j;
      if (n < N) store_y<YDT>(y, m * N + n, tile[r * Cfg::kPartPitch + c0 + j]);
    }
  }
}

// ----------------------------------------------------------------------------
// Host side.
// ----------------------------------------------------------------------------
constexpr int64_t kMaxW4K = int64_t{1} << 24;

int check_common(const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K, int group,
                 const void* x, int x_dtype, int64_t M, const void* y, int y_dtype) {
  if (!codes || !scales || !zeros || !x || !y) return QMM_EINVAL;
  if (N <= 0 || K <= 0 || M <= 0 || group <= 0 || K % group != 0) return QMM_EINVAL;
  if ((x_dtype != QMM_BF16 && x_dtype != QMM_F16 && x_dtype != QMM_F32 && x_dtype != QMM_I32) ||
      (y_dtype != QMM_BF16 && y_dtype != QMM_F16 && y_dtype != QMM_F32 && y_dtype != QMM_I32))
    return QMM_EINVAL;
  if (group != kGroup) return QMM_EUNSUPPORTED;
  // Lane and buffer offsets within a tile are 32-bit: at most 64 rows of
  // K / 2 code bytes or K x 2 activation bytes each stay below 2^31.
  if (K > kMaxW4K || N > INT32_MAX || M > INT32_MAX) return QMM_ERANGE;
  if (x_dtype != QMM_BF16 && x_dtype != QMM_F16) return QMM_EUNSUPPORTED;
  if (y_dtype != x_dtype && y_dtype != QMM_F32) return QMM_EUNSUPPORTED;
  if (!aligned(codes, 16) || !aligned(x, 16) || !aligned(scales, 4) || !aligned(y, y_dtype == QMM_F32 ? 4 : 2))
    return QMM_EALIGN;
  return QMM_OK;
}

template <int XDT, int YDT, int B, int KW>
void launch_valu_kw(const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K,
                    const uint16_t* x, void* y, hipStream_t s) {
  constexpr int R = 8;   // rows per wavefront: 8 x 16 bytes in flight per lane
  const dim3 grid(static_cast<unsigned>(ceil_div(N, R * (kValuWaves / KW))));
  gemv_valu_kernel<XDT, YDT, B, R, KW><<<grid, dim3(kValuWaves * kWave), 0, s>>>(codes, scales, zeros, N, K, x, y);
}

// Four wavefronts along K once a row has more than 6144 weights, two above
// 2048, else one.
template <int XDT, int YDT, int B>
void launch_valu(const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K,
                 const uint16_t* x, void* y, hipStream_t s) {
  if (K > 6144) launch_valu_kw<XDT, YDT, B, 4>(codes, scales, zeros, N, K, x, y, s);
  else if (K > 2048) launch_valu_kw<XDT, YDT, B, 2>(codes, scales, zeros, N, K, x, y, s);
  else launch_valu_kw<XDT, YDT, B, 1>(codes, scales, zeros, N, K, x, y, s);
}

template <int XDT, int YDT>
void launch_valu_b(int64_t B, const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K,
                   const uint16_t* x, void* y, hipStream_t s) {
  // One or two tokens (more go to the MFMA kernels).
  if (B == 1) launch_valu<XDT, YDT, 1>(codes, scales, zeros, N, K, x, y, s);
  else launch_valu<XDT, YDT, 2>(codes, scales, zeros, N, K, x, y, s);
}

// Wavefronts per block for the skinny MFMA kernel: split K further when the
// grid alone would leave compute units short of wavefronts.
// The per-block reduction buffer (nw * out_per_wave floats) stays within 64 KiB.
int skinny_waves(int64_t blocks, int64_t G, int64_t out_per_wave) {
  const int64_t target = static_cast<int64_t>(device_cus()) * 16;   // wavefronts wanted in flight
  int nw = 4;
  while (nw < 8 && blocks * nw < target && G >= 4 * nw * 2 &&
         2 * nw * out_per_wave * static_cast<int64_t>(sizeof(float)) <= 65536)
    nw *= 2;
  return nw;
}

template <int XDT, int YDT, int RT>
void launch_skinny(const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K,
                   const uint16_t* x, int64_t M, void* y, hipStream_t s) {
  const int64_t bx = ceil_div(N, 16 * RT);
  const int64_t by = ceil_div(M, 16);
  const int64_t G = K / kGroup;
  const int nw = skinny_waves(bx * by, ceil_div(G, 2) * 2, static_cast<int64_t>(RT) * 4 * kWave);
  const size_t lds = static_cast<size_t>(nw) * RT * 4 * kWave * sizeof(float);
  const dim3 grid(static_cast<unsigned>(bx), static_cast<unsigned>(by));
  if (G % 2 == 0)
    w4_mfma_skinny_kernel<XDT, YDT, RT, true><<<grid, dim3(nw * kWave), lds, s>>>(codes, scales, zeros, N, K, x, M, y);
  else
    w4_mfma_skinny_kernel<XDT, YDT, RT, false><<<grid, dim3(nw * kWave), lds, s>>>(codes, scales, zeros, N, K, x, M,
                                                                                  y);
}

// Four 16-row tiles per wavefront halve the activation re-reads per code
// byte; narrow matrices keep two so that enough blocks exist.
template <int XDT, int YDT>
void launch_skinny_m(int64_t M, const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N,
                     int64_t K, const uint16_t* x, void* y, hipStream_t s) {
  if (N >= static_cast<int64_t>(device_cus()) * 64)
    launch_skinny<XDT, YDT, 4>(codes, scales, zeros, N, K, x, M, y, s);
  else
    launch_skinny<XDT, YDT, 2>(codes, scales, zeros, N, K, x, M, y, s);
}

// LDS-tiled kernel: MT = 16 for up to 16 tokens, else 32.  Returns false
// (nothing launched) when the zero-point table would not fit in LDS.
template <int XDT, int YDT, int MT, int NT>
bool launch_lds_t(const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K,
                  const uint16_t* x, int64_t M, void* y, hipStream_t s) {
  using Cfg = LdsCfg<MT, NT>;
  const int64_t G = K / kGroup;
  const size_t lds = static_cast<size_t>(kLdsWaves) * Cfg::kWaveBytes +
                    static_cast<size_t>(Cfg::kRows) * zero_pitch(static_cast<int>((G + 1) / 2));
  if (lds > kLdsBytesMax) return false;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&w4_lds_kernel<XDT, YDT, MT, NT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  const int64_t tiles = ceil_div(M, MT) * ceil_div(N, Cfg::kRows);
  const dim3 grid(static_cast<unsigned>(ceil_div(tiles, 8) * 8));
  w4_lds_kernel<XDT, YDT, MT, NT><<<grid, dim3(kLdsWaves * kWave), lds, s>>>(codes, scales, zeros, N, K, x, M, y);
  return true;
}

// 32 weight rows per block instead of 64 when 64-row tiles would leave
// compute units without a block.
template <int XDT, int YDT, int MT>
bool launch_lds_m(const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K,
                  const uint16_t* x, int64_t M, void* y, hipStream_t s) {
  if (ceil_div(M, MT) * ceil_div(N, kLdsRows) < static_cast<int64_t>(device_cus()))
    return launch_lds_t<XDT, YDT, MT, 2>(codes, scales, zeros, N, K, x, M, y, s);
  return launch_lds_t<XDT, YDT, MT, 4>(codes, scales, zeros, N, K, x, M, y, s);
}

template <int XDT, int YDT, int BM>
bool launch_tile_t(const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K,
                   const uint16_t* x, int64_t M, void* y, hipStream_t s) {
  using Cfg = TileCfg<BM>;
  const int64_t G = K / kGroup;
  const size_t lds = static_cast<size_t>(kTileSlots) * Cfg::kSlotBytes +
                    static_cast<size_t>(kTileN) * zero_pitch(static_cast<int>((G + 1) / 2));
  if (lds > kLdsBytesMax) return false;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&w4_tile_kernel<XDT, YDT, BM>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  const int64_t tiles = ceil_div(M, BM) * ceil_div(N, kTileN);
  const dim3 grid(static_cast<unsigned>(ceil_div(tiles, 8) * 8));
  w4_tile_kernel<XDT, YDT, BM><<<grid, dim3(kLdsWaves * kWave), lds, s>>>(codes, scales, zeros, N, K, x, M, y);
  return true;
}

// The shared-tile kernel with the caller's column sums (fp32 out); false
// (nothing launched) where w4a16_gemm would not choose that kernel: up to
// 64 tokens, fewer 64 x 128 tiles than compute units, or a zero-point table
// too large for LDS.
template <int XDT>
bool launch_tile_colsums(const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K,
                         const uint16_t* x, const float* xsum, int64_t M, float* y, hipStream_t s) {
  using Cfg = TileCfg<64, true>;
  if (M <= 64 || ceil_div(M, 64) * ceil_div(N, kTileN) < static_cast<int64_t>(device_cus())) return false;
  const int64_t G = K / kGroup;
  // the plain kernel's LDS must fit too, or w4a16_gemm would not pick it
  const size_t plain = static_cast<size_t>(kTileSlots) * TileCfg<64>::kSlotBytes +
                       static_cast<size_t>(kTileN) * zero_pitch(static_cast<int>((G + 1) / 2));
  const size_t lds = static_cast<size_t>(kTileSlots) * Cfg::kSlotBytes +
                     static_cast<size_t>(kTileN) * zero_pitch(static_cast<int>((G + 1) / 2));
  if (plain > kLdsBytesMax || lds > kLdsBytesMax) return false;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&w4_tile_kernel<XDT, QMM_F32, 64, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  const int64_t tiles = ceil_div(M, 64) * ceil_div(N, kTileN);
  const dim3 grid(static_cast<unsigned>(ceil_div(tiles, 8) * 8));
  w4_tile_kernel<XDT, QMM_F32, 64, true><<<grid, dim3(kLdsWaves * kWave), lds, s>>>(codes, scales, zeros, N, K, x, M,
                                                                                    y, xsum);
  return true;
}

template <int XDT, int YDT, int NT, int S, int TT = 1, int H = 1, int NW = 4>
bool launch_rows_t(const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K,
                   const uint16_t* x, int64_t M, void* y, hipStream_t s) {
  using Cfg = RowsCfg<NT, S, TT, H, NW>;
  const int64_t G = K / kGroup;
  const size_t lds = S * static_cast<size_t>(Cfg::kStageBytes) +
                    static_cast<size_t>(Cfg::kRows) * zero_pitch(static_cast<int>((G + 1) / 2));
  if (lds > kLdsBytesMax) return false;
  // the activation buffer of a block tile (tokens x K x 2 bytes) is addressed with 32-bit offsets
  if (static_cast<int64_t>(Cfg::kTokens) * K * 2 > INT32_MAX) return false;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&w4_rows_kernel<XDT, YDT, NT, S, TT, H, NW>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  const int64_t tiles = ceil_div(M, Cfg::kTokens) * ceil_div(N, Cfg::kRows);
  const dim3 grid(static_cast<unsigned>(ceil_div(tiles, 8) * 8));
  w4_rows_kernel<XDT, YDT, NT, S, TT, H, NW><<<grid, dim3(NW * kWave), lds, s>>>(codes, scales, zeros, N, K, x, M,
                                                                               y);
  return true;
}

// The cooperative-load kernel, up to 64 tokens: 64 weight rows per block
// when that gives at least three quarters of the compute units a block, 32
// rows when that gives most units two; otherwise false (few rows, long K: one
// block per unit would serialize its steps on the barrier), and the split-K
// kernel, whose wavefronts run independently, takes the call.  Token tiles:
// 16 up to 16 tokens, 32 up to 32, 64 beyond (each code slice read and
// expanded once per block instead of once per 16 tokens).  Two stages and
// four wavefronts: on 14336 x 4096 (224 blocks) measured against three or
// four stages, eight wavefronts (64 or 32 rows each) and 32-row blocks, this
// was fastest or within noise at 16, 32 and 64 tokens.
template <int XDT, int YDT>
bool launch_rows(const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K,
                 const uint16_t* x, int64_t M, void* y, hipStream_t s) {
  const int64_t cus = device_cus();
  if (M > 16 && 4 * ceil_div(M, M > 32 ? 64 : 32) * ceil_div(N, 64) >= 3 * cus) {
    if (M > 32 && launch_rows_t<XDT, YDT, 4, 2, 2, 2>(codes, scales, zeros, N, K, x, M, y, s)) return true;
    if (M <= 32 && launch_rows_t<XDT, YDT, 4, 2, 2, 1>(codes, scales, zeros, N, K, x, M, y, s)) return true;
  }
  const int64_t mt = ceil_div(M, 16);
  if (4 * mt * ceil_div(N, 64) >= 3 * cus) return launch_rows_t<XDT, YDT, 4, 2>(codes, scales, zeros, N, K, x, M, y, s);
  if (2 * mt * ceil_div(N, 32) >= 3 * cus) return launch_rows_t<XDT, YDT, 2, 2>(codes, scales, zeros, N, K, x, M, y, s);
  return false;
}

template <int XDT, int YDT>
bool launch_lds(const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K,
                const uint16_t* x, int64_t M, void* y, hipStream_t s) {
  if (M <= 64 && launch_rows<XDT, YDT>(codes, scales, zeros, N, K, x, M, y, s)) return true;
  if (M <= 16) return launch_lds_m<XDT, YDT, 16>(codes, scales, zeros, N, K, x, M, y, s);
  // The shared-tile kernel once its 64 x 128 tiles give every compute unit a
  // block; below that the split-K kernel's smaller tiles keep more units busy.
  if (M > 32 && ceil_div(M, 64) * ceil_div(N, kTileN) >= static_cast<int64_t>(device_cus()) &&
      launch_tile_t<XDT, YDT, 64>(codes, scales, zeros, N, K, x, M, y, s))
    return true;
  return launch_lds_m<XDT, YDT, 32>(codes, scales, zeros, N, K, x, M, y, s);
}

// Tokens >= 2 (or the GEMM): the LDS-tiled kernels, else the skinny kernel
// when their zero-point table does not fit in LDS.
template <int XDT, int YDT>
void launch_mfma_t(const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K,
                   const uint16_t* x, int64_t M, void* y, hipStream_t s) {
  if (!launch_lds<XDT, YDT>(codes, scales, zeros, N, K, x, M, y, s))
    launch_skinny_m<XDT, YDT>(M, codes, scales, zeros, N, K, x, y, s);
}

void launch_mfma(int x_dtype, int y_dtype, const uint8_t* codes, const float* scales, const uint8_t* zeros,
                 int64_t N, int64_t K, const uint16_t* x, int64_t M, void* y, hipStream_t s) {
  if (x_dtype == QMM_BF16) {
    if (y_dtype == QMM_F32) launch_mfma_t<QMM_BF16, QMM_F32>(codes, scales, zeros, N, K, x, M, y, s);
    else launch_mfma_t<QMM_BF16, QMM_BF16>(codes, scales, zeros, N, K, x, M, y, s);
  } else {
    if (y_dtype == QMM_F32) launch_mfma_t<QMM_F16, QMM_F32>(codes, scales, zeros, N, K, x, M, y, s);
    else launch_mfma_t<QMM_F16, QMM_F16>(codes, scales, zeros, N, K, x, M, y, s);
  }
}

}  // namespace
}  // namespace qmm

using namespace qmm;

extern "C" int w4a16_gemv(const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K,
                          int group, const void* x, int x_dtype, int64_t B, void* y, int y_dtype, void* stream) {
  if (group != kGroup) {   // other group sizes: the stored formats with fp32 scales
    if (B > 8) return QMM_EUNSUPPORTED;
    return matmul_fmt(codes, scales, zeros, N, K, group, 4, QMM_F32, x, x_dtype, B, y, y_dtype, stream);
  }
  int st = check_common(codes, scales, zeros, N, K, group, x, x_dtype, B, y, y_dtype);
  if (st != QMM_OK) return st;
  if (B > 8) return QMM_EUNSUPPORTED;
  hipStream_t s = as_stream(stream);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  // Two tokens still stream the weights fastest on the vector ALUs (measured
  // 26-28 us against 30-35 us for the MFMA kernels on the 70B-class
  // matrices); from three on the MFMA kernels win.
  if (B >= 3) {
    launch_mfma(x_dtype, y_dtype, codes, scales, zeros, N, K, xp, B, y, s);
    return launch_status();
  }
  if (x_dtype == QMM_BF16) {
    if (y_dtype == QMM_F32) launch_valu_b<QMM_BF16, QMM_F32>(B, codes, scales, zeros, N, K, xp, y, s);
    else launch_valu_b<QMM_BF16, QMM_BF16>(B, codes, scales, zeros, N, K, xp, y, s);
  } else {
    if (y_dtype == QMM_F32) launch_valu_b<QMM_F16, QMM_F32>(B, codes, scales, zeros, N, K, xp, y, s);
    else launch_valu_b<QMM_F16, QMM_F16>(B, codes, scales, zeros, N, K, xp, y, s);
  }
  return launch_status();
}

namespace qmm {

int w4a16_gemm_colsums(const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K,
                       const uint16_t* X, const float* xsum, int x_dtype, int64_t M, float* Y, hipStream_t s) {
  int st = check_common(codes, scales, zeros, N, K, kGroup, X, x_dtype, M, Y, QMM_F32);
  if (st != QMM_OK) return st;
  if (!xsum || !aligned(xsum, 16)) return QMM_EINVAL;
  const bool done = x_dtype == QMM_BF16
                        ? launch_tile_colsums<QMM_BF16>(codes, scales, zeros, N, K, X, xsum, M, Y, s)
                        : launch_tile_colsums<QMM_F16>(codes, scales, zeros, N, K, X, xsum, M, Y, s);
  if (done) return launch_status();
  return w4a16_gemm(codes, scales, zeros, N, K, kGroup, X, x_dtype, M, Y, QMM_F32, s);
}

}  // namespace qmm

extern "C" int w4a16_gemm(const uint8_t* codes, const float* scales, const uint8_t* zeros, int64_t N, int64_t K,
                          int group, const void* X, int x_dtype, int64_t M, void* Y, int y_dtype, void* stream) {
  if (group != kGroup)
    return matmul_fmt(codes, scales, zeros, N, K, group, 4, QMM_F32, X, x_dtype, M, Y, y_dtype, stream);
  int st = check_common(codes, scales, zeros, N, K, group, X, x_dtype, M, Y, y_dtype);
  if (st != QMM_OK) return st;
  hipStream_t s = as_stream(stream);
  const uint16_t* xp = static_cast<const uint16_t*>(X);
  launch_mfma(x_dtype, y_dtype, codes, scales, zeros, N, K, xp, M, Y, s);
  return launch_status();
}
