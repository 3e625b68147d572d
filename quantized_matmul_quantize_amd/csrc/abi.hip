// abi.hip -- host-only entry points of libqmm (status strings, sizes), the
// per-device CU-count cache used to size persistent grids, and the plain
// streaming read used to measure the bandwidth the HBM-bound kernels can reach.

#include <atomic>

#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace qmm

extern "C" const char* qmm_status_string(int status) {
  switch (status) {
    case QMM_OK: return "QMM_OK";
    case QMM_EINVAL: return "QMM_EINVAL: invalid argument (null pointer, non-positive size, K % group != 0 or bad dtype)";
    case QMM_EUNSUPPORTED: return "QMM_EUNSUPPORTED: valid but not implemented (bits, group size or dtype)";
    case QMM_EALIGN: return "QMM_EALIGN: tensor pointer not aligned";
    case QMM_EWORKSPACE: return "QMM_EWORKSPACE: workspace missing or too small";
    case QMM_EHIP: return "QMM_EHIP: HIP launch failed";
    case QMM_ERANGE: return "QMM_ERANGE: size outside the range the arithmetic guarantees";
    default: return "QMM_E?: unknown status";
  }
}

extern "C" int qmm_version(void) { return 10000; }

extern "C" int qmm_w4_sizes(int64_t N, int64_t K, int group, size_t* codes_bytes, size_t* scales_bytes,
                            size_t* zeros_bytes) {
  if (N <= 0 || K <= 0 || group <= 0 || K % group != 0) return QMM_EINVAL;
  const int64_t G = K / group;
  if (codes_bytes) *codes_bytes = static_cast<size_t>(N) * static_cast<size_t>((K + 1) / 2);
  if (scales_bytes) *scales_bytes = static_cast<size_t>(N) * static_cast<size_t>(G) * 4u;
  if (zeros_bytes) *zeros_bytes = static_cast<size_t>(N) * static_cast<size_t>((G + 1) / 2);
  return QMM_OK;
}

namespace qmm {
namespace {

__global__ __launch_bounds__(256) void stream_zero_kernel(uint32_t* out) { *out = 0u; }

// Every 16-byte piece read once, all folded by XOR into one word so that no
// load can be dropped; one atomic per wavefront.  Block b reads the
// contiguous range [b per, (b + 1) per) of pieces, eight 1 KiB wavefront
// loads in flight at a time (128 bytes per lane).
constexpr int kReadUnroll = 8;

__global__ __launch_bounds__(256) void stream_read_kernel(const uint8_t* __restrict__ p, int64_t pieces, int64_t per,
                                                          uint32_t* __restrict__ out) {
  const int64_t begin = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t end = (begin + per < pieces) ? begin + per : pieces;
  uint32_t acc = 0u;
  for (int64_t i = begin + threadIdx.x; i < end; i += kReadUnroll * 256) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const int64_t j = i + u * 256;
      v[u] = (j < end) ? ld16_nt(p + 16 * j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (int o = 32; o > 0; o >>= 1) acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), o, kWave));
  if ((threadIdx.x & (kWave - 1)) == 0) atomicXor(out, acc);
}

}  // namespace
}  // namespace qmm

extern "C" int qmm_stream_read(const void* data, size_t bytes, uint32_t* out, void* stream) {
  using namespace qmm;
  if (!data || !out || bytes == 0) return QMM_EINVAL;
  if (!aligned(data, 16) || bytes % 16 != 0 || !aligned(out, 4)) return QMM_EALIGN;
  hipStream_t s = as_stream(stream);
  const int64_t pieces = static_cast<int64_t>(bytes / 16);
  // ranges of whole 8-load rounds, at most four blocks per compute unit
  const int64_t round = int64_t{kReadUnroll} * 256;
  const int64_t cap = static_cast<int64_t>(device_cus()) * 4;
  const int64_t per = ceil_div(ceil_div(pieces, cap), round) * round;
  const int64_t blocks = ceil_div(pieces, per);
  stream_zero_kernel<<<1, 1, 0, s>>>(out);
  stream_read_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(static_cast<const uint8_t*>(data), pieces, per,
                                                                   out);
  return launch_status();
}
