// abi.hip -- host-only entry points of libqmm (status strings, sizes) and the
// per-device CU-count cache used to size persistent grids.

#include <atomic>

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
