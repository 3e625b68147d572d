// qmm_internal.h -- host-side helpers shared by the libqmm entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmm.h"

namespace qmm {

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Status of the launches just made on this thread.
inline int launch_status() { return hipGetLastError() == hipSuccess ? QMM_OK : QMM_EHIP; }

// Compute units of the current device (cached per device ordinal).
int device_cus();

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace qmm
