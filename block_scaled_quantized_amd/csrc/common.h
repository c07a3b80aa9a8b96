// common.h -- internal helpers shared by the HIP sources of libmxgemm.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxgemm.h"

#define MX_HD __host__ __device__ __forceinline__
#define MX_DEV __device__ __forceinline__

namespace mx {

// Status of the most recent launch on this thread: hipGetLastError after a kernel launch.
inline int launch_status() { return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_LAUNCH; }

// 0 when the current device is gfx950, MX_ERR_ARCH otherwise (cached per device id).
int check_arch();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

template <typename T>
MX_HD T ceil_div(T a, T b) { return (a + b - 1) / b; }

}  // namespace mx
