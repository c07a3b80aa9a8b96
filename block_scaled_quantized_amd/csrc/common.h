// common.h -- internal helpers shared by the HIP sources of libmxgemm.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "mxgemm.h"

#define MX_HD __host__ __device__ __forceinline__
#define MX_DEV __device__ __forceinline__

namespace mx {

// Status of the most recent launch on this thread: hipGetLastError after a kernel launch.
inline int launch_status() { return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_LAUNCH; }

// The MX_SYNC_CHECK debug switch (environment variable, read at every call; set and not "0"): a GPU
// entry point whose work was queued waits for its stream and returns MX_ERR_LAUNCH when the stream
// reports an error, so an asynchronous fault surfaces at the call that caused it. Off by default:
// entry points then never synchronise.
inline int sync_check(int status, hipStream_t st) {
  if (status != MX_OK) return status;
  const char* e = std::getenv("MX_SYNC_CHECK");
  if (!e || e[0] == '\0' || (e[0] == '0' && e[1] == '\0')) return status;
  if (hipStreamSynchronize(st) != hipSuccess) {
    (void)hipGetLastError();
    return MX_ERR_LAUNCH;
  }
  return status;
}

// 0 when the current device is gfx950, MX_ERR_ARCH otherwise (cached per device id).
int check_arch();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

template <typename T>
MX_HD T ceil_div(T a, T b) { return (a + b - 1) / b; }

}  // namespace mx
