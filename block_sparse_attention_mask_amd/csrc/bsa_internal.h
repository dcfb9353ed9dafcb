// Internal helpers shared by the library's HIP translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsattn.h"

#define BSA_LAUNCH_CHECK()                        \
  do {                                            \
    if (hipGetLastError() != hipSuccess) return BSA_ERR_HIP; \
  } while (0)

#define BSA_HIP(call)                             \
  do {                                            \
    if ((call) != hipSuccess) return BSA_ERR_HIP; \
  } while (0)

static inline hipStream_t bsa_hip_stream(bsa_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

static inline bool bsa_aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Wave-wide helpers (wavefront size 64 on CDNA).
__device__ __forceinline__ uint64_t bsa_lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}
