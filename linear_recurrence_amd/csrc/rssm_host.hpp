// Host-side helpers shared by the C-ABI entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "replayssm.h"

namespace rssm {

// Dynamic LDS a decode workgroup may request.
constexpr size_t kMaxLds = 64 * 1024;

static inline bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

static inline bool valid_dtype(int32_t t) { return t == RSSM_F32 || t == RSSM_BF16; }

// Launch with the error code of the launch itself (not a stale one left in
// the thread's last-error slot by earlier runtime calls).
template <typename Args>
static inline int launch_kernel(const void* fn, unsigned grid, unsigned block,
                                size_t lds, hipStream_t stream, const Args& a) {
  void* kargs[] = {const_cast<Args*>(&a)};
  const hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(block), kargs, lds, stream);
  return e == hipSuccess ? RSSM_OK : RSSM_ELAUNCH;
}

}  // namespace rssm
