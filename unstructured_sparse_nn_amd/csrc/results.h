// results.h -- result words written by kernels (into the caller's pinned
// host words, or into device words that are copied back).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace snk {

// Store of a result word at system scope, so that it has reached host memory
// when the kernel ends: with pinned host words the host reads it once a later
// completion word arrives, without a stream sync.
__device__ __forceinline__ void store_result(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

}  // namespace snk
