// Device-side load helpers shared by the matrix-core kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pa {

// Wave-uniform read of memory that no launch of the calling kernel writes (block tables,
// int8/int4 scales), through the scalar cache.  Going through the constant address space keeps
// these reads off the vector-memory counter, so waiting for a table entry never waits for the
// K/V tiles requested before it (vector loads complete in order).
template <typename T>
__device__ __forceinline__ T uniform_load(const T* base, int64_t idx) {
  const __attribute__((address_space(4))) T* p = (const __attribute__((address_space(4))) T*)base;
  return p[idx];
}

}  // namespace pa
