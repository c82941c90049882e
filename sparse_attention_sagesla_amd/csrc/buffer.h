// Buffer-resource addressing for the HBM-bound kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sagesla {

typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Raw buffer resource over nbytes from p (gfx9 descriptor: 32-bit data format, no stride,
// no swizzle). Each access adds a 32-bit lane offset and a scalar offset in hardware, so
// no 64-bit lane address is formed; loads past nbytes read zero and stores past it are
// dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)nbytes, 0x00020000);
}

// A value that every lane holds alike, moved to scalar registers, so that what is built
// from it stays scalar.
__device__ __forceinline__ size_t scalar_off(size_t u) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return ((size_t)hi << 32) | lo;
}

}  // namespace sagesla
