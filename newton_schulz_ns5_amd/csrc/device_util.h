// Device helpers for the gfx950 kernels: bf16 conversion, wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bf16, round to nearest even; NaN stays NaN (quiet).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

// Sum over the 64 lanes of a wavefront with an xor butterfly.  Every lane
// ends with the same, bitwise identical value (each pairwise step adds the
// same two operands on both partners), and the order depends only on the
// lane layout, so the result is deterministic.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Load one element of either dtype as float.
__device__ __forceinline__ float load_elem(const void* base, int64_t idx, bool bf16) {
  return bf16 ? bf2f(((const uint16_t*)base)[idx]) : ((const float*)base)[idx];
}

__device__ __forceinline__ void store_elem(void* base, int64_t idx, float v, bool bf16) {
  if (bf16) ((uint16_t*)base)[idx] = f2bf(v);
  else ((float*)base)[idx] = v;
}

// Launch a kernel taking one parameter block by value, 256 threads per
// workgroup; returns the launch's own status.
template <typename P>
inline hipError_t launch_kernel(void (*kernel)(const P), dim3 grid, const P& p, hipStream_t s) {
  void* args[] = {const_cast<P*>(&p)};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, dim3(256), args, 0, s);
}

}  // namespace muon
