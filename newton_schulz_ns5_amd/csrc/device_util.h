// Device helpers for the gfx950 kernels: bf16 conversion, wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bf16 pair, round to nearest even, NaN kept (quiet): one
// v_cvt_pk_bf16_f32.  On gfx950 it gives the same bits as rounding the fp32
// pattern in integer arithmetic (add 0x7fff plus the kept lsb, set the quiet
// bit of a NaN), checked over ties, denormals, overflow and NaNs.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint16_t f2bf(float f) { return (uint16_t)pack_bf2(f, 0.f); }

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
