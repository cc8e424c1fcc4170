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

// s_waitcnt with only a vector-memory count (expcnt and lgkmcnt left open).
// On gfx950 the count covers vector-memory loads and stores alike, and they
// complete in issue order.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Buffer descriptor of a byte range as four words (base address, size),
// made explicitly wave-uniform, for the assembly loads below.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 rsrc_words(const void* base, int64_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)(uint32_t)bytes);
  r[3] = 0x00020000;
  return r;
}

// One 16-byte-per-lane HBM -> LDS load issued as assembly: lane l's 16 bytes
// from base + voff + soff land at LDS byte address lds + 16 l.  The compiler
// does not see it as an LDS write, so it does not make later LDS reads wait
// for every load in flight (it would before each transpose read); a kernel
// using it orders these loads itself with explicit vmcnt waits and barriers.
// The LDS address reaches the instruction through M0, passed as an input
// operand bound to that register: the compiler writes M0 itself and knows
// it is read here, so nothing the compiler keeps in M0 is overwritten.
__device__ __forceinline__ void lds_dma16_asm(i32x4 rsrc, uint32_t lds, int voff, int soff) {
  asm volatile("buffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "{m0}"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc),
                 "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory");
}

// Launch a kernel taking one parameter block by value, `threads` (256 unless
// given) threads per workgroup; returns the launch's own status.
template <typename P>
inline hipError_t launch_kernel(void (*kernel)(const P), dim3 grid, const P& p, hipStream_t s, int threads = 256) {
  void* args[] = {const_cast<P*>(&p)};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, dim3(threads), args, 0, s);
}

}  // namespace muon
