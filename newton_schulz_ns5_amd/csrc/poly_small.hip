// Split-K Gram sum and the polynomial of one Newton-Schulz iteration, fused,
// for matrices whose short side pads to 128 (e.g. the 128-row heads of
// per-head Newton-Schulz, "Muon under AutoTP orthogonalizes each shard ...",
// option 3).
//
// The iteration's polynomial B = b A + c A^2 ("core.optimizer.
// layer_sharded_muon", use_syrk) is, at m = 128, 4 MFLOP: a launch of the
// tiled GEMM for it is all latency.  Here one workgroup per matrix
//   1. sums the fp32 chunk products of the split-K Gram in chunk order,
//      scales by rs^2 (first iteration) and rounds to bf16 once: A exactly
//      as the separate sum would store it, but into LDS only;
//   2. computes A A with v_mfma_f32_32x32x16_bf16 (A is symmetric, so both
//      operands are rows of A), each of the four waves a 64 x 64 quadrant;
//   3. writes B = bf16(c (A A) + b A) through LDS with 16-byte stores.
#include "muon_internal.h"
#include "device_util.h"
#include "muon_mi355x.h"

namespace muon {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int N = 128;         // matrix edge
constexpr int PITCH = N + 8;   // bf16 per LDS row (272 bytes: 16 rows cover all 64 banks)

__global__ __launch_bounds__(256) void poly128_kernel(const Poly128Params p) {
  __shared__ __attribute__((aligned(16))) uint16_t As[N * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[N * PITCH];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t mm = (int64_t)N * N;

  // 1. A = bf16(rs^2 * sum_s part[b][s]); thread -> 8 chunks of 8 elements.
  // All of a chunk's ksplit partial loads are issued before the first add
  // (one workgroup reads the whole ksplit x 64 KiB, so it needs them in
  // flight together); the adds then run in chunk order.
  const float rsb = p.rs ? p.rs[b] : 1.f;
  const float alpha = rsb * rsb;
  const float* part = p.part + (int64_t)b * p.ksplit * mm;
  const int ks = p.ksplit;
#pragma unroll 1
  for (int u = 0; u < 8; ++u) {
    const int e8 = (tid + 256 * u) * 8;
    const float* src = part + e8;
    f32x4 t[kMaxKsplit][2];
#pragma unroll
    for (int k = 0; k < kMaxKsplit; ++k)
      if (k < ks) {
        t[k][0] = *(const f32x4*)(src + k * mm);
        t[k][1] = *(const f32x4*)(src + k * mm + 4);
      }
    f32x4 s0 = t[0][0], s1 = t[0][1];
#pragma unroll
    for (int k = 1; k < kMaxKsplit; ++k)
      if (k < ks) {
        s0 += t[k][0];
        s1 += t[k][1];
      }
    u32x4 w;
    w[0] = pack_bf2(alpha * s0[0], alpha * s0[1]);
    w[1] = pack_bf2(alpha * s0[2], alpha * s0[3]);
    w[2] = pack_bf2(alpha * s1[0], alpha * s1[1]);
    w[3] = pack_bf2(alpha * s1[2], alpha * s1[3]);
    const int i = e8 / N, j = e8 % N;
    *(u32x4*)(As + i * PITCH + j) = w;
  }
  __syncthreads();

  // 2. Wave (wm, wn) computes rows 64 wm .., columns 64 wn .. of A A as 2 x 2
  // blocks of 32 x 32.  MFMA operands: lane l supplies row l % 32 of the
  // block with the 8 K values 8 (l / 32) .. + 7 of the 16-wide K step (for
  // the B operand: column l % 32, i.e. row l % 32 of the symmetric A).
  const int wm = wave >> 1, wn = wave & 1;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int kl = 8 * (lane >> 5);
#pragma unroll
  for (int k0 = 0; k0 < N; k0 += 16) {
    bf16x8 a[2], q[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      a[i] = __builtin_bit_cast(bf16x8, *(const u32x4*)(As + (64 * wm + 32 * i + (lane & 31)) * PITCH + k0 + kl));
      q[i] = __builtin_bit_cast(bf16x8, *(const u32x4*)(As + (64 * wn + 32 * i + (lane & 31)) * PITCH + k0 + kl));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], q[j], acc[i][j], 0, 0, 0);
  }

  // 3. Accumulator register r of a block holds row 8 (r / 4) + 4 (l / 32) +
  // r % 4 and column l % 32.  B = bf16(c acc + b A), staged in LDS.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 64 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = 64 * wn + 32 * j + (lane & 31);
        const float v = p.c * acc[i][j][r] + p.b * bf2f(As[row * PITCH + col]);
        Bs[row * PITCH + col] = f2bf(v);
      }
  __syncthreads();
  uint16_t* const out = (uint16_t*)p.B + (int64_t)b * p.b_bs;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int e8 = (tid + 256 * u) * 8;
    const int i = e8 / N, j = e8 % N;
    *(u32x4*)(out + i * p.ldb + j) = *(const u32x4*)(Bs + i * PITCH + j);
  }
}

}  // namespace

hipError_t launch_poly128(const Poly128Params& p, int nb, hipStream_t s) {
  if (nb <= 0) return hipSuccess;
  if (p.ksplit < 1 || p.ksplit > kMaxKsplit || p.ldb < N || p.ldb % 8 != 0) return hipErrorInvalidValue;
  return launch_kernel(poly128_kernel, dim3(nb), p, s);
}

}  // namespace muon
