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
// One launch covers up to eight such problems (e.g. the q and k heads of a
// layer), the workgroup index picking the problem.
#include "muon_internal.h"
#include "device_util.h"
#include "muon_mi355x.h"

namespace muon {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int N = 128;         // matrix edge
constexpr int PITCH = N + 8;   // bf16 per LDS row (272 bytes: 16 rows cover all 64 banks)

// KSM: the most chunks any problem of the launch has (4, 8 or 16).  Each
// thread sums UB = 16 / KSM chunks of 8 elements at a time, so that every
// thread has up to 32 16-byte loads in flight whatever the chunk count.
template <int KSM>
__global__ __launch_bounds__(256) void poly128_kernel(const Poly128Group grp) {
  __shared__ __attribute__((aligned(16))) uint16_t As[N * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[N * PITCH];
  int pi = 0;
  while (pi + 1 < grp.nprob && (int)blockIdx.x >= grp.start[pi + 1]) ++pi;
  const Poly128Params& p = grp.prob[pi];
  const int b = blockIdx.x - grp.start[pi], tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t mm = (int64_t)N * N;

  // 1. A = bf16(rs^2 * sum_s part[b][s]); thread -> 8 chunks of 8 elements,
  // UB at a time.  All partial loads of those UB chunks are issued before
  // the first add (one workgroup reads the whole ksplit x 64 KiB, so it
  // needs many in flight together); the adds then run in chunk order.
  constexpr int U = N * N / 8 / 256;
  constexpr int UB = 16 / KSM;
  static_assert(U % UB == 0, "whole rounds");
  const float rsb = p.rs ? p.rs[b] : 1.f;
  const float alpha = rsb * rsb;
  const float* part = p.part + (int64_t)b * p.ksplit * mm;
  const int ks = p.ksplit;
#pragma unroll 1
  for (int u0 = 0; u0 < U; u0 += UB) {
    f32x4 t[UB][KSM][2];
#pragma unroll
    for (int v = 0; v < UB; ++v) {
      const float* src = part + (tid + 256 * (u0 + v)) * 8;
#pragma unroll
      for (int k = 0; k < KSM; ++k)
        if (k < ks) {
          t[v][k][0] = *(const f32x4*)(src + k * mm);
          t[v][k][1] = *(const f32x4*)(src + k * mm + 4);
        }
    }
#pragma unroll
    for (int v = 0; v < UB; ++v) {
      f32x4 s0 = t[v][0][0], s1 = t[v][0][1];
#pragma unroll
      for (int k = 1; k < KSM; ++k)
        if (k < ks) {
          s0 += t[v][k][0];
          s1 += t[v][k][1];
        }
      u32x4 w;
      w[0] = pack_bf2(alpha * s0[0], alpha * s0[1]);
      w[1] = pack_bf2(alpha * s0[2], alpha * s0[3]);
      w[2] = pack_bf2(alpha * s1[0], alpha * s1[1]);
      w[3] = pack_bf2(alpha * s1[2], alpha * s1[3]);
      const int e8 = (tid + 256 * (u0 + v)) * 8;
      const int i = e8 / N, j = e8 % N;
      *(u32x4*)(As + i * PITCH + j) = w;
    }
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

hipError_t launch_poly128(const Poly128Group& g, hipStream_t s) {
  if (g.nprob < 1 || g.nprob > kMaxPoly128 || g.start[0] != 0) return hipErrorInvalidValue;
  int ksm = 0;
  for (int i = 0; i < g.nprob; ++i) {
    const Poly128Params& p = g.prob[i];
    if (p.ksplit < 1 || p.ksplit > kMaxKsplit || p.ldb < N || p.ldb % 8 != 0) return hipErrorInvalidValue;
    if (g.start[i + 1] < g.start[i]) return hipErrorInvalidValue;
    ksm = p.ksplit > ksm ? p.ksplit : ksm;
  }
  const int grid = g.start[g.nprob];
  if (grid <= 0) return hipSuccess;
  if (ksm <= 4) return launch_kernel(poly128_kernel<4>, dim3(grid), g, s);
  if (ksm <= 8) return launch_kernel(poly128_kernel<8>, dim3(grid), g, s);
  return launch_kernel(poly128_kernel<16>, dim3(grid), g, s);
}

}  // namespace muon
