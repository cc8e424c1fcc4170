// Split-K Gram sum and the polynomial of one Newton-Schulz iteration, fused,
// for matrices whose short side pads to 128 (e.g. the 128-row heads of
// per-head Newton-Schulz, "Muon under AutoTP orthogonalizes each shard ...",
// option 3).
//
// The iteration's polynomial B = b A + c A^2 ("core.optimizer.
// layer_sharded_muon", use_syrk) is, at m = 128, 4 MFLOP: a launch of the
// tiled GEMM for it is all latency.  Here one workgroup of eight waves per
// matrix
//   0. on the first iteration, finalizes the Frobenius norm (rs) from the
//      prep kernel's partials;
//   1. sums the fp32 chunk products of the split-K Gram in chunk order,
//      scales by rs^2 (first iteration) and rounds to bf16 once: A exactly
//      as the separate sum would store it, but into LDS only.  A is
//      symmetric and the chunk products hold their 32 x 32 blocks on and
//      above the diagonal only (10 of 16, the diagonal ones exactly
//      symmetric), so those are read and each is written to LDS twice, as
//      itself and as its mirror;
//   2. computes A A with v_mfma_f32_32x32x16_bf16 (A is symmetric, so both
//      operands are rows of A), each wave two 32 x 32 blocks;
//   3. writes B = bf16(c (A A) + b A) through LDS with 16-byte stores.
// The matrix is read by one workgroup, so its loads are all issued before
// the first add.  One launch covers up to eight such problems (e.g. the q
// and k heads of a layer), the workgroup index picking the problem.
#include "muon_internal.h"
#include "device_util.h"
#include "muon_mi355x.h"

namespace muon {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int N = 128;         // matrix edge
constexpr int PITCH = N + 8;   // bf16 per LDS row (272 bytes: 16 rows cover all 64 banks)
constexpr int NT = 512;        // threads per workgroup
constexpr int UPT = 10 * 256 / NT;  // 16-byte units (4 fp32) of the 10 upper blocks per thread

// Upper block t (0..9) in row order: (0,0) (0,1) (0,2) (0,3) (1,1) (1,2)
// (1,3) (2,2) (2,3) (3,3).
__device__ __forceinline__ void upper_block(int t, int& bi, int& bj) {
  bi = t < 4 ? 0 : (t < 7 ? 1 : (t < 9 ? 2 : 3));
  const int first = bi == 0 ? 0 : (bi == 1 ? 4 : (bi == 2 ? 7 : 9));
  bj = bi + (t - first);
}

// KSM: the most chunks any problem of the launch has (4, 8 or 16).  A
// thread owns UPT units and loads UB of them (all their chunks) at a time.
template <int KSM>
__global__ __launch_bounds__(NT) void poly128_kernel(const Poly128Group grp) {
  __shared__ __attribute__((aligned(16))) uint16_t As[N * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[N * PITCH];
  int pi = 0;
  while (pi + 1 < grp.nprob && (int)blockIdx.x >= grp.start[pi + 1]) ++pi;
  const Poly128Params& p = grp.prob[pi];
  const int b = blockIdx.x - grp.start[pi], tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t mm = (int64_t)N * N;

  // 1. A = bf16(rs^2 * sum_s part[b][s]) on and above the diagonal blocks.
  // Unit u = tid + NT v of the upper blocks is row (u % 256) / 8, columns
  // 4 (u % 8) .. + 3 of upper block u / 256 = 2 v + tid / 256 (one block per
  // wave and v).
  constexpr int UB = KSM <= 8 ? UPT : 1;
  static_assert(UPT % UB == 0, "whole rounds");
  float rsb;
  if (p.nsum) {
    // rs = 1 / (sqrt(||X||_F^2) + eps) from the norm partials, summed as the
    // norm finalize sums them (its 256 threads are waves 0..3 here), NaN
    // when the sum is not finite.
    __shared__ float red[4];
    if (tid < 256) {
      const float* src = p.nsum + (int64_t)b * p.ntiles;
      float sq = 0.f;
      for (int i = tid; i < p.ntiles; i += 256) sq += src[i];
      sq = wave_sum(sq);
      if (lane == 0) red[wave] = sq;
    }
    __syncthreads();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    rsb = __builtin_isfinite(tot) ? 1.f / (sqrtf(tot) + p.eps) : __builtin_nanf("");
    if (tid == 0) p.rs_out[b] = rsb;
  } else {
    rsb = p.rs ? p.rs[b] : 1.f;
  }
  const float alpha = rsb * rsb;
  const float* part = p.part + (int64_t)b * p.ksplit * mm;
  const int ks = p.ksplit;
  const int r32 = (tid & 255) >> 3, c4 = (tid & 7) * 4;
#pragma unroll 1
  for (int v0 = 0; v0 < UPT; v0 += UB) {
    f32x4 t[UB][KSM];
#pragma unroll
    for (int v = 0; v < UB; ++v) {
      int bi, bj;
      upper_block(2 * (v0 + v) + (tid >> 8), bi, bj);
      const float* src = part + (32 * bi + r32) * N + 32 * bj + c4;
#pragma unroll
      for (int k = 0; k < KSM; ++k)
        if (k < ks) t[v][k] = *(const f32x4*)(src + k * mm);
    }
#pragma unroll
    for (int v = 0; v < UB; ++v) {
      f32x4 s0 = t[v][0];
#pragma unroll
      for (int k = 1; k < KSM; ++k)
        if (k < ks) s0 += t[v][k];
      int bi, bj;
      upper_block(2 * (v0 + v) + (tid >> 8), bi, bj);
      const int i = 32 * bi + r32, j = 32 * bj + c4;
      u32x2 w;
      w[0] = pack_bf2(alpha * s0[0], alpha * s0[1]);
      w[1] = pack_bf2(alpha * s0[2], alpha * s0[3]);
      *(u32x2*)(As + i * PITCH + j) = w;
      if (bi != bj) {
        As[(j + 0) * PITCH + i] = (uint16_t)(w[0] & 0xffffu);
        As[(j + 1) * PITCH + i] = (uint16_t)(w[0] >> 16);
        As[(j + 2) * PITCH + i] = (uint16_t)(w[1] & 0xffffu);
        As[(j + 3) * PITCH + i] = (uint16_t)(w[1] >> 16);
      }
    }
  }
  __syncthreads();

  // 2. Wave (wm, wn) computes rows 32 wm .., columns 64 wn .. of A A as two
  // 32 x 32 blocks.  MFMA operands: lane l supplies row l % 32 of the block
  // with the 8 K values 8 (l / 32) .. + 7 of the 16-wide K step (for the B
  // operand: column l % 32, i.e. row l % 32 of the symmetric A).
  const int wm = wave >> 1, wn = wave & 1;
  f32x16 acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  const int kl = 8 * (lane >> 5);
#pragma unroll
  for (int k0 = 0; k0 < N; k0 += 16) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(As + (32 * wm + (lane & 31)) * PITCH + k0 + kl));
    bf16x8 q[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      q[j] = __builtin_bit_cast(bf16x8, *(const u32x4*)(As + (64 * wn + 32 * j + (lane & 31)) * PITCH + k0 + kl));
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q[j], acc[j], 0, 0, 0);
  }

  // 3. Accumulator register r of a block holds row 8 (r / 4) + 4 (l / 32) +
  // r % 4 and column l % 32.  B = bf16(c acc + b A), staged in LDS.
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * wm + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      const int col = 64 * wn + 32 * j + (lane & 31);
      const float v = p.c * acc[j][r] + p.b * bf2f(As[row * PITCH + col]);
      Bs[row * PITCH + col] = f2bf(v);
    }
  __syncthreads();
  uint16_t* const out = (uint16_t*)p.B + (int64_t)b * p.b_bs;
#pragma unroll
  for (int u = 0; u < N * N / 8 / NT; ++u) {
    const int e8 = (tid + NT * u) * 8;
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
    if (p.nsum && (p.ntiles < 1 || !p.rs_out)) return hipErrorInvalidValue;
    if (g.start[i + 1] < g.start[i]) return hipErrorInvalidValue;
    ksm = p.ksplit > ksm ? p.ksplit : ksm;
  }
  const int grid = g.start[g.nprob];
  if (grid <= 0) return hipSuccess;
  if (ksm <= 4) return launch_kernel(poly128_kernel<4>, dim3(grid), g, s, NT);
  if (ksm <= 8) return launch_kernel(poly128_kernel<8>, dim3(grid), g, s, NT);
  return launch_kernel(poly128_kernel<16>, dim3(grid), g, s, NT);
}

}  // namespace muon
