// fp32 GEMMs of one Newton-Schulz iteration (fp32 compute mode) on gfx950.
//
// Same three products and the same tile scheduling as the bf16 path, in
// true fp32: operands are fp32 in LDS and products run on
// v_mfma_f32_32x32x2_f32 (no reduced-precision inputs).  A workgroup of 256
// threads owns a 64 x 64 tile as a 2x2 arrangement of waves with one 32x32
// MFMA block each; K advances 16 at a time through two LDS stages.
#include "muon_internal.h"
#include "device_util.h"
#include "muon_mi355x.h"

namespace muon {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BT = 64;        // tile edge
constexpr int BKF = 16;       // K step
constexpr int LDF = BKF + 1;  // padded LDS row (floats)

template <bool SYRK>
__device__ __forceinline__ void decode_tile_f32(const GemmParams& p, int& b, int& tm, int& tn) {
  const int G = gridDim.x, wg = blockIdx.x, per = G >> 3;
  const int pid = wg < (per << 3) ? (wg & 7) * per + (wg >> 3) : wg;
  b = pid / p.tiles_per_batch;
  int t = pid - b * p.tiles_per_batch;
  if constexpr (SYRK) {
    const int T = p.tiles_m;
    tm = 0;
    while (t >= T - tm) { t -= T - tm; ++tm; }
    tn = tm + t;
  } else {
    tm = t / p.tiles_n;
    tn = t - tm * p.tiles_n;
  }
}

template <bool NN, bool SYRK>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const GemmParams p) {
  __shared__ float Ps[2][BT * LDF];
  __shared__ float Qs[2][BT * LDF];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int b, tm, tn;
  decode_tile_f32<SYRK>(p, b, tm, tn);

  const float* Pg = (const float*)p.P + (int64_t)b * p.sP + (int64_t)tm * BT * p.ldp;
  const float* Qg = NN ? (const float*)p.Q + (int64_t)b * p.sQ + (int64_t)tn * BT
                       : (const float*)p.Q + (int64_t)b * p.sQ + (int64_t)tn * BT * p.ldq;
  f32x4 pr, qr;
  auto gload = [&](int k0) {
    pr = *(const f32x4*)(Pg + (int64_t)(tid >> 2) * p.ldp + k0 + (tid & 3) * 4);
    if constexpr (NN)
      qr = *(const f32x4*)(Qg + (int64_t)(k0 + (tid >> 4)) * p.ldq + (tid & 15) * 4);
    else
      qr = *(const f32x4*)(Qg + (int64_t)(tid >> 2) * p.ldq + k0 + (tid & 3) * 4);
  };
  auto sstore = [&](int s) {
#pragma unroll
    for (int e = 0; e < 4; ++e) Ps[s][(tid >> 2) * LDF + (tid & 3) * 4 + e] = pr[e];
    if constexpr (NN) {
#pragma unroll
      for (int e = 0; e < 4; ++e) Qs[s][((tid & 15) * 4 + e) * LDF + (tid >> 4)] = qr[e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) Qs[s][(tid >> 2) * LDF + (tid & 3) * 4 + e] = qr[e];
    }
  };

  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  // MFMA 32x32x2: lane l supplies A[l % 32][l / 32] and B[l / 32][l % 32].
  auto compute = [&](int s) {
    const float* pa = &Ps[s][(wm * 32 + (lane & 31)) * LDF + (lane >> 5)];
    const float* qa = &Qs[s][(wn * 32 + (lane & 31)) * LDF + (lane >> 5)];
#pragma unroll
    for (int ks = 0; ks < BKF / 2; ++ks)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(pa[ks * 2], qa[ks * 2], acc, 0, 0, 0);
  };

  const int KT = p.K / BKF;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * BKF);
    compute(cur);
    if (kt + 1 < KT) sstore(cur ^ 1);
    __syncthreads();
  }

  const float rsb = p.rs ? p.rs[b] : 1.f;
  const float alpha = p.alpha * (p.alpha_pow == 2 ? rsb * rsb : (p.alpha_pow == 1 ? rsb : 1.f));
  const float beta = p.beta * (p.beta_pow == 1 ? rsb : 1.f);
  const float* Dg = p.D ? (const float*)p.D + (int64_t)b * p.sD : nullptr;
  const int j = tn * BT + wn * 32 + (lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = tm * BT + wm * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
    float v = alpha * acc[r];
    if (Dg) v += beta * Dg[(int64_t)i * p.ldd + j];
    if constexpr (SYRK) {
      float* Cg = (float*)p.C + (int64_t)b * p.sC;
      if (tm < tn || i <= j) Cg[(int64_t)i * p.ldc + j] = v;
      if (tm < tn || i < j) Cg[(int64_t)j * p.ldc + i] = v;
    } else {
      const bool obf = p.c_dtype == MUON_BF16;
      uint8_t* Cg = (uint8_t*)p.C + (int64_t)b * p.sC * (obf ? 2 : 4);
      if (i < p.Mreal && j < p.Nreal) {
        const int64_t idx = p.c_trans ? (int64_t)j * p.ldc + i : (int64_t)i * p.ldc + j;
        store_elem(Cg, idx, v, obf);
      }
    }
  }
}

template <bool NN, bool SYRK>
hipError_t launch_one(const GemmParams& p, hipStream_t s) {
  const int64_t grid = (int64_t)p.batch * p.tiles_per_batch;
  if (grid <= 0) return hipSuccess;
  return launch_kernel(gemm_f32_kernel<NN, SYRK>, dim3((unsigned)grid), p, s);
}

}  // namespace

hipError_t launch_gemm_f32(const GemmParams& p, bool nn, bool syrk, hipStream_t s) {
  if (syrk) return launch_one<false, true>(p, s);
  return nn ? launch_one<true, false>(p, s) : launch_one<false, false>(p, s);
}

}  // namespace muon
