// fp32 GEMMs of one Newton-Schulz iteration (fp32 compute mode) on gfx950.
//
// The same three products as the bf16 path ("core.optimizer.layer_sharded_muon",
// use_syrk: A = X X^T and B = b A + c A^2 one triangle only, then X <- a X +
// B X), in true fp32 on v_mfma_f32_32x32x2_f32.  fp32 mode serves small
// problems (a 256 x 256 gradient has 10 to 16 output tiles of 64 x 64), so
// the kernel is built for parallelism and latency rather than tile reuse:
//  - one workgroup per 32 x 32 output tile, its four waves splitting K
//    round-robin in stages of 32 (wave w takes stages w, w + 4, ...), each
//    wave accumulating the whole 32 x 32 block over its stages;
//  - every wave streams its own stages HBM -> LDS (direct buffer loads) through
//    a ring of four slots of its own, so the K loop has no barrier: a wave
//    waits only on its own loads;
//  - the four partial blocks are added in wave order through LDS (a fixed
//    order, so a matrix's result does not depend on its batch), then scaled,
//    D added and stored (SYRK: mirrored, so the result is exactly symmetric).
#include "muon_internal.h"
#include "device_util.h"
#include "muon_mi355x.h"

namespace muon {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BT = 32;                 // tile edge
constexpr int SK = 32;                 // K values per stage
constexpr int NSW = 4;                 // ring slots per wave
constexpr int OPB = BT * SK * 4;       // bytes of one operand of one stage (4 KiB)
constexpr int SLOT = 2 * OPB;          // P and Q of one stage
constexpr int WAVE_LDS = NSW * SLOT;   // 32 KiB per wave
constexpr int RPITCH = BT + 1;         // floats per row of a staged partial block
static_assert(4 * WAVE_LDS <= 160 * 1024, "LDS of one workgroup");
static_assert(4 * BT * RPITCH * 4 <= 4 * WAVE_LDS, "partials fit in the ring");

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

// LDS layout of one slot (byte offsets): P rows [32][32 K] fp32, 128 bytes per
// row, the eight 16-byte chunks XOR-swizzled by (row / 2) % 8; Q the same
// (NT: rows of Q^T) or, NN, [32 K][32 N] fp32 rows unswizzled.
//
// MFMA 32x32x2 f32: lane l supplies row (A) / column (B) l % 32 at one K
// position per instruction, K position l / 32.  Each pair of instructions 2 s,
// 2 s + 1 covers the stage's K values 4 s .. 4 s + 3: lane half h = l / 32 takes
// K = 4 s + 2 h in the first and 4 s + 2 h + 1 in the second (A and B agree,
// so every K value is summed once), which lets the NT operands be read as one
// 8-byte load per pair.
template <bool NN, bool SYRK>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * WAVE_LDS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int b, tm, tn;
  decode_tile_f32<SYRK>(p, b, tm, tn);

  const int ldp = __builtin_amdgcn_readfirstlane((int)p.ldp);
  const int ldq = __builtin_amdgcn_readfirstlane((int)p.ldq);
  const float* Pg = (const float*)p.P + (int64_t)b * p.sP + (int64_t)tm * BT * ldp;
  const float* Qg = NN ? (const float*)p.Q + (int64_t)b * p.sQ + (int64_t)tn * BT
                       : (const float*)p.Q + (int64_t)b * p.sQ + (int64_t)tn * BT * ldq;
  const i32x4 prw = rsrc_words(Pg, (int64_t)BT * ldp * 4);
  const i32x4 qrw = rsrc_words(Qg, NN ? (int64_t)p.K * ldq * 4 : (int64_t)BT * ldq * 4);
  const uint32_t lds0 =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem);
  const uint32_t wbase = lds0 + (uint32_t)(wave * WAVE_LDS);

  // Stages of this wave: global stage s = wave + 4 i, i = 0 .. cnt - 1.
  const int nst = p.K / SK;
  const int cnt = nst > wave ? (nst - wave + 3) / 4 : 0;

  // DMA of one stage: 4 instructions per operand, each 8 rows x 128 bytes;
  // lane l lands at row 8 q + l / 8, chunk l % 8 of the slot.
  const int r8 = lane >> 3;
  auto dma_stage = [&](int i) {
    const int s = wave + 4 * i;
    const uint32_t dst = wbase + (uint32_t)((i % NSW) * SLOT);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 8 * q + r8;
      const int gc = (lane & 7) ^ ((row >> 1) & 7);
      lds_dma16_asm(prw, dst + (uint32_t)(q * 1024), r8 * ldp * 4 + gc * 16, 8 * q * ldp * 4 + s * SK * 4);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (NN) {
        lds_dma16_asm(qrw, dst + (uint32_t)(OPB + q * 1024), r8 * ldq * 4 + (lane & 7) * 16,
                      (s * SK + 8 * q) * ldq * 4);
      } else {
        const int row = 8 * q + r8;
        const int gc = (lane & 7) ^ ((row >> 1) & 7);
        lds_dma16_asm(qrw, dst + (uint32_t)(OPB + q * 1024), r8 * ldq * 4 + gc * 16, 8 * q * ldq * 4 + s * SK * 4);
      }
    }
  };

  // Fragment addresses within a slot (lane-fixed): NT row l % 32 at chunk s ^
  // ((l % 32) / 2 % 8), byte 8 h; NN column l % 32 of K row 4 s + 2 h (+ 1).
  const int h = lane >> 5, r = lane & 31;
  const int sw = (r >> 1) & 7;
  f32x16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;

#pragma unroll
  for (int i = 0; i < NSW; ++i)
    if (i < cnt) dma_stage(i);
#pragma unroll 1
  for (int i = 0; i < cnt; ++i) {
    // Stage i has landed once at most the stages issued after it are pending.
    const int after = cnt - 1 - i < NSW - 1 ? cnt - 1 - i : NSW - 1;
    if (after >= 3) wait_vmcnt<24>();
    else if (after == 2) wait_vmcnt<16>();
    else if (after == 1) wait_vmcnt<8>();
    else wait_vmcnt<0>();
    typedef __attribute__((address_space(3))) float lds_f32;
    typedef __attribute__((address_space(3))) f32x2_t lds_f32x2;
    const uint32_t slot = wbase + (uint32_t)((i % NSW) * SLOT);
#pragma unroll
    for (int s = 0; s < SK / 4; ++s) {
      const f32x2_t a = *(const lds_f32x2*)(uintptr_t)(slot + r * 128 + ((s ^ sw) << 4) + 8 * h);
      f32x2_t q;
      if constexpr (NN) {
        q[0] = *(const lds_f32*)(uintptr_t)(slot + OPB + ((4 * s + 2 * h) * BT + r) * 4);
        q[1] = *(const lds_f32*)(uintptr_t)(slot + OPB + ((4 * s + 2 * h + 1) * BT + r) * 4);
      } else {
        q = *(const lds_f32x2*)(uintptr_t)(slot + OPB + r * 128 + ((s ^ sw) << 4) + 8 * h);
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0], q[0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[1], q[1], acc, 0, 0, 0);
    }
    // The slot is refilled with stage i + NSW once this wave's reads of it
    // have returned.
    if (i + NSW < cnt) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      dma_stage(i + NSW);
    }
  }

  // Partial blocks through LDS (the ring is free once every wave is here):
  // accumulator register e holds row 8 (e / 4) + 4 (l / 32) + e % 4, column
  // l % 32.  Thread t then owns row t / 8, columns 4 (t % 8) .. + 3.
  __syncthreads();
  float* const red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int row = 8 * (e >> 2) + 4 * h + (e & 3);
    red[(wave * BT + row) * RPITCH + r] = acc[e];
  }
  __syncthreads();

  const float rsb = p.rs ? p.rs[b] : 1.f;
  const float alpha = p.alpha * (p.alpha_pow == 2 ? rsb * rsb : (p.alpha_pow == 1 ? rsb : 1.f));
  const float beta = p.beta * (p.beta_pow == 1 ? rsb : 1.f);
  const float* Dg = p.D ? (const float*)p.D + (int64_t)b * p.sD : nullptr;
  const int li = tid >> 3, lj0 = (tid & 7) * 4;
  const int i = tm * BT + li;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int lj = lj0 + e, j = tn * BT + lj;
    const float s01 = red[(0 * BT + li) * RPITCH + lj] + red[(1 * BT + li) * RPITCH + lj];
    const float s2 = s01 + red[(2 * BT + li) * RPITCH + lj];
    float v = alpha * (s2 + red[(3 * BT + li) * RPITCH + lj]);
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
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  return launch_kernel(gemm_f32_kernel<NN, SYRK>, dim3((unsigned)grid), p, s);
}

}  // namespace

int gemm_f32_tile() { return BT; }

hipError_t launch_gemm_f32(const GemmParams& p, bool nn, bool syrk, hipStream_t s) {
  // M, N and K are multiples of the tile edge and of the stage (the fp32
  // workspace pads to 64); a SYRK product is square.
  if (p.M % BT || p.N % BT || p.K % SK || p.K <= 0) return hipErrorInvalidValue;
  if (syrk && (nn || p.M != p.N)) return hipErrorInvalidValue;
  if (syrk) return launch_one<false, true>(p, s);
  return nn ? launch_one<true, false>(p, s) : launch_one<false, false>(p, s);
}

}  // namespace muon
