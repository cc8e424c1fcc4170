// bf16 MFMA GEMMs of one Newton-Schulz iteration on gfx950 (CDNA4).
//
// The three products of an iteration ("core.optimizer.layer_sharded_muon",
// LayerShardedMuon, use_syrk: A = X X^T and B = b A + c A^2 are symmetric and
// need one triangle only; the update X <- a X + B X is a full product):
//
//   Gram   A = alpha X X^T        NT, SYRK (upper tiles, mirrored store)
//   Poly   B = c A A + b A        NT, SYRK (A symmetric, so A A = A A^T)
//   Update X' = B X + a X         NN (X is [K][N]; transposed on its way to LDS)
//
// One kernel template serves all three.  A workgroup of 256 threads (four
// wave64s in a 2x2 arrangement) owns a BM x BN output tile; each wave owns a
// (BM/2) x (BN/2) sub-tile made of 32x32 blocks computed with
// v_mfma_f32_32x32x16_bf16 (fp32 accumulation).  K advances in steps of 64
// through two LDS stages: the next K slice is fetched from HBM into registers
// while the current one feeds the MFMAs, then written to the other stage.
// LDS rows are padded by 16 bytes so that the 16-byte fragment reads of 16
// consecutive rows fall in distinct banks.
//
// Every output tile is computed by the same instruction sequence whatever the
// batch size or the tile's position, so a matrix's result is bitwise
// independent of the batch it is in.
#include "muon_internal.h"
#include "device_util.h"
#include "muon_mi355x.h"

namespace muon {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64;
constexpr int LDK = BK + 8;  // padded LDS row, in bf16 elements (144 bytes)

// Workgroup -> (batch, tile row, tile col).
//
// Workgroups are dispatched round-robin over the 8 XCDs (workgroup w runs on
// XCD w % 8); the remap gives each XCD a contiguous range of logical tiles so
// that tiles sharing operand panels share that XCD's L2.  Full tiles are then
// ordered in groups of 4 tile rows (all tile columns of a group before the
// next group), SYRK tiles row by row over the upper triangle.
template <bool SYRK>
__device__ __forceinline__ void decode_tile(const GemmParams& p, int& b, int& tm, int& tn) {
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
    constexpr int GM = 4;
    const int span = GM * p.tiles_n;
    const int grp = t / span, first = grp * GM;
    const int gsz = min(p.tiles_m - first, GM);
    const int r = t - grp * span;
    tm = first + r % gsz;
    tn = r / gsz;
  }
}

template <int BM, int BN, bool NN, bool SYRK>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(const GemmParams p) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int PL = BM * BK / 8 / 256;          // 16-byte P chunks per thread
  constexpr int QL = NN ? 8 : BN * BK / 8 / 256;  // Q chunks per thread
  constexpr int NB8 = BN / 8;                     // NN: 8x8 blocks along N (x 8 along K)
  constexpr int PS = BM * LDK, QS = BN * LDK;     // one LDS stage of P / Q, in bf16 elements
  constexpr int RH = BM / 2;                      // epilogue: tile rows staged per pass
  constexpr int RP = RH + 1;                      // epilogue: odd LDS pitch (floats)
  static_assert(BN * RP * 4 <= 2 * (PS + QS) * 2, "epilogue staging must fit in the main-loop LDS");
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (PS + QS)];
  uint16_t* const Ps = smem;            // [2][BM][LDK]
  uint16_t* const Qs = smem + 2 * PS;   // [2][BN][LDK]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  int b, tm, tn;
  decode_tile<SYRK>(p, b, tm, tn);

  const uint16_t* Pg = (const uint16_t*)p.P + (int64_t)b * p.sP + (int64_t)tm * BM * p.ldp;
  const uint16_t* Qg = NN ? (const uint16_t*)p.Q + (int64_t)b * p.sQ + (int64_t)tn * BN
                          : (const uint16_t*)p.Q + (int64_t)b * p.sQ + (int64_t)tn * BN * p.ldq;

  u32x4 pr[PL], qr[QL];
  const int kb = tid & 7, nb = tid >> 3;  // NN: this thread's 8x8 block (k block, n block)
  const bool q_active = !NN || nb < NB8;

  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int c = tid + 256 * i, row = c >> 3, kc = c & 7;
      pr[i] = *(const u32x4*)(Pg + (int64_t)row * p.ldp + k0 + kc * 8);
    }
    if constexpr (NN) {
      if (q_active) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          qr[j] = *(const u32x4*)(Qg + (int64_t)(k0 + kb * 8 + j) * p.ldq + nb * 8);
      }
    } else {
#pragma unroll
      for (int i = 0; i < QL; ++i) {
        const int c = tid + 256 * i, row = c >> 3, kc = c & 7;
        qr[i] = *(const u32x4*)(Qg + (int64_t)row * p.ldq + k0 + kc * 8);
      }
    }
  };

  auto sstore = [&](int s) {
    uint16_t* const ps = Ps + s * PS;
    uint16_t* const qs = Qs + s * QS;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int c = tid + 256 * i, row = c >> 3, kc = c & 7;
      *(u32x4*)(ps + row * LDK + kc * 8) = pr[i];
    }
    if constexpr (NN) {
      if (q_active) {
        // qr[j] holds Q[k0 + 8 kb + j][8 nb .. 8 nb + 7]; write column 8 nb + i
        // of the tile as the K-contiguous LDS row Qs[8 nb + i][8 kb .. 8 kb + 7].
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int w = i >> 1;
          u32x4 o;
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const uint32_t lo = qr[2 * h][w], hi = qr[2 * h + 1][w];
            o[h] = (i & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
          }
          *(u32x4*)(qs + (nb * 8 + i) * LDK + kb * 8) = o;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < QL; ++i) {
        const int c = tid + 256 * i, row = c >> 3, kc = c & 7;
        *(u32x4*)(qs + row * LDK + kc * 8) = qr[i];
      }
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[fm][fn][r] = 0.f;

  // MFMA operand layout (32x32x16): lane l supplies row (l % 32) of the A
  // block and column (l % 32) of the B block, each with the 8 K values
  // 8 (l / 32) .. 8 (l / 32) + 7 of the 16-wide K step.  Fragments of the
  // next K step are read from LDS while the MFMAs of the current one run.
  auto compute = [&](int s) {
    const uint16_t* pa = Ps + s * PS + (wm * WM + (lane & 31)) * LDK + (lane >> 5) * 8;
    const uint16_t* qa = Qs + s * QS + (wn * WN + (lane & 31)) * LDK + (lane >> 5) * 8;
    bf16x8 af[2][FM], bq[2][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) af[0][fm] = __builtin_bit_cast(bf16x8, *(const u32x4*)(pa + fm * 32 * LDK));
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) bq[0][fn] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qa + fn * 32 * LDK));
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < BK / 16) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
          af[cur ^ 1][fm] = __builtin_bit_cast(bf16x8, *(const u32x4*)(pa + fm * 32 * LDK + (ks + 1) * 16));
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          bq[cur ^ 1][fn] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qa + fn * 32 * LDK + (ks + 1) * 16));
      }
      // Keep the reads of step ks+1 ahead of the MFMAs of step ks.
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][fm], bq[cur][fn], acc[fm][fn], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int KT = p.K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * BK);
    compute(cur);
    if (kt + 1 < KT) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue --------------------------------------------------------------
  // Accumulator register r of a 32x32 block holds row 8 (r / 4) + 4 (l / 32)
  // + (r % 4) and column l % 32.  The tile is staged through LDS in two
  // passes of BM/2 rows (the waves with wm == pass write theirs) as
  // S[col][row] fp32 with an odd pitch; all register indices are compile-time
  // constants.  A cooperative loop then applies alpha, beta * D and the
  // rounding, and writes C row-major (consecutive threads -> consecutive
  // columns) and/or transposed (consecutive threads -> consecutive rows).
  float* const S = reinterpret_cast<float*>(smem);
  const float rsb = p.rs ? p.rs[b] : 1.f;
  const float alpha = p.alpha * (p.alpha_pow == 2 ? rsb * rsb : (p.alpha_pow == 1 ? rsb : 1.f));
  const float beta = p.beta * (p.beta_pow == 1 ? rsb : 1.f);
  const uint16_t* Dg = p.D ? (const uint16_t*)p.D + (int64_t)b * p.sD : nullptr;
  const bool obf = SYRK || p.c_dtype == MUON_BF16;
  uint8_t* const Cg = (uint8_t*)p.C + (int64_t)b * p.sC * (obf ? 2 : 4);
  const bool do_rows = SYRK || !p.c_trans;
  const bool do_trans = SYRK || p.c_trans;
  const int Mlim = SYRK ? p.M : p.Mreal, Nlim = SYRK ? p.N : p.Nreal;

#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    if (wm == pass) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = fm * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
            const int col = wn * WN + fn * 32 + (lane & 31);
            S[col * RP + row] = acc[fm][fn][r];
          }
    }
    __syncthreads();
    const int i0 = tm * BM + pass * RH;
    const int j0 = tn * BN;
    {  // row-major pass: thread -> column, loop over rows
      constexpr int TPC = 256 / BN;  // threads per column
      const int jj = tid % BN, rsub = tid / BN;
      const int j = j0 + jj;
      for (int rr = rsub; rr < RH; rr += TPC) {
        const int i = i0 + rr;
        float v = alpha * S[jj * RP + rr];
        if (Dg) v += beta * bf2f(Dg[(int64_t)i * p.ldd + j]);
        S[jj * RP + rr] = v;
        if (do_rows && i < Mlim && j < Nlim && (!SYRK || tm < tn || i <= j))
          store_elem(Cg, (int64_t)i * p.ldc + j, v, obf);
      }
    }
    if (do_trans) {
      __syncthreads();
      for (int idx = tid; idx < RH * BN; idx += 256) {
        const int rr = idx % RH, jj = idx / RH;
        const int i = i0 + rr, j = j0 + jj;
        if (i < Mlim && j < Nlim && (!SYRK || tm < tn || i < j))
          store_elem(Cg, (int64_t)j * p.ldc + i, S[jj * RP + rr], obf);
      }
    }
    __syncthreads();
  }
}

template <int BM, int BN, bool NN, bool SYRK>
hipError_t launch_one(const GemmParams& p, hipStream_t s) {
  const int64_t grid = (int64_t)p.batch * p.tiles_per_batch;
  if (grid <= 0) return hipSuccess;
  return launch_kernel(gemm_bf16_kernel<BM, BN, NN, SYRK>, dim3((unsigned)grid), p, s);
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmParams& p, bool nn, bool syrk, int tile, hipStream_t s) {
  if (tile == 256) {
    if (syrk) return launch_one<256, 256, false, true>(p, s);
    return nn ? launch_one<256, 256, true, false>(p, s) : launch_one<256, 256, false, false>(p, s);
  }
  if (syrk) return launch_one<128, 128, false, true>(p, s);
  return nn ? launch_one<128, 128, true, false>(p, s) : launch_one<128, 128, false, false>(p, s);
}

}  // namespace muon
