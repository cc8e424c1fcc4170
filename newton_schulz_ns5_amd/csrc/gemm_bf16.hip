// bf16 MFMA GEMMs of one Newton-Schulz iteration on gfx950 (CDNA4).
//
// The three products of an iteration ("core.optimizer.layer_sharded_muon",
// LayerShardedMuon, use_syrk: A = X X^T and B = b A + c A^2 are symmetric and
// need one triangle only; the update X <- a X + B X is a full product) are
// all computed here as C = alpha P op(Q) + beta D with P stored K-contiguous:
//
//   Gram   A  = alpha X X^T       NT: P = Q = X,               SYRK
//   Poly   B  = c A A + b A       NT: P = Q = A (A = A^T),     SYRK, D = A
//   Update X' = B X + a X         NN: P = B, Q = X ([K][N]),   D = X
//
// In the poly and the update the D tile is the transposed Q tile, so beta D
// is added inside the products.  NN fragments come from the LDS transpose
// read (ds_read_b64_tr_b16), so the iterate is only ever stored row-major.
//
// Work decomposition: one workgroup per BT x BT output tile: at BT = 256
// eight wave64s (2 x 4, two per SIMD, so one wave's MFMAs run while the other
// waits on a load, a fragment read or the barrier), each owning a 128 x 64
// sub-tile; at BT = 128 four (2 x 2, two workgroups per CU), each owning
// 64 x 64.  Sub-tiles are 32x32 blocks computed with
// v_mfma_f32_32x32x16_bf16 (fp32 accumulation).  K advances 64 at a time:
// each operand row contributes one 128-byte line per slice, brought by direct
// HBM -> LDS buffer loads (buffer_load_dwordx4 ... lds) into a ring of five
// operand slots (160 KiB for BT = 256), about one and a half slices ahead of
// the multiply.  One barrier per slice.  The loads, the LDS fragment reads and the MFMAs are
// interleaved in fixed slots, so no burst of loads holds the MFMAs back.
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

#define MUON_LDS(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int KS = 64;        // K per slice: one 128-byte line of each operand row
constexpr int NSLOT = 5;      // LDS ring of operand slots (one operand's rows of one slice each)
constexpr int ROWB = KS * 2;  // bytes per LDS row

// Workgroup -> (problem, batch, tile row, tile col).
//
// Workgroups are dispatched round-robin over the 8 XCDs (workgroup w runs on
// XCD w % 8, as the k = w / 8-th of that XCD's queue), and each XCD's 32 CUs
// drain their own queue.  The launch's tiles are numbered problem after
// problem, longest K first.  Two orders:
//  - rounds (default): the tile numbers are handed out in rounds of 8 x 32,
//    XCD x taking the 32 consecutive tiles [x*32, x*32 + 32) of each round,
//    so tiles that share operand panels run together on one XCD's L2 while
//    every XCD moves through the problem list at the same pace;
//  - balanced (g.balance): every XCD gets an equal share of every problem
//    and works through the problems in order, so the last waves of all XCDs
//    end together when long and short tiles mix (with rounds, the XCDs that
//    draw the long tiles of the round where the long problems end finish
//    far behind the others).  XCD x's share of a problem whose tiles are
//    numbered c0 .. c1 - 1 is the number of i in [c0, c1) with i % 8 == x,
//    so the shares add up to exactly the workgroups each XCD is sent.
//    Within a problem the XCDs still move together in rounds of 8 x 32
//    tiles; the tail after the last full round is cut into 8 contiguous
//    pieces, one per XCD.
// Within a problem, tiles are ordered in bands of 4 tile rows (a band's tile
// columns one after the other, before the next band), so 32 consecutive
// tiles read about 12 operand panels; SYRK bands cover the upper triangle
// only.
template <bool SYRK>
__device__ __forceinline__ const GemmParams& decode_tile(const GemmGroup& g, int& b, int& tm, int& tn) {
  constexpr int CH = 32;
  const int wg = blockIdx.x, x = wg & 7, k = wg >> 3;
  int pi = 0, local;
  if (!g.balance) {
    const int G = gridDim.x;
    const int full = (G / (8 * CH)) * (8 * CH);
    const int pid = wg < full ? (k / CH) * (8 * CH) + x * CH + (k % CH) : wg;
    while (pi + 1 < g.nprob && pid >= g.tile_start[pi + 1]) ++pi;
    local = pid - g.tile_start[pi];
  } else {
    // Number of i in [0, n) with i % 8 == xx (n >= 0).
    auto share = [](int n, int xx) { return (n + 7 - xx) >> 3; };
    while (pi + 1 < g.nprob && k >= share(g.tile_start[pi + 1], x)) ++pi;
    const int c0 = g.tile_start[pi], c1 = g.tile_start[pi + 1];
    const int j = k - share(c0, x);  // position in XCD x's share of this problem
    const int rounds = (c1 - c0) / (8 * CH);
    if (j < rounds * CH) {
      local = (j / CH) * (8 * CH) + x * CH + j % CH;
    } else {
      local = rounds * 8 * CH + (j - rounds * CH);
      for (int xx = 0; xx < x; ++xx) local += share(c1, xx) - share(c0, xx) - rounds * CH;
    }
  }
  const GemmParams& p = g.prob[pi];
  b = local / p.tiles_per_batch;
  int t = local - b * p.tiles_per_batch;
  if constexpr (SYRK) {
    // Upper-triangle tiles in bands of GM tile rows r0 .. r0 + g - 1; within
    // a band, column by column from column r0 on, rows r0 .. min(tn, last).
    constexpr int GM = 4;
    const int T = p.tiles_m;
    int r0 = 0;
    for (;;) {
      const int g = min(T - r0, GM);
      const int tri = g * (g + 1) / 2;
      const int size = tri + (T - r0 - g) * g;
      if (t < size) {
        if (t < tri) {
          int c = 0;
          while (t >= c + 1) { t -= c + 1; ++c; }
          tn = r0 + c;
          tm = r0 + t;
        } else {
          t -= tri;
          tn = r0 + g + t / g;
          tm = r0 + t % g;
        }
        break;
      }
      t -= size;
      r0 += g;
    }
  } else {
    constexpr int GM = 4;
    const int span = GM * p.tiles_n;
    const int grp = t / span, first = grp * GM;
    const int gsz = min(p.tiles_m - first, GM);
    const int r = t - grp * span;
    tm = first + r % gsz;
    tn = r / gsz;
  }
  return p;
}

// Buffer descriptor of a panel: base address and size in bytes, both made
// explicitly wave-uniform so the descriptor lives in SGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const int n = __builtin_amdgcn_readfirstlane((int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, n, 0x00020000);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// NN: Q is stored [K][N] (N contiguous) instead of [N][K]; its fragments are
// read with the LDS transpose read (ds_read_b64_tr_b16).
template <int BT, bool SYRK, bool NN, int NW>
__global__ __launch_bounds__(NW * 64, 1) void gemm_nt_bf16_kernel(const GemmGroup grp) {
  static_assert(!(SYRK && NN), "SYRK products are NT");
  static_assert(NW == 4 || NW == 8, "2 x 2 or 2 x 4 waves");
  constexpr int NTH = NW * 64;        // threads per workgroup
  constexpr int WT = BT / 2;          // wave tile rows (two rows of waves)
  constexpr int WC = BT / (NW / 2);   // wave tile columns
  constexpr int F = WT / 32;          // 32x32 MFMA block rows per wave tile
  constexpr int FN = WC / 32;         // 32x32 MFMA block columns per wave tile
  constexpr int MPS = F / 2;          // MFMAs per slot of a quarter
  constexpr int NSL = F * FN / MPS;   // slots per quarter
  constexpr int OPB = BT * ROWB;      // bytes of one slot
  constexpr int RPW = BT / NW;        // operand rows each wave loads per slice
  constexpr int DPW = RPW / 8;        // DMA instructions per wave per operand slice (8 rows each)
  constexpr int DQ = DPW / 2;         // DMA instructions per quarter step
  static_assert(2 * DQ <= NSL && F + FN <= 2 * NSL, "one DMA instruction per even slot, two fragment reads per slot");
  constexpr int RH = BT / 2;          // epilogue: tile rows staged per pass
  constexpr int EPI = RH * (BT + 4) * 4;  // epilogue staging bytes
  constexpr int LDS_BYTES = (NSLOT * OPB > EPI) ? NSLOT * OPB : EPI;
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / (NW / 2), wn = wave % (NW / 2);

  int b, tm, tn;
  const GemmParams& p = decode_tile<SYRK>(grp, b, tm, tn);

  // Split K (SYRK only): batch entry b is chunk ch of matrix bm, covering K
  // values [k0, k0 + Kc); chunk edges are multiples of 128.
  int bm = b, k0 = 0, Kc = p.K;
  if constexpr (SYRK) {
    if (p.ksplit > 1) {
      bm = b / p.ksplit;
      const int ch = b - bm * p.ksplit, kb = p.K / 128;
      k0 = 128 * (int)((int64_t)ch * kb / p.ksplit);
      Kc = 128 * (int)((int64_t)(ch + 1) * kb / p.ksplit) - k0;
    }
  }
  const int ldp = __builtin_amdgcn_readfirstlane((int)p.ldp);
  const int ldq = __builtin_amdgcn_readfirstlane((int)p.ldq);
  const uint16_t* Pg = (const uint16_t*)p.P + (int64_t)bm * p.sP + (int64_t)tm * BT * p.ldp + k0;
  const uint16_t* Qg =
      (const uint16_t*)p.Q + (int64_t)bm * p.sQ + (NN ? (int64_t)tn * BT : (int64_t)tn * BT * p.ldq + k0);
  const int64_t qbytes = (NN ? (int64_t)p.K : (int64_t)BT) * p.ldq * 2;
  const __amdgpu_buffer_rsrc_t prs = make_rsrc(Pg, (int64_t)BT * p.ldp * 2);
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Qg, qbytes);
  const i32x4 prw = rsrc_words(Pg, (int64_t)BT * p.ldp * 2);
  const i32x4 qrw = rsrc_words(Qg, qbytes);

  // LDS layout: a slot holds BT rows of 128 bytes (64 K values of one
  // operand row); its eight 16-byte chunks are XOR-swizzled by (row / 2) mod
  // 8.  A 16-byte fragment read is served 16 lanes (256 bytes, all 64 banks)
  // at a time; its 16 lanes read 16 consecutive rows at one logical chunk,
  // and the pairs (row parity, swizzle) are then all distinct.
  // Slice t's P rows live in slot 2t mod 5, its Q rows in slot 2t + 1 mod 5.
  //
  // DMA: instruction j of a wave fills rows wave*RPW + 8 j .. +7 of a slot;
  // lane l lands at row (l / 8), chunk (l % 8) and therefore fetches the
  // global chunk (l % 8) ^ ((row / 2) % 8), where (row / 2) % 8 =
  // (4 j + l / 16) % 8.  Eight lanes cover one 128-byte line.
  //
  // NN Q slot: 64 K rows of the tile's BT columns, QROWB bytes each, with the
  // 32-byte blocks of a row XOR-swizzled by 2 (row % 4) (see the transpose
  // reads).  Wave w fills rows QW w .. QW w + QW - 1 (QW = 64 / NW), QRPI rows
  // per instruction; lane l lands at row l / QCH, chunk l % QCH.
  constexpr int QROWB = NN ? BT * 2 : ROWB;
  constexpr int QCH = QROWB / 16;      // 16-byte chunks per Q slot row
  constexpr int QRPI = 1024 / QROWB;   // Q slot rows per DMA instruction
  constexpr int QW = KS / NW;          // Q slot rows per wave (NN)
  static_assert(!NN || QW == DPW * QRPI, "the NN Q rows of a slice take DPW instructions per wave");
  const int prow = wave * RPW + (lane >> 3);
  int pvo[2], qvo[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int dkc = (lane & 7) ^ ((4 * par + (lane >> 4)) & 7);
    pvo[par] = prow * ldp * 2 + dkc * 16;
    if constexpr (NN) {
      const int rl = lane / QCH, cl = lane % QCH;
      const int key = (par * QRPI + rl) & 3;
      qvo[par] = rl * ldq * 2 + (2 * ((cl >> 1) ^ (2 * key)) + (cl & 1)) * 16;
    } else {
      qvo[par] = prow * ldq * 2 + dkc * 16;
    }
  }
  const int KT = Kc / KS;
  auto slot = [&](int t, int op) { return smem + ((2 * t + op) % NSLOT) * OPB; };
  // A SYRK diagonal tile multiplies a panel by itself: its Q rows are its P
  // rows, so the Q loads are skipped and the Q fragments read the P slot.
  // The waits below stay right: the loads a wait may leave in flight are
  // still the youngest P loads.
  const bool same_pq = SYRK && tm == tn && p.P == p.Q && p.ldp == p.ldq && p.sP == p.sQ;
  const uint32_t smem_lds =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem);

  // DMA instruction j (0 .. DPW-1) of operand op (0: P, 1: Q) of slice t.
  // Slices past the last one (the pipeline runs ahead) re-read the last
  // slice into a slot nobody reads any more, so every step has one shape.
  auto dma = [&](int t, int op, int j) {
    const int tc = t < KT ? t : KT - 1;
    const int k0b = tc * ROWB;
    if constexpr (NN) {
      const uint32_t sl = smem_lds + (uint32_t)(((2 * t + op) % NSLOT) * OPB);
      if (op == 0) {
        lds_dma16_asm(prw, sl + (wave * RPW + 8 * j) * ROWB, pvo[j & 1], 8 * j * ldp * 2 + k0b);
      } else {
        const uint32_t krow = (uint32_t)tc * KS + wave * QW + j * QRPI;
        lds_dma16_asm(qrw, sl + (wave * QW + j * QRPI) * QROWB, qvo[j & 1], (int)(krow * (uint32_t)ldq * 2u));
      }
    } else {
      uint8_t* const dst = slot(t, op) + (wave * RPW + 8 * j) * ROWB;
      if (op == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(prs, MUON_LDS(dst), 16, pvo[j & 1], 8 * j * ldp * 2 + k0b, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, MUON_LDS(dst), 16, qvo[j & 1], 8 * j * ldq * 2 + k0b, 0, 0);
    }
  };

  // MFMA operand layout (32x32x16): lane l supplies row (l % 32) of the A
  // block and column (l % 32) of the B block, each with the 8 K values
  // 8 (l / 32) .. 8 (l / 32) + 7 of the 16-wide K step, i.e. chunk
  // 2 ks + l / 32 of quarter ks.  Blocks start at multiples of 32 rows, so a
  // row's swizzle is ((l % 32) / 2) % 8.
  const int prd = (wm * WT + (lane & 31)) * ROWB;
  const int qrd = (wn * WC + (lane & 31)) * ROWB;
  // NN: lane l of 16-lane group g = l / 16 supplies row 8 (g / 2) + (l % 16) / 4
  // (+ 16 ks + 4 r) and the four columns 4 (l % 4) .. + 3 of the 16-column half
  // g % 2 of a 32-column block; the transpose read then hands lane l column
  // l % 32 with the four K values 8 (l / 32) + 4 r .. + 3, the MFMA B layout.
  // Lanes 0..31 cover four rows and all eight 32-byte blocks of a 256-byte
  // span under the 2 (row % 4) swizzle: no bank is read twice.
  const int trow = (8 * (lane >> 5) + ((lane & 15) >> 2)) * QROWB;
  int tcol[FN];
#pragma unroll
  for (int f = 0; f < FN; ++f)
    tcol[f] = ((((wn * WC + 32 * f) >> 4) + ((lane >> 4) & 1)) ^ (2 * ((lane & 15) >> 2))) * 32 + (lane & 3) * 8;
  auto trq = [&](int t, int ks, int f) {
    const uint8_t* base = slot(t, 1) + 16 * ks * QROWB + trow + tcol[f];
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)MUON_LDS(base));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)MUON_LDS(base + 4 * QROWB));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // Fragment u (0 .. F+FN-1) of quarter ks of slice t, in the order the MFMAs
  // first need them: a[0], q[0 .. FN-1], a[1 .. F-1].
  auto frag = [&](int t, int ks, int u, bf16x8 (&a)[F], bf16x8 (&q)[FN]) {
    const int so = ((2 * ks + (lane >> 5)) ^ (((lane & 31) >> 1) & 7)) * 16;
    if (u == 0)
      a[0] = __builtin_bit_cast(bf16x8, *(const u32x4*)(slot(t, 0) + prd + so));
    else if (u <= FN) {
      if constexpr (NN)
        q[u - 1] = trq(t, ks, u - 1);
      else
        q[u - 1] = __builtin_bit_cast(bf16x8, *(const u32x4*)(slot(t, same_pq ? 0 : 1) + qrd + (u - 1) * 32 * ROWB + so));
    }
    else
      a[u - FN] = __builtin_bit_cast(bf16x8, *(const u32x4*)(slot(t, 0) + prd + (u - FN) * 32 * ROWB + so));
  };

  const float rsb = p.rs ? p.rs[bm] : 1.f;
  const float alpha = p.alpha * (p.alpha_pow == 2 ? rsb * rsb : (p.alpha_pow == 1 ? rsb : 1.f));
  const float beta = p.beta * (p.beta_pow == 1 ? rsb : 1.f);

  // beta D with D = Q^T on this tile (p.dq) is added inside the products: in
  // the quarters whose 16 K values are 16 of this wave's tile rows, block row
  // bi also takes E Q^T, where E is (beta / alpha) on the matching diagonal
  // and zero elsewhere, so that alpha (P Q^T + E Q^T) = alpha P Q^T + beta D.
  // The factor enters as two bf16 terms (hi + lo, within 2^-16 of it).
  // Fragment eh[h] / el[h] covers the K half h (rows 16h .. 16h + 15) of a
  // 32-row block: lane l holds row l % 32 and K 8 (l / 32) .. + 7.
  bf16x8 eh[2], el[2];
  if (p.dq) {
    const float e = beta / alpha;
    const uint32_t hb = f2bf(e);
    const uint32_t lb = f2bf(e - bf2f((uint16_t)hb));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int pos = (lane & 31) - 16 * h - 8 * (lane >> 5);
      u32x4 vh, vl;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        vh[w] = (pos == 2 * w ? hb : 0u) | (pos == 2 * w + 1 ? hb << 16 : 0u);
        vl[w] = (pos == 2 * w ? lb : 0u) | (pos == 2 * w + 1 ? lb << 16 : 0u);
      }
      eh[h] = __builtin_bit_cast(bf16x8, vh);
      el[h] = __builtin_bit_cast(bf16x8, vl);
    }
  }

  f32x16 acc[F][FN];
#pragma unroll
  for (int i = 0; i < F; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // One quarter of a slice (16 K): its F x FN MFMAs on (ac, qc), MPS per
  // slot over NSL slots; the first slots also read two fragments each (F + FN
  // in all) of quarter rks of slice rt into (an, qn), and even slots issue DMA
  // instructions j0 .. j0 + DQ - 1 of operand dop of slice dt.  Straight-line code, so the
  // compiler waits on exactly the fragment reads each MFMA needs, and the
  // loads never hold the MFMAs back in one burst.
  auto diag_mfmas = [&](auto bi_c, auto h_c, const bf16x8 (&qc)[FN]) {
    constexpr int bi = decltype(bi_c)::value, h = decltype(h_c)::value;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      acc[bi][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(eh[h], qc[j], acc[bi][j], 0, 0, 0);
      acc[bi][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(el[h], qc[j], acc[bi][j], 0, 0, 0);
    }
  };
  // SD >= 0: the slice multiplied is the SD-th of the tile's own rows, whose
  // K values 16 cq .. 16 cq + 15 are rows 16 (cq % 2) .. of block row
  // bi = 2 (SD % (F/2)) + cq / 2 of wave SD / (F/2); that wave adds E Q^T.
  auto quarter = [&](auto cq_c, auto sd_c, int rt, int rks, bf16x8 (&an)[F], bf16x8 (&qn)[FN],
                     const bf16x8 (&ac)[F], const bf16x8 (&qc)[FN], int dt, int dop, int j0) {
    constexpr int cq = decltype(cq_c)::value, SD = decltype(sd_c)::value;
#pragma unroll
    for (int u = 0; u < NSL; ++u) {
      if ((u & 1) == 0 && (u >> 1) < DQ && !(dop == 1 && same_pq)) dma(dt, dop, j0 + (u >> 1));
      if (2 * u < F + FN) frag(rt, rks, 2 * u, an, qn);
      if (2 * u + 1 < F + FN) frag(rt, rks, 2 * u + 1, an, qn);
#pragma unroll
      for (int m = u * MPS; m < (u + 1) * MPS; ++m)
        acc[m / FN][m % FN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ac[m / FN], qc[m % FN], acc[m / FN][m % FN], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (SD >= 0) {
      constexpr int HW = F / 2;  // slices of one wave's rows
      if (wm == SD / HW)
        diag_mfmas(std::integral_constant<int, 2 * (SD % HW) + cq / 2>{}, std::integral_constant<int, cq & 1>{}, qc);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using Q0 = std::integral_constant<int, 0>;
  using Q1 = std::integral_constant<int, 1>;
  using Q2 = std::integral_constant<int, 2>;
  using Q3 = std::integral_constant<int, 3>;

  // Pipeline over the KT slices of 64 K.  Step t multiplies slice t in four
  // quarters q0..q3 and, between q2 and q3, waits for its own loads of slice
  // t + 1 and meets the other waves at a barrier.  That barrier publishes
  // slice t + 1 (q3 already reads its first quarter) and, since each wave has
  // finished its reads of slice t before it (q3's fragments are read in q2),
  // frees slice t's slots.  Loads, each into slots freed by the barrier before
  // them:
  //   q3 of step t - 1, q0 of step t:  Q rows of slice t + 1 (two halves)
  //   q1, q2 of step t:                P rows of slice t + 2
  // so at step t's barrier the loads issued after slice t + 1's are the DPW
  // of P(t + 2).
  bf16x8 a0[F], q0[FN], a1[F], q1[FN];
#pragma unroll
  for (int j = 0; j < DPW; ++j) dma(0, 0, j);
#pragma unroll
  for (int j = 0; j < DPW; ++j)
    if (!same_pq) dma(0, 1, j);
#pragma unroll
  for (int j = 0; j < DPW; ++j) dma(1, 0, j);
#pragma unroll
  for (int j = 0; j < DQ; ++j)
    if (!same_pq) dma(1, 1, j);
  if (same_pq)
    wait_vmcnt<DPW>();  // P(1) may stay in flight
  else
    wait_vmcnt<DPW + DQ>();
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int u = 0; u < F + FN; ++u) frag(0, 0, u, a0, q0);
  __builtin_amdgcn_sched_barrier(0);
  auto step = [&](int t, auto sd_c) {
    quarter(Q0{}, sd_c, t, 1, a1, q1, a0, q0, t + 1, 1, DQ);
    quarter(Q1{}, sd_c, t, 2, a0, q0, a1, q1, t + 2, 0, 0);
    quarter(Q2{}, sd_c, t, 3, a1, q1, a0, q0, t + 2, 0, DQ);
    wait_vmcnt<DPW>();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of slice t are done
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    quarter(Q3{}, sd_c, t + 1, 0, a0, q0, a1, q1, t + 2, 1, 0);
  };
  // The tile's own rows are slices td .. td + PEEL - 1 (K = M here); those
  // steps are peeled so that the loops carry no branch.
  constexpr int PEEL = BT / KS;
  using SN = std::integral_constant<int, -1>;
  const int td = p.dq ? tm * BT / KS : KT;
  int t = 0;
  for (; t < td; ++t) step(t, SN{});
  if (p.dq) {
    step(t, std::integral_constant<int, 0>{});
    step(t + 1, std::integral_constant<int, 1>{});
    if constexpr (PEEL == 4) {
      step(t + 2, std::integral_constant<int, 2>{});
      step(t + 3, std::integral_constant<int, 3>{});
    }
    t += PEEL;
  }
  for (; t < KT; ++t) step(t, SN{});
  // Every wave is done with the LDS ring, and its loads past the last slice
  // have landed, before the ring is reused (explicit: the NN kernel's loads
  // are invisible to the compiler).
  wait_vmcnt<0>();
  __syncthreads();

  // ---- epilogue --------------------------------------------------------------
  // Accumulator register r of a 32x32 block holds row 8 (r / 4) + 4 (l / 32)
  // + (r % 4) and column l % 32.  The tile is staged through LDS in two
  // passes of BT/2 rows as a row-major fp32 array S with a 16-byte aligned
  // pitch; register indices are compile-time constants.  Pass p stages block
  // rows F/2 p .. F/2 p + F/2 - 1 of all four waves, so every wave writes in
  // every pass: staged row s is tile row WT (s / HWT) + HWT p + s % HWT.
  // Then, with 16-byte global accesses:
  //  - row pass: thread -> (row, 8 consecutive columns); v = alpha S
  //    (+ beta D when D is not folded into the products) is written back to S
  //    and stored row-major to C;
  //  - transposed pass: thread -> (column, 8 consecutive rows), stored to
  //    T[j][i .. i+7] (SYRK: the mirrored half of C; the final output of a
  //    tall matrix: X'^T).
  // Ragged edges and an explicit D take a compact generic path with element
  // stores where needed.
  float* const S = reinterpret_cast<float*>(smem);
  const uint16_t* __restrict__ Dg = p.D ? (const uint16_t*)p.D + (int64_t)b * p.sD : nullptr;
  const bool obf = p.c_dtype == MUON_BF16;  // fp32: split-K partial products
  const int esz = obf ? 2 : 4;
  uint8_t* const Cg = p.C ? (uint8_t*)p.C + (int64_t)b * p.sC * esz : nullptr;
  uint8_t* const Tg = SYRK ? Cg : (p.Ct ? (uint8_t*)p.Ct + (int64_t)b * p.sCt * esz : nullptr);
  const int64_t ldc = p.ldc, ldt = SYRK ? p.ldc : p.ldct;
  const int Mlim = p.Mreal, Nlim = p.Nreal;
  const bool diag = SYRK && tm == tn;
  // 16-byte stores need the row starts aligned: ld * esz and the base.
  const bool cvec = Cg && ((ldc * esz) & 15) == 0 && (((uintptr_t)Cg) & 15) == 0;
  const bool tvec = Tg && ((ldt * esz) & 15) == 0 && (((uintptr_t)Tg) & 15) == 0;

  // Store v[0..7] at elements base[idx .. idx+7]; `valid` leading elements only.
  auto store8 = [&](uint8_t* base, int64_t idx, const float* v, int valid, bool vec) {
    if (vec && valid >= 8) {
      if (obf) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack_bf2(v[2 * e], v[2 * e + 1]);
        *(u32x4*)(base + idx * 2) = w;
      } else {
        f32x4 w0, w1;
#pragma unroll
        for (int e = 0; e < 4; ++e) { w0[e] = v[e]; w1[e] = v[4 + e]; }
        *(f32x4*)(base + idx * 4) = w0;
        *(f32x4*)(base + idx * 4 + 16) = w1;
      }
    } else {
      for (int e = 0; e < 8; ++e)
        if (e < valid) store_elem(base, idx + e, v[e], obf);
    }
  };

  constexpr int PITCH = BT + 4;      // floats per staged row
  constexpr int HWT = WT / 2;        // rows of one wave's quadrant staged per pass
  constexpr int CPR = BT / 8;        // 8-column chunks per row
  constexpr int RPI = NTH / CPR;     // rows per step of the row pass
  constexpr int NIT = RH / RPI;      // steps of the row pass
  constexpr int R8 = RH / 8;         // 8-row chunks per pass (transposed pass)
  static_assert(RH * PITCH * 4 <= LDS_BYTES, "epilogue staging must fit");

  // The two passes are instantiated separately (compile-time pass index), so
  // the accumulators are dead after the second pass's staging.
  auto epilogue_pass = [&](auto pass_c) {
    constexpr int pass = decltype(pass_c)::value;
#pragma unroll
    for (int ii = 0; ii < F / 2; ++ii)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * HWT + ii * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          const int col = wn * WC + j * 32 + (lane & 31);
          S[row * PITCH + col] = acc[pass * (F / 2) + ii][j][r];
        }
    __syncthreads();
    // tile row of staged row s (8-row chunks never straddle a quadrant band)
    auto trow = [&](int s) { return (s / HWT) * WT + pass * HWT + (s % HWT); };
    const int i0 = tm * BT;
    const int j0 = tn * BT;
    // Almost every tile: all its rows and columns are stored, no D, aligned
    // rows.  Then both passes store alpha S (bf16, or fp32 for split-K
    // partial products) in whole 8-element chunks with 16-byte stores; the
    // transposed pass recomputes alpha S, so its values are bitwise those of
    // the row pass.  On a SYRK diagonal tile the row pass stores the chunks
    // that reach the diagonal or above it and the transposed pass mirrors the
    // chunks that reach below it.  Where the diagonal crosses a chunk, both
    // passes store it, so the 8 x 8 diagonal blocks of the staged rows are
    // first made symmetric in S (lower elements := their upper mirrors, all
    // within one pass: 8-row chunks never straddle a quadrant band): then
    // both passes store the same bits there, and the stored matrix is exactly
    // symmetric.
    const bool fast = !Dg && i0 + BT <= Mlim && j0 + BT <= Nlim && (!Cg || cvec) && (!Tg || tvec);
    // Store v[0..7] at dst (bf16 or fp32) with one or two 16-byte stores.
    auto put8 = [&](uint8_t* dst, const float (&v)[8]) {
      if (obf) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack_bf2(v[2 * e], v[2 * e + 1]);
        *(u32x4*)dst = w;
      } else {
        f32x4 w0, w1;
#pragma unroll
        for (int e = 0; e < 4; ++e) { w0[e] = v[e]; w1[e] = v[4 + e]; }
        *(f32x4*)dst = w0;
        *(f32x4*)(dst + 16) = w1;
      }
    };
    if (fast && diag) {
      // Diagonal block d (staged rows 8 d .. 8 d + 7, tile rows and columns
      // trow(8 d) ..): element (r, c) with r > c takes (c, r).
      for (int idx = tid; idx < R8 * 64; idx += NTH) {
        const int s0 = (idx >> 6) * 8, r = (idx >> 3) & 7, c = idx & 7;
        const int t0 = trow(s0);
        if (r > c) S[(s0 + r) * PITCH + t0 + c] = S[(s0 + c) * PITCH + t0 + r];
      }
      __syncthreads();
    }
    if (fast) {
      if (Cg) {
        const int c8 = (tid % CPR) * 8, r0 = tid / CPR;
#pragma unroll 4
        for (int it = 0; it < NIT; ++it) {
          const int rr = r0 + it * RPI;
          const float* srow = S + rr * PITCH + c8;
          const f32x4 s0 = *(const f32x4*)srow, s1 = *(const f32x4*)(srow + 4);
          float v[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) { v[e] = alpha * s0[e]; v[4 + e] = alpha * s1[e]; }
          const int tr = trow(rr);
          uint8_t* const dst = Cg + ((int64_t)(i0 + tr) * ldc + j0 + c8) * esz;
          if (!diag || tr < c8 + 8) put8(dst, v);  // the chunk reaches the diagonal or above
        }
      }
      if (Tg) {
#pragma unroll 2
        for (int idx = tid; idx < BT * R8; idx += NTH) {
          const int jj = idx % BT, i8 = (idx / BT) * 8;
          // mirrored to row jj, columns trow(i8) .. + 7: on a diagonal tile
          // only where some of them are below the diagonal
          const int ti = trow(i8);
          if (diag && jj <= ti) continue;
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = alpha * S[(i8 + e) * PITCH + jj];
          uint8_t* const dst = Tg + ((int64_t)(j0 + jj) * ldt + i0 + ti) * esz;
          put8(dst, v);
        }
      }
    } else {
      // Ragged edges or an explicit D: element-wise where needed, through
      // v = alpha S (+ beta D) written back to S.
      const int c8 = (tid % CPR) * 8, r0 = tid / CPR;
      const int j = j0 + c8;
#pragma unroll 1
      for (int it = 0; it < NIT; ++it) {
        const int rr = r0 + it * RPI;
        const int i = i0 + trow(rr);
        float* srow = S + rr * PITCH + c8;
        f32x4 s0 = *(const f32x4*)srow, s1 = *(const f32x4*)(srow + 4);
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) { v[e] = alpha * s0[e]; v[4 + e] = alpha * s1[e]; }
        if (Dg && i < Mlim && j < Nlim) {  // D is padded like the output: whole chunks are in bounds
          const u32x4 dv = *(const u32x4*)(Dg + (int64_t)i * p.ldd + j);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[2 * e] += beta * __uint_as_float(dv[e] << 16);
            v[2 * e + 1] += beta * __uint_as_float(dv[e] & 0xffff0000u);
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) { s0[e] = v[e]; s1[e] = v[4 + e]; }
        *(f32x4*)srow = s0;
        *(f32x4*)(srow + 4) = s1;
        if (Cg && i < Mlim) {
          if (diag) {
            for (int e = 0; e < 8; ++e)
              if (i <= j + e) store_elem(Cg, (int64_t)i * ldc + j + e, v[e], obf);
          } else {
            store8(Cg, (int64_t)i * ldc + j, v, Nlim - j, cvec);
          }
        }
      }
      if (Tg) {
        __syncthreads();
#pragma unroll 1
        for (int idx = tid; idx < BT * R8; idx += NTH) {
          const int jj = idx % BT, i8 = (idx / BT) * 8;
          const int jt = j0 + jj, it8 = i0 + trow(i8);
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = S[(i8 + e) * PITCH + jj];
          if (jt < Nlim) {
            if (diag) {
              for (int e = 0; e < 8; ++e)
                if (it8 + e < jt) store_elem(Tg, (int64_t)jt * ldt + it8 + e, v[e], obf);
            } else {
              store8(Tg, (int64_t)jt * ldt + it8, v, Mlim - it8, tvec);
            }
          }
        }
      }
    }
    __syncthreads();
  };
  epilogue_pass(std::integral_constant<int, 0>{});
  epilogue_pass(std::integral_constant<int, 1>{});
}

template <int BT, bool SYRK, bool NN>
hipError_t launch_one(const GemmGroup& g, hipStream_t s) {
  const int64_t grid = g.tile_start[g.nprob];
  if (grid <= 0) return hipSuccess;
  constexpr int NW = BT == 256 ? 8 : 4;
  return launch_kernel(gemm_nt_bf16_kernel<BT, SYRK, NN, NW>, dim3((unsigned)grid), g, s, NW * 64);
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmGroup& g, bool syrk, bool nn, int tile, hipStream_t s) {
  // Every K is a multiple of 128 and at least the tile edge (the pipeline and
  // the peeled diagonal slices rely on it); SYRK products are NT.
  // Products are either symmetric NT (Gram, polynomial) or NN (update).
  for (int i = 0; i < g.nprob; ++i)
    if (g.prob[i].K % 128 != 0 || g.prob[i].K < tile) return hipErrorInvalidValue;
  if (syrk == nn) return hipErrorInvalidValue;
  if (tile == 256) return syrk ? launch_one<256, true, false>(g, s) : launch_one<256, false, true>(g, s);
  return syrk ? launch_one<128, true, false>(g, s) : launch_one<128, false, true>(g, s);
}

}  // namespace muon
