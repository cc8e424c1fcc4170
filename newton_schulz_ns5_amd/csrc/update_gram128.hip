// The update of one Newton-Schulz iteration fused with the Gram of the next,
// for matrices whose short side pads to 128 rows (e.g. the 128-row heads of
// per-head Newton-Schulz, "Muon under AutoTP orthogonalizes each shard ...",
// "What could be done" option 3).
//
// An iteration ends with X' = B X + a X (B = b A + c A^2, exactly symmetric;
// "core.optimizer.layer_sharded_muon", use_syrk) and the next one starts with
// A' = X' X'^T.  With 128 rows a column strip of X' holds every row, so the
// split-K products of the next Gram over that strip's columns come straight
// from the strip.  One workgroup per (matrix, column chunk):
//   1. keeps B in LDS (32 KiB, loaded once) and streams its chunk of X in
//      128-column sub-tiles through three LDS buffers, two sub-tiles ahead
//      (direct HBM -> LDS loads);
//   2. computes X'^T = X^T B with v_mfma_f32_32x32x16_bf16: the A operand is
//      X read column-wise with the LDS transpose read, the B operand rows of
//      B, so each lane's accumulators hold four consecutive columns of one
//      row of X';
//   3. adds beta X inside the products (MFMAs of X^T with (beta / alpha) I on
//      the K steps that meet its diagonal, as the tiled update does), rounds
//      to bf16 and writes the sub-tile into LDS as rows of K values -- the
//      layout the Gram's operands are read in -- from where it goes to HBM
//      with 16-byte stores;
//   4. accumulates the chunk's Gram product X'_c X'_c^T over its sub-tiles
//      (fp32) and finally stores its 32 x 32 blocks on and above the
//      diagonal (the diagonal ones exactly symmetric), straight from the
//      accumulators, as chunk c of the split-K product the next iteration's
//      sum-and-polynomial kernel reads.
// The same kernel without steps 2-3 computes the first iteration's chunk
// products from X itself (and, when asked, the chunk's sum of squares, the
// norm's partial), and without step 4 an update alone.
// Eight waves (two per SIMD) share each sub-tile's products, so one wave's
// MFMAs run while the other waits on LDS.  Waves 0-3 issue every HBM -> LDS
// load and waves 4-7 every X' store, so no wave waits on a count that
// mixes loads and stores.  Every LDS address a lane uses is
// fixed up front, so the loop issues its LDS accesses with immediate offsets.
// The chunk edges are the split-K Gram's, multiples of 128 that depend on the
// matrix shape only, and every sub-tile is computed by the same instruction
// sequence, so a matrix's result does not depend on its batch.
#include "muon_internal.h"
#include "device_util.h"
#include "muon_mi355x.h"

namespace muon {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int M = 128;                 // rows of X (and the update's K)
constexpr int SUB = 128;               // columns per sub-tile
constexpr int NT_SLICE = M * 128;      // 64 K values of 128 rows, 128 bytes per row: 16 KiB
constexpr int B_BYTES = 2 * NT_SLICE;  // B: 32 KiB
constexpr int XROWB = SUB * 2;         // bytes of one row of an X sub-tile
constexpr int X_BYTES = M * XROWB;     // one X sub-tile: 32 KiB
constexpr int NXB = 3;                 // X sub-tile buffers
constexpr int Y_BYTES = 2 * NT_SLICE;  // the X' sub-tile as Gram operand rows: 32 KiB
constexpr int LDS_BYTES = B_BYTES + NXB * X_BYTES + Y_BYTES;
static_assert(LDS_BYTES <= 160 * 1024, "LDS of one workgroup");

// LDS layouts (byte offsets):
//  - NT operand (B, and the X' sub-tile Y): slice s (K values 64 s .. 64 s +
//    63) of row r at s NT_SLICE + 128 r; its eight 16-byte chunks are
//    XOR-swizzled by (r / 2) mod 8, so a 16-lane fragment read of 16
//    consecutive rows at one logical chunk touches all 64 banks once.
//  - X sub-tile: row k (a K index of the update) at XROWB k, its eight
//    32-byte blocks (16 columns each) XOR-swizzled by 2 (k mod 4), so a
//    transpose read of 32 lanes covers every bank once.
// MODE: kUpdGram (update, then the next Gram's chunk products), kUpdOnly
// (update only) or kGramOnly (the chunk products of X itself: the first
// iteration's Gram; B, Y, alpha and beta are unused).
enum { kUpdGram = 0, kUpdOnly = 1, kGramOnly = 2 };

// Workgroup -> (problem, matrix, chunk).  Workgroup w runs on XCD w % 8 as the
// (w / 8)-th of that XCD's queue.  The launch's matrices are numbered problem
// after problem, and matrix g is given to XCD g % 8 with all its chunks: the
// chunk products a workgroup writes are read by the next launch's workgroups
// of the same matrix on the same XCD, from its L2.  XCD x's queue holds its
// matrices in order, each as its chunks in order; the grid is 8 times the
// longest queue, and the workgroups past the end of a shorter queue return
// at once (xcd_slot false).
__device__ __forceinline__ bool xcd_slot(const UpdGram128Group& g, int& pi, int& b, int& ch) {
  const int x = (int)blockIdx.x & 7;
  int k = (int)blockIdx.x >> 3;
  auto share = [x](int n) { return (n + 7 - x) >> 3; };  // g < n with g % 8 == x
  int g0 = 0;
  for (pi = 0; pi < g.nprob; ++pi) {
    const int ks = g.prob[pi].ksplit;
    const int nb = (g.start[pi + 1] - g.start[pi]) / ks;
    const int cnt = share(g0 + nb) - share(g0);  // this problem's matrices on XCD x
    if (k < cnt * ks) {
      const int j = k / ks;
      ch = k - j * ks;
      b = ((x - g0) & 7) + 8 * j;  // the j-th matrix g >= g0 with g % 8 == x, minus g0
      return true;
    }
    k -= cnt * ks;
    g0 += nb;
  }
  return false;
}

// Grid of a launch: 8 x the longest XCD queue.
int xcd_grid(const UpdGram128Group& g) {
  int longest = 0;
  for (int x = 0; x < 8; ++x) {
    int q = 0, g0 = 0;
    for (int i = 0; i < g.nprob; ++i) {
      const int ks = g.prob[i].ksplit;
      const int nb = (g.start[i + 1] - g.start[i]) / ks;
      q += (((g0 + nb + 7 - x) >> 3) - ((g0 + 7 - x) >> 3)) * ks;
      g0 += nb;
    }
    longest = q > longest ? q : longest;
  }
  return 8 * longest;
}

template <int MODE>
__global__ __launch_bounds__(512, 1) void updgram128_kernel(const UpdGram128Group grp) {
  constexpr bool UPD = MODE != kGramOnly, GRAM = MODE != kUpdOnly;
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7, two per SIMD
  const int wa = wave >> 1, wb = wave & 1;                     // wa 0..3: a 32-wide block row

  int pi, b, ch;
  if (!xcd_slot(grp, pi, b, ch)) return;  // a padding workgroup: no work
  const UpdGram128Params& p = grp.prob[pi];
  const int ks = p.ksplit;
  const int kb = p.np / SUB;
  const int j0 = (int)((int64_t)ch * kb / ks);
  const int nsub = (int)((int64_t)(ch + 1) * kb / ks) - j0;
  const int ldx = __builtin_amdgcn_readfirstlane(p.np);

  const uint16_t* const Bg = (const uint16_t*)p.B + (int64_t)b * p.b_bs;
  const uint16_t* const Xg = (const uint16_t*)p.X + (int64_t)b * p.x_bs + (int64_t)j0 * SUB;
  uint16_t* const Yg = (uint16_t*)p.Y + (int64_t)b * p.y_bs + (int64_t)j0 * SUB;
  const int64_t chunk_bytes = ((int64_t)(M - 1) * ldx + (int64_t)nsub * SUB) * 2;
  const i32x4 brw = rsrc_words(Bg, (int64_t)M * M * 2);
  const i32x4 xrw = rsrc_words(Xg, chunk_bytes);
  const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)Yg, (short)0, __builtin_amdgcn_readfirstlane((int)chunk_bytes), 0x00020000);
  // LDS byte addresses (the ds instructions take a 32-bit address plus an
  // immediate offset): B, the X buffers and the X' sub-tile Y.
  const uint32_t lds0 =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem);
  const uint32_t Bs = lds0, Xs = lds0 + B_BYTES, Ys = Xs + NXB * X_BYTES;

  const float rsb = p.rs ? p.rs[b] : 1.f;
  const float alpha = p.alpha * (p.alpha_pow == 2 ? rsb * rsb : (p.alpha_pow == 1 ? rsb : 1.f));
  const float beta = p.beta * (p.beta_pow == 1 ? rsb : 1.f);

  // B (waves 0-3): instruction q (0..7) of a wave fills rows 8 g .. 8 g + 7
  // (g = 4 wave + q % 4) of slice q / 4; lane l lands at row 8 g + l / 8,
  // chunk l % 8 and therefore fetches the chunk (l % 8) ^ ((row / 2) % 8) of
  // that row.
  if (UPD && wave < 4) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int s = q >> 2, g = wave * 4 + (q & 3);
      const int voff = (lane >> 3) * (M * 2) + ((lane & 7) ^ ((4 * g + (lane >> 4)) & 7)) * 16;
      lds_dma16_asm(brw, Bs + (uint32_t)(s * NT_SLICE + 8 * g * 128), voff, 8 * g * (M * 2) + s * 128);
    }
  }
  // X sub-tile jj (waves 0-3), update modes: instruction q (0..7) of a wave
  // fills rows 32 wave + 4 q .. + 3; lane l lands at row 32 wave + 4 q +
  // l / 16, 16-byte chunk l % 16, fetching the chunk whose 32-byte block is
  // swizzled by 2 (row % 4) = 2 (l / 16).
  // Gram only: the sub-tile goes into the NT layout (it is the Gram's operand
  // as it stands), filled as B is: instruction q fills rows 8 g .. 8 g + 7
  // (g = 4 wave + q % 4) of slice q / 4.
  const int xvoff = UPD ? (lane >> 4) * ldx * 2 + (2 * (((lane & 15) >> 1) ^ (2 * (lane >> 4))) + (lane & 1)) * 16
                        : (lane >> 3) * ldx * 2;
  auto dma_x = [&](int jj, int buf) {
    if (wave >= 4) return;
    const uint32_t dst = Xs + (uint32_t)(buf * X_BYTES);
    if constexpr (UPD) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int row = 32 * wave + 4 * q;
        lds_dma16_asm(xrw, dst + (uint32_t)(row * XROWB), xvoff, row * ldx * 2 + jj * SUB * 2);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int s = q >> 2, g = wave * 4 + (q & 3);
        const int voff = xvoff + ((lane & 7) ^ ((4 * g + (lane >> 4)) & 7)) * 16;
        lds_dma16_asm(xrw, dst + (uint32_t)(s * NT_SLICE + 8 * g * 128), voff, 8 * g * ldx * 2 + s * 128 + jj * SUB * 2);
      }
    }
  };

  // ---- per-lane LDS addresses, fixed for the whole kernel ------------------
  // MFMA 32x32x16 operands: lane l supplies row (A) or column (B) l % 32 of a
  // block with the 8 K values 8 (l / 32) .. + 7 of the 16-wide K step kk.
  // NT operand (B and Y) rows r = r0 + l % 32 with r0 a multiple of 32, so
  // the chunk swizzle (r / 2) % 8 is the lane's own sw; the 16-byte chunk of
  // K step kk is 2 (kk % 4) + l / 32, in slice kk / 4.
  const int sw = ((lane & 31) >> 1) & 7;
  uint32_t ntl[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) ntl[t] = (uint32_t)((lane & 31) * 128 + (((2 * t + (lane >> 5)) ^ sw) << 4));
  auto nt_frag = [&](uint32_t base, int kk) {  // base: operand + 128 r0 (+ slice added here)
    typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
    return __builtin_bit_cast(bf16x8, *(const lds_u32x4*)(uintptr_t)(base + ntl[kk & 3] + (kk >> 2) * NT_SLICE));
  };
  // X^T fragment: columns n0 + l % 32 of an X sub-tile (n0 = 32 wa),
  // K rows 16 kk + 8 (l / 32) .. + 7, from two transpose reads.  Within each
  // 16-lane group lane l supplies row 8 (l / 32) + (l % 16) / 4 (+ 16 kk, + 4
  // for the second read) and columns 4 (l % 4) .. + 3 of the 16-column half
  // (l / 16) % 2; that row's 32-byte blocks are swizzled by 2 ((l % 16) / 4).
  uint32_t xtl;
  {
    const int blk = ((2 * wa + ((lane >> 4) & 1)) ^ (2 * ((lane & 15) >> 2)));
    xtl = (uint32_t)((8 * (lane >> 5) + ((lane & 15) >> 2)) * XROWB + blk * 32 + (lane & 3) * 8);
  }
  auto xt_frag = [&](uint32_t xbase, int kk) {  // xbase: X buffer + xtl
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(xbase + 16 * kk * XROWB));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(xbase + 16 * kk * XROWB + 4 * XROWB));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // Epilogue writes: X'(m, n .. n + 3) with m = 64 wb + 32 j + l % 32 and n =
  // 64 wa + 8 c + 4 (l / 32), c = 4 i + q, lands in slice wa of Y at row m,
  // chunk c ^ sw, byte 8 (l / 32) of the chunk.
  uint32_t ywl[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    ywl[q] = Ys + (uint32_t)((wa >> 1) * NT_SLICE + (64 * wb + (lane & 31)) * 128 + (((4 * (wa & 1) + q) ^ sw) << 4) +
                             8 * (lane >> 5));
  // X' rows to HBM (waves 4-7, t2 = tid - 256): thread -> 16-byte chunk
  // t2 % 16 of rows t2 / 16 + 16 u (u = 0..7); row t2 / 16 + 16 u has the
  // swizzle (t2 / 32) % 8 whatever u.
  const int t2 = tid & 255;
  const uint32_t yrd = Ys + (uint32_t)(((t2 >> 3) & 1) * NT_SLICE + (t2 >> 4) * 128 +
                                       (((t2 & 7) ^ ((t2 >> 5) & 7)) << 4));
  const int yvoff = ((t2 >> 4) * ldx + (t2 & 15) * 8) * 2;

  // beta X is added inside the products: X'^T = X^T (B + E) with E = (beta /
  // alpha) I, entered as two bf16 terms (hi + lo, within 2^-16 of the
  // factor).  For block column j (rows m0 = 64 wb + 32 j of B) the K steps
  // 4 wb + 2 j + h (h = 0, 1) meet E's diagonal; there the B-operand fragment
  // eh[h] / el[h] of lane l holds the factor at K position (l % 32) - 16 h -
  // 8 (l / 32) when that lies in 0..7.
  bf16x8 eh[2], el[2];
  {
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

  f32x16 accg[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) accg[j][r] = 0.f;
  // Gram only, with nsq: this thread's share of the chunk's sum of squares,
  // the 16-byte pieces tid + 512 i (i = 0..3) of every sub-tile, added in
  // sub-tile, piece and element order.
  float sq = 0.f;

  // Pipeline.  Waves 0-3 issue only loads, in this order: B (8, update
  // modes), X_0 (8), X_1 (8 when nsub > 1), then per sub-tile jj X_{jj+2} (8
  // when jj + 2 < nsub).  Loads complete in issue order, so waiting until at
  // most the 8 loads of X_{jj+1} are pending means X_jj has landed; the
  // barrier after it publishes X_jj to every wave.  Waves 4-7 issue only the
  // X' stores and never wait on them: a store may complete before loads
  // issued ahead of it, so a count that mixed the two could return with a
  // load still in flight.
  dma_x(0, 0);
  if (nsub > 1) dma_x(1, 1);
#pragma unroll 1
  for (int jj = 0; jj < nsub; ++jj) {
    const int buf = jj % NXB;
    if (wave < 4) {
      if (jj + 1 < nsub) wait_vmcnt<8>(); else wait_vmcnt<0>();
    }
    __syncthreads();  // X_jj (and B) visible; every wave is done with sub-tile jj - 1
    if (jj + 2 < nsub) dma_x(jj + 2, (jj + 2) % NXB);
    const uint32_t xb = Xs + (uint32_t)(buf * X_BYTES);
    // The Gram's operand: the X' sub-tile, or (Gram only) the X sub-tile.
    const uint32_t gop = UPD ? Ys : xb;

    if constexpr (UPD) {
      const uint32_t xa0 = xb + xtl;
      // X'^T block j of wave (wa, wb): columns 32 wa .. of X' (its rows here),
      // rows 64 wb + 32 j .. of X' (its columns here).
      f32x16 acc[2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 xa = xt_frag(xa0, kk);
        bf16x8 bq[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) bq[j] = nt_frag(Bs + (uint32_t)((64 * wb + 32 * j) * 128), kk);
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, bq[j], acc[j], 0, 0, 0);
        if ((kk >> 2) == wb) {  // K step 4 wb + 2 j + h meets E's diagonal for block column j
          const int j = (kk >> 1) & 1, h = kk & 1;
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, eh[h], acc[j], 0, 0, 0);
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, el[h], acc[j], 0, 0, 0);
        }
      }
      if (alpha != 1.f) {  // first iteration: alpha = 1 / (||U|| + eps)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[j][r] *= alpha;
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          u32x2 w;
          w[0] = pack_bf2(acc[j][4 * q], acc[j][4 * q + 1]);
          w[1] = pack_bf2(acc[j][4 * q + 2], acc[j][4 * q + 3]);
          typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
          *(lds_u32x2*)(uintptr_t)(ywl[q] + 32 * j * 128) = w;
        }
      __syncthreads();  // the X' sub-tile is complete in LDS
      if (wave >= 4) {
        typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
        u32x4 yv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) yv[u] = *(const lds_u32x4*)(uintptr_t)(yrd + 2048 * u);
#pragma unroll
        for (int u = 0; u < 8; ++u)
          __builtin_amdgcn_raw_buffer_store_b128(yv[u], yrs, yvoff,
                                                 __builtin_amdgcn_readfirstlane(16 * u * ldx * 2 + jj * SUB * 2), 0);
      }
    }
    if constexpr (!UPD) {
      if (p.nsq) {
        typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4 w = *(const lds_u32x4*)(uintptr_t)(xb + (uint32_t)(16 * tid + 8192 * i));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float lo = __uint_as_float(w[e] << 16), hi = __uint_as_float(w[e] & 0xffff0000u);
            sq += lo * lo;
            sq += hi * hi;
          }
        }
      }
    }
    // Gram block j of wave (wa, wb): rows 32 wa .., columns 64 wb + 32 j ...
    if constexpr (GRAM) {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 ya = nt_frag(gop + (uint32_t)((32 * wa) * 128), kk);
        bf16x8 yq[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) yq[j] = nt_frag(gop + (uint32_t)((64 * wb + 32 * j) * 128), kk);
#pragma unroll
        for (int j = 0; j < 2; ++j) accg[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ya, yq[j], accg[j], 0, 0, 0);
      }
    }
  }
  if constexpr (!GRAM) return;
  if constexpr (!UPD) {
    if (p.nsq) {
      // Wave sums into the (unused) X' area, then added in wave order.
      typedef __attribute__((address_space(3))) float lds_f32;
      sq = wave_sum(sq);
      if (lane == 0) *(lds_f32*)(uintptr_t)(Ys + 4 * wave) = sq;
      __syncthreads();
      if (tid == 0) {
        float t = 0.f;
        for (int w = 0; w < 8; ++w) t += *(const lds_f32*)(uintptr_t)(Ys + 4 * w);
        p.nsq[(int64_t)b * ks + ch] = t;
      }
    }
  }

  // The chunk's Gram product from the accumulators: register 4 q + e of
  // block j holds G(R + e, C) with R = 32 wa + 8 q + 4 (l / 32) and C = 64 wb
  // + 32 j + l % 32.  Its reader (the sum-and-polynomial kernel) takes the
  // 32 x 32 blocks on and above the diagonal only, so those are stored: a
  // block above the diagonal (block row wa below block column 2 wb + j) as
  // it is, a diagonal block exactly symmetric (G(R + e, C) when R + e <= C,
  // and as its mirror G(C, R + e) when R + e < C); blocks below are skipped.
  float* const out = p.part + ((int64_t)b * ks + ch) * M * M;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int bi = wa, bj = 2 * wb + j;
      if (bi > bj) continue;
      const f32x16& a = accg[j];
      const int C = 32 * bj + (lane & 31);
      if (bi < bj) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int R = 32 * bi + 8 * q + 4 * (lane >> 5);
#pragma unroll
          for (int e = 0; e < 4; ++e) out[(R + e) * M + C] = a[4 * q + e];
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int R = 32 * bi + 8 * q + 4 * (lane >> 5);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (R + e <= C) out[(R + e) * M + C] = a[4 * q + e];
            if (R + e < C) out[C * M + R + e] = a[4 * q + e];
          }
        }
      }
    }
}

}  // namespace

hipError_t launch_updgram128(const UpdGram128Group& g, hipStream_t s) {
  if (g.nprob < 1 || g.nprob > kMaxUpdGram128 || g.start[0] != 0) return hipErrorInvalidValue;
  for (int i = 0; i < g.nprob; ++i) {
    const UpdGram128Params& p = g.prob[i];
    if (p.np <= 0 || p.np % SUB != 0 || p.ksplit < 1 || p.ksplit > p.np / SUB) return hipErrorInvalidValue;
    if (g.start[i + 1] < g.start[i] || (g.start[i + 1] - g.start[i]) % p.ksplit != 0) return hipErrorInvalidValue;
  }
  if (g.start[g.nprob] <= 0) return hipSuccess;
  const int grid = xcd_grid(g);
  // One variant per launch: the Gram products are computed for every problem
  // or for none.
  const bool gram = g.prob[0].part != nullptr;
  for (int i = 1; i < g.nprob; ++i)
    if ((g.prob[i].part != nullptr) != gram) return hipErrorInvalidValue;
  return gram ? launch_kernel(updgram128_kernel<kUpdGram>, dim3(grid), g, s, 512)
              : launch_kernel(updgram128_kernel<kUpdOnly>, dim3(grid), g, s, 512);
}

hipError_t launch_gram128(const UpdGram128Group& g, hipStream_t s) {
  if (g.nprob < 1 || g.nprob > kMaxUpdGram128 || g.start[0] != 0) return hipErrorInvalidValue;
  for (int i = 0; i < g.nprob; ++i) {
    const UpdGram128Params& p = g.prob[i];
    if (p.np <= 0 || p.np % SUB != 0 || p.ksplit < 1 || p.ksplit > p.np / SUB || !p.X || !p.part)
      return hipErrorInvalidValue;
    if (g.start[i + 1] < g.start[i] || (g.start[i + 1] - g.start[i]) % p.ksplit != 0) return hipErrorInvalidValue;
  }
  if (g.start[g.nprob] <= 0) return hipSuccess;
  return launch_kernel(updgram128_kernel<kGramOnly>, dim3(xcd_grid(g)), g, s, 512);
}

}  // namespace muon
