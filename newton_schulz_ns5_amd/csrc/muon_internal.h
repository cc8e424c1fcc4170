// Internal declarations shared by the host entry points and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace muon {

// Pointer tables travel in kernel arguments; a launch covers at most this
// many parameters.
constexpr int kMaxParams = 32;

// Padding granule of the oriented workspace matrices.  Pad rows and columns
// are zero and stay zero through every iteration (zero columns add nothing to
// X X^T; zero rows of B give zero rows of B X), so the GEMMs need no bounds
// checks in their main loops.
constexpr int kPadBf16 = 128;
constexpr int kPadF32 = 64;
constexpr int kPrepTile = 64;   // tile edge of the load / momentum kernel

// ---- GEMM: C[b] = alpha_b * P[b] * op(Q[b]) + beta_b * D[b] -------------------
// P is [M][K] row-major.  NT: Q is [N][K] (both operands K-contiguous).
// NN: Q is [K][N].  SYRK: only tiles with tile_n >=
// tile_m are computed and each value is also written to the mirrored
// position, so C is exactly symmetric.
struct GemmParams {
  const void* P; int64_t ldp; int64_t sP;
  const void* Q; int64_t ldq; int64_t sQ;
  const void* D; int64_t ldd; int64_t sD;   // may be null
  void* C; int64_t ldc; int64_t sC;         // row-major result, may be null (bf16 kernels)
  void* Ct; int64_t ldct; int64_t sCt;      // transposed result: (i, j) -> Ct[j*ldct + i] (bf16 kernels)
  int32_t c_dtype;        // MUON_BF16 / MUON_F32
  int32_t c_trans;        // fp32 kernels: store C^T into C instead of C
  int32_t dq;             // bf16 kernels: D = Q^T on every tile (D itself unused, alpha != 0);
                          // beta D is then added inside the products
  int32_t M, N, K;        // padded problem (multiples of the tile edges)
  int32_t Mreal, Nreal;   // only i < Mreal, j < Nreal are stored
  float alpha, beta;
  const float* rs;        // per-batch factor, may be null
  int32_t alpha_pow, beta_pow;  // alpha_b = alpha * rs[b]^alpha_pow ...
  int32_t batch;
  int32_t tiles_m, tiles_n, tiles_per_batch;
  int32_t ksplit;         // bf16 SYRK: > 1 splits K into this many chunks (cut at multiples
                          // of 128); batch entry b is chunk b % ksplit of matrix
                          // b / ksplit (P, Q, rs), and C[b] receives that chunk's product
  double flop, bytes;     // host bookkeeping for launch timing (not read by kernels)
};

// Several GEMM problems of one kind (same tile edge, same SYRK flag) in one
// launch: workgroups [tile_start[i], tile_start[i+1]) belong to problem i.
constexpr int kMaxProblems = 8;
struct GemmGroup {
  GemmParams prob[kMaxProblems];
  int32_t nprob;
  int32_t tile_start[kMaxProblems + 1];
  int32_t balance;  // 1: every XCD takes an equal share of every problem (else rounds of 8 x 32 tiles)
};

// ---- load / momentum / orientation / norm partials ------------------------
struct PrepParams {
  int32_t mode;           // 0: U = x (plain load); 1: Nesterov momentum
  int32_t tall;           // oriented X = U^T
  int32_t rows, cols;     // one NS matrix in parameter orientation
  int32_t mp, np;         // padded oriented dims
  int32_t heads;          // NS matrices per parameter (mode 1)
  int32_t src_dtype;      // x (mode 0) or grad (mode 1)
  int32_t mom_dtype;      // mode 1
  int32_t x_bf16;         // X0 storage dtype is bf16
  float mu; int32_t nesterov;
  const void* x; int64_t x_bs, x_rs;          // mode 0
  int64_t param_cols;                          // mode 1: row stride of a parameter
  const void* grad[kMaxParams];                // mode 1
  void* mom[kMaxParams];                       // mode 1
  void* X; int64_t X_bs;                       // oriented, padded output
  float* partial;                              // [b][tiles]
  int32_t no_x;                                // mode 0: partials only, X not written
};

struct NormParams {
  const float* partial; int32_t tiles;
  float eps;
  float* rs;              // rs[b] = 1 / (sqrt(sum partial) + eps)
};

// ---- split-K Gram: sum of the chunks' partial products -----------------------
// A[b] = bf16(rs[b]^2 * sum_s part[b][s]) over full mp x mp matrices (rs may be
// null: factor 1); the chunks are added in order s = 0, 1, ...
struct SplitSumParams {
  const float* part; int32_t ksplit; int32_t mp;
  void* A; int64_t lda; int64_t a_bs;
  const float* rs;
};

// ---- split-K Gram sum fused with the polynomial, 128 x 128 matrices ----------
// B[b] = bf16(c A A + b A) with A = bf16(rs[b]^2 * sum_s part[b][s]) (rs may
// be null: factor 1); one workgroup per matrix.
constexpr int kMaxKsplit = 16;   // K chunks of a split Gram, at most
// With nsum set (the first iteration), the workgroup of matrix b first
// computes rs[b] itself from the matrix's ntiles Frobenius-norm partials,
// exactly as the norm finalize does, uses it and stores it to rs_out[b] for
// the iteration's update; rs is then unused.
struct Poly128Params {
  const float* part; int32_t ksplit;
  const float* rs;
  float b, c;
  void* B; int64_t ldb; int64_t b_bs;
  const float* nsum; int32_t ntiles; float eps; float* rs_out;
};

// ---- NorMuon statistics ---------------------------------------------------
struct RowStatParams {
  const void* O; int32_t o_dtype; int64_t o_bs, o_rs;
  int32_t rows, cols;
  float* v_tab[kMaxParams];       // per-matrix variance pointers (table mode)
  float* v_base; int64_t v_bs;    // strided mode when v_base != null
  float beta2, eps;
  float* d; float* ms; float* q;  // workspace [b][rows]
};

struct RhoParams {
  const float* ms; const float* q; int32_t rows;
  float* rho;
};

// ---- weight update / in-place scaling ------------------------------------
struct ApplyParams {
  int32_t mode;           // 0: weight update; 1: o <- rho * d_r * o in place
  const void* O; int32_t o_dtype; int64_t o_bs, o_rs;
  int32_t rows, cols;
  const float* d; const float* rho;   // null without NorMuon
  float lr_eff, decay;    // decay = 1 - lr * wd
  float* w[kMaxParams];
  void* wm[kMaxParams];   // bf16 model copy or null
  int32_t vec;            // 1: 16-byte vector path is valid
};

// Launchers (return hipSuccess or the launch error).
// bf16: symmetric NT products (syrk) or NN products (nn), exactly one of the two.
hipError_t launch_gemm_bf16(const GemmGroup& g, bool syrk, bool nn, int tile, hipStream_t s);
hipError_t launch_gemm_f32(const GemmParams& p, bool nn, bool syrk, hipStream_t s);
int gemm_f32_tile();    // output tile edge of the fp32 GEMM (divides kPadF32)
// The load kernel and the norm finalize take several problems per launch:
// load-kernel problem i owns grid z indices zstart[i] .. zstart[i + 1] - 1,
// one per matrix (at most 65535 in all), norm problem i owns workgroups
// start[i] .. start[i + 1] - 1.  A PrepParams carries two pointer tables, so a
// load launch holds at most four problems.
constexpr int kMaxPrep = 4;
struct PrepGroup {
  PrepParams prob[kMaxPrep];
  int32_t zstart[kMaxPrep + 1];
  int32_t nprob;
};
static_assert(sizeof(PrepGroup) <= 4096, "kernel argument block of one launch");
hipError_t launch_prep_group(const PrepGroup& g, hipStream_t s);
constexpr int kMaxNorm = 8;
struct NormGroup {
  NormParams prob[kMaxNorm];
  int32_t start[kMaxNorm + 1];
  int32_t nprob;
};
hipError_t launch_norm_group(const NormGroup& g, hipStream_t s);
hipError_t launch_split_sum(const SplitSumParams& p, int nb, hipStream_t s);
// Up to kMaxPoly128 such problems in one launch; problem i owns workgroups
// start[i] .. start[i + 1] - 1, one per matrix.
constexpr int kMaxPoly128 = 8;
struct Poly128Group {
  Poly128Params prob[kMaxPoly128];
  int32_t start[kMaxPoly128 + 1];
  int32_t nprob;
};
hipError_t launch_poly128(const Poly128Group& g, hipStream_t s);
// ---- update fused with the next Gram's chunk products, 128-row matrices -----
// Y[b] = alpha_b B[b] X[b] + beta_b X[b] (bf16, [128][np] row-major; alpha_b
// = alpha rs[b]^alpha_pow, beta_b = beta rs[b]^beta_pow, rs may be null) and,
// when part is not null, part[b * ksplit + c] = Y_c Y_c^T (fp32 [128][128],
// its 32 x 32 blocks on and above the diagonal only, the diagonal blocks
// exactly symmetric; the blocks below are not written) over the columns of
// chunk c, whose edges are those of the split-K Gram (128 * floor(c * (np /
// 128) / ksplit)).  B is exactly symmetric.
struct UpdGram128Params {
  const void* B; int64_t b_bs;       // [128][128] bf16, row stride 128
  const void* X; int64_t x_bs;       // [128][np] bf16, row stride np
  void* Y; int64_t y_bs;             // [128][np] bf16, row stride np
  float* part;                       // [nb * ksplit][128][128] fp32, or null
  float* nsq;                        // Gram only: [nb][ksplit] sums of squares of X's chunks, or null
  int32_t np, ksplit;                // np a multiple of 128; 1 <= ksplit <= np / 128
  float alpha, beta;
  const float* rs; int32_t alpha_pow, beta_pow;
};
// Up to kMaxUpdGram128 such problems in one launch; problem i owns workgroups
// start[i] .. start[i + 1] - 1 (nb_i * ksplit_i, one per matrix and chunk).
constexpr int kMaxUpdGram128 = 8;
struct UpdGram128Group {
  UpdGram128Params prob[kMaxUpdGram128];
  int32_t start[kMaxUpdGram128 + 1];
  int32_t nprob;
};
hipError_t launch_updgram128(const UpdGram128Group& g, hipStream_t s);
// The chunk products of X X^T alone (the first iteration's Gram), chunked as
// above, and (nsq) each chunk's sum of squares; only X, x_bs, part, nsq, np
// and ksplit are used.
hipError_t launch_gram128(const UpdGram128Group& g, hipStream_t s);
hipError_t launch_rowstat(const RowStatParams& p, int nb, hipStream_t s);
hipError_t launch_rho(const RhoParams& p, int nb, hipStream_t s);
hipError_t launch_apply(const ApplyParams& p, int nb, hipStream_t s);
// The same three for several problems per launch (the step's shape groups):
// problem i owns matrices start[i] .. start[i + 1] - 1 of the launch.
constexpr int kMaxRowStat = 4, kMaxRho = 8, kMaxApply = 4;
struct RowStatGroup {
  RowStatParams prob[kMaxRowStat];
  int32_t start[kMaxRowStat + 1];
  int32_t nprob;
};
struct RhoGroup {
  RhoParams prob[kMaxRho];
  int32_t start[kMaxRho + 1];
  int32_t nprob;
};
struct ApplyGroup {
  ApplyParams prob[kMaxApply];
  int32_t start[kMaxApply + 1];
  int32_t nprob;
};
static_assert(sizeof(RowStatGroup) <= 4096 && sizeof(ApplyGroup) <= 4096, "kernel argument block of one launch");
hipError_t launch_rowstat_group(const RowStatGroup& g, hipStream_t s);
hipError_t launch_rho_group(const RhoGroup& g, hipStream_t s);
hipError_t launch_apply_group(const ApplyGroup& g, hipStream_t s);

// Tile edge the bf16 GEMM uses for an M x N output (depends on shape only).
// An output of at most 512 rows has at most 2 tile rows of 256 (a symmetric
// one at most 3 upper-triangle tiles, against 10 of 128): such problems
// are short-K or few-tile, and 128-edge tiles fill the chip better.
inline int bf16_tile_for(int M, int N) {
  if (M <= 512) return 128;
  return (M % 256 == 0 && N % 256 == 0) ? 256 : 128;
}

}  // namespace muon
