// Host side of the C ABI: validation, geometry, workspace carve-up and the
// launch sequence of one Muon / NorMuon step on the caller's stream.
//
// Failure policy ("core.optimizer.layer_sharded_muon", _validate_ns_config:
// one error kind, raised up front, never a silent switch of kernels; "Fix
// convolution flattening in megabatches and NorMuon normalization",
// "Compatibility": reject before mutating any state, empty shards are valid):
// every argument is checked before the first enqueue, so a call that returns
// an error has changed nothing.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "muon_internal.h"
#include "muon_mi355x.h"

using namespace muon;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return MUON_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MUON_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool dtype_ok(int32_t d) { return d == MUON_F32 || d == MUON_BF16; }
size_t esize(int32_t d) { return d == MUON_BF16 ? 2 : 4; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
int64_t round_up(int64_t x, int64_t g) { return (x + g - 1) / g * g; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// ---- geometry ---------------------------------------------------------------
// One NS problem is rows x cols in parameter orientation; it runs oriented as
// m x n with m = min, n = max (a tall matrix goes through its transpose), in
// workspace buffers padded to mp x np.
struct Geom {
  int64_t rows, cols, m, n, mp, np;
  bool tall, bf;
};

Geom make_geom(int64_t rows, int64_t cols, int32_t compute) {
  Geom g;
  g.rows = rows;
  g.cols = cols;
  g.tall = rows > cols;
  g.m = g.tall ? cols : rows;
  g.n = g.tall ? rows : cols;
  g.bf = compute == MUON_BF16;
  const int64_t pad = g.bf ? kPadBf16 : kPadF32;
  g.mp = round_up(g.m, pad);
  g.np = round_up(g.n, pad);
  return g;
}

// K chunks of the Gram A = X X^T of a bf16 geometry (1: no split).  A matrix
// with m <= 256 has one to three Gram tiles, too few workgroups to fill the
// chip over a long K = n; its Gram is then computed in chunks of about
// max(4 m, 1024) columns (at most 16), whose fp32 products are summed
// afterwards (shorter chunks would move more partial products than they save
// in latency).  A 128-row matrix takes chunks of about 683 columns (6 for
// n = 4096): its chunks are also the workgroups of the fused update / Gram
// kernel, and 40 heads of 4096 columns then fit one wave of workgroups over
// the chip (8 chunks, 320 workgroups, would need two).  The count depends on
// the shape only, so a matrix's result does not depend on its batch.
int gram_ksplit(const Geom& g) {
  if (!g.bf || g.mp > 256) return 1;
  const int64_t s = g.mp == 128 ? g.np * 3 / 2048 : g.np / std::max<int64_t>(4 * g.mp, 1024);
  return s < 2 ? 1 : (s > kMaxKsplit ? kMaxKsplit : (int)s);
}

// The 128-row path with a split Gram (fused update/Gram kernels; the norm
// is finalized by the first iteration's sum-and-polynomial kernel).
bool path128(const Geom& g) { return g.mp == 128 && gram_ksplit(g) > 1; }

// Column chunks (workgroups per matrix) of the last update of a 128-row
// matrix written straight to the output by the fused kernel.  No Gram
// follows, so the chunking is free: every 128-column sub-tile is computed
// the same way whatever chunk it is in.
int last_chunks128(const Geom& g) {
  const int kb = (int)(g.np / 128);
  return std::max(1, std::min(kb, kb / 8));
}

// Workspace of `nb` NS problems.
struct Layout {
  size_t X0, X1, A, B, partial, rs, part, total;
  int tiles;
};

Layout make_layout(const Geom& g, int64_t nb) {
  Layout L{};
  const size_t es = g.bf ? 2 : 4;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off = align256(off + bytes); return at; };
  L.tiles = (int)((g.mp / kPrepTile) * (g.np / kPrepTile));
  L.X0 = take((size_t)nb * g.mp * g.np * es);
  L.X1 = take((size_t)nb * g.mp * g.np * es);
  L.A = take((size_t)nb * g.mp * g.mp * es);
  L.B = take((size_t)nb * g.mp * g.mp * es);
  L.partial = take((size_t)nb * L.tiles * 4);
  L.rs = take((size_t)nb * 4);
  const int ks = gram_ksplit(g);
  L.part = ks > 1 ? take((size_t)nb * ks * g.mp * g.mp * 4) : 0;
  L.total = off;
  return L;
}

// ---- launch timing ------------------------------------------------------------
struct Pending {
  hipEvent_t a, b;
  int cls;
  double flop, bytes;
};
struct ClassTotals {
  int64_t launches = 0;
  double ms = 0, flop = 0, bytes = 0;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
uint32_t g_prof_mask = (1u << MUON_K_COUNT) - 1;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_event_pool;
ClassTotals g_totals[MUON_K_COUNT];

hipError_t get_event(hipEvent_t* e) {
  if (!g_event_pool.empty()) {
    *e = g_event_pool.back();
    g_event_pool.pop_back();
    return hipSuccess;
  }
  return hipEventCreate(e);
}

// Launch through `fn`, bracketed by events when timing is on.
template <class F>
hipError_t run(int cls, double flop, double bytes, hipStream_t s, F&& fn) {
  if (!g_prof_on || !((g_prof_mask >> cls) & 1u)) return fn();
  std::lock_guard<std::mutex> lk(g_prof_mu);
  Pending pd{nullptr, nullptr, cls, flop, bytes};
  hipError_t e = get_event(&pd.a);
  if (e == hipSuccess) e = get_event(&pd.b);
  if (e == hipSuccess) e = hipEventRecord(pd.a, s);
  if (e != hipSuccess) return e;
  e = fn();
  if (e != hipSuccess) return e;
  e = hipEventRecord(pd.b, s);
  if (e != hipSuccess) return e;
  g_pending.push_back(pd);
  return hipSuccess;
}

hipError_t drain_pending() {
  for (auto& pd : g_pending) {
    hipError_t e = hipEventSynchronize(pd.b);
    if (e != hipSuccess) return e;
    float ms = 0;
    e = hipEventElapsedTime(&ms, pd.a, pd.b);
    if (e != hipSuccess) return e;
    ClassTotals& t = g_totals[pd.cls];
    t.launches += 1;
    t.ms += ms;
    t.flop += pd.flop;
    t.bytes += pd.bytes;
    g_event_pool.push_back(pd.a);
    g_event_pool.push_back(pd.b);
  }
  g_pending.clear();
  return hipSuccess;
}

// ---- validation helpers ------------------------------------------------------
int check_cfg(const muon_ns_config* c) {
  if (!c) return fail(MUON_ERR_INVALID_ARG, "ns config is NULL");
  if (c->steps < 1 || c->steps > MUON_NS_MAX_STEPS) return fail(MUON_ERR_INVALID_ARG, "steps must be in 1..MUON_NS_MAX_STEPS (got %d)", c->steps);
  if (!dtype_ok(c->compute_dtype)) return fail(MUON_ERR_UNSUPPORTED, "compute_dtype %d is not MUON_BF16 or MUON_F32", c->compute_dtype);
  if (c->schedule != 0 && c->schedule != 1) return fail(MUON_ERR_INVALID_ARG, "schedule must be 0 or 1 (got %d)", c->schedule);
  if (c->max_batch < 0) return fail(MUON_ERR_INVALID_ARG, "max_batch must be >= 0");
  if (!std::isfinite(c->a) || !std::isfinite(c->b) || !std::isfinite(c->c) || !std::isfinite(c->eps) || c->eps < 0)
    return fail(MUON_ERR_INVALID_ARG, "coefficients must be finite and eps >= 0");
  if (c->schedule)
    for (int k = 0; k < c->steps; ++k)
      for (int j = 0; j < 3; ++j)
        if (!std::isfinite(c->coeffs[k][j])) return fail(MUON_ERR_INVALID_ARG, "coeffs[%d][%d] is not finite", k, j);
  return MUON_OK;
}

// Rows and columns per matrix: a 256-row operand panel of the padded long
// side must stay below 2^31 bytes (the GEMMs address panels through buffer
// descriptors with 32-bit sizes and offsets).
constexpr int64_t kMaxDim = ((int64_t)1 << 22) - kPadBf16;

int check_dims(int64_t n, int64_t rows, int64_t cols) {
  if (n < 0 || rows < 0 || cols < 0) return fail(MUON_ERR_INVALID_ARG, "negative size (n=%lld rows=%lld cols=%lld)", (long long)n, (long long)rows, (long long)cols);
  if (rows > kMaxDim || cols > kMaxDim) return fail(MUON_ERR_INVALID_ARG, "rows/cols above %lld", (long long)kMaxDim);
  const int64_t mp = round_up(rows < cols ? rows : cols, kPadBf16), np = round_up(rows < cols ? cols : rows, kPadBf16);
  if (mp * np >= ((int64_t)1 << 31)) return fail(MUON_ERR_INVALID_ARG, "matrix of %lld x %lld is too large", (long long)rows, (long long)cols);
  return MUON_OK;
}

// ---- the Newton-Schulz iterations on X0 already in the workspace --------------
struct FinalOut {
  void* C;
  int32_t dtype;
  int64_t ldc, sC;
};

// One fp32-compute GEMM launch.
hipError_t gemm_f32(GemmParams& p, bool nn, bool syrk, int cls, double flop, double bytes, hipStream_t s) {
  const int t = gemm_f32_tile();
  p.tiles_m = p.M / t;
  p.tiles_n = p.N / t;
  p.tiles_per_batch = syrk ? p.tiles_m * (p.tiles_m + 1) / 2 : p.tiles_m * p.tiles_n;
  return run(cls, flop, bytes, s, [&]() { return launch_gemm_f32(p, nn, syrk, s); });
}

// One pass of Newton-Schulz over nb same-shape matrices already loaded (X0,
// norm scales) into their own workspace region.
struct NsJob {
  Geom g;
  int64_t nb;
  char* ws;
  Layout L;
  FinalOut out;
  // The caller's bf16 input, read in place by the first iteration instead of
  // a copy in X0 (null: X0 holds the input), and its batch stride.
  const void* x0 = nullptr;
  int64_t x0_bs = 0;
};

// Estimated end of a launch's slowest XCD, in units of K: XCD x runs, in
// problem order, its tiles of each problem p (which ones: the kernel's tile
// order, rounds or balanced), each taking dur[p], on whichever of its 32 CUs
// frees first.
double xcd_makespan(const GemmGroup& g, const int* dur, bool balance) {
  constexpr int CH = 32, NCU = 32;
  const int G = g.tile_start[g.nprob];
  const int full = (G / (8 * CH)) * (8 * CH);
  // Tiles numbered below n that XCD x runs (n a problem boundary).
  auto before = [&](int n, int x) -> int64_t {
    if (balance) return (n + 7 - x) / 8;
    if (n <= full) return (int64_t)(n / (8 * CH)) * CH + std::min(std::max(n % (8 * CH) - x * CH, 0), CH);
    return (int64_t)(full / (8 * CH)) * CH + (n - full + 7 - x) / 8;
  };
  double worst = 0;
  for (int x = 0; x < 8; ++x) {
    double f[NCU] = {};  // CU free times, ascending
    for (int p = 0; p < g.nprob; ++p) {
      int64_t n = before(g.tile_start[p + 1], x) - before(g.tile_start[p], x);
      const double d = dur[p];
      while (n > 0) {
        if (n >= NCU && f[NCU - 1] - f[0] <= d) {
          // Every CU takes one tile of each batch of NCU (a CU that takes a
          // tile frees after all the others).
          const int64_t k = n / NCU;
          for (double& v : f) v += (double)k * d;
          n -= k * NCU;
          continue;
        }
        double v = f[0] + d;
        int i = 1;
        for (; i < NCU && f[i] < v; ++i) f[i - 1] = f[i];
        f[i - 1] = v;
        --n;
      }
    }
    worst = std::max(worst, f[NCU - 1]);
  }
  return worst;
}

// Launch one phase (Gram, poly or update) of several jobs: problems with the
// same tile edge share a launch (at most kMaxProblems each), longest K first
// so that the long tiles start in the first waves.  Where K differs between
// the problems of a launch, the balanced tile order is taken if it is
// expected to end the launch at least 3 % sooner.
hipError_t launch_phase(std::vector<GemmParams>& probs, bool syrk, bool nn, int cls, hipStream_t s) {
  for (int tile : {256, 128}) {
    std::vector<GemmParams*> sel;
    for (auto& p : probs)
      if (bf16_tile_for(p.M, p.N) == tile) sel.push_back(&p);
    // K per workgroup: a split-K problem's chunks are about K / ksplit long.
    auto kwg = [](const GemmParams* x) { return x->ksplit > 1 ? x->K / x->ksplit : x->K; };
    std::stable_sort(sel.begin(), sel.end(), [&](const GemmParams* x, const GemmParams* y) { return kwg(x) > kwg(y); });
    for (size_t i0 = 0; i0 < sel.size(); i0 += kMaxProblems) {
      GemmGroup grp{};
      grp.nprob = 0;
      int64_t tiles = 0;
      for (size_t i = i0; i < sel.size() && i < i0 + kMaxProblems; ++i) {
        GemmParams& p = *sel[i];
        p.tiles_m = p.M / tile;
        p.tiles_n = p.N / tile;
        p.tiles_per_batch = syrk ? p.tiles_m * (p.tiles_m + 1) / 2 : p.tiles_m * p.tiles_n;
        grp.tile_start[grp.nprob] = (int32_t)tiles;
        grp.prob[grp.nprob++] = p;
        tiles += (int64_t)p.batch * p.tiles_per_batch;
      }
      // Tile indices are 32-bit in the kernel (and a grid holds < 2^31 workgroups).
      if (tiles > INT32_MAX) return hipErrorInvalidValue;
      grp.tile_start[grp.nprob] = (int32_t)tiles;
      grp.balance = 0;
      int dur[kMaxProblems];
      bool mixed = false;
      for (int i = 0; i < grp.nprob; ++i) {
        dur[i] = kwg(&grp.prob[i]);
        mixed |= dur[i] != dur[0];
      }
      if (mixed && xcd_makespan(grp, dur, true) < 0.97 * xcd_makespan(grp, dur, false)) grp.balance = 1;
      double fl = 0, by = 0;  // algorithmic FLOPs and bytes of this launch
      for (int i = 0; i < grp.nprob; ++i) {
        fl += grp.prob[i].flop;
        by += grp.prob[i].bytes;
      }
      hipError_t e = run(cls, fl, by, s, [&]() { return launch_gemm_bf16(grp, syrk, nn, tile, s); });
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// (a, b, c) of iteration `it`.
struct Coeffs { float a, b, c; };
Coeffs coeffs_of(const muon_ns_config& cfg, int it) {
  if (cfg.schedule) return {cfg.coeffs[it][0], cfg.coeffs[it][1], cfg.coeffs[it][2]};
  return {cfg.a, cfg.b, cfg.c};
}

// bf16 mode: Gram and poly are symmetric NT products, the update is NN and
// reads X row-major.  X ping-pongs between two buffers; the last update
// writes the output in parameter orientation instead.
// A problem of the fused 128-row kernel with its batch and modelled cost.
struct UpdGram { UpdGram128Params p; int nb; double flop, bytes; };

// Launches of the fused 128-row kernel over `v`, kMaxUpdGram128 problems at a
// time: the update (with the next Gram when the problems have `part`), or the
// Gram only (`gram_only`).
hipError_t launch_updgram_groups(const std::vector<UpdGram>& v, int kclass, bool gram_only, hipStream_t s) {
  for (size_t i0 = 0; i0 < v.size(); i0 += kMaxUpdGram128) {
    UpdGram128Group ug{};
    double flop = 0, bytes = 0;
    for (size_t i = i0; i < v.size() && i < i0 + kMaxUpdGram128; ++i) {
      ug.prob[ug.nprob] = v[i].p;
      ug.start[ug.nprob + 1] = ug.start[ug.nprob] + v[i].nb * v[i].p.ksplit;
      ++ug.nprob;
      flop += v[i].flop;
      bytes += v[i].bytes;
    }
    const hipError_t e = run(kclass, flop, bytes, s, [&]() {
      return gram_only ? launch_gram128(ug, s) : launch_updgram128(ug, s);
    });
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t ns_iterations_bf16(const std::vector<NsJob>& jobs, const muon_ns_config& cfg, hipStream_t s) {
  std::vector<int> cur(jobs.size(), 0);
  for (int it = 0; it < cfg.steps; ++it) {
    const bool first = it == 0, last = it == cfg.steps - 1;
    const Coeffs cf = coeffs_of(cfg, it);
    std::vector<GemmParams> gram, poly, upd;
    struct Sum { SplitSumParams p; int nb; double bytes; };
    struct Fused { Poly128Params p; int nb; double flop, bytes; };
    std::vector<Sum> sums;
    std::vector<Fused> fused;
    std::vector<UpdGram> updgram, gram128, updonly;
    for (size_t k = 0; k < jobs.size(); ++k) {
      const NsJob& J = jobs[k];
      const Geom& g = J.g;
      const double m = (double)g.m, n = (double)g.n, B = (double)J.nb;
      char* ws = J.ws;
      void* X[2] = {ws + J.L.X0, ws + J.L.X1};
      void* A = ws + J.L.A;
      void* Bm = ws + J.L.B;
      const float* rs = (const float*)(ws + J.L.rs);
      const int64_t sx = g.mp * g.np, sa = g.mp * g.mp;
      const int c = cur[k];
      // The iterate this iteration reads: the caller's input itself on the
      // first iteration when it is read in place.
      const bool direct = first && J.x0;
      void* const Xin = direct ? const_cast<void*>(J.x0) : X[c];
      const int64_t sxin = direct ? J.x0_bs : sx;
      {  // A = X X^T (times rs^2 on the first iteration, which folds in the normalization)
        GemmParams p{};
        p.P = Xin; p.ldp = g.np; p.sP = sxin;
        p.Q = Xin; p.ldq = g.np; p.sQ = sxin;
        p.C = A; p.ldc = g.mp; p.sC = sa; p.c_dtype = MUON_BF16;
        p.M = p.N = (int)g.mp; p.K = (int)g.np; p.Mreal = p.Nreal = (int)g.mp;
        p.alpha = 1.f;
        p.rs = first ? rs : nullptr; p.alpha_pow = 2;
        p.batch = (int)J.nb;
        p.flop = B * m * m * n; p.bytes = B * (m * n + m * m) * 2;
        const int ks = gram_ksplit(g);
        // A 128-row matrix's Gram after the first iteration was computed by
        // the previous iteration's update (update_gram128): its chunk
        // products are already in the workspace.
        const bool prev_fused = path128(g) && !first;
        if (path128(g)) {
          // fp32 product of each K chunk, summed by the fused kernel that also
          // computes B (A is not stored)
          Poly128Params q{};
          q.part = (const float*)(ws + J.L.part); q.ksplit = ks;
          q.rs = p.rs;
          if (first) {  // the norm is finalized here from the first Gram's chunk sums of squares
            q.rs = nullptr;
            q.nsum = (const float*)(ws + J.L.partial); q.ntiles = ks;
            q.eps = cfg.eps; q.rs_out = (float*)(ws + J.L.rs);
          }
          q.b = cf.b; q.c = cf.c;
          q.B = Bm; q.ldb = g.mp; q.b_bs = sa;
          fused.push_back({q, (int)J.nb, B * m * m * m, B * (ks * m * m * 4 + m * m * 2)});
        } else if (ks > 1) {
          // fp32 product of each K chunk; the sum below scales and rounds
          SplitSumParams q{};
          q.part = (const float*)(ws + J.L.part); q.ksplit = ks; q.mp = (int)g.mp;
          q.A = A; q.lda = g.mp; q.a_bs = sa;
          q.rs = p.rs;
          sums.push_back({q, (int)J.nb, B * (ks * m * m * 4 + m * m * 2)});
        }
        if (ks > 1) {
          p.C = ws + J.L.part; p.sC = sa; p.c_dtype = MUON_F32;
          p.rs = nullptr;
          p.batch = (int)(J.nb * ks);
          p.ksplit = ks;
          p.bytes += B * (ks - 1) * m * m * 4;
        }
        if (path128(g) && first) {
          // The first Gram of a 128-row matrix: chunk products straight from
          // X by the Gram-only variant of the fused kernel (same chunks), with
          // each chunk's sum of squares (the norm's partials: no load-kernel
          // partials and no norm launch on this path).
          UpdGram128Params u{};
          u.X = Xin; u.x_bs = sxin;
          u.part = (float*)(ws + J.L.part);
          u.nsq = (float*)(ws + J.L.partial);
          u.np = (int)g.np; u.ksplit = ks;
          gram128.push_back({u, (int)J.nb, p.flop, B * (m * n * 2 + ks * m * m * 4)});
        } else if (!prev_fused) {
          gram.push_back(p);
        }
      }
      {  // B = c A A + b A; A is stored exactly symmetric, so the b A term is
         // A^T restricted to each tile and is added inside the products
        GemmParams p{};
        p.P = A; p.ldp = g.mp; p.sP = sa;
        p.Q = A; p.ldq = g.mp; p.sQ = sa;
        if (cf.c != 0.f) {
          p.dq = 1;
        } else {
          p.D = A; p.ldd = g.mp; p.sD = sa;
        }
        p.C = Bm; p.ldc = g.mp; p.sC = sa; p.c_dtype = MUON_BF16;
        p.M = p.N = p.K = (int)g.mp; p.Mreal = p.Nreal = (int)g.mp;
        p.alpha = cf.c; p.beta = cf.b;
        p.batch = (int)J.nb;
        p.flop = B * m * m * m; p.bytes = B * 2 * m * m * 2;
        if (!path128(g)) poly.push_back(p);
      }
      {  // X' = B X + a X (times rs on the first iteration): NN with Q = X,
         // whose transposed tile is the D tile, so a X is added inside the
         // products
        GemmParams p{};
        p.P = Bm; p.ldp = g.mp; p.sP = sa;
        p.Q = Xin; p.ldq = g.np; p.sQ = sxin;
        p.dq = 1;
        p.M = (int)g.mp; p.N = (int)g.np; p.K = (int)g.mp;
        p.alpha = 1.f; p.beta = cf.a;
        p.rs = first ? rs : nullptr; p.alpha_pow = 1; p.beta_pow = 1;
        p.batch = (int)J.nb;
        if (last) {
          p.c_dtype = J.out.dtype;
          if (g.tall) { p.Ct = J.out.C; p.ldct = J.out.ldc; p.sCt = J.out.sC; }
          else { p.C = J.out.C; p.ldc = J.out.ldc; p.sC = J.out.sC; }
          p.Mreal = (int)g.m; p.Nreal = (int)g.n;
        } else {
          p.c_dtype = MUON_BF16;
          p.C = X[c ^ 1]; p.ldc = g.np; p.sC = sx;
          p.Mreal = (int)g.mp; p.Nreal = (int)g.np;
        }
        p.flop = B * 2 * m * m * n; p.bytes = B * (m * m + 2 * m * n) * 2;
        const int ks = gram_ksplit(g);
        // The last update of a 128-row matrix whose output is the bf16
        // iterate's own layout (128 real rows, rows np apart, no padded
        // columns, 16-byte aligned) is written by the fused kernel's
        // update-only variant.
        const bool out128 = path128(g) && last && J.out.dtype == MUON_BF16 && !g.tall && g.m == g.mp &&
                            g.n == g.np && J.out.ldc == g.np && (J.out.sC % 8) == 0 &&
                            ((uintptr_t)J.out.C & 15) == 0;
        if (path128(g) && !last) {
          // Fused with the next iteration's Gram: X' to the other X buffer
          // and the chunk products of X' X'^T to the split-K buffer.
          UpdGram128Params u{};
          u.B = Bm; u.b_bs = sa;
          u.X = Xin; u.x_bs = sxin;
          u.Y = X[c ^ 1]; u.y_bs = sx;
          u.part = (float*)(ws + J.L.part);
          u.np = (int)g.np; u.ksplit = ks;
          u.alpha = 1.f; u.beta = cf.a;
          u.rs = p.rs; u.alpha_pow = 1; u.beta_pow = 1;
          updgram.push_back({u, (int)J.nb, B * 3 * m * m * n, B * ((m * m + 2 * m * n) * 2 + ks * m * m * 4)});
        } else if (out128) {
          UpdGram128Params u{};
          u.B = Bm; u.b_bs = sa;
          u.X = Xin; u.x_bs = sxin;
          u.Y = J.out.C; u.y_bs = J.out.sC;
          u.np = (int)g.np; u.ksplit = last_chunks128(g);
          u.alpha = 1.f; u.beta = cf.a;
          u.rs = p.rs; u.alpha_pow = 1; u.beta_pow = 1;
          updonly.push_back({u, (int)J.nb, p.flop, p.bytes});
        } else {
          upd.push_back(p);
        }
      }
    }
    hipError_t e;
    if ((e = launch_phase(gram, true, false, MUON_K_GRAM, s)) != hipSuccess) return e;
    if ((e = launch_updgram_groups(gram128, MUON_K_GRAM, true, s)) != hipSuccess) return e;
    for (const Sum& u : sums)
      if ((e = run(MUON_K_GRAM, 0, u.bytes, s, [&]() { return launch_split_sum(u.p, u.nb, s); })) != hipSuccess)
        return e;
    for (size_t i0 = 0; i0 < fused.size(); i0 += kMaxPoly128) {
      Poly128Group pg{};
      double flop = 0, bytes = 0;
      for (size_t i = i0; i < fused.size() && i < i0 + kMaxPoly128; ++i) {
        pg.prob[pg.nprob] = fused[i].p;
        pg.start[pg.nprob + 1] = pg.start[pg.nprob] + fused[i].nb;
        ++pg.nprob;
        flop += fused[i].flop;
        bytes += fused[i].bytes;
      }
      if ((e = run(MUON_K_POLY, flop, bytes, s, [&]() { return launch_poly128(pg, s); })) != hipSuccess) return e;
    }
    if ((e = launch_phase(poly, true, false, MUON_K_POLY, s)) != hipSuccess) return e;
    if ((e = launch_phase(upd, false, true, MUON_K_UPDATE, s)) != hipSuccess) return e;
    if ((e = launch_updgram_groups(updgram, MUON_K_UPDATE, false, s)) != hipSuccess) return e;
    if ((e = launch_updgram_groups(updonly, MUON_K_UPDATE, false, s)) != hipSuccess) return e;
    for (auto& c : cur) c ^= 1;
  }
  return hipSuccess;
}

// fp32 mode: Gram and poly NT (SYRK), update NN reading X itself.
hipError_t ns_iterations_f32(const Geom& g, int64_t nb, const muon_ns_config& cfg, char* ws, const Layout& L,
                             const FinalOut& out, hipStream_t s) {
  const int32_t wdt = g.bf ? MUON_BF16 : MUON_F32;
  const double es = g.bf ? 2 : 4;
  const double m = (double)g.m, n = (double)g.n, B = (double)nb;
  void* xin = ws + L.X0;
  void* xout = ws + L.X1;
  void* A = ws + L.A;
  void* Bm = ws + L.B;
  const float* rs = (const float*)(ws + L.rs);
  const int64_t sx = g.mp * g.np, sa = g.mp * g.mp;
  for (int it = 0; it < cfg.steps; ++it) {
    const bool first = it == 0, last = it == cfg.steps - 1;
    const Coeffs cf = coeffs_of(cfg, it);
    hipError_t e;
    {  // A = X X^T (times rs^2 on the first iteration, which folds in the normalization)
      GemmParams p{};
      p.P = xin; p.ldp = g.np; p.sP = sx;
      p.Q = xin; p.ldq = g.np; p.sQ = sx;
      p.C = A; p.ldc = g.mp; p.sC = sa; p.c_dtype = wdt;
      p.M = p.N = (int)g.mp; p.K = (int)g.np; p.Mreal = p.Nreal = (int)g.mp;
      p.alpha = 1.f; p.beta = 0.f;
      p.rs = first ? rs : nullptr; p.alpha_pow = 2;
      p.batch = (int)nb;
      e = gemm_f32(p, false, true, MUON_K_GRAM, B * m * m * n, B * (m * n + m * m) * es, s);
      if (e != hipSuccess) return e;
    }
    {  // B = c A A + b A
      GemmParams p{};
      p.P = A; p.ldp = g.mp; p.sP = sa;
      p.Q = A; p.ldq = g.mp; p.sQ = sa;
      p.D = A; p.ldd = g.mp; p.sD = sa;
      p.C = Bm; p.ldc = g.mp; p.sC = sa; p.c_dtype = wdt;
      p.M = p.N = p.K = (int)g.mp; p.Mreal = p.Nreal = (int)g.mp;
      p.alpha = cf.c; p.beta = cf.b;
      p.batch = (int)nb;
      e = gemm_f32(p, false, true, MUON_K_POLY, B * m * m * m, B * 2 * m * m * es, s);
      if (e != hipSuccess) return e;
    }
    {  // X' = B X + a X (times rs on the first iteration)
      GemmParams p{};
      p.P = Bm; p.ldp = g.mp; p.sP = sa;
      p.Q = xin; p.ldq = g.np; p.sQ = sx;
      p.D = xin; p.ldd = g.np; p.sD = sx;
      p.M = (int)g.mp; p.N = (int)g.np; p.K = (int)g.mp;
      p.alpha = 1.f; p.beta = cf.a;
      p.rs = first ? rs : nullptr; p.alpha_pow = 1; p.beta_pow = 1;
      p.batch = (int)nb;
      if (last) {
        p.C = out.C; p.c_dtype = out.dtype; p.ldc = out.ldc; p.sC = out.sC;
        p.c_trans = g.tall ? 1 : 0;
        p.Mreal = (int)g.m; p.Nreal = (int)g.n;
      } else {
        p.C = xout; p.c_dtype = wdt; p.ldc = g.np; p.sC = sx;
        p.Mreal = (int)g.mp; p.Nreal = (int)g.np;
      }
      e = gemm_f32(p, true, false, MUON_K_UPDATE, B * 2 * m * m * n, B * (m * m + 3 * m * n) * es, s);
      if (e != hipSuccess) return e;
    }
    std::swap(xin, xout);
  }
  return hipSuccess;
}

hipError_t ns_iterations(const std::vector<NsJob>& jobs, const muon_ns_config& cfg, hipStream_t s) {
  if (jobs.empty()) return hipSuccess;
  if (cfg.compute_dtype == MUON_BF16) return ns_iterations_bf16(jobs, cfg, s);
  for (const NsJob& J : jobs) {
    hipError_t e = ns_iterations_f32(J.g, J.nb, cfg, J.ws, J.L, J.out, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// The norm finalize of the matrices of one workspace region.
NormParams norm_params(const Layout& L, float eps, char* ws) {
  NormParams np{};
  np.partial = (const float*)(ws + L.partial);
  np.tiles = L.tiles;
  np.eps = eps;
  np.rs = (float*)(ws + L.rs);
  return np;
}

// Load-kernel and norm-finalize work of one pass, gathered over every group
// and launched a few problems at a time.
struct StageLaunches {
  struct Prep { PrepParams pp; int nb; double bytes; };
  std::vector<Prep> preps;
  std::vector<std::pair<NormParams, int>> norms;
};

hipError_t launch_stage(const StageLaunches& st, hipStream_t s) {
  for (size_t i0 = 0; i0 < st.preps.size();) {
    PrepGroup g{};
    double bytes = 0;
    size_t i = i0;
    for (; i < st.preps.size() && g.nprob < kMaxPrep && g.zstart[g.nprob] + st.preps[i].nb <= 65535; ++i) {
      g.prob[g.nprob] = st.preps[i].pp;
      g.zstart[g.nprob + 1] = g.zstart[g.nprob] + st.preps[i].nb;
      ++g.nprob;
      bytes += st.preps[i].bytes;
    }
    const hipError_t e = run(MUON_K_PREP, 0, bytes, s, [&]() { return launch_prep_group(g, s); });
    if (e != hipSuccess) return e;
    i0 = i;
  }
  for (size_t i0 = 0; i0 < st.norms.size(); i0 += kMaxNorm) {
    NormGroup g{};
    double bytes = 0;
    for (size_t i = i0; i < st.norms.size() && i < i0 + kMaxNorm; ++i) {
      g.prob[g.nprob] = st.norms[i].first;
      g.start[g.nprob + 1] = g.start[g.nprob] + st.norms[i].second;
      ++g.nprob;
      bytes += (double)st.norms[i].second * st.norms[i].first.tiles * 4;
    }
    const hipError_t e = run(MUON_K_NORM, 0, bytes, s, [&]() { return launch_norm_group(g, s); });
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Matrices (or parameters) processed per pass; the grid's z extent bounds it.
int64_t chunk_of(int64_t n, int64_t max_batch) {
  int64_t c = max_batch > 0 && max_batch < n ? max_batch : n;
  return c < 65535 ? c : 65535;
}


// Byte span [lo, hi) reached by a strided batch of matrices.
struct Span { uintptr_t lo, hi; };
Span span_of(const void* p, int32_t dt, int64_t bs, int64_t rs, int64_t n, int64_t rows, int64_t cols) {
  const uintptr_t lo = (uintptr_t)p;
  return {lo, lo + (uintptr_t)(((n - 1) * bs + (rows - 1) * rs + cols) * (int64_t)esize(dt))};
}

bool ns_empty(const muon_ns_problem& q) { return q.n == 0 || q.rows == 0 || q.cols == 0; }

// The argument checks of one Newton-Schulz problem (the config is checked by
// the caller); an empty problem passes once its sizes and dtypes do.
int check_ns_problem(const muon_ns_problem& q) {
  int rc = check_dims(q.n, q.rows, q.cols);
  if (rc) return rc;
  if (!dtype_ok(q.x_dtype) || !dtype_ok(q.y_dtype)) return fail(MUON_ERR_UNSUPPORTED, "x/y dtype must be MUON_F32 or MUON_BF16");
  if (ns_empty(q)) return MUON_OK;
  if (!q.x || !q.y) return fail(MUON_ERR_INVALID_ARG, "x or y is NULL");
  if (q.x_row_stride < q.cols || q.y_row_stride < q.cols) return fail(MUON_ERR_INVALID_ARG, "row stride smaller than cols");
  if (q.x_batch_stride < 0 || q.y_batch_stride < 0) return fail(MUON_ERR_INVALID_ARG, "negative batch stride");
  if (q.n > 1 && q.y_batch_stride < (q.rows - 1) * q.y_row_stride + q.cols)
    return fail(MUON_ERR_INVALID_ARG, "output batches overlap");
  if (((uintptr_t)q.x % esize(q.x_dtype)) || ((uintptr_t)q.y % esize(q.y_dtype)))
    return fail(MUON_ERR_INVALID_ARG, "x/y not aligned to their element size");
  // In place needs equal layouts, so that the final store of a matrix only
  // overwrites that matrix's own (already read) input.  Any other overlap of
  // the output with the input is refused: when the work is cut into passes
  // (max_batch, or more than 65535 matrices) an earlier pass would overwrite
  // inputs of a later one.
  if (q.y == q.x) {
    if (q.x_dtype != q.y_dtype || q.x_batch_stride != q.y_batch_stride || q.x_row_stride != q.y_row_stride)
      return fail(MUON_ERR_INVALID_ARG, "in-place call needs identical dtype and strides");
  } else {
    const Span xs = span_of(q.x, q.x_dtype, q.x_batch_stride, q.x_row_stride, q.n, q.rows, q.cols);
    const Span ys = span_of(q.y, q.y_dtype, q.y_batch_stride, q.y_row_stride, q.n, q.rows, q.cols);
    if (xs.lo < ys.hi && ys.lo < xs.hi) return fail(MUON_ERR_INVALID_ARG, "output overlaps the input (only y == x is allowed)");
  }
  return MUON_OK;
}

// Workspace bytes of one problem: its region holds one pass of at most
// max_batch matrices.
size_t ns_region_bytes(const muon_ns_problem& q, const muon_ns_config& cfg) {
  if (ns_empty(q)) return 0;
  return make_layout(make_geom(q.rows, q.cols, cfg.compute_dtype), chunk_of(q.n, cfg.max_batch)).total;
}

int check_workspace(const void* ws, size_t have, size_t need) {
  if (!ws) return fail(MUON_ERR_INVALID_ARG, "workspace is NULL");
  if ((uintptr_t)ws & 255) return fail(MUON_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (have < need) return fail(MUON_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, have);
  return MUON_OK;
}

// No problem's output span meets another problem's input or output span.
int check_disjoint(const muon_ns_problem* q, int64_t nq) {
  auto meet = [](Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; };
  for (int64_t i = 0; i < nq; ++i) {
    if (ns_empty(q[i])) continue;
    const Span yi = span_of(q[i].y, q[i].y_dtype, q[i].y_batch_stride, q[i].y_row_stride, q[i].n, q[i].rows, q[i].cols);
    for (int64_t j = 0; j < nq; ++j) {
      if (j == i || ns_empty(q[j])) continue;
      const Span xj = span_of(q[j].x, q[j].x_dtype, q[j].x_batch_stride, q[j].x_row_stride, q[j].n, q[j].rows, q[j].cols);
      const Span yj = span_of(q[j].y, q[j].y_dtype, q[j].y_batch_stride, q[j].y_row_stride, q[j].n, q[j].rows, q[j].cols);
      if (meet(yi, xj) || meet(yi, yj))
        return fail(MUON_ERR_INVALID_ARG, "output of problem %lld overlaps problem %lld", (long long)i, (long long)j);
    }
  }
  return MUON_OK;
}

// Newton-Schulz of every (checked, non-empty or empty) problem.  Problem i
// owns a region of ns_region_bytes at the running offset in ws and is cut
// into passes of chunk_of(n_i, max_batch) matrices; pass k loads and
// normalizes chunk k of every problem that has one, and one set of
// iteration launches then covers them all.
hipError_t ns_run_passes(const muon_ns_problem* q, int64_t nq, const muon_ns_config& cfg, char* ws, hipStream_t s) {
  struct Live { const muon_ns_problem* q; Geom g; int64_t chunk; Layout L; char* ws; };
  std::vector<Live> live;
  size_t off = 0;
  int64_t passes = 0;
  for (int64_t i = 0; i < nq; ++i) {
    if (ns_empty(q[i])) continue;
    Live v{&q[i], make_geom(q[i].rows, q[i].cols, cfg.compute_dtype), chunk_of(q[i].n, cfg.max_batch), {}, nullptr};
    v.L = make_layout(v.g, v.chunk);
    v.ws = ws + off;
    off += v.L.total;
    passes = std::max(passes, (q[i].n + v.chunk - 1) / v.chunk);
    live.push_back(v);
  }
  for (int64_t k = 0; k < passes; ++k) {
    std::vector<NsJob> jobs;
    StageLaunches st;
    for (const Live& v : live) {
      const muon_ns_problem& p = *v.q;
      const int64_t c0 = k * v.chunk;
      if (c0 >= p.n) continue;
      const int64_t nb = std::min(v.chunk, p.n - c0);
      const size_t xe = esize(p.x_dtype), ye = esize(p.y_dtype);
      PrepParams pp{};
      pp.mode = 0;
      pp.tall = v.g.tall;
      pp.rows = (int)p.rows; pp.cols = (int)p.cols;
      pp.mp = (int)v.g.mp; pp.np = (int)v.g.np;
      pp.heads = 1;
      pp.src_dtype = p.x_dtype;
      pp.x_bf16 = v.g.bf;
      pp.x = (const char*)p.x + c0 * p.x_batch_stride * xe;
      pp.x_bs = p.x_batch_stride; pp.x_rs = p.x_row_stride;
      pp.X = v.ws + v.L.X0; pp.X_bs = v.g.mp * v.g.np;
      pp.partial = (float*)(v.ws + v.L.partial);
      // A bf16 input already laid out as the iterate (not transposed, no
      // padding, rows np apart, 16-byte aligned) and not overwritten by the
      // output is read in place by the first iteration: the load kernel then
      // computes the norm partials only.
      const bool direct = v.g.bf && p.x_dtype == MUON_BF16 && !v.g.tall && v.g.mp == p.rows && v.g.np == p.cols &&
                          p.x_row_stride == p.cols && (p.x_batch_stride % 8) == 0 && ((uintptr_t)p.x & 15) == 0 &&
                          p.y != p.x;
      pp.no_x = direct ? 1 : 0;
      // A 128-row matrix's norm comes from its first Gram (the fused kernel's
      // chunk sums of squares), so an input read in place needs no load launch.
      if (!(direct && path128(v.g)))
        st.preps.push_back({pp, (int)nb, (double)nb * p.rows * p.cols * (xe + (direct ? 0 : (v.g.bf ? 2 : 4)))});
      if (!path128(v.g)) st.norms.push_back({norm_params(v.L, cfg.eps, v.ws), (int)nb});
      FinalOut out{(char*)p.y + c0 * p.y_batch_stride * ye, p.y_dtype, p.y_row_stride, p.y_batch_stride};
      NsJob job{v.g, nb, v.ws, v.L, out};
      if (direct) {
        job.x0 = pp.x;
        job.x0_bs = p.x_batch_stride;
      }
      jobs.push_back(job);
    }
    // The load kernel and the norm finalize for every problem of the pass,
    // several problems per launch.
    hipError_t e = launch_stage(st, s);
    if (e != hipSuccess) return e;
    e = ns_iterations(jobs, cfg, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

int ns_run(const muon_ns_problem* q, int64_t nq, const muon_ns_config& cfg, char* ws, hipStream_t s) {
  hipError_t e = ns_run_passes(q, nq, cfg, ws, s);
  if (e != hipSuccess) return hip_fail(e, "Newton-Schulz kernels");
  return ok();
}

// ---- the workspace of muon_ns_batched_noalloc --------------------------------
// A fixed array in the library's device code: every GPU the library runs on
// holds its own copy until the process ends.  On the host, `scratch` names a
// stand-in, not a device address; the address of each GPU's copy comes from
// hipGetSymbolAddress with that GPU current, looked up on the first call on
// that GPU and kept per device ordinal.
static __device__ __align__(256) unsigned char scratch[MUON_NS_NOALLOC_WORKSPACE_BYTES];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;

// Device address of the scratch array on the device that runs `s` (the
// current device for the null stream).
int scratch_for(hipStream_t s, char** out) {
  int dev = -1;
  hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "device of the stream");
  if (dev < 0) return fail(MUON_ERR_HIP, "no device for the stream");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "hipSetDevice");
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the scratch array");
    if (!p || ((uintptr_t)p & 255)) return fail(MUON_ERR_HIP, "scratch array address %p is null or not 256-byte aligned", p);
    g_scratch_ptr[dev] = p;
  }
  *out = (char*)g_scratch_ptr[dev];
  return MUON_OK;
}

}  // namespace

// =============================================================================
extern "C" {

void muon_ns_default_config(muon_ns_config* cfg) {
  if (!cfg) return;
  std::memset(cfg, 0, sizeof *cfg);
  cfg->steps = 5;
  cfg->a = 3.4445f;
  cfg->b = -4.7750f;
  cfg->c = 2.0315f;
  cfg->eps = 1e-7f;
  cfg->compute_dtype = MUON_BF16;
  cfg->max_batch = 0;
  for (int k = 0; k < MUON_NS_MAX_STEPS; ++k) {
    cfg->coeffs[k][0] = cfg->a;
    cfg->coeffs[k][1] = cfg->b;
    cfg->coeffs[k][2] = cfg->c;
  }
}

void muon_default_hparams(muon_hparams* hp) {
  if (!hp) return;
  std::memset(hp, 0, sizeof *hp);
  hp->lr = 0.05f;
  hp->momentum = 0.95f;
  hp->nesterov = 1;
  hp->weight_decay = 0.f;
  hp->extra_scale = 1.f;
  hp->normuon = 0;
  hp->beta2 = 0.95f;
  hp->norm_eps = 1e-8f;
  muon_ns_default_config(&hp->ns);
}

int muon_abi_version(void) { return MUON_ABI_VERSION; }
int muon_state_layout_version(void) { return MUON_STATE_LAYOUT_VERSION; }

const char* muon_status_string(int status) {
  switch (status) {
    case MUON_OK: return "ok";
    case MUON_ERR_INVALID_ARG: return "invalid argument";
    case MUON_ERR_UNSUPPORTED: return "unsupported";
    case MUON_ERR_WORKSPACE: return "workspace too small";
    case MUON_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* muon_last_error(void) { return g_err.c_str(); }

int muon_ns_workspace_bytes(int64_t n, int64_t rows, int64_t cols, const muon_ns_config* cfg, size_t* bytes) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if ((rc = check_dims(n, rows, cols))) return rc;
  if (!bytes) return fail(MUON_ERR_INVALID_ARG, "bytes is NULL");
  if (n == 0 || rows == 0 || cols == 0) { *bytes = 0; return ok(); }
  const Geom g = make_geom(rows, cols, cfg->compute_dtype);
  *bytes = make_layout(g, chunk_of(n, cfg->max_batch)).total;
  return ok();
}

int muon_ns_batched(const void* x, int32_t x_dtype, int64_t x_batch_stride, int64_t x_row_stride,
                    void* y, int32_t y_dtype, int64_t y_batch_stride, int64_t y_row_stride,
                    int64_t n, int64_t rows, int64_t cols, const muon_ns_config* cfg,
                    void* workspace, size_t workspace_bytes, void* stream) {
  const muon_ns_problem q{x, x_dtype, x_batch_stride, x_row_stride, y, y_dtype, y_batch_stride, y_row_stride,
                          n, rows, cols};
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if ((rc = check_ns_problem(q))) return rc;
  if (ns_empty(q)) return ok();
  const size_t need = make_layout(make_geom(rows, cols, cfg->compute_dtype), chunk_of(n, cfg->max_batch)).total;
  if ((rc = check_workspace(workspace, workspace_bytes, need))) return rc;
  return ns_run(&q, 1, *cfg, (char*)workspace, (hipStream_t)stream);
}

int muon_ns_batched_noalloc(const void* x, int32_t x_dtype, int64_t x_batch_stride, int64_t x_row_stride,
                            void* y, int32_t y_dtype, int64_t y_batch_stride, int64_t y_row_stride,
                            int64_t n, int64_t rows, int64_t cols, const muon_ns_config* cfg, void* stream) {
  const muon_ns_problem q{x, x_dtype, x_batch_stride, x_row_stride, y, y_dtype, y_batch_stride, y_row_stride,
                          n, rows, cols};
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if ((rc = check_ns_problem(q))) return rc;
  if (ns_empty(q)) return ok();
  const size_t need = make_layout(make_geom(rows, cols, cfg->compute_dtype), chunk_of(n, cfg->max_batch)).total;
  if (need > MUON_NS_NOALLOC_WORKSPACE_BYTES)
    return fail(MUON_ERR_WORKSPACE,
                "this problem needs %zu bytes of workspace, above the %zu-byte scratch array of "
                "muon_ns_batched_noalloc; set cfg->max_batch lower or call muon_ns_batched with a workspace",
                need, (size_t)MUON_NS_NOALLOC_WORKSPACE_BYTES);
  char* ws = nullptr;
  if ((rc = scratch_for((hipStream_t)stream, &ws))) return rc;
  return ns_run(&q, 1, *cfg, ws, (hipStream_t)stream);
}

int muon_ns_groups_workspace_bytes(const muon_ns_problem* probs, int64_t nprob, const muon_ns_config* cfg,
                                   size_t* bytes) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (!bytes) return fail(MUON_ERR_INVALID_ARG, "bytes is NULL");
  if (nprob < 0 || nprob > 4096) return fail(MUON_ERR_INVALID_ARG, "nprob must be in 0..4096");
  if (nprob > 0 && !probs) return fail(MUON_ERR_INVALID_ARG, "probs is NULL");
  size_t total = 0;
  for (int64_t i = 0; i < nprob; ++i) {
    if ((rc = check_dims(probs[i].n, probs[i].rows, probs[i].cols))) return rc;
    total += ns_region_bytes(probs[i], *cfg);
  }
  *bytes = total;
  return ok();
}

int muon_ns_groups(const muon_ns_problem* probs, int64_t nprob, const muon_ns_config* cfg,
                   void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (nprob < 0 || nprob > 4096) return fail(MUON_ERR_INVALID_ARG, "nprob must be in 0..4096");
  if (nprob > 0 && !probs) return fail(MUON_ERR_INVALID_ARG, "probs is NULL");
  size_t need = 0;
  for (int64_t i = 0; i < nprob; ++i) {
    if ((rc = check_ns_problem(probs[i]))) return fail(rc, "problem %lld: %s", (long long)i, g_err.c_str());
    need += ns_region_bytes(probs[i], *cfg);
  }
  if ((rc = check_disjoint(probs, nprob))) return rc;
  if (need == 0) return ok();
  if ((rc = check_workspace(workspace, workspace_bytes, need))) return rc;
  return ns_run(probs, nprob, *cfg, (char*)workspace, (hipStream_t)stream);
}

int normuon_workspace_bytes(int64_t n, int64_t rows, int64_t cols, size_t* bytes) {
  int rc = check_dims(n, rows, cols);
  if (rc) return rc;
  if (!bytes) return fail(MUON_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = align256((size_t)n * rows * 4) * 3 + align256((size_t)n * 4);
  return ok();
}

int normuon_normalize(void* o, int32_t o_dtype, int64_t o_batch_stride, int64_t o_row_stride,
                      int64_t n, int64_t rows, int64_t cols,
                      float* v, int64_t v_batch_stride, float beta2, float eps,
                      void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_dims(n, rows, cols);
  if (rc) return rc;
  if (!dtype_ok(o_dtype)) return fail(MUON_ERR_UNSUPPORTED, "o dtype must be MUON_F32 or MUON_BF16");
  if (!(beta2 >= 0.f && beta2 <= 1.f) || !(eps >= 0.f) || !std::isfinite(eps)) return fail(MUON_ERR_INVALID_ARG, "beta2 must be in [0,1] and eps >= 0");
  if (n == 0 || rows == 0 || cols == 0) return ok();
  if (!o || !v) return fail(MUON_ERR_INVALID_ARG, "o or v is NULL");
  if (o_row_stride < cols || o_batch_stride < 0 || v_batch_stride < 0) return fail(MUON_ERR_INVALID_ARG, "bad strides");
  if (n > 1 && (v_batch_stride < rows || o_batch_stride < (rows - 1) * o_row_stride + cols)) return fail(MUON_ERR_INVALID_ARG, "batches overlap");
  if (((uintptr_t)o % esize(o_dtype)) || ((uintptr_t)v & 3)) return fail(MUON_ERR_INVALID_ARG, "o/v not aligned to their element size");
  size_t need = 0;
  normuon_workspace_bytes(n, rows, cols, &need);
  if (!workspace) return fail(MUON_ERR_INVALID_ARG, "workspace is NULL");
  if ((uintptr_t)workspace & 255) return fail(MUON_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (workspace_bytes < need) return fail(MUON_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
  if (n > 65535) return fail(MUON_ERR_INVALID_ARG, "n above 65535");
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const size_t per = align256((size_t)n * rows * 4);
  float* d = (float*)ws;
  float* ms = (float*)(ws + per);
  float* q = (float*)(ws + 2 * per);
  float* rho = (float*)(ws + 3 * per);
  const double es = (double)esize(o_dtype);
  RowStatParams rp{};
  rp.O = o; rp.o_dtype = o_dtype; rp.o_bs = o_batch_stride; rp.o_rs = o_row_stride;
  rp.rows = (int)rows; rp.cols = (int)cols;
  rp.v_base = v; rp.v_bs = v_batch_stride;
  rp.beta2 = beta2; rp.eps = eps;
  rp.d = d; rp.ms = ms; rp.q = q;
  hipError_t e = run(MUON_K_ROWSTAT, 0, (double)n * rows * (cols * es + 8), s, [&]() { return launch_rowstat(rp, (int)n, s); });
  if (e != hipSuccess) return hip_fail(e, "row statistics kernel");
  RhoParams hp{ms, q, (int)rows, rho};
  e = run(MUON_K_RHO, 0, (double)n * rows * 8, s, [&]() { return launch_rho(hp, (int)n, s); });
  if (e != hipSuccess) return hip_fail(e, "rho kernel");
  ApplyParams ap{};
  ap.mode = 1;
  ap.O = o; ap.o_dtype = o_dtype; ap.o_bs = o_batch_stride; ap.o_rs = o_row_stride;
  ap.rows = (int)rows; ap.cols = (int)cols;
  ap.d = d; ap.rho = rho;
  e = run(MUON_K_APPLY, 0, (double)n * rows * cols * 2 * es, s, [&]() { return launch_apply(ap, (int)n, s); });
  if (e != hipSuccess) return hip_fail(e, "scale kernel");
  return ok();
}

// Sizes, heads and row splits of one group.
static int check_group_shape(const muon_group* g) {
  int rc = check_dims(g->n, g->rows, g->cols);
  if (rc) return rc;
  if (g->heads < 1) return fail(MUON_ERR_INVALID_ARG, "heads must be >= 1");
  if (g->rows % g->heads) return fail(MUON_ERR_INVALID_ARG, "rows (%lld) not divisible by heads (%lld)", (long long)g->rows, (long long)g->heads);
  if (g->nsplit < 0 || g->nsplit > 4096) return fail(MUON_ERR_INVALID_ARG, "nsplit must be in 0..4096");
  if (g->nsplit > 0) {
    if (!g->split_rows) return fail(MUON_ERR_INVALID_ARG, "split_rows is NULL");
    if (g->heads != 1) return fail(MUON_ERR_INVALID_ARG, "row splits need heads == 1");
    int64_t sum = 0;
    for (int64_t k = 0; k < g->nsplit; ++k) {
      if (g->split_rows[k] <= 0) return fail(MUON_ERR_INVALID_ARG, "split_rows[%lld] must be > 0", (long long)k);
      sum += g->split_rows[k];
    }
    if (sum != g->rows) return fail(MUON_ERR_INVALID_ARG, "split_rows sum to %lld, rows is %lld", (long long)sum, (long long)g->rows);
  }
  return MUON_OK;
}

static int check_group(const muon_group* g, const muon_hparams* hp) {
  if (!g || !hp) return fail(MUON_ERR_INVALID_ARG, "group or hparams is NULL");
  int rc = check_cfg(&hp->ns);
  if (rc) return rc;
  if ((rc = check_group_shape(g))) return rc;
  if (!dtype_ok(g->grad_dtype) || !dtype_ok(g->mom_dtype)) return fail(MUON_ERR_UNSUPPORTED, "grad/mom dtype must be MUON_F32 or MUON_BF16");
  if (g->model_dtype != -1 && g->model_dtype != MUON_BF16) return fail(MUON_ERR_UNSUPPORTED, "model_dtype must be MUON_BF16 or -1");
  if (g->reserved != 0) return fail(MUON_ERR_INVALID_ARG, "reserved field must be 0");
  if (!std::isfinite(hp->lr) || !std::isfinite(hp->momentum) || !std::isfinite(hp->weight_decay) || !std::isfinite(hp->extra_scale))
    return fail(MUON_ERR_INVALID_ARG, "lr, momentum, weight_decay and extra_scale must be finite");
  if (hp->normuon && (!(hp->beta2 >= 0.f && hp->beta2 <= 1.f) || !(hp->norm_eps >= 0.f) || !std::isfinite(hp->norm_eps)))
    return fail(MUON_ERR_INVALID_ARG, "beta2 must be in [0,1] and norm_eps >= 0");
  if (hp->fan_out < 0 || hp->fan_in < 0) return fail(MUON_ERR_INVALID_ARG, "fan_out/fan_in must be >= 0");
  if (g->n == 0 || g->rows == 0 || g->cols == 0) return MUON_OK;
  if (!g->w_master || !g->grad || !g->mom) return fail(MUON_ERR_INVALID_ARG, "w_master, grad and mom arrays are required");
  if (hp->normuon && !g->var) return fail(MUON_ERR_INVALID_ARG, "var array is required with normuon");
  if (g->model_dtype == MUON_BF16 && !g->w_model) return fail(MUON_ERR_INVALID_ARG, "w_model array is required for a bf16 model copy");
  for (int64_t i = 0; i < g->n; ++i) {
    if (!g->w_master[i] || !g->grad[i] || !g->mom[i]) return fail(MUON_ERR_INVALID_ARG, "NULL tensor pointer for parameter %lld", (long long)i);
    if (!aligned16(g->w_master[i]) || !aligned16(g->grad[i]) || !aligned16(g->mom[i]))
      return fail(MUON_ERR_INVALID_ARG, "parameter %lld: tensors must be 16-byte aligned", (long long)i);
    if (hp->normuon && (!g->var[i] || ((uintptr_t)g->var[i] & 3))) return fail(MUON_ERR_INVALID_ARG, "bad var pointer for parameter %lld", (long long)i);
    if (g->model_dtype == MUON_BF16 && (!g->w_model[i] || !aligned16(g->w_model[i])))
      return fail(MUON_ERR_INVALID_ARG, "bad w_model pointer for parameter %lld", (long long)i);
  }
  return MUON_OK;
}

}  // extern "C"

namespace {

// One row block of a group: rows [r0, r0 + h) of every parameter, split into
// H heads of hb rows for Newton-Schulz.
struct Block {
  int64_t r0, h, H, hb;
  Geom ge;
  Layout L;
  size_t off;              // of the block's region within the group's region
};

// Where each group of a step call lives in the workspace and how it is cut
// into passes of at most pc parameters.
struct GroupPlan {
  const muon_group* g;
  bool live;               // non-empty group
  bool split;              // row blocks: O is assembled in its own buffer
  int64_t pc, pelems;
  std::vector<Block> blocks;
  size_t obuf_off;         // split groups: O [pc][rows][cols]
  size_t nm_d, nm_ms, nm_q, nm_rho;  // NorMuon scratch: [pc][rows] x 3, [pc]
  size_t offset;           // of the group's region in the workspace
};

int plan_groups(const muon_group* groups, int64_t ng, const muon_hparams* hp, std::vector<GroupPlan>& plans,
                size_t* total) {
  if (ng < 0 || ng > 4096) return fail(MUON_ERR_INVALID_ARG, "ngroups must be in 0..4096");
  if (ng > 0 && !groups) return fail(MUON_ERR_INVALID_ARG, "groups is NULL");
  if (!hp) return fail(MUON_ERR_INVALID_ARG, "hparams is NULL");
  plans.clear();
  size_t off = 0;
  for (int64_t i = 0; i < ng; ++i) {
    const muon_group* g = &groups[i];
    GroupPlan P{};
    P.g = g;
    P.live = !(g->n == 0 || g->rows == 0 || g->cols == 0);
    if (P.live) {
      P.split = g->nsplit > 0;
      P.pc = chunk_of(g->n, hp->ns.max_batch);
      P.pelems = g->rows * g->cols;
      size_t goff = 0;
      auto take = [&](size_t bytes) { size_t at = goff; goff = align256(goff + bytes); return at; };
      int64_t r0 = 0;
      const int64_t nb = P.split ? g->nsplit : 1;
      for (int64_t k = 0; k < nb; ++k) {
        Block B{};
        B.r0 = r0;
        B.h = P.split ? g->split_rows[k] : g->rows;
        B.H = P.split ? 1 : g->heads;
        B.hb = B.h / B.H;
        B.ge = make_geom(B.hb, g->cols, hp->ns.compute_dtype);
        B.L = make_layout(B.ge, P.pc * B.H);
        B.off = take(B.L.total);
        if (P.pc * B.H > 65535)
          return fail(MUON_ERR_INVALID_ARG, "group %lld: parameters x heads per pass above 65535; set ns.max_batch", (long long)i);
        P.blocks.push_back(B);
        r0 += B.h;
      }
      const size_t oes = hp->ns.compute_dtype == MUON_BF16 ? 2 : 4;
      if (P.split) P.obuf_off = take((size_t)P.pc * P.pelems * oes);
      if (hp->normuon) {
        P.nm_d = take((size_t)P.pc * g->rows * 4);
        P.nm_ms = take((size_t)P.pc * g->rows * 4);
        P.nm_q = take((size_t)P.pc * g->rows * 4);
        P.nm_rho = take((size_t)P.pc * 4);
      }
      P.offset = off;
      off = align256(off + goff);
    }
    plans.push_back(P);
  }
  *total = off;
  return MUON_OK;
}

int check_groups(const muon_group* groups, int64_t ng, const muon_hparams* hp) {
  if (ng < 0 || ng > 4096) return fail(MUON_ERR_INVALID_ARG, "ngroups must be in 0..4096");
  if (ng > 0 && !groups) return fail(MUON_ERR_INVALID_ARG, "groups is NULL");
  for (int64_t i = 0; i < ng; ++i) {
    int rc = check_group(&groups[i], hp);
    if (rc) return rc;
  }
  if (ng == 0 && !hp) return fail(MUON_ERR_INVALID_ARG, "hparams is NULL");
  return ng == 0 ? check_cfg(&hp->ns) : MUON_OK;
}

// Momentum (+ orientation and norm partials) and the norm finalize of one pass
// of one group, appended to `st` (launched once all groups are staged), and
// one Newton-Schulz job per row block, appended to `jobs`; *obuf receives
// where the pass's O [np_][rows][cols] is assembled.
int stage_group(const GroupPlan& P, const muon_hparams* hp, char* ws, int64_t c0, int64_t np_, StageLaunches& st,
                std::vector<NsJob>& jobs, void** obuf) {
  const muon_group* g = P.g;
  const double ges = (double)esize(g->grad_dtype), mes = (double)esize(g->mom_dtype);
  for (const Block& B : P.blocks) {
    const Geom& ge = B.ge;
    const Layout& L = B.L;
    char* const bws = ws + B.off;
    const double oes = ge.bf ? 2 : 4;
    for (int64_t s0 = 0; s0 < np_; s0 += kMaxParams) {
      const int64_t k = (np_ - s0) < kMaxParams ? (np_ - s0) : kMaxParams;
      PrepParams pp{};
      pp.mode = 1;
      pp.tall = ge.tall;
      pp.rows = (int)B.hb; pp.cols = (int)g->cols;
      pp.mp = (int)ge.mp; pp.np = (int)ge.np;
      pp.heads = (int)B.H;
      pp.src_dtype = g->grad_dtype; pp.mom_dtype = g->mom_dtype;
      pp.x_bf16 = ge.bf;
      pp.mu = hp->momentum; pp.nesterov = hp->nesterov ? 1 : 0;
      pp.param_cols = g->cols;
      for (int64_t i = 0; i < k; ++i) {
        pp.grad[i] = (const char*)g->grad[c0 + s0 + i] + (size_t)(B.r0 * g->cols) * (size_t)ges;
        pp.mom[i] = (char*)g->mom[c0 + s0 + i] + (size_t)(B.r0 * g->cols) * (size_t)mes;
      }
      pp.X = bws + L.X0 + (size_t)(s0 * B.H) * ge.mp * ge.np * (size_t)oes;
      pp.X_bs = ge.mp * ge.np;
      pp.partial = (float*)(bws + L.partial) + s0 * B.H * L.tiles;
      st.preps.push_back({pp, (int)(k * B.H), (double)k * B.h * g->cols * (ges + 2 * mes + oes)});
    }
    if (!path128(ge)) st.norms.push_back({norm_params(L, hp->ns.eps, bws), (int)(np_ * B.H)});
    // The last update writes O in parameter orientation ([n][rows][cols],
    // contiguous): a whole group into the X buffer its last iteration does not
    // read, row blocks into the group's O buffer at their row offset.
    const int32_t odt = ge.bf ? MUON_BF16 : MUON_F32;
    FinalOut out;
    if (P.split) {
      out = FinalOut{ws + P.obuf_off + (size_t)(B.r0 * g->cols) * (size_t)oes, odt, g->cols, P.pelems};
      *obuf = ws + P.obuf_off;
    } else {
      void* o = bws + ((hp->ns.steps % 2) ? L.X1 : L.X0);
      out = FinalOut{o, odt, g->cols, B.hb * g->cols};
      *obuf = o;
    }
    jobs.push_back(NsJob{ge, np_ * B.H, bws, L, out});
  }
  return MUON_OK;
}

// NorMuon and weight-update work of one pass, gathered over every group and
// launched a few problems at a time (row statistics of every group, then
// their rho, then the updates).
struct FinishLaunches {
  struct RS { RowStatParams p; int nb; double bytes; };
  struct RH { RhoParams p; int nb; double bytes; };
  struct AP { ApplyParams p; int nb; double bytes; };
  std::vector<RS> rowstats;
  std::vector<RH> rhos;
  std::vector<AP> applies;
};

// Launches of one grouped kernel over `v`, at most `kmax` problems and 65535
// matrices per launch.
template <typename Group, typename Item, typename Launch>
hipError_t launch_grouped(const std::vector<Item>& v, int kmax, int cls, hipStream_t s, Launch&& launch) {
  for (size_t i0 = 0; i0 < v.size();) {
    Group g{};
    double bytes = 0;
    size_t i = i0;
    for (; i < v.size() && g.nprob < kmax && g.start[g.nprob] + v[i].nb <= 65535; ++i) {
      g.prob[g.nprob] = v[i].p;
      g.start[g.nprob + 1] = g.start[g.nprob] + v[i].nb;
      ++g.nprob;
      bytes += v[i].bytes;
    }
    const hipError_t e = run(cls, 0, bytes, s, [&]() { return launch(g, s); });
    if (e != hipSuccess) return e;
    i0 = i;
  }
  return hipSuccess;
}

hipError_t launch_finish(const FinishLaunches& f, hipStream_t s) {
  hipError_t e = launch_grouped<RowStatGroup>(f.rowstats, kMaxRowStat, MUON_K_ROWSTAT, s, launch_rowstat_group);
  if (e != hipSuccess) return e;
  if ((e = launch_grouped<RhoGroup>(f.rhos, kMaxRho, MUON_K_RHO, s, launch_rho_group)) != hipSuccess) return e;
  return launch_grouped<ApplyGroup>(f.applies, kMaxApply, MUON_K_APPLY, s, launch_apply_group);
}

// NorMuon (when on) and the weight update of one pass of one group, appended
// to `f`.
void finish_group(const GroupPlan& P, const muon_hparams* hp, char* ws, int64_t c0, int64_t np_, void* obuf,
                  FinishLaunches& f) {
  const muon_group* g = P.g;
  const bool nm = hp->normuon != 0;
  const int32_t odt = hp->ns.compute_dtype == MUON_BF16 ? MUON_BF16 : MUON_F32;
  const double oes = odt == MUON_BF16 ? 2 : 4;
  const int64_t fan_out = hp->fan_out ? hp->fan_out : g->rows;
  const int64_t fan_in = hp->fan_in ? hp->fan_in : g->cols;
  const double ratio = (double)fan_out / (double)fan_in;
  const float lr_eff = (float)((double)hp->lr * std::sqrt(ratio > 1.0 ? ratio : 1.0) * (double)hp->extra_scale);
  const float decay = (float)(1.0 - (double)hp->lr * (double)hp->weight_decay);
  if (nm) {
    for (int64_t s0 = 0; s0 < np_; s0 += kMaxParams) {
      const int64_t k = (np_ - s0) < kMaxParams ? (np_ - s0) : kMaxParams;
      RowStatParams r2{};
      r2.O = (char*)obuf + (size_t)s0 * P.pelems * (size_t)oes;
      r2.o_dtype = odt; r2.o_bs = P.pelems; r2.o_rs = g->cols;
      r2.rows = (int)g->rows; r2.cols = (int)g->cols;
      r2.beta2 = hp->beta2; r2.eps = hp->norm_eps;
      r2.d = (float*)(ws + P.nm_d) + s0 * g->rows;
      r2.ms = (float*)(ws + P.nm_ms) + s0 * g->rows;
      r2.q = (float*)(ws + P.nm_q) + s0 * g->rows;
      for (int64_t i = 0; i < k; ++i) r2.v_tab[i] = g->var[c0 + s0 + i];
      f.rowstats.push_back({r2, (int)k, (double)k * (P.pelems * oes + g->rows * 8)});
    }
    RhoParams hpm{(float*)(ws + P.nm_ms), (float*)(ws + P.nm_q), (int)g->rows, (float*)(ws + P.nm_rho)};
    f.rhos.push_back({hpm, (int)np_, (double)np_ * g->rows * 8});
  }
  for (int64_t s0 = 0; s0 < np_; s0 += kMaxParams) {
    const int64_t k = (np_ - s0) < kMaxParams ? (np_ - s0) : kMaxParams;
    ApplyParams ap{};
    ap.mode = 0;
    ap.O = (char*)obuf + (size_t)s0 * P.pelems * (size_t)oes;
    ap.o_dtype = odt; ap.o_bs = P.pelems; ap.o_rs = g->cols;
    ap.rows = (int)g->rows; ap.cols = (int)g->cols;
    ap.d = nm ? (float*)(ws + P.nm_d) + s0 * g->rows : nullptr;
    ap.rho = nm ? (float*)(ws + P.nm_rho) + s0 : nullptr;
    ap.lr_eff = lr_eff; ap.decay = decay;
    ap.vec = (g->cols % 8) == 0 ? 1 : 0;
    for (int64_t i = 0; i < k; ++i) {
      ap.w[i] = g->w_master[c0 + s0 + i];
      ap.wm[i] = g->model_dtype == MUON_BF16 ? g->w_model[c0 + s0 + i] : nullptr;
    }
    const double wb = g->model_dtype == MUON_BF16 ? 10 : 8;
    f.applies.push_back({ap, (int)k, (double)k * P.pelems * (oes + wb)});
  }
}

}  // namespace

extern "C" {

int muon_step_groups_workspace_bytes(const muon_group* groups, int64_t ngroups, const muon_hparams* hp,
                                     size_t* bytes) {
  if (!bytes) return fail(MUON_ERR_INVALID_ARG, "bytes is NULL");
  if (!hp) return fail(MUON_ERR_INVALID_ARG, "hparams is NULL");
  int rc = check_cfg(&hp->ns);
  if (rc) return rc;
  if (ngroups < 0 || ngroups > 4096) return fail(MUON_ERR_INVALID_ARG, "ngroups must be in 0..4096");
  if (ngroups > 0 && !groups) return fail(MUON_ERR_INVALID_ARG, "groups is NULL");
  for (int64_t i = 0; i < ngroups; ++i) {
    if ((rc = check_group_shape(&groups[i]))) return rc;
  }
  std::vector<GroupPlan> plans;
  size_t total = 0;
  if ((rc = plan_groups(groups, ngroups, hp, plans, &total))) return rc;
  *bytes = total;
  return ok();
}

int muon_step_workspace_bytes(const muon_group* g, const muon_hparams* hp, size_t* bytes) {
  if (!g) return fail(MUON_ERR_INVALID_ARG, "group is NULL");
  return muon_step_groups_workspace_bytes(g, 1, hp, bytes);
}

int muon_step_groups(const muon_group* groups, int64_t ngroups, const muon_hparams* hp, void* workspace,
                     size_t workspace_bytes, void* stream) {
  int rc = check_groups(groups, ngroups, hp);
  if (rc) return rc;
  std::vector<GroupPlan> plans;
  size_t total = 0;
  if ((rc = plan_groups(groups, ngroups, hp, plans, &total))) return rc;
  if (total == 0) return ok();
  if (!workspace) return fail(MUON_ERR_INVALID_ARG, "workspace is NULL");
  if ((uintptr_t)workspace & 255) return fail(MUON_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (workspace_bytes < total) return fail(MUON_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", total, workspace_bytes);

  hipStream_t s = (hipStream_t)stream;
  int64_t passes = 0;
  for (const GroupPlan& P : plans)
    if (P.live) passes = std::max<int64_t>(passes, (P.g->n + P.pc - 1) / P.pc);
  // Pass c of every group runs together: its Newton-Schulz launches cover all
  // groups at once (a matrix's result does not depend on who shares a launch).
  for (int64_t c = 0; c < passes; ++c) {
    std::vector<NsJob> jobs;
    std::vector<std::pair<const GroupPlan*, void*>> who;
    StageLaunches st;
    for (const GroupPlan& P : plans) {
      if (!P.live || c * P.pc >= P.g->n) continue;
      const int64_t c0 = c * P.pc, np_ = std::min<int64_t>(P.pc, P.g->n - c0);
      void* obuf = nullptr;
      if ((rc = stage_group(P, hp, (char*)workspace + P.offset, c0, np_, st, jobs, &obuf))) return rc;
      who.emplace_back(&P, obuf);
    }
    hipError_t e = launch_stage(st, s);
    if (e != hipSuccess) return hip_fail(e, "momentum or norm kernel");
    e = ns_iterations(jobs, hp->ns, s);
    if (e != hipSuccess) return hip_fail(e, "Newton-Schulz kernels");
    FinishLaunches f;
    for (const auto& [pp, obuf] : who) {
      const GroupPlan& P = *pp;
      const int64_t c0 = c * P.pc, np_ = std::min<int64_t>(P.pc, P.g->n - c0);
      finish_group(P, hp, (char*)workspace + P.offset, c0, np_, obuf, f);
    }
    if ((e = launch_finish(f, s)) != hipSuccess) return hip_fail(e, "NorMuon or update kernels");
  }
  return ok();
}

int muon_step_group(const muon_group* g, const muon_hparams* hp, void* workspace, size_t workspace_bytes, void* stream) {
  if (!g || !hp) return fail(MUON_ERR_INVALID_ARG, "group or hparams is NULL");
  return muon_step_groups(g, 1, hp, workspace, workspace_bytes, stream);
}

// ---- launch timing ------------------------------------------------------------
int muon_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  return ok();
}

int muon_profile_classes(uint32_t mask) {
  if (mask >> MUON_K_COUNT) return fail(MUON_ERR_INVALID_ARG, "mask 0x%x names classes above %d", mask, MUON_K_COUNT - 1);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_mask = mask;
  return ok();
}

int muon_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  hipError_t e = drain_pending();
  for (auto& t : g_totals) t = ClassTotals{};
  if (e != hipSuccess) return hip_fail(e, "event synchronize");
  return ok();
}

int muon_profile_query(int kernel_class, int64_t* launches, double* total_ms, double* total_flop, double* total_bytes) {
  if (kernel_class < 0 || kernel_class >= MUON_K_COUNT) return fail(MUON_ERR_INVALID_ARG, "kernel class %d out of range", kernel_class);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  hipError_t e = drain_pending();
  if (e != hipSuccess) return hip_fail(e, "event synchronize");
  const ClassTotals& t = g_totals[kernel_class];
  if (launches) *launches = t.launches;
  if (total_ms) *total_ms = t.ms;
  if (total_flop) *total_flop = t.flop;
  if (total_bytes) *total_bytes = t.bytes;
  return ok();
}

const char* muon_kernel_class_name(int kernel_class) {
  static const char* names[MUON_K_COUNT] = {"prep", "norm", "gram", "poly", "update", "rowstat", "rho", "apply"};
  return (kernel_class >= 0 && kernel_class < MUON_K_COUNT) ? names[kernel_class] : "unknown";
}

}  // extern "C"
