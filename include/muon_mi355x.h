/*
 * muon_mi355x.h -- C ABI of the gfx950 (MI355X) Muon / NorMuon step library.
 *
 * The library computes, on one GPU, the data-parallel hot path of one Muon
 * optimizer step: Nesterov momentum, Frobenius normalization, five quintic
 * Newton-Schulz iterations per matrix (batched over same-shape matrices,
 * megabatch slices or attention heads, never across them), the optional
 * NorMuon per-output-channel normalization with its norm-preserving rescale,
 * and the spectrally scaled weight update.
 *
 * Sources, by page title and section:
 *  [AutoTP]   "Muon under AutoTP orthogonalizes each shard, so the update
 *             depends on the TP degree" -- "Why it happens" (normalize by the
 *             matrix norm, iterate on X X^T), "What could be done" option 3
 *             (per-head Newton-Schulz over row blocks).
 *  [LSMuon]   "core.optimizer.layer_sharded_muon" -- class LayerShardedMuon
 *             (momentum 0.95, nesterov, quintic coefficients, 5 steps,
 *             spectral scale mode, extra_scale_factor, ns_batch_size,
 *             use_syrk: A = X X^T and B = b A + c A^2 computed one triangle
 *             only), _validate_ns_config (one error, raised up front, no
 *             silent kernel switch), _run_ns (same-shape batching capped by
 *             ns_batch_size), _apply_update (fused multiply-add, one rounding
 *             on store).
 *  [ConvFix]  "Fix convolution flattening in megabatches and NorMuon
 *             normalization" -- "Problem and fix" (megabatch [N, out,
 *             prod(rest)], fan_out = out, fan_in = prod(rest)), "What it does"
 *             (one NorMuon variance per output channel on the flattened
 *             matrix), "Compatibility" (norm-preserving rescale, empty shards).
 *
 * Conventions shared by every entry point
 *  - Every function returns an int status (MUON_OK or a negative MUON_ERR_*).
 *    No C++ exception crosses the ABI.  muon_last_error() gives a readable
 *    detail for the calling thread.
 *  - All arguments are validated before anything is enqueued: a call that
 *    fails leaves every buffer untouched.
 *  - Device pointers are plain HIP device pointers; every buffer (inputs,
 *    outputs, optimizer state, workspace) is owned and allocated by the
 *    caller.  The library never allocates device memory and never
 *    synchronizes: work is only enqueued on `stream` (a hipStream_t; NULL is
 *    the default stream) and the call returns after the enqueue.
 *  - Matrices are row-major with unit column stride; row and batch strides
 *    are in elements.  Matrix pointers of muon_ns_batched, muon_ns_groups
 *    and normuon_normalize need only be aligned to their element size; the
 *    per-parameter tensors of the step entry points must be 16-byte aligned
 *    (as every tensor allocation is).  Workspaces must be 256-byte aligned.
 *  - Zero-sized problems (n == 0, rows == 0 or cols == 0) are valid no-ops.
 *  - With launch timing off (the default) a call only launches kernels on
 *    `stream`: no allocation, no memset, no synchronization.  A call can
 *    therefore be captured into a HIP graph and replayed (the pointers and
 *    scalars are fixed at capture; the data they point to may change between
 *    replays).  Calls made while timing is on record events and must not be
 *    captured.
 *  - Size limits: rows and cols of one matrix at most 4194176 (2^22 - 128),
 *    and (rows rounded up to 128) x (cols rounded up to 128) below 2^31;
 *    larger matrices fail with MUON_ERR_INVALID_ARG.
 *  - Results for one matrix are bitwise independent of how many other
 *    matrices share the call and of its position in the batch.
 *  - Input range: the Frobenius normalization is folded into the first
 *    iteration, whose products accumulate the unnormalized input in fp32, and
 *    ||U||_F^2 is summed in fp32 (for a matrix whose short side pads to 128
 *    and whose Gram is split over column chunks, from U as rounded to bf16,
 *    by the first Gram).  Any input with ||U||_F below 1.8e19 (its
 *    square within the fp32 range) is supported, down to the smallest normal
 *    values; above it the output is NaN (never a silent zero).  Entries so
 *    small that their squares fall below the fp32 normal range leave
 *    ||U||_F far below eps, where the first iteration is a scaling by
 *    a / (||U||_F + eps) that does not square the entries.
 */
#ifndef MUON_MI355X_H
#define MUON_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MUON_ABI_VERSION 4
/* Layout of the caller-owned optimizer state: momentum has the parameter's
 * shape and dtype; the NorMuon variance is one fp32 value per output channel
 * ([ConvFix] "What it does"). */
#define MUON_STATE_LAYOUT_VERSION 1

/* ---- status codes ------------------------------------------------------ */
#define MUON_OK 0
#define MUON_ERR_INVALID_ARG (-1)  /* null pointer, bad size/stride, rows % heads != 0 ... */
#define MUON_ERR_UNSUPPORTED (-2)  /* a dtype combination or option the library does not run */
#define MUON_ERR_WORKSPACE (-3)    /* workspace_bytes smaller than the query returned */
#define MUON_ERR_HIP (-4)          /* a HIP runtime call or kernel launch failed */

/* ---- element types ----------------------------------------------------- */
#define MUON_F32 0
#define MUON_BF16 1

/* Newton-Schulz configuration ([LSMuon] LayerShardedMuon: coefficient_type
 * 'quintic', num_ns_steps 5; [AutoTP] "Why it happens").
 * One iteration on the oriented matrix X (m x n, m <= n):
 *     A = X X^T,   B = b A + c A A,   X <- a X + B X.
 * X0 = U / (||U||_F + eps).  A matrix with more rows than columns is
 * orthogonalized through its transpose and returned in its own orientation.
 * compute_dtype MUON_BF16: X, A, B are stored in bf16 between kernels and all
 * products accumulate in fp32 on bf16 MFMA; MUON_F32: everything is fp32
 * (fp32 MFMA).
 * schedule 1 runs iteration k with coeffs[k] instead of (a, b, c): a
 * per-iteration coefficient schedule (the Polar-Express-style schedules
 * [ConvFix] mentions; the pages give no values). */
#define MUON_NS_MAX_STEPS 64
typedef struct muon_ns_config {
  int32_t steps;          /* iterations, 1..MUON_NS_MAX_STEPS (5) */
  float a, b, c;          /* (3.4445, -4.7750, 2.0315) */
  float eps;              /* added to the Frobenius norm (1e-7) */
  int32_t compute_dtype;  /* MUON_BF16 or MUON_F32 */
  int32_t schedule;       /* 0: (a, b, c) in every iteration; 1: coeffs[k] in iteration k */
  int64_t max_batch;      /* most matrices (or parameters, for muon_step_group)
                             processed at once; 0 = all.  Bounds the workspace
                             like ns_batch_size ([LSMuon] _run_ns); results do
                             not depend on it. */
  float coeffs[MUON_NS_MAX_STEPS][3];  /* per-iteration (a, b, c); entries past `steps` unused */
} muon_ns_config;

/* Fills *cfg with steps 5, the quintic coefficients above (also in every row
 * of coeffs), schedule 0, eps 1e-7, compute_dtype MUON_BF16, max_batch 0. */
void muon_ns_default_config(muon_ns_config* cfg);

int muon_abi_version(void);
int muon_state_layout_version(void);
/* Static string for a status code. */
const char* muon_status_string(int status);
/* Detail of the last failed call on this thread ("" if none).  Valid until
 * the next call on the same thread. */
const char* muon_last_error(void);

/* ---- batched Newton-Schulz --------------------------------------------- */

/* Bytes of workspace muon_ns_batched needs for this problem.  Depends only on
 * (n or cfg->max_batch, rows, cols, cfg->compute_dtype). */
int muon_ns_workspace_bytes(int64_t n, int64_t rows, int64_t cols,
                            const muon_ns_config* cfg, size_t* bytes);

/* y[i] = NS5(x[i]) for i < n, each x[i] a rows x cols matrix.
 *
 * [AutoTP] "Why it happens"; [LSMuon] _run_ns (same-shape batch).
 * x      device, x_dtype (MUON_F32 / MUON_BF16); element (i, r, c) at
 *        x + i*x_batch_stride + r*x_row_stride + c.
 * y      device, y_dtype, same indexing with its own strides.  y may equal x
 *        (in place) when the dtypes and strides are equal; any other overlap
 *        of the bytes y reaches with the bytes x reaches is refused
 *        (MUON_ERR_INVALID_ARG).
 * Layouts covered by the strides:
 *   - a megabatch [N, out, F] of flattened parameters ([ConvFix] "Problem and
 *     fix"): batch stride out*F, row stride F;
 *   - per-head NS of one [H*hb, F] projection ([AutoTP] option 3): n = H,
 *     rows = hb, batch stride hb*row_stride.
 * Requires x_row_stride >= cols, y_row_stride >= cols, batch strides >= 0.
 * workspace: device, at least muon_ns_workspace_bytes() bytes, 256-byte
 *            aligned; its contents on entry do not matter.
 * Errors: MUON_ERR_INVALID_ARG (null pointers for a non-empty problem,
 * negative sizes, strides too small, overlapping x and y, steps outside
 * 1..64, schedule not 0 or 1, max_batch < 0, non-finite coefficients),
 * MUON_ERR_UNSUPPORTED (unknown dtype), MUON_ERR_WORKSPACE, MUON_ERR_HIP. */
int muon_ns_batched(const void* x, int32_t x_dtype, int64_t x_batch_stride, int64_t x_row_stride,
                    void* y, int32_t y_dtype, int64_t y_batch_stride, int64_t y_row_stride,
                    int64_t n, int64_t rows, int64_t cols, const muon_ns_config* cfg,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Size of the scratch array muon_ns_batched_noalloc works in: 256 MiB. */
#define MUON_NS_NOALLOC_WORKSPACE_BYTES ((size_t)256 << 20)

/* muon_ns_batched without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The call allocates nothing: its
 * workspace is a fixed array of MUON_NS_NOALLOC_WORKSPACE_BYTES in the
 * library's device code, one copy per GPU, held from the library's load on
 * that GPU until the process ends (the first call on a GPU looks up that
 * GPU's copy; no allocation and no stream work).  Its contents on entry do
 * not matter, and it keeps the last call's contents.
 * Every call on one GPU works in that GPU's one array: calls that can run
 * at the same time on one GPU (on different streams, or from threads whose
 * calls are not ordered on one stream) race and give wrong results.  Calls
 * enqueued on one stream are ordered and safe.
 * Arguments, results and errors as for muon_ns_batched, and
 * MUON_ERR_WORKSPACE when the problem's muon_ns_workspace_bytes exceeds
 * MUON_NS_NOALLOC_WORKSPACE_BYTES (nothing is enqueued; a smaller
 * cfg->max_batch lowers it). */
int muon_ns_batched_noalloc(const void* x, int32_t x_dtype, int64_t x_batch_stride, int64_t x_row_stride,
                            void* y, int32_t y_dtype, int64_t y_batch_stride, int64_t y_row_stride,
                            int64_t n, int64_t rows, int64_t cols, const muon_ns_config* cfg, void* stream);

/* One problem of muon_ns_groups: the arguments of one muon_ns_batched call. */
typedef struct muon_ns_problem {
  const void* x;
  int32_t x_dtype;
  int64_t x_batch_stride, x_row_stride;
  void* y;
  int32_t y_dtype;
  int64_t y_batch_stride, y_row_stride;
  int64_t n, rows, cols;
} muon_ns_problem;

/* Workspace bytes muon_ns_groups needs for these nprob problems: the sum of
 * muon_ns_workspace_bytes over them. */
int muon_ns_groups_workspace_bytes(const muon_ns_problem* probs, int64_t nprob,
                                   const muon_ns_config* cfg, size_t* bytes);

/* muon_ns_batched on each of nprob problems (host array, read during the call
 * only), with every Newton-Schulz launch shared by all of them: e.g. the
 * per-head views of q_proj [32, 128, 4096] and k_proj [8, 128, 4096] of one
 * layer ([AutoTP] option 3) in one launch per kernel instead of one per
 * projection ([LSMuon] _run_ns: the per-matrix loop is launch-bound, so
 * batch).  Each y[i] of each problem is bitwise what muon_ns_batched gives.
 * With cfg->max_batch > 0 each problem is cut into chunks of at most
 * max_batch matrices, and pass k covers chunk k of every problem.
 * A problem's output span (first to last byte its strides reach) must not
 * overlap another problem's input or output span.  nprob is in 0..4096.
 * workspace: device, at least muon_ns_groups_workspace_bytes() bytes, 256-byte
 *            aligned; its contents on entry do not matter.
 * Errors as for muon_ns_batched, checked for every problem before anything
 * is enqueued; MUON_ERR_INVALID_ARG also for overlapping problems. */
int muon_ns_groups(const muon_ns_problem* probs, int64_t nprob, const muon_ns_config* cfg,
                   void* workspace, size_t workspace_bytes, void* stream);

/* ---- NorMuon normalization --------------------------------------------- */

int normuon_workspace_bytes(int64_t n, int64_t rows, int64_t cols, size_t* bytes);

/* In place on o[i] (rows x cols, one flattened parameter or megabatch slice),
 * with v[i] its per-output-channel (per-row) fp32 variance state:
 *   ms_r = mean_j o_rj^2;  v_r <- beta2 v_r + (1 - beta2) ms_r;
 *   o_rj <- o_rj / (sqrt(v_r) + eps);  then o <- o * ||o_before||_F / ||o||_F
 * (o = 0 when the normalized matrix is zero).
 * [ConvFix] "Adjacent bug", "What it does" (one variance per output channel,
 * rows of the [out, prod(rest)] view), "Compatibility" (norm-preserving
 * rescale).  The variance is the uncentered mean of squares kept as an
 * exponential moving average without bias correction.
 * o: device, o_dtype, element (i, r, c) at o + i*o_batch_stride + r*o_row_stride + c.
 * v: device fp32, element (i, r) at v + i*v_batch_stride + r.
 * Errors as for muon_ns_batched. */
int normuon_normalize(void* o, int32_t o_dtype, int64_t o_batch_stride, int64_t o_row_stride,
                      int64_t n, int64_t rows, int64_t cols,
                      float* v, int64_t v_batch_stride, float beta2, float eps,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ---- one optimizer step for a group of same-shape parameters ------------ */

/* n parameters of identical shape [rows = out, cols = prod(rest)], each given
 * by host arrays of n device pointers (read during the call only).  Each
 * parameter's tensors are contiguous (row stride = cols). */
typedef struct muon_group {
  int64_t n;
  int64_t rows;            /* out (fan_out) */
  int64_t cols;            /* prod(rest) (fan_in) */
  int64_t heads;           /* >= 1; NS runs on each of the `heads` row blocks */
  int32_t grad_dtype;      /* MUON_BF16 or MUON_F32 */
  int32_t mom_dtype;       /* MUON_BF16 or MUON_F32 */
  int32_t model_dtype;     /* MUON_BF16 for a bf16 model copy, or -1 for none */
  int32_t reserved;        /* must be 0 */
  float* const* w_master;  /* n x fp32 [rows][cols], updated in place */
  void* const* w_model;    /* n x bf16 [rows][cols] written = RNE(w_master); NULL if model_dtype == -1 */
  const void* const* grad; /* n x grad_dtype [rows][cols] */
  void* const* mom;        /* n x mom_dtype [rows][cols], updated in place */
  float* const* var;       /* n x fp32 [rows] NorMuon variance, updated in place; NULL without NorMuon */
  int64_t nsplit;          /* 0, or the number of row blocks (heads must then be 1) */
  const int64_t* split_rows; /* nsplit block heights (host, read during the call), > 0, summing to rows:
                                NS runs on each block [r0, r0 + h) of every parameter (a fused
                                q/k/v weight split on its rows); momentum, NorMuon and the update
                                act on the whole parameter */
} muon_group;

/* Step hyper-parameters.  [LSMuon] LayerShardedMuon: lr, momentum,
 * nesterov, weight_decay with decoupled decay, extra_scale_factor,
 * scale_mode 'spectral'; [ConvFix] "Problem and fix": fan_out = out,
 * fan_in = prod(rest) of one parameter. */
typedef struct muon_hparams {
  float lr;
  float momentum;
  int32_t nesterov;        /* 1: U = G + mu M_new; 0: U = M_new */
  float weight_decay;      /* decoupled: W <- W - lr*wd*W */
  float extra_scale;       /* lr_eff = lr * sqrt(max(1, fan_out/fan_in)) * extra_scale */
  int32_t normuon;         /* 1: apply the NorMuon normalization */
  float beta2;             /* NorMuon EMA factor (0.95) */
  float norm_eps;          /* NorMuon eps (1e-8) */
  int64_t fan_out;         /* 0 = rows */
  int64_t fan_in;          /* 0 = cols */
  muon_ns_config ns;       /* ns.max_batch counts parameters here */
} muon_hparams;

/* lr 0.05, momentum 0.95, nesterov 1, weight_decay 0, extra_scale 1,
 * normuon 0, beta2 0.95, norm_eps 1e-8, fan_out = fan_in = 0, default ns. */
void muon_default_hparams(muon_hparams* hp);

/* Workspace bytes muon_step_group needs for this group (0 for an empty one). */
int muon_step_workspace_bytes(const muon_group* g, const muon_hparams* hp, size_t* bytes);

/* One Muon (or NorMuon) step for every parameter of the group:
 *   M <- mu M + G;  U = G + mu M (nesterov) or U = M;
 *   O = NS5(U) per parameter, or per head row block when heads > 1;
 *   O_hat = NorMuon(O, var) when hp->normuon, else O;
 *   W <- W - lr*wd*W - lr_eff * O_hat  (fp32, one rounding on store);
 *   w_model <- RNE_bf16(W) when requested.
 * Momentum is stored in mom_dtype (bf16 rounding to nearest even).
 * Errors as for muon_ns_batched; additionally MUON_ERR_INVALID_ARG when
 * rows % heads != 0 or a pointer array / entry is NULL. */
int muon_step_group(const muon_group* g, const muon_hparams* hp,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes muon_step_groups needs for these ngroups groups. */
int muon_step_groups_workspace_bytes(const muon_group* groups, int64_t ngroups,
                                     const muon_hparams* hp, size_t* bytes);

/* One step over several groups (one per parameter shape, e.g. every matrix
 * of a layer): [LSMuon] _run_ns batches same-shape matrices only, and
 * [ConvFix] "Problem and fix" builds one megabatch per shape; this call
 * steps all of them at once.  groups: host array of ngroups (0..4096)
 * descriptors as for muon_step_group; hp applies to every group, with
 * fan_out / fan_in taken from each group's rows / cols unless set.  The
 * Newton-Schulz launches of the different groups are shared, so small
 * groups fill the GPU together; each parameter's results are bitwise
 * identical to a muon_step_group call on its own group.  Errors as for
 * muon_step_group (nothing is enqueued when any group is invalid). */
int muon_step_groups(const muon_group* groups, int64_t ngroups, const muon_hparams* hp,
                     void* workspace, size_t workspace_bytes, void* stream);

/* ---- launch timing ------------------------------------------------------ */

/* Kernel classes the library launches. */
#define MUON_K_PREP 0       /* momentum / load, orientation, norm partials */
#define MUON_K_NORM 1       /* Frobenius-norm finalize */
#define MUON_K_GRAM 2       /* A = X X^T (upper-triangle tiles, mirrored) */
#define MUON_K_POLY 3       /* B = b A + c A A (upper-triangle tiles, mirrored) */
#define MUON_K_UPDATE 4     /* X <- a X + B X */
#define MUON_K_ROWSTAT 5    /* NorMuon row statistics and variance update */
#define MUON_K_RHO 6        /* NorMuon norm-preserving factor */
#define MUON_K_APPLY 7      /* weight update (or NorMuon in-place scaling) */
#define MUON_K_COUNT 8

/* When enabled, every launch is bracketed by HIP events on its stream, and
 * the launch count, summed event time and summed algorithmic FLOPs and bytes
 * are kept per kernel class.  Off by default; enabling or disabling clears
 * nothing.  Reading synchronizes on the recorded events. */
int muon_profile_enable(int on);
/* Kernel classes whose launches are bracketed while timing is on: bit c of
 * mask for class c (default all, (1u << MUON_K_COUNT) - 1).  Fewer events
 * disturb the timed work less: an event pair serializes the launch
 * boundaries it sits on. */
int muon_profile_classes(uint32_t mask);
int muon_profile_reset(void);
int muon_profile_query(int kernel_class, int64_t* launches, double* total_ms,
                       double* total_flop, double* total_bytes);
const char* muon_kernel_class_name(int kernel_class);

#ifdef __cplusplus
}
#endif

#endif /* MUON_MI355X_H */
