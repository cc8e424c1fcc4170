"""CPU float64 oracle for the Muon / NorMuon optimizer step with quintic
Newton-Schulz orthogonalization.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link
or execute anything in this package: only the test suite, the smoke check of
the package entry module and the CPU-baseline leg of the benchmark use it.  It
shares no code with the HIP library: plain numpy in float64, one matrix at a
time, no blocking or fusion beyond what the method states.

Sources (pages are cited by title and section):

* "Muon under AutoTP orthogonalizes each shard, so the update depends on the TP
  degree" (DeepSpeed issue), section "Why it happens": Newton-Schulz first
  normalizes by the matrix norm and then iterates on X @ X^T; section "What
  could be done", option 3: per-head Newton-Schulz batches over row blocks.
* "core.optimizer.layer_sharded_muon" (Megatron Core API docs), class
  LayerShardedMuon: Nesterov momentum 0.95, quintic coefficients, 5 steps,
  spectral lr scaling, decoupled weight decay; the SYRK note names the two
  symmetric products X X^T and b A + c A^2; _apply_update: one fused
  multiply-add in the promoted precision with a single rounding on store.
* "Fix convolution flattening in megabatches and NorMuon normalization" (dion
  pull request): "Problem and fix" (megabatch [N, out, prod(rest)], fan_out=out,
  fan_in=prod(rest)), "Adjacent bug" and "What it does" (one NorMuon variance
  per output channel on the flattened matrix, norm-preserving rescale);
  "Design" (review): split_sizes row blocks cut on dim -2 before Newton-Schulz.

Parity status per function (see also the test suite):

* newton_schulz5, ns5_megabatch, ns5_per_head, ns5_row_split, flatten_param: pinned (SVD
  closed form, scalar fixed points, invariances, the shard-vs-whole figures
  printed on the AutoTP page).
* nesterov_momentum: pinned by the two-step closed form.
* normuon: pinned by its invariants (norm preservation, equal row RMS at step
  one, the two-step closed form); the exact variance definition is a reading
  of the pages (see normuon's docstring) and its numbers are otherwise
  parity unpinned.
* spectral_lr / muon_step: pinned by the closed-form update of one step.
"""
from .bf16 import round_bf16, round_f32  # noqa: F401
from .ns5 import (  # noqa: F401
    QUINTIC, newton_schulz5, ns5_megabatch, ns5_per_head, ns5_row_split, frobenius_normalize,
)
from .muon import (  # noqa: F401
    flatten_param, nesterov_momentum, normuon, spectral_lr, muon_step, MuonHParams,
)
