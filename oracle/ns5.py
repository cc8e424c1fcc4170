"""Quintic Newton-Schulz orthogonalization, five iterations (test infrastructure only).

Follows "Muon under AutoTP orthogonalizes each shard, so the update depends on
the TP degree", section "Why it happens": the input is divided by its matrix
(Frobenius) norm and the iteration then works on the Gram matrix X X^T.  The
iteration itself is the one whose two symmetric products are named in
"core.optimizer.layer_sharded_muon", LayerShardedMuon, parameter use_syrk:
A = X X^T and B = b A + c A^2, after which X <- a X + B X.  The coefficients
(a, b, c) = (3.4445, -4.7750, 2.0315) are the quintic ones of the workload
definition and are used unchanged in all five iterations.

A per-iteration schedule (one (a, b, c) triple per iteration, as the
Polar-Express-style schedules that "Fix convolution flattening in megabatches
and NorMuon normalization" mentions; the pages print none) runs iteration k
with the k-th triple.

Readings where the pages are silent:
* eps is added to the norm: X0 = G / (||G||_F + eps).
* A matrix with more rows than columns is transposed first and transposed back
  at the end, so the Gram matrix is min(rows, cols) square.  p(X X^T) X equals
  X p(X^T X), so this only changes rounding.
"""
import numpy as np

QUINTIC = (3.4445, -4.7750, 2.0315)


def frobenius_normalize(g, eps=1e-7):
    g = np.array(g, dtype=np.float64, copy=True, order="C")
    return g / (np.sqrt(np.sum(g * g)) + eps)


def schedule(coeffs, steps):
    """The (a, b, c) of each iteration: one triple for all, or one per iteration."""
    t = np.asarray(coeffs, dtype=np.float64)
    if t.shape == (3,):
        return [tuple(float(v) for v in t)] * int(steps)
    if t.shape == (int(steps), 3):
        return [tuple(float(v) for v in row) for row in t]
    raise ValueError("coeffs must be (a, b, c) or one (a, b, c) per iteration")


def newton_schulz5(g, steps=5, coeffs=QUINTIC, eps=1e-7):
    """Orthogonalize one matrix.  float64 in, float64 out, same shape."""
    g = np.asarray(g, dtype=np.float64)
    if g.ndim != 2:
        raise ValueError("newton_schulz5 takes one 2-D matrix")
    x = frobenius_normalize(g, eps)
    tall = x.shape[0] > x.shape[1]
    if tall:
        x = np.ascontiguousarray(x.T)
    for a, b, c in schedule(coeffs, steps):
        gram = x @ x.T                       # A = X X^T
        poly = b * gram + c * (gram @ gram)  # B = b A + c A^2
        x = a * x + poly @ x                 # X <- a X + B X
    if tall:
        x = x.T
    return np.ascontiguousarray(x)


def ns5_megabatch(stack, **kw):
    """A megabatch [N, out, F] is N independent problems: one call per slice.

    "Fix convolution flattening in megabatches and NorMuon normalization",
    "Problem and fix": the megabatch axis is kept, never folded into columns.
    """
    stack = np.asarray(stack, dtype=np.float64)
    if stack.ndim != 3:
        raise ValueError("megabatch must be [N, out, F]")
    return np.stack([newton_schulz5(np.array(s, copy=True, order="C"), **kw)
                     for s in stack]) if len(stack) else np.zeros_like(stack)


def ns5_per_head(p, heads, **kw):
    """Per-head Newton-Schulz: row block h = rows [h*out/H, (h+1)*out/H).

    "Muon under AutoTP orthogonalizes each shard...", "What could be done",
    option 3: per-head NS batches over the head (row-block) axis.
    """
    p = np.asarray(p, dtype=np.float64)
    out = p.shape[0]
    if heads < 1 or out % heads:
        raise ValueError("rows must divide evenly into heads")
    hb = out // heads
    res = np.empty_like(p)
    for h in range(heads):
        res[h * hb:(h + 1) * hb] = newton_schulz5(
            np.array(p[h * hb:(h + 1) * hb], copy=True, order="C"), **kw)
    return res


def ns5_row_split(p, split_rows, **kw):
    """Row-split Newton-Schulz: block k = rows [r_k, r_k + h_k) with the
    heights h_k in order, each block orthogonalized on its own.

    "Fix convolution flattening in megabatches and NorMuon normalization",
    "Design" (review): a split_sizes list cuts a parameter into row blocks on
    dim -2 before Newton-Schulz; "core.optimizer.layer_sharded_muon",
    LayerShardedMuon (split_qkv, qkv_split_shapes) applies it to fused q/k/v
    weights.  Reading taken: the heights are listed top to bottom and must
    cover the rows exactly.
    """
    p = np.asarray(p, dtype=np.float64)
    hs = [int(h) for h in split_rows]
    if any(h <= 0 for h in hs) or sum(hs) != p.shape[0]:
        raise ValueError("split_rows must be positive and sum to the row count")
    res = np.empty_like(p)
    r0 = 0
    for h in hs:
        res[r0:r0 + h] = newton_schulz5(np.array(p[r0:r0 + h], copy=True, order="C"), **kw)
        r0 += h
    return res

