"""One Muon / NorMuon optimizer step for one parameter (test infrastructure only).

Order of the step, as the Megatron page ("core.optimizer.layer_sharded_muon",
LayerShardedMuon.step) lists it for the single-rank case: momentum on the
parameter, full-matrix Newton-Schulz, then p -= lr * update.  NorMuon inserts
its normalization between the orthogonalization and the update
("Fix convolution flattening in megabatches and NorMuon normalization",
"What it does").
"""
from dataclasses import dataclass

import numpy as np

from .bf16 import round_bf16, round_f32
from .ns5 import QUINTIC, newton_schulz5, ns5_per_head, ns5_row_split


def flatten_param(p):
    """A parameter [out, *rest] is the matrix [out, prod(rest)].

    "Fix convolution flattening...", "Problem and fix" and "What it does".
    """
    p = np.asarray(p)
    return p.reshape(p.shape[0], -1) if p.ndim != 2 else p


def nesterov_momentum(g, m, mu=0.95, nesterov=True):
    """SGD-style Nesterov momentum.  Returns (new momentum, NS input).

    M <- mu M + G;  U = G + mu M (with the updated M), or U = M without
    Nesterov.  The pages fix only "momentum 0.95, nesterov=True"
    ("core.optimizer.layer_sharded_muon", LayerShardedMuon); this form is the
    reading taken.  The EMA form differs from it by the factor (1 - mu) on U,
    which the Frobenius normalization removes.
    """
    g = np.asarray(g, dtype=np.float64)
    m_new = mu * np.asarray(m, dtype=np.float64) + g
    u = g + mu * m_new if nesterov else m_new
    return m_new, u


def normuon(o, v, beta2=0.95, eps=1e-8):
    """NorMuon normalization of one orthogonalized matrix O [out, F].

    "Fix convolution flattening...", "Adjacent bug" / "What it does": one
    variance per output channel (neuron), taken along the input axis of the
    flattened matrix, then a rescale that preserves the Frobenius norm
    ("Compatibility": norm-preserving rescale).  Reading taken for what the
    pages leave open: the "variance" is the uncentered mean of squares along
    the row, kept as an exponential moving average without bias correction,
    and the row is divided by sqrt(v) + eps.  If the normalized matrix is all
    zero the result is zero.

    Returns (O_hat, v_new).
    """
    o = np.asarray(o, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if o.shape[0] == 0 or o.shape[1] == 0:
        return o.copy(), v.copy()
    ms = np.mean(o * o, axis=1)
    v_new = beta2 * v + (1.0 - beta2) * ms
    ohat = o / (np.sqrt(v_new) + eps)[:, None]
    n_o = np.sqrt(np.sum(o * o))
    n_hat = np.sqrt(np.sum(ohat * ohat))
    ohat = ohat * (n_o / n_hat) if n_hat > 0 else np.zeros_like(ohat)
    return ohat, v_new


def spectral_lr(lr, fan_out, fan_in, extra_scale=1.0):
    """lr * sqrt(max(1, fan_out / fan_in)) * extra_scale.

    fan_out = out and fan_in = prod(rest) of one parameter ("Fix convolution
    flattening...", "Problem and fix"; "core.optimizer.layer_sharded_muon",
    scale_mode='spectral', extra_scale_factor).
    """
    return float(lr) * np.sqrt(max(1.0, float(fan_out) / float(fan_in))) * float(extra_scale)


@dataclass
class MuonHParams:
    lr: float = 0.05
    momentum: float = 0.95
    nesterov: bool = True
    weight_decay: float = 0.0
    extra_scale: float = 1.0
    ns_steps: int = 5
    coeffs: tuple = QUINTIC
    ns_eps: float = 1e-7
    heads: int = 1
    split_rows: tuple = None    # row-block heights of a fused weight (heads must be 1)
    normuon: bool = False
    beta2: float = 0.95
    norm_eps: float = 1e-8
    mom_dtype: str = "f32"      # storage of the momentum buffer: "f32" or "bf16"


def _store(x, dtype):
    return round_bf16(x) if dtype == "bf16" else round_f32(x)


def muon_step(w, g, m, v=None, hp=MuonHParams()):
    """One optimizer step of one parameter, all arithmetic in float64.

    w: fp32 master weight values [out, *rest]; g: gradient; m: momentum;
    v: NorMuon variance [out] (required when hp.normuon).  With
    hp.split_rows only Newton-Schulz runs per row block; momentum, NorMuon
    (its norm-preserving rescale included) and the spectral scale act on the
    whole parameter, whose shape is the one the lr adjustment uses ("Fix
    convolution flattening...", "Problem and fix").  This whole-parameter
    scope is a reading: the pages do not say.  Inputs are the
    exact stored values widened to float64.

    Returns a dict with the stored results (w rounded to fp32, m rounded to
    its storage dtype, v rounded to fp32, w_bf16 = bf16 copy of the stored w)
    and the float64 intermediates u (NS input), o (NS output) and o_hat (the
    update direction after NorMuon).
    """
    shape = np.shape(w)
    w2 = flatten_param(np.asarray(w, dtype=np.float64))
    g2 = flatten_param(np.asarray(g, dtype=np.float64))
    m2 = flatten_param(np.asarray(m, dtype=np.float64))
    out, fan_in = w2.shape
    m_new, u = nesterov_momentum(g2, m2, hp.momentum, hp.nesterov)
    kw = dict(steps=hp.ns_steps, coeffs=hp.coeffs, eps=hp.ns_eps)
    if out == 0 or fan_in == 0:
        o = np.zeros_like(u)
    elif hp.split_rows:
        if hp.heads != 1:
            raise ValueError("row splits take heads == 1")
        o = ns5_row_split(u, hp.split_rows, **kw)
    elif hp.heads > 1:
        o = ns5_per_head(u, hp.heads, **kw)
    else:
        o = newton_schulz5(u, **kw)
    v_new = None
    if hp.normuon:
        o_hat, v_new = normuon(o, np.asarray(v, dtype=np.float64), hp.beta2, hp.norm_eps)
    else:
        o_hat = o
    lr_eff = spectral_lr(hp.lr, out, fan_in, hp.extra_scale) if out and fan_in else 0.0
    w_new = w2 - hp.lr * hp.weight_decay * w2 - lr_eff * o_hat
    w_store = round_f32(w_new)
    return {
        "w": w_store.reshape(shape),
        "w_bf16": round_bf16(w_store).reshape(shape),
        "m": _store(m_new, hp.mom_dtype).reshape(shape),
        "v": None if v_new is None else round_f32(v_new),
        "u": u, "o": o, "o_hat": o_hat, "lr_eff": lr_eff,
    }
