"""Storage rounding used by the oracle (test infrastructure only).

The oracle computes in float64 and rounds a state tensor once, when it is
stored, to the dtype the workload gives it (bf16 momentum, fp32 master weight,
bf16 model copy).  This follows the single-rounding-on-store rule of
"core.optimizer.layer_sharded_muon", LayerShardedMuon._apply_update.
"""
import numpy as np


def round_f32(x):
    """float64 -> nearest float32 (ties to even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_bf16(x):
    """float64 -> nearest bfloat16 (ties to even), returned as float64.

    Rounds the float64 value directly to an 8-bit significand: with
    x = m * 2^e, m in [0.5, 1), the quantum is 2^(e-8), floored at the bfloat16
    subnormal quantum 2^-133.  Values whose rounding reaches 2^128 become inf.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    if fin.any():
        xf = x[fin]
        _, e = np.frexp(xf)
        q = np.maximum(e - 8, -133).astype(np.float64)
        scale = np.exp2(q)
        r = np.rint(xf / scale) * scale  # rint rounds half to even
        r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, r), r)
        out[fin] = r
    return out
