"""Seeded synthetic input generators.

Every draw comes from ``numpy.random.Generator(PCG64(SeedSequence(key)))`` with
``key = (workload, layer, matrix, step, role)``, is made in float64 and is then
rounded to the storage dtype the workload names.  Rounding to bfloat16 goes
float64 -> float32 (round to nearest even) -> bfloat16 (round to nearest even);
both sides receive the exact stored bits, so neither side depends on that choice.

Roles (the last component of the key):

=====  =====================================================
0      gradient, i.i.d. N(0, 1)
1      initial master weight, N(0, 0.02^2)
2      Haar factor U of a power-law gradient
3      Haar factor V of a power-law gradient
4      noise term of a power-law gradient
=====  =====================================================

Power-law gradients follow the workload description of one Llama-3-8B-shaped
layer: ``G = U diag(s) V^T + 0.1 N(0,1)`` with Haar-random U (r x k) and V (c x k),
``k = min(r, c)`` and ``s_i = i^-0.7``.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "ROLE_GRAD", "ROLE_WEIGHT", "ROLE_U", "ROLE_V", "ROLE_NOISE",
    "generator", "f64_to_bf16_bits", "bf16_bits_to_f64", "bf16_bits_to_f32",
    "store", "gaussian", "haar", "power_law", "power_law_many", "power_law_signal",
    "power_law_from_signal", "power_law_device", "key_seed",
    "LLAMA3_8B_LAYER", "conv_megabatches",
]

ROLE_GRAD, ROLE_WEIGHT, ROLE_U, ROLE_V, ROLE_NOISE = 0, 1, 2, 3, 4

# One Llama-3-8B decoder layer's projection shapes, [out, in].
LLAMA3_8B_LAYER = (
    ("q", (4096, 4096)),
    ("k", (1024, 4096)),
    ("v", (1024, 4096)),
    ("o", (4096, 4096)),
    ("gate", (14336, 4096)),
    ("up", (14336, 4096)),
    ("down", (4096, 14336)),
)


def conv_megabatches():
    """The convolution megabatch workload: (name, N, param shape)."""
    return (("conv2d", 64, (256, 128, 3, 3)), ("conv1d", 32, (512, 512, 5)))


def generator(*key: int) -> np.random.Generator:
    """A PCG64 generator seeded by the integer key tuple."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to bfloat16 (via float32, both steps nearest-even).

    Returns the raw 16-bit patterns as uint16.
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32)
    # uint32 arithmetic wraps only for NaN patterns, which are replaced below.
    r = ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        r = np.where(nan, np.uint16(0x7FC0), r)
    return r


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float64."""
    return bf16_bits_to_f32(bits).astype(np.float64)


def store(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 draws to the storage dtype.

    ``"f32"`` returns a float32 array; ``"bf16"`` returns uint16 bit patterns.
    """
    if dtype == "f32":
        return np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == "bf16":
        return f64_to_bf16_bits(x64)
    raise ValueError(f"unknown storage dtype {dtype!r}")


def gaussian(shape, key, dtype: str = "f32", std: float = 1.0) -> np.ndarray:
    """``std * N(0,1)`` draws of the given shape, rounded to ``dtype``."""
    g = generator(*key)
    return store(std * g.standard_normal(size=tuple(shape)), dtype)


def haar(n: int, k: int, key) -> np.ndarray:
    """An n x k matrix with orthonormal columns, Haar distributed (float64).

    The Q factor, with positive diag(R), of the QR factorization of an n x k
    Gaussian matrix.  For n >= 2k the factor is computed by two passes of
    Cholesky QR (the same Q in exact arithmetic; a tall Gaussian matrix is
    well conditioned, so the result is orthonormal to rounding), otherwise by
    Householder QR with the signs of diag(R) moved into Q.
    """
    g = generator(*key)
    z = g.standard_normal(size=(n, k))
    if n >= 2 * k:
        q = z
        for _ in range(2):
            r = np.linalg.cholesky(q.T @ q).T          # upper triangular, positive diagonal
            q = q @ _inv_upper(r)
        return q
    q, r = np.linalg.qr(z, mode="reduced")
    d = np.sign(np.diag(r))
    d[d == 0] = 1.0
    return q * d[None, :]


def _inv_upper(r):
    """Inverse of an upper-triangular matrix."""
    import scipy.linalg
    return scipy.linalg.solve_triangular(r, np.eye(r.shape[0]), lower=False)


def power_law(shape, key_uv, key_noise, dtype: str = "bf16", alpha: float = 0.7,
              noise: float = 0.1) -> np.ndarray:
    """``U diag(i^-alpha) V^T + noise * N(0,1)`` rounded to ``dtype``.

    ``key_uv`` seeds U (role 2) and V (role 3); ``key_noise`` seeds the noise.
    Keys are tuples without the role component.
    """
    return power_law_many(shape, key_uv, [key_noise], dtype, alpha, noise)[0]


def power_law_signal(shape, key_uv, alpha: float = 0.7) -> np.ndarray:
    """The low-rank part ``U diag(i^-alpha) V^T`` (float64) of a power-law matrix."""
    r, c = int(shape[0]), int(shape[1])
    k = min(r, c)
    u = haar(r, k, tuple(key_uv) + (ROLE_U,))
    v = haar(c, k, tuple(key_uv) + (ROLE_V,))
    s = np.arange(1, k + 1, dtype=np.float64) ** (-alpha)
    return (u * s[None, :]) @ v.T


def power_law_from_signal(signal: np.ndarray, key_noise, dtype: str = "bf16", noise: float = 0.1) -> np.ndarray:
    """``signal + noise * N(0,1)`` with the noise seeded by ``key_noise``, rounded to ``dtype``."""
    gnoise = generator(*(tuple(key_noise) + (ROLE_NOISE,)))
    g = noise * gnoise.standard_normal(size=signal.shape)
    g += signal
    return store(g, dtype)


def power_law_many(shape, key_uv, keys_noise, dtype: str = "bf16", alpha: float = 0.7,
                   noise: float = 0.1):
    """Several power-law matrices sharing U, V and s, each with its own noise.

    Entry i equals ``power_law(shape, key_uv, keys_noise[i], ...)``.
    """
    signal = power_law_signal(shape, key_uv, alpha)
    return [power_law_from_signal(signal, kn, dtype, noise) for kn in keys_noise]


def key_seed(key) -> int:
    """A 63-bit seed derived from an integer key tuple (for device generators)."""
    w = np.random.SeedSequence([int(k) for k in key]).generate_state(2, np.uint32)
    return (int(w[0]) << 31) ^ int(w[1])


def power_law_device(signal_f32, key_noise, noise: float = 0.1):
    """A bf16 power-law matrix drawn on the GPU: ``signal + noise * N(0,1)``.

    ``signal_f32`` is the low-rank part as a float32 CUDA tensor; the noise
    comes from torch's device generator seeded by ``key_seed(key_noise +
    (ROLE_NOISE,))`` and the sum is rounded to bfloat16 (nearest even).  This
    is a different generator from the host one: the same key gives different
    noise.  Used where host generation of billions of values would dominate.
    """
    import torch
    gen = torch.Generator(device=signal_f32.device)
    gen.manual_seed(key_seed(tuple(key_noise) + (ROLE_NOISE,)))
    g = torch.randn(signal_f32.shape, generator=gen, device=signal_f32.device, dtype=torch.float32)
    g.mul_(noise).add_(signal_f32)
    return g.to(torch.bfloat16)
