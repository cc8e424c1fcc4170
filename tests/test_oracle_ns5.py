"""Pins of the oracle's Newton-Schulz against the mathematics.

Newton-Schulz with the quintic p(x) = a x + b x^3 + c x^5 acts on singular
values only: NS5(G) = U diag(phi^5(sigma_i / (||G||_F + eps))) V^T with the
thin SVD of G.  The tests below compare the oracle's matrix iteration with that
closed form (numpy's SVD, a different algorithm), with scalar fixed points
computed in exact rational arithmetic, and with invariances that any correct
implementation has.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import newton_schulz5, ns5_megabatch, ns5_per_head, ns5_row_split

A, B, C = oracle.QUINTIC


def rel(x, y):
    return float(np.linalg.norm(np.asarray(x) - np.asarray(y)) / np.linalg.norm(np.asarray(y)))


def scalar_phi5(sigma, steps=5):
    """The quintic applied `steps` times to one singular value (float64)."""
    s = float(sigma)
    for _ in range(steps):
        s = A * s + B * s ** 3 + C * s ** 5
    return s


def exact_phi5(sigma: Fraction, steps=5):
    a, b, c = Fraction("3.4445"), Fraction("-4.7750"), Fraction("2.0315")
    s = sigma
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def svd_closed_form(g, eps=1e-7, steps=5):
    g = np.asarray(g, dtype=np.float64)
    u, s, vt = np.linalg.svd(g, full_matrices=False)
    nrm = np.sqrt(np.sum(g * g)) + eps
    mapped = np.array([scalar_phi5(x / nrm, steps) if x > 0 else 0.0 for x in s])
    return (u * mapped[None, :]) @ vt


@pytest.mark.parametrize("shape", [(7, 5), (5, 7), (16, 16), (33, 20), (3, 64)])
def test_svd_closed_form(shape):
    g = np.random.default_rng(sum(shape)).standard_normal(shape)
    assert rel(newton_schulz5(g), svd_closed_form(g)) < 1e-12


def test_svd_closed_form_rank_deficient():
    rng = np.random.default_rng(3)
    g = rng.standard_normal((8, 3)) @ rng.standard_normal((3, 12))  # rank 3
    out = newton_schulz5(g)
    assert rel(out, svd_closed_form(g)) < 1e-10
    assert np.linalg.matrix_rank(out, tol=1e-8) == 3


@pytest.mark.parametrize("steps", [1, 2, 5])
def test_closed_form_other_step_counts(steps):
    g = np.random.default_rng(11).standard_normal((9, 13))
    assert rel(newton_schulz5(g, steps=steps), svd_closed_form(g, steps=steps)) < 1e-12


def test_scalar_fixed_points_exact():
    # phi(1) = a + b + c = 0.701 exactly; phi^5(1) from exact rationals.
    assert exact_phi5(Fraction(1), steps=1) == Fraction("0.701")
    # 15-digit decimal values of the exact rationals.
    assert abs(float(exact_phi5(Fraction(1))) - 0.696436409469752) < 5e-15
    assert abs(float(exact_phi5(Fraction(1, 16))) - 1.070524447724669) < 5e-15
    assert abs(float(exact_phi5(Fraction(1, 64))) - 0.902525752966620) < 5e-15


def test_rank_one_maps_to_phi5_of_one():
    rng = np.random.default_rng(5)
    u = rng.standard_normal(24); u /= np.linalg.norm(u)
    v = rng.standard_normal(40); v /= np.linalg.norm(v)
    g = 3.7 * np.outer(u, v)
    expect = float(exact_phi5(Fraction(1))) * np.outer(u, v)
    # eps = 1e-7 against ||G|| = 3.7 perturbs sigma by ~3e-8 relative.
    assert rel(newton_schulz5(g), expect) < 1e-7
    assert rel(newton_schulz5(g, eps=0.0), expect) < 1e-13


@pytest.mark.parametrize("n,const", [(256, "1/16"), (4096, "1/64")])
def test_orthogonal_input(n, const):
    if n > 1024:
        # A diagonal orthogonal matrix (signs) keeps the 4096 case cheap; the
        # singular values are all 1 exactly as for any orthogonal matrix.
        q = np.diag(np.where(np.random.default_rng(1).random(n) < 0.5, -1.0, 1.0))
    else:
        q, _ = np.linalg.qr(np.random.default_rng(2).standard_normal((n, n)))
    scale = float(exact_phi5(Fraction(const)))
    assert rel(newton_schulz5(q, eps=0.0), scale * q) < 1e-12


def test_diagonal_acts_elementwise():
    d = np.array([3.0, -1.0, 0.5, 0.0, 2.0])
    g = np.diag(d)
    nrm = np.linalg.norm(d)
    expect = np.diag([np.sign(x) * scalar_phi5(abs(x) / nrm) for x in d])
    assert np.max(np.abs(newton_schulz5(g, eps=0.0) - expect)) < 1e-14


def test_zero_matrix_gives_zero():
    z = newton_schulz5(np.zeros((6, 9)))
    assert np.all(z == 0.0)


@pytest.mark.parametrize("c", [1e-3, 7.5, 1e4])
def test_scale_invariance(c):
    g = np.random.default_rng(7).standard_normal((20, 30))
    # Only eps breaks exact invariance: sigma/(||G||+eps) vs c sigma/(c||G||+eps).
    assert rel(newton_schulz5(c * g), newton_schulz5(g)) < 1e-6 / min(c, 1.0)


def test_transpose_equivariance_bitwise_for_rectangular():
    g = np.random.default_rng(8).standard_normal((12, 31))
    a = newton_schulz5(g.T.copy())
    b = newton_schulz5(g).T
    assert np.array_equal(a, b)


def test_transpose_equivariance_square():
    g = np.random.default_rng(9).standard_normal((17, 17))
    assert rel(newton_schulz5(g.T.copy()), newton_schulz5(g).T) < 1e-12


def test_zero_padding_leaves_real_entries():
    # "Fix convolution flattening...", Review 1, Correctness: zero columns add
    # nothing to X X^T, so the real columns come back unchanged.
    g = np.random.default_rng(10).standard_normal((10, 14))
    padded_cols = np.concatenate([g, np.zeros((10, 5))], axis=1)
    padded_rows = np.concatenate([g, np.zeros((3, 14))], axis=0)
    ref = newton_schulz5(g)
    pc = newton_schulz5(padded_cols)
    pr = newton_schulz5(padded_rows)
    assert rel(pc[:, :14], ref) < 1e-13 and np.all(pc[:, 14:] == 0)
    assert rel(pr[:10], ref) < 1e-13 and np.all(pr[10:] == 0)


def test_permutation_and_sign_commute():
    rng = np.random.default_rng(12)
    g = rng.standard_normal((9, 15))
    p = np.eye(9)[rng.permutation(9)] * np.where(rng.random(9) < 0.5, -1, 1)[:, None]
    q = np.eye(15)[rng.permutation(15)] * np.where(rng.random(15) < 0.5, -1, 1)[None, :]
    assert rel(newton_schulz5(p @ g @ q), p @ newton_schulz5(g) @ q) < 1e-12


def test_megabatch_is_loop_bitwise():
    stack = np.random.default_rng(13).standard_normal((5, 8, 36))
    mb = ns5_megabatch(stack)
    for i in range(5):
        assert np.array_equal(mb[i], newton_schulz5(stack[i].copy()))


def test_megabatch_reversal_bitwise():
    stack = np.random.default_rng(14).standard_normal((3, 6, 10))
    assert np.array_equal(ns5_megabatch(stack[::-1].copy())[::-1], ns5_megabatch(stack))


def test_per_head_slice_bitwise():
    # "Muon under AutoTP...", "What could be done", option 3 (0.00e+00).
    p = np.random.default_rng(15).standard_normal((32 * 8, 64))
    whole = ns5_per_head(p, 32)
    part = ns5_per_head(p[8 * 8:16 * 8].copy(), 8)
    assert np.array_equal(part, whole[8 * 8:16 * 8])


def test_per_head_with_one_head_is_plain_ns():
    p = np.random.default_rng(16).standard_normal((12, 20))
    assert np.array_equal(ns5_per_head(p, 1), newton_schulz5(p))


def test_per_head_rejects_uneven_heads():
    with pytest.raises(ValueError):
        ns5_per_head(np.ones((10, 4)), 3)


# ---- row-split geometry (fused q/k/v weights) --------------------------------
# "Fix convolution flattening...", "Design": split_sizes row blocks on dim -2.
def test_row_split_blocks_follow_their_own_svd_closed_form():
    # Blocks of unequal height, tall and wide, at very different scales: each
    # block is normalized by its own norm and orthogonalized alone.
    rng = np.random.default_rng(40)
    hs = [5, 3, 9, 1]
    p = rng.standard_normal((sum(hs), 7)) * np.repeat([1.0, 1e3, 1e-2, 5.0], hs)[:, None]
    out = ns5_row_split(p, hs)
    r0 = 0
    for h in hs:
        assert rel(out[r0:r0 + h], svd_closed_form(p[r0:r0 + h])) < 1e-12, h
        r0 += h


def test_row_split_differs_from_whole_matrix():
    p = np.random.default_rng(41).standard_normal((12, 16))
    assert rel(ns5_row_split(p, [4, 8]), newton_schulz5(p)) > 0.1


def test_row_split_blocks_are_independent_bitwise():
    rng = np.random.default_rng(42)
    p = rng.standard_normal((10, 6))
    q = p.copy()
    q[4:] = rng.standard_normal((6, 6))          # change the second block only
    a, b = ns5_row_split(p, [4, 6]), ns5_row_split(q, [4, 6])
    assert np.array_equal(a[:4], b[:4])
    assert not np.array_equal(a[4:], b[4:])


def test_row_split_of_equal_heights_is_per_head():
    p = np.random.default_rng(43).standard_normal((24, 10))
    assert np.array_equal(ns5_row_split(p, [6, 6, 6, 6]), ns5_per_head(p, 4))
    assert np.array_equal(ns5_row_split(p, [24]), newton_schulz5(p))


@pytest.mark.parametrize("hs", [[5, 4], [10, 0, 0], [11, -1], []])
def test_row_split_rejects_bad_heights(hs):
    with pytest.raises(ValueError):
        ns5_row_split(np.ones((10, 4)), hs)


# ---- per-iteration coefficient schedules ------------------------------------
CLASSICAL = (15 / 8, -10 / 8, 3 / 8)   # p(s) = (15 s - 10 s^3 + 3 s^5) / 8: p(1) = 1, p'(1) = 0


def _phi(coeffs, s):
    a, b, c = coeffs
    return a * s + b * s ** 3 + c * s ** 5


def test_schedule_of_identical_rows_equals_constant_coefficients():
    g = np.random.default_rng(11).standard_normal((24, 40))
    assert np.array_equal(oracle.newton_schulz5(g, coeffs=[oracle.QUINTIC] * 5), oracle.newton_schulz5(g))


def test_schedule_svd_closed_form():
    # NS with (a_k, b_k, c_k) maps every singular value s of G/(||G||+eps)
    # through phi_K o ... o phi_1 and keeps the singular vectors.
    rng = np.random.default_rng(12)
    g = rng.standard_normal((30, 50))
    sched = [oracle.QUINTIC] * 3 + [CLASSICAL] * 2
    u, sv, vt = np.linalg.svd(g, full_matrices=False)
    s = sv / (np.sqrt(np.sum(g * g)) + 1e-7)
    for co in sched:
        s = _phi(co, s)
    want = (u * s[None, :]) @ vt
    got = oracle.newton_schulz5(g, steps=5, coeffs=sched)
    assert np.max(np.abs(got - want)) < 1e-12


def test_schedule_order_matters():
    g = np.random.default_rng(13).standard_normal((16, 32))
    sched = [oracle.QUINTIC, oracle.QUINTIC, CLASSICAL]
    rev = sched[::-1]
    assert np.max(np.abs(oracle.newton_schulz5(g, steps=3, coeffs=sched)
                         - oracle.newton_schulz5(g, steps=3, coeffs=rev))) > 1e-3


def test_classical_tail_converges_to_the_polar_factor():
    # Quintic steps bring every singular value near 1; the classical
    # polynomial (fixed point 1, zero derivative there) then converges to the
    # exact polar factor U V^T of G.
    rng = np.random.default_rng(14)
    u, _ = np.linalg.qr(rng.standard_normal((20, 20)))
    v, _ = np.linalg.qr(rng.standard_normal((36, 20)))
    g = (u * np.linspace(0.2, 1.0, 20)[None, :]) @ v.T
    sched = [oracle.QUINTIC] * 5 + [CLASSICAL] * 6
    got = oracle.newton_schulz5(g, steps=11, coeffs=sched)
    assert np.max(np.abs(got - u @ v.T)) < 1e-10


def test_schedule_shape_is_checked():
    with pytest.raises(ValueError):
        oracle.newton_schulz5(np.eye(4), steps=5, coeffs=[oracle.QUINTIC] * 4)
