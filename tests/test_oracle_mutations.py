"""The pins are strong enough to catch plausible mistakes.

Each mutant below is the oracle's Newton-Schulz or NorMuon with one planted
mistake (a dropped term, a wrong sign, a swapped coefficient, a transposed
operand, a misplaced eps, a wrong reduction axis).  The same pins that the
oracle passes must reject every mutant.  Everything here runs on the CPU.
"""
import numpy as np
import pytest

import oracle
from test_oracle_ns5 import svd_closed_form
from test_oracle_step import rel

A, B, C = oracle.QUINTIC


def ns_variant(g, mutation=None, steps=5, eps=1e-7):
    g = np.asarray(g, dtype=np.float64)
    a, b, c = A, B, C
    if mutation == "swap_bc":
        b, c = c, b
    if mutation == "neg_b":
        b = -b
    if mutation == "eps_in_sqrt":
        x = g / np.sqrt(np.sum(g * g) + eps)
    elif mutation == "no_normalize":
        x = g.copy()
    elif mutation == "max_norm":
        x = g / (np.max(np.abs(g)) + eps)
    else:
        x = g / (np.sqrt(np.sum(g * g)) + eps)
    tall = x.shape[0] > x.shape[1]
    if tall and mutation != "no_orient":
        x = x.T.copy()
    for it in range(steps - (1 if mutation == "four_steps" else 0)):
        # "gram_swapped": X^T X where X X^T belongs (shape-valid only when square).
        gram = x.T @ x if (mutation == "gram_swapped" and x.shape[0] == x.shape[1]) else x @ x.T
        if mutation == "drop_cA2":
            poly = b * gram
        elif mutation == "A_cubed":
            poly = b * gram + c * (gram @ gram @ gram)
        else:
            poly = b * gram + c * (gram @ gram)
        if mutation == "drop_aX":
            x = poly @ x
        elif mutation == "update_right":
            # B applied from the wrong side on the (square) iterate.
            x = a * x + (x @ poly if x.shape[0] == x.shape[1] else poly @ x)
        else:
            x = a * x + poly @ x
    if tall and mutation != "no_orient":
        x = x.T
    return x


NS_MUTANTS = ["swap_bc", "neg_b", "eps_in_sqrt", "no_normalize", "max_norm", "four_steps",
              "drop_cA2", "A_cubed", "drop_aX", "gram_swapped", "update_right"]


def ns_pins_pass(ns):
    rng = np.random.default_rng(0)
    for shape in [(7, 5), (5, 7), (16, 16)]:
        g = rng.standard_normal(shape) * 1e-3   # small norm: eps placement matters
        if rel(ns(g), svd_closed_form(g)) > 1e-12:
            return False
    return True


def test_unmutated_passes():
    assert ns_pins_pass(lambda g: ns_variant(g))
    assert ns_pins_pass(oracle.newton_schulz5)


@pytest.mark.parametrize("mutation", NS_MUTANTS)
def test_ns_mutant_is_caught(mutation):
    assert not ns_pins_pass(lambda g: ns_variant(g, mutation))


def test_orientation_mutant_is_caught_by_transpose_pin():
    # Without the orientation rule a tall input runs on its larger Gram;
    # mathematically equal, so the closed form alone cannot see it, but the
    # bitwise transpose equivariance of the oracle can.
    g = np.random.default_rng(1).standard_normal((31, 12))
    assert not np.array_equal(ns_variant(g, "no_orient"), ns_variant(g.T.copy(), "no_orient").T)
    assert np.array_equal(oracle.newton_schulz5(g), oracle.newton_schulz5(g.T.copy()).T)


def normuon_variant(o, v, mutation=None, beta2=0.95, eps=1e-8):
    axis = 0 if mutation == "col_stats" else 1
    ms = np.mean(o * o, axis=axis)
    if mutation == "centered":
        ms = np.var(o, axis=axis)
    v_new = beta2 * v + (1 - beta2) * ms if mutation != "swap_beta" else (1 - beta2) * v + beta2 * ms
    den = np.sqrt(v_new) + eps
    ohat = o / (den[:, None] if axis == 1 else den[None, :])
    if mutation != "no_rescale":
        ohat = ohat * (np.linalg.norm(o) / np.linalg.norm(ohat))
    return ohat, v_new


NORMUON_MUTANTS = ["col_stats", "centered", "swap_beta", "no_rescale"]


def normuon_pins_pass(fn):
    beta2, out, f = 0.95, 8, 8
    rng = np.random.default_rng(4)
    o1 = rng.standard_normal((out, f)) * np.linspace(0.5, 2, out)[:, None] + 0.3
    o2 = rng.standard_normal((out, f)) * np.linspace(2, 0.5, out)[:, None] - 0.2
    _, v1 = fn(o1, np.zeros(out))
    ohat2, v2 = fn(o2, v1)
    ms1, ms2 = np.mean(o1 ** 2, 1), np.mean(o2 ** 2, 1)
    d = 1.0 / np.sqrt(beta2 * (1 - beta2) * ms1 + (1 - beta2) * ms2)
    expect = o2 * d[:, None]
    expect *= np.linalg.norm(o2) / np.linalg.norm(expect)
    return rel(ohat2, expect) < 1e-6 and abs(np.linalg.norm(ohat2) - np.linalg.norm(o2)) < 1e-9


def test_normuon_unmutated_passes():
    assert normuon_pins_pass(lambda o, v: normuon_variant(o, v))
    assert normuon_pins_pass(lambda o, v: oracle.normuon(o, v))


@pytest.mark.parametrize("mutation", NORMUON_MUTANTS)
def test_normuon_mutant_is_caught(mutation):
    assert not normuon_pins_pass(lambda o, v: normuon_variant(o, v, mutation))


# ---- row-split geometry -----------------------------------------------------
def split_variant(p, hs, mutation=None):
    p = np.asarray(p, dtype=np.float64)
    if mutation == "reversed_heights":
        hs = list(hs)[::-1]
    whole = np.sqrt(np.sum(p * p)) + 1e-7
    res = np.empty_like(p)
    r0 = 0
    for h in hs:
        blk = p[r0:r0 + h]
        if mutation == "whole_norm":
            # every block scaled by the whole matrix's norm instead of its own
            res[r0:r0 + h] = ns_variant(blk / whole, "no_normalize")
        else:
            res[r0:r0 + h] = ns_variant(blk)
        r0 += h
    return res


def split_pins_pass(fn):
    rng = np.random.default_rng(1)
    hs = [5, 3, 9, 1]
    p = rng.standard_normal((sum(hs), 7))
    out = fn(p, hs)
    r0 = 0
    for h in hs:
        if rel(out[r0:r0 + h], svd_closed_form(p[r0:r0 + h])) > 1e-12:
            return False
        r0 += h
    return True


def test_split_unmutated_passes():
    assert split_pins_pass(lambda p, hs: split_variant(p, hs))
    assert split_pins_pass(oracle.ns5_row_split)


@pytest.mark.parametrize("mutation", ["reversed_heights", "whole_norm"])
def test_split_mutant_is_caught(mutation):
    assert not split_pins_pass(lambda p, hs: split_variant(p, hs, mutation))
