"""Pins of the oracle's momentum, NorMuon, update and storage rounding.

Closed forms used:
* momentum from M0 = 0: U1 = (1 + mu) G1 and U2 = (1 + mu) G2 + mu^2 G1;
* NorMuon: the rescale preserves ||O||_F; at step one (v0 = 0) every row of
  the result has the same RMS and beta2 cancels; at step two the row scale is
  1 / sqrt(beta2 (1 - beta2) ms1 + (1 - beta2) ms2) before the rescale;
* update: W1 - W0 = -lr * sqrt(max(1, out / F)) * O_hat (+ decoupled decay);
* a convolution [out, *rest] steps exactly like the [out, prod(rest)] matrix
  ("Fix convolution flattening...", "What it does": exact-equivalence oracle);
* a row-split (fused q/k/v) weight: each block's own SVD closed form, with
  the scale and NorMuon over the whole parameter.
"""
import json
import os

import numpy as np
import pytest

import synth
from oracle import (MuonHParams, flatten_param, muon_step, nesterov_momentum, newton_schulz5,
                    normuon, ns5_megabatch, round_bf16, round_f32, spectral_lr)
from test_oracle_ns5 import svd_closed_form

MU = 0.95


def rel(x, y):
    return float(np.linalg.norm(np.asarray(x) - np.asarray(y)) / np.linalg.norm(np.asarray(y)))


def test_momentum_two_step_closed_form():
    rng = np.random.default_rng(0)
    g1, g2 = rng.standard_normal((2, 5, 7))
    m1, u1 = nesterov_momentum(g1, np.zeros_like(g1), MU)
    m2, u2 = nesterov_momentum(g2, m1, MU)
    assert np.allclose(u1, (1 + MU) * g1, rtol=0, atol=1e-15)
    assert np.allclose(u2, (1 + MU) * g2 + MU ** 2 * g1, rtol=0, atol=1e-14)
    assert np.allclose(m2, MU * g1 + g2, rtol=0, atol=1e-15)


def test_momentum_plain():
    g = np.ones((2, 2)); m = np.full((2, 2), 2.0)
    m_new, u = nesterov_momentum(g, m, 0.5, nesterov=False)
    assert np.all(m_new == 2.0) and np.all(u == 2.0)


def test_normuon_preserves_norm():
    o = np.random.default_rng(1).standard_normal((16, 40)) * np.linspace(0.1, 3, 16)[:, None]
    ohat, _ = normuon(o, np.zeros(16))
    assert abs(np.linalg.norm(ohat) - np.linalg.norm(o)) < 1e-12 * np.linalg.norm(o)


@pytest.mark.parametrize("beta2", [0.95, 0.5])
def test_normuon_step_one_equal_row_rms(beta2):
    out, f = 12, 30
    o = np.random.default_rng(2).standard_normal((out, f)) * np.linspace(0.2, 5, out)[:, None]
    target = np.linalg.norm(o) / np.sqrt(out * f)
    ohat, v = normuon(o, np.zeros(out), beta2=beta2, eps=0.0)
    rms = np.sqrt(np.mean(ohat ** 2, axis=1))
    assert np.max(np.abs(rms - target)) < 1e-13 * target
    # With eps = 1e-8 the rows differ only by eps / sqrt(v) (about 2e-7 here).
    ohat, _ = normuon(o, np.zeros(out), beta2=beta2)
    rms = np.sqrt(np.mean(ohat ** 2, axis=1))
    assert np.max(np.abs(rms - target)) < 1e-6 * target
    assert np.allclose(v, (1 - beta2) * np.mean(o * o, axis=1), rtol=1e-15, atol=0)


def test_normuon_step_one_beta2_cancels():
    o = np.random.default_rng(3).standard_normal((6, 9)) * np.arange(1, 7)[:, None]
    a, _ = normuon(o, np.zeros(6), beta2=0.95)
    b, _ = normuon(o, np.zeros(6), beta2=0.5)
    assert rel(a, b) < 1e-7


def test_normuon_step_two_closed_form():
    beta2, out, f = 0.95, 8, 20
    rng = np.random.default_rng(4)
    o1 = rng.standard_normal((out, f)) * np.linspace(0.5, 2, out)[:, None]
    o2 = rng.standard_normal((out, f)) * np.linspace(2, 0.5, out)[:, None]
    _, v1 = normuon(o1, np.zeros(out), beta2=beta2, eps=0.0)
    ohat2, v2 = normuon(o2, v1, beta2=beta2, eps=0.0)
    ms1, ms2 = np.mean(o1 ** 2, 1), np.mean(o2 ** 2, 1)
    d = 1.0 / np.sqrt(beta2 * (1 - beta2) * ms1 + (1 - beta2) * ms2)
    expect = o2 * d[:, None]
    expect *= np.linalg.norm(o2) / np.linalg.norm(expect)
    assert rel(ohat2, expect) < 1e-13
    assert rel(v2, beta2 * (1 - beta2) * ms1 + (1 - beta2) * ms2) < 1e-15


def test_normuon_zero_matrix():
    ohat, v = normuon(np.zeros((3, 4)), np.zeros(3))
    assert np.all(ohat == 0) and np.all(v == 0)


def test_spectral_lr_values():
    assert spectral_lr(0.05, 4096, 4096) == 0.05
    assert spectral_lr(0.05, 1024, 4096) == 0.05
    assert abs(spectral_lr(1.0, 14336, 4096) - np.sqrt(3.5)) < 1e-15
    assert abs(spectral_lr(1.0, 14336, 4096) - 1.8708286933869707) < 1e-15
    assert spectral_lr(0.05, 4096, 14336) == 0.05
    assert spectral_lr(2.0, 10, 5, extra_scale=0.5) == 2.0 * np.sqrt(2.0) * 0.5


@pytest.mark.parametrize("shape,normuon_on", [((14, 6), False), ((6, 14), True), ((8, 4, 3, 3), True)])
def test_one_step_update_closed_form(shape, normuon_on):
    rng = np.random.default_rng(5)
    w = round_f32(0.02 * rng.standard_normal(shape))
    g = rng.standard_normal(shape)
    hp = MuonHParams(lr=0.05, normuon=normuon_on, mom_dtype="f32")
    out = shape[0]; f = int(np.prod(shape[1:]))
    r = muon_step(w, g, np.zeros(shape), np.zeros(out), hp)
    o = newton_schulz5((1 + MU) * flatten_param(g))
    if normuon_on:
        o, _ = normuon(o, np.zeros(out))
    lr_eff = 0.05 * np.sqrt(max(1.0, out / f))
    expect = round_f32(flatten_param(w) - lr_eff * o).reshape(shape)
    assert np.array_equal(r["w"], expect)


@pytest.mark.parametrize("normuon_on", [False, True])
def test_row_split_step_closed_form(normuon_on):
    # A fused [q; k; v] weight of 24 x 8 with blocks 16, 4, 4: Newton-Schulz
    # per block (each block's SVD), the spectral scale and NorMuon on the
    # whole parameter (24 / 8: lr * sqrt(3)).
    rng = np.random.default_rng(8)
    hs = (16, 4, 4)
    w = round_f32(0.02 * rng.standard_normal((24, 8)))
    g = rng.standard_normal((24, 8))
    hp = MuonHParams(lr=0.05, normuon=normuon_on, split_rows=hs, mom_dtype="f32")
    r = muon_step(w, g, np.zeros((24, 8)), np.zeros(24), hp)
    u = (1 + MU) * g
    o = np.concatenate([svd_closed_form(u[0:16]), svd_closed_form(u[16:20]), svd_closed_form(u[20:24])])
    assert rel(r["o"], o) < 1e-12
    if normuon_on:
        assert abs(np.linalg.norm(r["o_hat"]) - np.linalg.norm(r["o"])) < 1e-12 * np.linalg.norm(r["o"])
        o, _ = normuon(o, np.zeros(24))
    expect = flatten_param(w) - 0.05 * np.sqrt(3.0) * o
    assert np.all(np.abs(r["w"] - expect) <= 2.0 ** -24 * np.abs(expect) + 1e-12)   # one fp32 rounding


def test_row_split_needs_one_head():
    with pytest.raises(ValueError):
        muon_step(np.zeros((8, 4)), np.ones((8, 4)), np.zeros((8, 4)), hp=MuonHParams(heads=2, split_rows=(4, 4)))


def test_decoupled_weight_decay():
    rng = np.random.default_rng(6)
    w = round_f32(rng.standard_normal((5, 5)))
    g = rng.standard_normal((5, 5))
    a = muon_step(w, g, np.zeros((5, 5)), hp=MuonHParams(lr=0.1, weight_decay=0.0))
    b = muon_step(w, g, np.zeros((5, 5)), hp=MuonHParams(lr=0.1, weight_decay=0.5))
    assert np.allclose(b["w"] - a["w"], round_f32(w * (1 - 0.05)) - w, atol=1e-6)


def test_constant_gradient_keeps_direction():
    # With G_t = G every step, U_t is a positive multiple of G, so NS(U_t) = NS(G).
    g = np.random.default_rng(7).standard_normal((6, 10))
    m = np.zeros_like(g)
    for _ in range(3):
        m, u = nesterov_momentum(g, m, MU)
        assert rel(newton_schulz5(u), newton_schulz5(g)) < 1e-7


def test_conv_equals_reshaped_linear_bitwise():
    # "Fix convolution flattening...", "What it does": [out, *rest] under
    # flatten must step exactly like [out, prod(rest)].
    rng = np.random.default_rng(8)
    for shape in [(8, 4, 3, 3), (5, 3, 7), (4, 2, 2, 2, 2)]:
        w = round_f32(0.02 * rng.standard_normal(shape))
        g = rng.standard_normal(shape)
        hp = MuonHParams(normuon=True)
        a = muon_step(w, g, np.zeros(shape), np.zeros(shape[0]), hp)
        b = muon_step(w.reshape(shape[0], -1), g.reshape(shape[0], -1),
                      np.zeros((shape[0], int(np.prod(shape[1:])))), np.zeros(shape[0]), hp)
        assert np.array_equal(a["w"].reshape(shape[0], -1), b["w"])
        assert np.array_equal(a["v"], b["v"])


def test_negative_control_layer_mixing():
    # "Fix convolution flattening...", Validation: the defect presented
    # [2, 288] to Newton-Schulz instead of [2, 8, 36].
    fx = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "conv_negative_control.json")))
    n = fx["megabatch"]
    stack = np.random.default_rng(9).standard_normal([n] + fx["param_shape"])
    right = ns5_megabatch(stack.reshape(fx["correct_ns_view"]))
    wrong = newton_schulz5(stack.reshape(fx["defective_ns_view"])).reshape(fx["correct_ns_view"])
    assert rel(wrong, right) > 0.5
    for i in range(n):
        assert np.array_equal(right[i], newton_schulz5(stack[i].reshape(8, 36).copy()))


def test_round_bf16_against_brute_force():
    # Nearest bfloat16, ties to even, by exhaustive search over the bf16 grid
    # around each value.
    rng = np.random.default_rng(10)
    xs = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-30, 30, 2000),
                         [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 2.0 ** -130,
                          3.0 * 2.0 ** -134]])
    grid = synth.bf16_bits_to_f64(np.arange(0, 0x7F80, dtype=np.uint16))  # all finite positives
    for x in xs:
        a = abs(x)
        i = np.searchsorted(grid, a)
        cands = [grid[j] for j in (i - 1, i) if 0 <= j < len(grid)]
        best = min(cands, key=lambda y: (abs(y - a), int(np.float32(y).view(np.uint32) >> 16) & 1))
        assert round_bf16(np.array([x]))[0] == np.copysign(best, x), x


def test_round_bf16_specials():
    r = round_bf16(np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, 3.3893e38]))
    assert r[0] == 0 and np.signbit(r[1]) and r[2] == np.inf and r[3] == -np.inf
    assert r[4] == np.inf and r[5] == 255 * 2.0 ** 120
    assert np.isnan(round_bf16(np.array([np.nan])))[0]


def test_store_rounding_of_step_results():
    rng = np.random.default_rng(11)
    w = round_f32(rng.standard_normal((4, 6)))
    r = muon_step(w, rng.standard_normal((4, 6)), np.zeros((4, 6)), hp=MuonHParams(mom_dtype="bf16"))
    assert np.array_equal(r["m"], round_bf16(r["m"]))
    assert np.array_equal(r["w"], round_f32(r["w"]))
    assert np.array_equal(r["w_bf16"], round_bf16(r["w"]))


def test_empty_param_is_noop():
    r = muon_step(np.zeros((0, 5)), np.zeros((0, 5)), np.zeros((0, 5)), np.zeros(0),
                  MuonHParams(normuon=True))
    assert r["w"].shape == (0, 5) and r["v"].shape == (0,)
