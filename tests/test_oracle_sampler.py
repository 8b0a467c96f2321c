"""Pins of the oracle's sampler (oracle/sampler.py) against the pages' numbers, closed forms and
exact solutions of the flow ODE."""
import json
import math
import os

import numpy as np
import pytest

from oracle import sampler as S

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))


def test_timesteps_are_the_pages():
    np.testing.assert_array_equal(S.timesteps(), GOLD["sampler_timesteps"]["value"])
    assert S.N_STEPS == GOLD["sampler_steps"]["value"]
    assert (S.SHIFT_VIDEO, S.SHIFT_AUDIO) == (GOLD["sigma_shift"]["video"], GOLD["sigma_shift"]["audio"])


def test_shift_closed_forms():
    sig = np.linspace(0.0, 1.0, 101)
    np.testing.assert_array_equal(S.shift(sig, 1.0), sig)                  # s = 1: identity
    assert S.shift(0.0, 10.0) == 0.0 and S.shift(1.0, 10.0) == 1.0
    assert abs(S.shift(0.5, 10.0) - 10.0 / 11.0) < 1e-15
    assert abs(S.shift(0.125, 3.0) - 0.3) < 1e-15
    assert (np.diff(S.shift(sig, 10.0)) > 0).all()                         # monotone
    # the shift is the conjugation of sigma/(1-sigma) by the factor s
    r = S.shift(sig[1:-1], 7.0)
    np.testing.assert_allclose(r / (1 - r), 7.0 * sig[1:-1] / (1 - sig[1:-1]), rtol=1e-13)


def test_sigma_schedules():
    sv, sa = S.sigmas(10.0), S.sigmas(3.0)
    assert len(sv) == 9 and sv[-1] == 0.0 and sa[-1] == 0.0
    t = np.array(GOLD["sampler_timesteps"]["value"], float) / 1000.0
    np.testing.assert_allclose(sv[:8], 10 * t / (1 + 9 * t), rtol=1e-15)
    np.testing.assert_allclose(sa[:8], 3 * t / (1 + 2 * t), rtol=1e-15)
    assert abs(sa[7] - 0.3) < 1e-15 and abs(sa[4] - 0.75) < 1e-15       # t = 125, 500 with s = 3


def _lam(s):
    return math.log((1 - s) / s)


def test_constant_x0_model_is_exact_every_step():
    """A model whose velocity is that of a fixed (x0, eps) pair keeps the flow path exactly: every
    state is (1 - sigma) x0 + sigma eps, and the final latent is x0."""
    rng = np.random.default_rng(0)
    L, Lv, d = 40, 30, 8
    x0, eps = rng.standard_normal((L, d)), rng.standard_normal((L, d))
    sv, sa = S.sigmas(10.0), S.sigmas(3.0)

    def model(x, i, t):
        return eps - x0                               # v = eps - x0, whatever the state
    # start from the exact state at sigma_0: the path x = (1-s) x0 + s eps (the sampler's own start
    # sigma_0 eps is that path only for x0 = 0, tested below)
    def run(sig, rows):
        x = (1 - sig[0]) * x0[rows] + sig[0] * eps[rows]
        x0p = np.zeros_like(x)
        for i in range(8):
            x, x0p = S.step(x, model(x, i, 0)[rows], x0p, sig, i)
            np.testing.assert_allclose(x, (1 - sig[i + 1]) * x0[rows] + sig[i + 1] * eps[rows],
                                       rtol=0, atol=1e-12)
        return x
    np.testing.assert_allclose(run(sv, slice(0, Lv)), x0[:Lv], atol=1e-12)
    np.testing.assert_allclose(run(sa, slice(Lv, L)), x0[Lv:], atol=1e-12)
    # the sampler's start is the empty latent (x0 = 0) at sigma_0
    xs = S.sample(eps, lambda x, i, t: eps, Lv)
    np.testing.assert_allclose(xs, 0.0, atol=1e-12)


def _affine_exact(sig, i, A, B):
    """Exact ODE step for x0_hat(lambda) = A + B lambda: y = x / sigma, dy/dlambda = e^lambda x0_hat."""
    l0, l1 = _lam(sig[i]), _lam(sig[i + 1])
    F = lambda l: math.exp(l) * (A + B * (l - 1.0))    # an antiderivative of e^l (A + B l)
    return F, l0, l1


def test_second_order_step_exact_for_x0_affine_in_lambda():
    """Given the exact state and the estimates of a model whose x0_hat is affine in lambda, every
    second-order step lands on the exact ODE solution; a first-order step does not (so the
    (h - 1 + e^-h)/h_prev term is pinned)."""
    rng = np.random.default_rng(1)
    A, B = rng.standard_normal(5), rng.standard_normal(5)
    for s in (10.0, 3.0, 1.0):
        sig = S.sigmas(s)
        for i in range(1, 7):                          # steps with a previous estimate and sigma > 0 after
            l_prev, l0, l1 = _lam(sig[i - 1]), _lam(sig[i]), _lam(sig[i + 1])
            F = lambda l: np.exp(l) * (A + B * (l - 1.0))
            y0 = rng.standard_normal(5)                 # any x / sigma at step i
            x = sig[i] * y0
            x0h = A + B * l0
            v = (x - x0h) / sig[i]
            x_exact = sig[i + 1] * (y0 + F(l1) - F(l0))
            got, got_x0h = S.step(x, v, A + B * l_prev, sig, i)
            np.testing.assert_allclose(got_x0h, x0h, rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(got, x_exact, rtol=1e-11, atol=1e-11)
            _, a, b, c = S.step_coefficients(sig, i)
            first = a * x + (b + c) * x0h               # the same step with the slope term dropped
            assert np.abs(first - x_exact).max() > 1e-6


def test_last_step_returns_x0_hat_and_first_step_is_first_order():
    rng = np.random.default_rng(2)
    sig = S.sigmas(10.0)
    x, v = rng.standard_normal(6), rng.standard_normal(6)
    xn, x0h = S.step(x, v, np.full(6, np.nan), sig, 7)
    np.testing.assert_array_equal(xn, x0h)
    np.testing.assert_allclose(x0h, x - sig[7] * v, rtol=1e-15)
    _, a, b, c = S.step_coefficients(sig, 0)
    assert c == 0.0
    assert abs(b - ((1 - sig[1]) - (1 - sig[0]) * sig[1] / sig[0])) < 1e-14
