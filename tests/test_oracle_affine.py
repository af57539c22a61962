"""Pins of the closed-form centred affine fit (oracle/affine.py) and of the
library's host solve. CPU only."""
import numpy as np

import linear_global_attention_amd as zb
from oracle import affine as oaf


def _data(n, d, seed):
    rng = np.random.default_rng(seed)
    O = rng.standard_normal((n, d)) * rng.uniform(0.5, 2.0, d) + rng.standard_normal(d)
    return rng, O


def test_planted_affine_recovered():
    """t = m + A (o - mean o) + c exactly: with no ridge the fit returns A,
    and mu + b = m + c (the mean of t)."""
    rng, O = _data(2000, 64, 1)
    A = rng.standard_normal((64, 64)) * 0.3
    m, c = rng.standard_normal(64), rng.standard_normal(64)
    T = m + (O - O.mean(axis=0)) @ A.T + c
    W, b, mu = oaf.affine_fit(oaf.affine_stats(O, T), 0.0)
    assert np.allclose(W, A, atol=1e-9)
    assert np.allclose(mu, O.mean(axis=0), atol=1e-12)
    assert np.allclose(mu + b, m + c, atol=1e-9)
    assert np.allclose(oaf.apply_affine(O, W, b, mu), T, atol=1e-8)


def test_ridge_equals_augmented_least_squares():
    """The normal-equation fit from the statistics equals least squares on
    the augmented (ridge-as-ordinary) system built from the centred data."""
    rng, O = _data(500, 64, 2)
    T = rng.standard_normal((500, 64)) + O[:, ::-1] * 0.5
    for lam in (0.0, 1e-3, 0.5):
        W1, b1, mu1 = oaf.affine_fit(oaf.affine_stats(O, T), lam)
        W2, b2, mu2 = oaf.affine_fit_direct(O, T, lam)
        assert np.allclose(W1, W2, atol=1e-9), lam
        assert np.allclose(b1, b2, atol=1e-12) and np.allclose(mu1, mu2, atol=1e-12)


def test_one_channel_closed_form():
    """d = 1: W = cov(o, t) / (var(o) (1 + lambda_rel)), b = mean t - mean o."""
    rng = np.random.default_rng(3)
    o = rng.standard_normal((300, 1)) * 2 + 1
    t = 0.7 * o + rng.standard_normal((300, 1)) * 0.1 - 3
    lam = 0.25
    W, b, mu = oaf.affine_fit(oaf.affine_stats(o, t), lam, d=1)
    oc, tc = o[:, 0] - o.mean(), t[:, 0] - t.mean()
    assert np.isclose(W[0, 0], (oc @ tc) / ((oc @ oc) * (1 + lam)), rtol=1e-12)
    assert np.isclose(b[0], t.mean() - o.mean(), rtol=1e-12) and np.isclose(mu[0], o.mean(), rtol=1e-12)


def test_stats_pool_samples():
    """Statistics add: two halves accumulated separately give the whole."""
    rng, O = _data(400, 64, 4)
    T = rng.standard_normal((400, 64))
    s = oaf.affine_stats(O, T)
    s2 = oaf.affine_stats(O[:150], T[:150]) + oaf.affine_stats(O[150:], T[150:])
    assert np.allclose(s, s2, rtol=1e-12, atol=1e-9)


def test_library_solve_matches_oracle():
    """zebra_affine_solve (host code, no GPU) on the oracle's statistics
    returns the oracle's fit, to fp32 output precision; bad input is an
    error."""
    rng, O = _data(3000, 64, 5)
    T = rng.standard_normal((3000, 64)) * 0.2 + O @ (rng.standard_normal((64, 64)) * 0.1).T
    s = oaf.affine_stats(O, T)
    for lam in (0.0, 1e-2):
        W, b, mu = zb.affine_solve(s, lam)
        Wr, br, mur = oaf.affine_fit(s, lam)
        assert np.allclose(W, Wr, rtol=2e-6, atol=2e-6), np.abs(W - Wr).max()
        assert np.allclose(b, br, rtol=1e-6, atol=1e-6) and np.allclose(mu, mur, rtol=1e-6, atol=1e-6)
    bad = s.copy()
    bad[0] = 0.0
    try:
        zb.affine_solve(bad, 0.0)
        raise AssertionError("n = 0 accepted")
    except zb.ZebraError:
        pass
    # a rank-deficient Gram with no ridge is rejected, with a ridge solved
    O2 = np.repeat(O[:, :1], 64, axis=1)
    s2 = oaf.affine_stats(O2, T)
    try:
        zb.affine_solve(s2, 0.0)
        raise AssertionError("singular Gram accepted")
    except zb.ZebraError:
        pass
    zb.affine_solve(s2, 1e-3)
