"""Pins of the oracle's attention-mass coverage and landmark error
(Zebra3D pages, "Sensitive stages also concentrate their attention"):
a scalar brute force, the closed cases y = 0 and y = 1, Jensen's
inequality, identical-key tiles, nesting of the kept sets, scipy's softmax
for the special-key share, and planted mistakes that must fail."""
import math

import numpy as np
import pytest
from scipy.special import softmax

from oracle import coverage as ocov
from oracle import sparse as osp
from oracle.layout import TileMap


def _qkv(tm, H, seed, scale=1.0):
    g = np.random.default_rng(seed)
    return (g.standard_normal((tm.N, H, 64)) * scale, g.standard_normal((tm.N, H, 64)) * scale,
            g.standard_normal((tm.N, H, 64)))


def _brute(Q, K, tm, t, kept):
    """Row by row with math.exp over explicit key lists."""
    kbar = [[sum(K[j][c] for j in tm.tokens[u]) / len(tm.tokens[u]) for c in range(64)] for u in range(tm.T)]
    cov, err = [], []
    for i in tm.tokens[t]:
        dot = lambda a, b: sum(x * y for x, y in zip(a, b)) / 8.0  # noqa: E731
        lg = [dot(Q[i], K[j]) for j in range(tm.N)]
        m = max(lg)
        w = [math.exp(x - m) for x in lg]
        covered = sum(w[j] for u in kept for j in tm.tokens[u])
        cov.append(covered / sum(w))
        omitted = [u for u in range(tm.T) if u not in set(kept)]
        E = sum(w[j] for u in omitted for j in tm.tokens[u])
        Lm = sum(len(tm.tokens[u]) * math.exp(dot(Q[i], kbar[u]) - m) for u in omitted)
        err.append(1.0 - Lm / E if omitted else 0.0)
    return np.mean(cov), np.mean(err)


@pytest.mark.parametrize("y", [0.25, 0.5, 0.75])
def test_matches_scalar_brute_force(y):
    tm = TileMap(2, 2, 9, 11)
    Q, K, _ = _qkv(tm, 1, 1)
    cov, err = ocov.coverage_head(Q[:, 0], K[:, 0], tm, y)
    kbar, _, _ = osp.landmarks(K[:, 0], K[:, 0], tm)
    sel, _, _ = osp.select_tiles(Q[:, 0], kbar, tm, y)
    for t in range(tm.T):
        bc, be = _brute(Q[:, 0].tolist(), K[:, 0].tolist(), tm, t, sel[t].tolist())
        assert abs(cov[t] - bc) < 1e-12 and abs(err[t] - be) < 1e-12, t


def test_closed_cases_all_and_no_tiles():
    tm = TileMap(3, 0, 10, 12)  # no special tokens
    Q, K, _ = _qkv(tm, 2, 2)
    cov, err = ocov.coverage(Q, K, tm, 0.0)  # every tile kept
    assert np.allclose(cov, 1.0, atol=1e-14) and np.all(err == 0.0)
    cov, err = ocov.coverage(Q, K, tm, 1.0)  # no tile kept
    assert np.all(cov == 0.0)
    assert np.all(err >= 0.0) and np.all(err < 1.0)


def test_special_share_at_y0_matches_scipy():
    """With every tile kept, the uncovered mass is exactly the special keys'
    share of each row's softmax."""
    tm = TileMap(2, 5, 8, 8)
    Q, K, _ = _qkv(tm, 1, 3)
    cov, _ = ocov.coverage_head(Q[:, 0], K[:, 0], tm, 0.0)
    for t in range(tm.T):
        p = softmax(Q[tm.tokens[t], 0] @ K[:, 0].T / 8.0, axis=1)
        assert abs(cov[t] - (1.0 - p[:, tm.specials].sum(axis=1)).mean()) < 1e-13


def test_jensen_bound_and_identical_key_tiles():
    tm = TileMap(3, 1, 11, 9)
    Q, K, _ = _qkv(tm, 1, 4, scale=2.0)
    _, err = ocov.coverage_head(Q[:, 0], K[:, 0], tm, 0.6)
    assert np.all(err > 0.0) and np.all(err < 1.0)  # random keys: a strict gap
    for u in range(tm.T):  # every tile's keys identical: landmarks are exact
        K[tm.tokens[u]] = K[tm.tokens[u][0]]
    _, err = ocov.coverage_head(Q[:, 0], K[:, 0], tm, 0.6)
    assert np.abs(err).max() < 1e-12


def test_coverage_grows_as_more_tiles_are_kept():
    """Top-k lists are nested, so coverage cannot fall as y falls."""
    tm = TileMap(4, 2, 16, 16)
    Q, K, _ = _qkv(tm, 1, 5, scale=1.5)
    prev = None
    for y in (0.9, 0.75, 0.5, 0.25, 0.0):
        cov, _ = ocov.coverage_head(Q[:, 0], K[:, 0], tm, y)
        if prev is not None:
            assert np.all(cov >= prev - 1e-14)
        prev = cov


def test_planted_mistakes_fail(monkeypatch):
    tm = TileMap(2, 2, 9, 11)
    Q, K, _ = _qkv(tm, 1, 1)
    kbar, _, _ = osp.landmarks(K[:, 0], K[:, 0], tm)
    sel, _, _ = osp.select_tiles(Q[:, 0], kbar, tm, 0.5)
    bc, be = _brute(Q[:, 0].tolist(), K[:, 0].tolist(), tm, 0, sel[0].tolist())
    real_log = np.log
    # a landmark that forgets its ln n_u term
    monkeypatch.setattr(ocov.np, "log", lambda x: 0.0 * real_log(x))
    c, e = ocov.row_coverage(Q[:, 0], K[:, 0], tm, 0, sel[0], kbar)
    assert abs(e.mean() - be) > 1e-3
    monkeypatch.setattr(ocov.np, "log", real_log)
    # covering the omitted tiles instead of the kept ones
    omitted = np.setdiff1d(np.arange(tm.T), sel[0])
    c, _ = ocov.row_coverage(Q[:, 0], K[:, 0], tm, 0, omitted, kbar)
    assert abs(c.mean() - bc) > 1e-3
