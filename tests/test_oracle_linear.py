"""Pins of the oracle's linear path: RMSNorm, 2D rotary, channel-softmax
feature map, KV-state linear attention and the centred affine correction
(Zebra3D pages, "Speedup scales with the number of input views" and "A
closed-form fit avoids retraining from scratch"), checked against brute
force, closed forms, invariants and a hand-derived golden example."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import linear as olin
from oracle.layout import TileMap

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_zero_qk():
    fx = json.load(open(os.path.join(GOLD, "linear_zero_qk_example.json")))
    tm = TileMap(1, 1, 8, 16)
    N, d = tm.N, 64
    Q = np.zeros((N, 1, d))
    K = np.zeros((N, 1, d))
    V = np.zeros((N, 1, d))
    V[0, 0, 0] = 1.0
    V[:, 0, 1] = 1.0
    V[78, 0, 2] = 1.0
    o = olin.linear_attention(Q, K, V, tm)
    W = 2 * np.eye(d)[None]
    b = np.zeros((1, d)); b[0, 0] = 0.5
    mu = np.zeros((1, d)); mu[0, 1] = 1.0
    yv = olin.linear_attention(Q, K, V, tm, W, b, mu)
    for ch in range(3):
        want_o = float(Fraction(fx["expected_o"][f"ch{ch}"]))
        assert np.allclose(o[:, 0, ch], want_o, atol=1e-14)
    assert np.allclose(yv[:, 0, 0], 2 / 129 + 0.5, atol=1e-14)
    assert np.allclose(yv[:, 0, 1], 1.0, atol=1e-14)
    assert np.allclose(yv[:, 0, 2], 2 / 129, atol=1e-14)
    assert np.allclose(yv[:, 0, 3:], 0.0, atol=1e-14)


def test_factored_equals_brute_force_quadratic_sum():
    """o_i = sum_j w_ij v_j / sum_j w_ij, w_ij = phi(q_i).phi(k_j), written
    out with explicit loops (O(N^2 d))."""
    tm = TileMap(2, 2, 3, 4)
    N, d = tm.N, 64
    g = np.random.default_rng(0)
    Q, K, V = (g.standard_normal((N, 1, d)) * 2 for _ in range(3))
    got = olin.linear_attention(Q, K, V, tm)[:, 0]
    pq = olin.featurize(Q[:, 0], tm)
    pk = olin.featurize(K[:, 0], tm)
    for i in range(N):
        num = [0.0] * d
        den = 0.0
        for j in range(N):
            w = sum(pq[i, a] * pk[j, a] for a in range(d))
            den += w
            for c in range(d):
                num[c] += w * V[j, 0, c]
        assert np.abs(got[i] - np.array(num) / den).max() < 1e-12


def test_feature_map_is_a_distribution_and_constant_v_passes_through():
    tm = TileMap(2, 3, 6, 7)
    g = np.random.default_rng(1)
    Q, K = g.standard_normal((2, tm.N, 1, 64)) * 3
    phi = olin.featurize(K[:, 0], tm)
    assert (phi > 0).all() and np.allclose(phi.sum(axis=1), 1.0, atol=1e-14)
    c = g.standard_normal(64)
    V = np.broadcast_to(c, (tm.N, 1, 64))
    assert np.abs(olin.linear_attention(Q, K, V, tm)[:, 0] - c).max() < 1e-12
    # the feature map equals a shifted-exponential normalisation
    x = g.standard_normal((5, 64))
    e = np.exp(x)
    assert np.allclose(olin.feature_map(x), e / e.sum(axis=1, keepdims=True), atol=1e-15)


def test_rms_norm_unit_mean_square_and_scale_invariance():
    g = np.random.default_rng(2)
    x = g.standard_normal((10, 64)) * 5
    y = olin.rms_norm(x, eps=0.0)
    assert np.allclose((y * y).mean(axis=1), 1.0, atol=1e-13)
    assert np.allclose(olin.rms_norm(7.0 * x, eps=0.0), y, atol=1e-13)
    gain = g.standard_normal(64)
    assert np.allclose(olin.rms_norm(x, gain, eps=0.0), y * gain, atol=1e-13)
    # eps = 1e-6 barely moves unit-scale rows and keeps zero rows finite
    assert np.allclose(olin.rms_norm(x), y, atol=1e-6)
    assert np.all(olin.rms_norm(np.zeros((1, 64))) == 0.0)


def test_rope_properties():
    g = np.random.default_rng(3)
    x = g.standard_normal((6, 64))
    pr = np.array([0, 1, 5, 36, 2, 0])
    pc = np.array([0, 3, 5, 0, 36, 9])
    y = olin.rope2d(x, pr, pc)
    # a rotation: norms are kept, position (0, 0) is the identity
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), atol=1e-12)
    assert np.array_equal(y[0], x[0])
    # relative: <R(p)a, R(p')b> depends only on p - p'
    a, b = g.standard_normal((2, 1, 64))
    ip = lambda p, q: float((olin.rope2d(a, *p) @ olin.rope2d(b, *q).T)[0, 0])  # noqa: E731
    P = lambda r, c: (np.array([r]), np.array([c]))  # noqa: E731
    assert ip(P(3, 7), P(1, 2)) == pytest.approx(ip(P(12, 20), P(10, 15)), abs=1e-12)
    assert ip(P(3, 7), P(1, 2)) != pytest.approx(ip(P(3, 7), P(2, 2)), abs=1e-6)
    # the row turns channels [0,32), the column [32,64); pair (j, j+16)
    # turns by p * 100^(-j/16): measure each pair's angle at p = 1
    e = np.zeros((1, 64)); e[0, :16] = 1.0; e[0, 32:48] = 1.0
    yr = olin.rope2d(e, np.array([1]), np.array([0]))
    yc = olin.rope2d(e, np.array([0]), np.array([1]))
    ang_r = np.arctan2(yr[0, 16:32], yr[0, :16])
    ang_c = np.arctan2(yc[0, 48:64], yc[0, 32:48])
    assert np.allclose(ang_r, 100.0 ** (-np.arange(16) / 16), atol=1e-14)
    assert np.allclose(ang_c, ang_r, atol=1e-14)
    assert np.array_equal(yr[0, 32:], e[0, 32:]) and np.array_equal(yc[0, :32], e[0, :32])
    assert ang_r[1] / ang_r[0] == pytest.approx(100.0 ** (-1 / 16))


def test_positions_specials_at_origin():
    tm = TileMap(2, 3, 4, 5)
    pr, pc = olin.positions(tm)
    assert pr[:3].tolist() == [0, 0, 0] and pc[:3].tolist() == [0, 0, 0]
    t = 23 + 3 + 2 * 5 + 4  # frame 1, patch (2, 4)
    assert (pr[t], pc[t]) == (2, 4)


def test_affine_orientation_and_identity():
    g = np.random.default_rng(4)
    o = g.standard_normal((9, 64))
    assert np.array_equal(olin.affine(o), o)
    mu = g.standard_normal(64)
    assert np.allclose(olin.affine(o, np.eye(64), None, mu), o, atol=1e-14)
    W = g.standard_normal((64, 64))
    b = g.standard_normal(64)
    y = olin.affine(o, W, b, mu)
    # y - W o is the same vector (I - W) mu + b for every row; W o written
    # out as sum_c W[a][c] o[c]
    Wo = np.array([[sum(W[a, c] * o[i, c] for c in range(64)) for a in range(64)] for i in range(9)])
    diff = y - Wo
    assert np.allclose(diff, diff[0], atol=1e-12)
    assert np.allclose(diff[0], mu - W @ mu + b, atol=1e-12)


def test_rows_and_mean_output():
    tm = TileMap(2, 2, 8, 9)
    g = np.random.default_rng(5)
    Q, K, V = g.standard_normal((3, tm.N, 2, 64))
    W = np.eye(64)[None].repeat(2, 0) + 0.01 * g.standard_normal((2, 64, 64))
    b = 0.01 * g.standard_normal((2, 64))
    mu = np.stack([olin.mean_output(Q[:, h], K[:, h], V[:, h], tm) for h in range(2)])
    full = olin.linear_attention(Q, K, V, tm, W, b, mu)
    rows = np.array([[0, 0], [0, 17], [1, 5], [1, tm.N - 1]])
    got = olin.linear_rows(Q, K, V, tm, rows, W, b, mu)
    assert np.abs(got - full[rows[:, 1], rows[:, 0]]).max() < 1e-13
    plain = olin.linear_attention(Q, K, V, tm)
    assert np.allclose(plain.mean(axis=0), mu, atol=1e-14)
    # centring: with mu the mean output, the corrected mean is mu + b
    assert np.allclose(full.mean(axis=0), mu + b, atol=1e-13)


def _brute_head(Q, K, V, tm, W, b, mu, gq, gk, eps, base):
    """One head's corrected linear output written out token by token with
    math-module scalars: RMSNorm with gain, the pair rotation by
    p * base^(-j/16) per 32-channel half, the channel softmax, the O(N^2)
    weighted sum and y_a = mu_a + b_a + sum_c W[a][c] (o_c - mu_c)."""
    N, d = Q.shape
    C = tm.C

    def pos(t):
        loc = t % tm.tpf
        return (0, 0) if loc < tm.S else divmod(loc - tm.S, C)

    def phi(x, g, t):
        ms = sum(c * c for c in x) / d
        r = math.sqrt(ms + eps)
        xn = [x[c] / r * g[c] for c in range(d)]
        out = list(xn)
        for half, p in enumerate(pos(t)):
            for j in range(16):
                a = p * base ** (-j / 16)
                lo, hi = xn[32 * half + j], xn[32 * half + 16 + j]
                out[32 * half + j] = lo * math.cos(a) - hi * math.sin(a)
                out[32 * half + 16 + j] = hi * math.cos(a) + lo * math.sin(a)
        m = max(out)
        e = [math.exp(c - m) for c in out]
        s = sum(e)
        return [c / s for c in e]

    pk = [phi(K[j], gk, j) for j in range(N)]
    Y = np.empty((N, d))
    for i in range(N):
        pq = phi(Q[i], gq, i)
        w = [sum(pq[a] * pk[j][a] for a in range(d)) for j in range(N)]
        den = sum(w)
        o = [sum(w[j] * V[j][c] for j in range(N)) / den for c in range(d)]
        Y[i] = [mu[a] + b[a] + sum(W[a][c] * (o[c] - mu[c]) for c in range(d)) for a in range(d)]
    return Y


def test_multi_head_wrapper_takes_each_heads_parameters():
    """linear_attention and linear_rows with per-head W, b, mu, RMSNorm gains,
    a non-default eps and rotary base: every head equals the scalar brute
    force of that head with that head's parameters, and swapping the heads'
    W (or gains) changes the result, so a per-head mix-up is caught."""
    tm = TileMap(2, 1, 3, 5)
    g = np.random.default_rng(8)
    H, d = 2, 64
    Q, K, V = g.standard_normal((3, tm.N, H, d))
    W = np.eye(d)[None].repeat(H, 0) + 0.3 * g.standard_normal((H, d, d))
    b = g.standard_normal((H, d))
    mu = g.standard_normal((H, d))
    gq = 0.5 + g.random((H, d))
    gk = 0.5 + g.random((H, d))
    eps, base = 1e-3, 10000.0
    got = olin.linear_attention(Q, K, V, tm, W, b, mu, gq, gk, eps, base)
    for h in range(H):
        want = _brute_head(Q[:, h], K[:, h], V[:, h], tm, W[h], b[h], mu[h], gq[h], gk[h], eps, base)
        assert np.abs(got[:, h] - want).max() < 1e-11, h
    rows = np.array([[0, 3], [1, 0], [1, tm.N - 1]])
    sub = olin.linear_rows(Q, K, V, tm, rows, W, b, mu, gq, gk, eps, base)
    assert np.abs(sub - got[rows[:, 1], rows[:, 0]]).max() < 1e-13
    swapped = olin.linear_attention(Q, K, V, tm, W[::-1], b, mu, gq, gk, eps, base)
    assert np.abs(swapped - got).max() > 1e-2
    swapped = olin.linear_attention(Q, K, V, tm, W, b, mu, gq[::-1], gk[::-1], eps, base)
    assert np.abs(swapped - got).max() > 1e-4
    # eps and base reach the result
    assert np.abs(olin.linear_attention(Q, K, V, tm, W, b, mu, gq, gk, 1e-6, base) - got).max() > 1e-6
    assert np.abs(olin.linear_attention(Q, K, V, tm, W, b, mu, gq, gk, eps, 100.0) - got).max() > 1e-4


def test_pins_catch_planted_mistakes(monkeypatch):
    tm = TileMap(2, 2, 3, 4)
    g = np.random.default_rng(0)
    Q, K, V = (g.standard_normal((tm.N, 1, 64)) * 2 for _ in range(3))
    good = olin.linear_attention(Q, K, V, tm)
    # transposed state: uses S^T instead of S
    real = olin.kv_state
    monkeypatch.setattr(olin, "kv_state", lambda pk, Vh: (real(pk, Vh)[0].T, real(pk, Vh)[1]))
    bad = olin.linear_attention(Q, K, V, tm)
    assert np.abs(bad - good).max() > 1e-3
