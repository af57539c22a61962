"""Pins of the oracle's backward passes (oracle/backward.py; Zebra3D pages,
"A closed-form fit avoids retraining from scratch", the optional training
stage after conversion).

Every gradient is pinned by central finite differences of the forward map it
differentiates (oracle.linear.linear_head, oracle.sparse.sparse_attention,
both pinned in their own tests), coordinate by coordinate over every token.
Besides: the tile-sparse backward at y = 0 against torch's float64 autograd
of dense softmax attention, exact invariants of softmax attention (the key
gradients sum to zero, the value gradients to the output gradients), the
RMSNorm scale invariance of the linear backward (q . dq = 0 at eps = 0), and
the sampled-row helpers against the full backward."""
import numpy as np
import pytest
import torch

from oracle import backward as ob
from oracle import linear as olin
from oracle import sparse as osp
from oracle.layout import TileMap, keep_count


def _rng_inputs(tm, H, seed, scale=(1.5, 1.5, 1.0)):
    g = np.random.default_rng(seed)
    Q, K, V = (g.standard_normal((tm.N, H, 64)) * s for s in scale)
    dY = g.standard_normal((tm.N, H, 64))
    return Q, K, V, dY, g


def _fd_check(loss, X, grad, coords, h, rtol):
    """Central differences of loss at the coordinates coords [(token, channel)]
    of X against grad; returns the largest relative error."""
    worst = 0.0
    scale = np.abs(grad).max()
    for (i, c) in coords:
        x0 = X[i, c]
        X[i, c] = x0 + h
        lp = loss()
        X[i, c] = x0 - h
        lm = loss()
        X[i, c] = x0
        fd = (lp - lm) / (2 * h)
        err = abs(fd - grad[i, c]) / scale
        worst = max(worst, err)
        assert err < rtol, (i, c, fd, grad[i, c])
    return worst


def _coords(n, g, per_token=1):
    return [(i, int(c)) for i in range(n) for c in g.choice(64, per_token, replace=False)]


@pytest.mark.parametrize("with_affine", [False, True])
def test_linear_backward_finite_differences(with_affine):
    """Every token, every tensor, against central differences of the
    linear-stage forward (with W, b, mu, gains, eps and base away from their
    defaults in one case; b and mu must not change the gradient)."""
    tm = TileMap(1, 2, 3, 5)
    Q, K, V, dY, g = _rng_inputs(tm, 1, 0)
    kw = {}
    if with_affine:
        kw = dict(W=np.eye(64) + 0.2 * g.standard_normal((64, 64)), gq=0.5 + g.random(64),
                  gk=0.5 + g.random(64), eps=1e-3, base=1000.0)
    b = mu = None
    if with_affine:
        b, mu = g.standard_normal(64), g.standard_normal(64)
    q, k, v, dy = Q[:, 0].copy(), K[:, 0].copy(), V[:, 0].copy(), dY[:, 0]
    dq, dk, dv = ob.linear_head_backward(q, k, v, dy, tm, **kw)
    fkw = {kk: kw[kk] for kk in ("W", "gq", "gk", "eps", "base") if kk in kw}

    def loss():
        return float((dy * olin.linear_head(q, k, v, tm, None, b=b, mu=mu, **fkw)).sum())

    for X, G in ((q, dq), (k, dk), (v, dv)):
        _fd_check(loss, X, G, _coords(tm.N, g, 3), 1e-5, 1e-7)


def test_linear_backward_rms_scale_invariance():
    """At eps = 0 RMSNorm is invariant to scaling its input, so the gradient
    of every q and k row is orthogonal to the row: q . dq = 0, k . dk = 0."""
    tm = TileMap(2, 1, 5, 6)
    Q, K, V, dY, g = _rng_inputs(tm, 2, 1)
    W = np.eye(64)[None] + 0.1 * g.standard_normal((2, 64, 64))
    dQ, dK, dV = ob.linear_backward(Q, K, V, dY, tm, W=W, eps=0.0)
    for X, G in ((Q, dQ), (K, dK)):
        dots = np.abs((X * G).sum(axis=2))
        assert dots.max() < 1e-12 * np.abs(X).max() * np.abs(G).max() * 64


def test_linear_backward_w_enters_as_dy_w():
    """The affine correction enters the backward only as dO = dY W: the
    gradients with W equal those with the identity and dY W."""
    tm = TileMap(2, 1, 4, 4)
    Q, K, V, dY, g = _rng_inputs(tm, 1, 2)
    W = g.standard_normal((1, 64, 64))
    a = ob.linear_backward(Q, K, V, dY, tm, W=W)
    b = ob.linear_backward(Q, K, V, dY @ W[0], tm)
    for x, y in zip(a, b):
        assert np.abs(x - y).max() < 1e-12 * np.abs(y).max()


def _sparse_case(tm, y, seed):
    Q, K, V, dO, g = _rng_inputs(tm, 1, seed)
    O, sel, tie = osp.sparse_attention(Q, K, V, tm, y)
    assert not tie.any()
    return Q, K, V, dO, sel, g


@pytest.mark.parametrize("y", [0.5, 1.0])
def test_sparse_backward_finite_differences(y):
    """Every token (special, in kept and in omitted tiles, in the 8x8, 8x1,
    1x8 and 1x1 tiles of a 9x9 grid), one or two channels each, of Q, K and V
    against central differences of the tile-sparse forward; the selection
    stays the forward's under the perturbation."""
    tm = TileMap(2, 2, 9, 9)
    Q, K, V, dO, sel, g = _sparse_case(tm, y, 3)
    assert sel.shape[2] == keep_count(y, tm.T)
    dQ, dK, dV = ob.sparse_backward(Q, K, V, dO, tm, y)

    def loss():
        O, s2, _ = osp.sparse_attention(Q, K, V, tm, y)
        assert np.array_equal(s2, sel)
        return float((dO * O).sum())

    for X, G in ((Q, dQ), (K, dK), (V, dV)):
        # X[:, 0, :] is a view: the perturbation reaches the forward's inputs
        _fd_check(loss, X[:, 0, :], G[:, 0, :], _coords(tm.N, g, 1), 1e-5, 1e-7)


def test_sparse_backward_y0_is_dense_autograd():
    """At y = 0 every tile is kept: the tile-sparse backward is the backward
    of dense softmax attention, here torch's float64 autograd of
    scaled_dot_product_attention on the CPU."""
    tm = TileMap(2, 3, 10, 7)
    Q, K, V, dO, _ = _rng_inputs(tm, 2, 4)
    got = ob.sparse_backward(Q, K, V, dO, tm, 0.0)
    t = [torch.tensor(np.ascontiguousarray(x.transpose(1, 0, 2)), dtype=torch.float64, requires_grad=True)
         for x in (Q, K, V)]
    out = torch.nn.functional.scaled_dot_product_attention(t[0], t[1], t[2])
    out.backward(torch.tensor(dO.transpose(1, 0, 2)))
    for a, x in zip(got, t):
        want = x.grad.numpy().transpose(1, 0, 2)
        assert np.abs(a - want).max() < 1e-12 * np.abs(want).max()


@pytest.mark.parametrize("y", [0.3, 0.7, 1.0])
def test_sparse_backward_softmax_invariants(y):
    """Every row's probabilities (over tokens, landmarks and its self key)
    sum to one and a landmark hands 1/n of its gradient to each of its n
    tokens, so the value gradients sum to the output gradients and the key
    gradients sum to zero (each row's logit gradients sum to zero and the
    landmark bias ln n does not depend on K)."""
    tm = TileMap(3, 1, 11, 13)
    Q, K, V, dO, _ = _rng_inputs(tm, 1, 5)
    dQ, dK, dV = ob.sparse_backward(Q, K, V, dO, tm, y)
    assert np.abs(dV.sum(axis=0) - dO.sum(axis=0)).max() < 1e-10
    assert np.abs(dK.sum(axis=0)).max() < 1e-10 * np.abs(dK).max() * tm.N


def test_sparse_dq_rows_matches_full_backward():
    tm = TileMap(2, 2, 9, 11)
    Q, K, V, dO, g = _rng_inputs(tm, 1, 6)
    y = 0.6
    dQ, _, _ = ob.sparse_head_backward(Q[:, 0], K[:, 0], V[:, 0], dO[:, 0], tm, y)
    toks = np.concatenate([tm.specials, g.choice(tm.N, 40, replace=False)])
    got = ob.sparse_dq_rows(Q[:, 0], K[:, 0], V[:, 0], dO[:, 0], tm, y, toks)
    assert np.abs(got - dQ[toks]).max() < 1e-12 * np.abs(dQ).max()
