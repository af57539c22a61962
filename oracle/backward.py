"""Gradients of the linear and the tile-sparse attention stages (oracle
side, float64): the vector-Jacobian products of the forward maps in
oracle.linear and oracle.sparse.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: Zebra3D pages, "A closed-form fit avoids retraining from scratch":
after the training-free conversion an optional training stage (task
supervision plus output, feature and relational distillation) fine-tunes the
converted model, so gradients flow back through its linear and tile-sparse
stages.

Readings (the pages give no backward pass):
  * the backward of a stage takes the gradient dY of its output Y and
    returns the gradients of sum(dY * Y) with respect to the stage inputs
    Q, K and V;
  * the centred affine correction (W, b, mu), the RMSNorm gains, eps and the
    rotary base are constants of the backward: the correction comes from the
    closed-form fit, not from gradient steps. b and mu drop out; W enters as
    dO = dY W;
  * the top-k tile selection is piecewise constant in Q and K, so it passes
    no gradient: the backward uses the tiles the forward kept;
  * a landmark is the mean of its tile's keys and values, so every token of
    an omitted tile receives 1/n_u of its landmark's key and value
    gradients; the ln n_u term of a landmark's logit is a constant.

Each function runs the forward map of one head again, keeping its
intermediates, then takes the chain rule back through the same steps in
reverse order.
"""
from __future__ import annotations

import math

import numpy as np

from .layout import TileMap
from . import linear as olin
from . import sparse as osp


# ---------------------------------------------------------------- linear

def rms_norm_backward(x, gain, eps, dy):
    """Gradient with respect to x of sum(dy * RMSNorm(x)) (oracle.linear.rms_norm):
    y = (x / r) g with r = sqrt(mean(x^2) + eps), so
    dx = (dy g) / r - x * sum((dy g) x) / (d r^3)."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    d = x.shape[-1]
    r = np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    dxh = dy if gain is None else dy * np.asarray(gain, dtype=np.float64)
    return dxh / r - x * (dxh * x).sum(axis=-1, keepdims=True) / (d * r ** 3)


def rope2d_backward(dy, prow, pcol, base=100.0):
    """Gradient through oracle.linear.rope2d. Each channel pair turns by an
    angle, an orthogonal map, so its transpose turns by minus that angle:
    the rotation at positions (-prow, -pcol)."""
    return olin.rope2d(dy, -np.asarray(prow), -np.asarray(pcol), base)


def feature_map_backward(u, du):
    """Gradient through the channel softmax u = softmax(x):
    dx = u * (du - sum(u * du))."""
    return u * (du - (u * du).sum(axis=-1, keepdims=True))


def linear_head_backward(Q_h, K_h, V_h, dY_h, tm: TileMap, W=None, gq=None, gk=None,
                         eps=1e-6, base=100.0):
    """Gradients (dQ, dK, dV), each [N][d] float64, of sum(dY * Y) for one
    head, where Y = oracle.linear.linear_head(Q, K, V, ...) over all N tokens
    (b and mu do not change the gradient)."""
    pr, pc = olin.positions(tm)
    # forward, keeping the intermediates
    u = olin.feature_map(olin.rope2d(olin.rms_norm(Q_h, gq, eps), pr, pc, base))   # phi(q)
    pk = olin.feature_map(olin.rope2d(olin.rms_norm(K_h, gk, eps), pr, pc, base))  # phi(k)
    V = np.asarray(V_h, dtype=np.float64)
    S, z = olin.kv_state(pk, V)          # S = phi(K)^T V, z = sum phi(k)
    num = u @ S                          # numerator of o
    den = u @ z                          # phi(q) . z
    o = num / den[:, None]
    # y = mu + (o - mu) W^T + b
    dY = np.asarray(dY_h, dtype=np.float64)
    do = dY if W is None else dY @ np.asarray(W, dtype=np.float64)
    # o = num / den
    dnum = do / den[:, None]
    dden = -(do * o).sum(axis=1) / den
    # num = u S, den = u . z
    du = dnum @ S.T + dden[:, None] * z[None, :]
    dS = u.T @ dnum
    dz = u.T @ dden
    # S = phi(K)^T V, z = sum of phi(k)
    dpk = V @ dS.T + dz[None, :]
    dV = pk @ dS
    dQ = rms_norm_backward(Q_h, gq, eps, rope2d_backward(feature_map_backward(u, du), pr, pc, base))
    dK = rms_norm_backward(K_h, gk, eps, rope2d_backward(feature_map_backward(pk, dpk), pr, pc, base))
    return dQ, dK, dV


def linear_backward(Q, K, V, dY, tm: TileMap, W=None, gq=None, gk=None, eps=1e-6, base=100.0):
    """All heads: (dQ, dK, dV), each [N][H][d] float64. W [H][d][d], gq, gk
    [H][d] (None: identity / ones)."""
    N, H, d = Q.shape
    out = [np.empty((N, H, d)) for _ in range(3)]
    pick = lambda a, h: None if a is None else np.asarray(a)[h]  # noqa: E731
    for h in range(H):
        g = linear_head_backward(Q[:, h], K[:, h], V[:, h], dY[:, h], tm, pick(W, h),
                                 pick(gq, h), pick(gk, h), eps, base)
        for a, b in zip(out, g):
            a[:, h] = b
    return tuple(out)


# ---------------------------------------------------------------- sparse

def _softmax_rows_backward(lg, Vals, dO):
    """Rows of softmax attention given the logits lg [r][m] (-inf where not
    visible) and the values Vals [m][d]: returns (P, ds) with P the
    probabilities and ds = P * (dP - sum(P * dP)) the logit gradients,
    dP = dO Vals^T."""
    m = lg.max(axis=1, keepdims=True)
    w = np.exp(lg - m)
    P = w / w.sum(axis=1, keepdims=True)
    dP = dO @ Vals.T
    return P, P * (dP - (P * dP).sum(axis=1, keepdims=True))


def sparse_head_backward(Q_h, K_h, V_h, dO_h, tm: TileMap, y: float, sel=None):
    """Gradients (dQ, dK, dV), each [N][d] float64, of sum(dO * O) for one
    head of the tile-sparse stage O = oracle.sparse.sparse_head(...) over all
    N query tokens. sel [T][k]: the kept tiles of every query tile (default:
    oracle.sparse.select_tiles on these inputs)."""
    N, d = Q_h.shape
    inv = 1.0 / math.sqrt(d)
    Q = np.asarray(Q_h, dtype=np.float64)
    K = np.asarray(K_h, dtype=np.float64)
    V = np.asarray(V_h, dtype=np.float64)
    dO = np.asarray(dO_h, dtype=np.float64)
    kbar, vbar, logn = osp.landmarks(K_h, V_h, tm)
    if sel is None:
        sel, _, _ = osp.select_tiles(Q_h, kbar, tm, y)
    kept = np.zeros((tm.T, tm.T), dtype=bool)   # kept[t][u]: query tile t keeps key tile u
    if sel.shape[1]:
        np.put_along_axis(kept, np.asarray(sel, dtype=np.int64), True, axis=1)
    dQ, dK, dV = np.zeros((N, d)), np.zeros((N, d)), np.zeros((N, d))
    dkbar, dvbar = np.zeros((tm.T, d)), np.zeros((tm.T, d))

    # special query rows: dense softmax attention over all N keys
    sp = tm.specials
    if len(sp):
        P, ds = _softmax_rows_backward(Q[sp] @ K.T * inv, V, dO[sp])
        dQ[sp] += ds @ K * inv
        dK += ds.T @ Q[sp] * inv
        dV += P.T @ dO[sp]

    # patch query rows, one query tile at a time. Visible keys of a row in
    # tile t: every special token, every token of a kept tile, the landmark
    # of every omitted tile (logit + ln n_u), and the row's own key when t
    # is not kept.
    special = tm.tile_of < 0
    tile_idx = np.where(special, 0, tm.tile_of)
    for t in range(tm.T):
        rows = tm.tokens[t]
        q = Q[rows]
        vis = special | (kept[t][tile_idx] & ~special)
        l_tok = np.where(vis[None, :], q @ K.T * inv, -np.inf)
        l_lm = np.where(kept[t][None, :], -np.inf, q @ kbar.T * inv + logn[None, :])
        l_self = np.full(len(rows), -np.inf) if kept[t][t] else (q * K[rows]).sum(axis=1) * inv
        # one softmax over [tokens | landmarks | self]
        lg = np.concatenate([l_tok, l_lm, l_self[:, None]], axis=1)
        m = lg.max(axis=1, keepdims=True)
        w = np.exp(lg - m)
        P = w / w.sum(axis=1, keepdims=True)
        dP = np.concatenate([dO[rows] @ V.T, dO[rows] @ vbar.T, (dO[rows] * V[rows]).sum(axis=1)[:, None]], axis=1)
        ds = P * (dP - (P * dP).sum(axis=1, keepdims=True))
        ds_tok, ds_lm, ds_self = ds[:, :N], ds[:, N:N + tm.T], ds[:, N + tm.T]
        P_tok, P_lm, P_self = P[:, :N], P[:, N:N + tm.T], P[:, N + tm.T]
        dQ[rows] += (ds_tok @ K + ds_lm @ kbar + ds_self[:, None] * K[rows]) * inv
        dK += ds_tok.T @ q * inv
        dV += P_tok.T @ dO[rows]
        dK[rows] += ds_self[:, None] * q * inv
        dV[rows] += P_self[:, None] * dO[rows]
        dkbar += ds_lm.T @ q * inv
        dvbar += P_lm.T @ dO[rows]

    # a landmark is the mean of its tile: 1/n_u of its gradient to each token
    for u in range(tm.T):
        dK[tm.tokens[u]] += dkbar[u] / tm.n[u]
        dV[tm.tokens[u]] += dvbar[u] / tm.n[u]
    return dQ, dK, dV


def sparse_backward(Q, K, V, dO, tm: TileMap, y: float, sel=None):
    """All heads: (dQ, dK, dV), each [N][H][d] float64. sel [H][T][k] or
    None (selection of the forward on these inputs)."""
    N, H, d = Q.shape
    out = [np.empty((N, H, d)) for _ in range(3)]
    for h in range(H):
        g = sparse_head_backward(Q[:, h], K[:, h], V[:, h], dO[:, h], tm, y,
                                 None if sel is None else sel[h])
        for a, b in zip(out, g):
            a[:, h] = b
    return tuple(out)


def sparse_dq_rows(Q_h, K_h, V_h, dO_h, tm: TileMap, y: float, toks, sel=None):
    """dQ of one head at the given query tokens only, [len(toks)][d]: a row's
    query gradient needs only its own softmax row (for sampled checks at
    sizes where the full backward is out of reach)."""
    N, d = Q_h.shape
    inv = 1.0 / math.sqrt(d)
    K = np.asarray(K_h, dtype=np.float64)
    V = np.asarray(V_h, dtype=np.float64)
    kbar, vbar, logn = osp.landmarks(K_h, V_h, tm)
    special = tm.tile_of < 0
    tile_idx = np.where(special, 0, tm.tile_of)
    out = np.empty((len(toks), d))
    for r, i in enumerate(np.asarray(toks, dtype=np.int64)):
        q = np.asarray(Q_h[i], dtype=np.float64)
        do = np.asarray(dO_h[i], dtype=np.float64)
        if special[i]:
            lg, keys, vals = q @ K.T * inv, K, V
        else:
            t = tm.tile_of[i]
            if sel is None:
                kt, _, _ = osp.select_tiles(Q_h, kbar, tm, y, query_tiles=[t])
                kt = kt[0]
            else:
                kt = np.asarray(sel[t], dtype=np.int64)
            keep = np.zeros(tm.T, dtype=bool)
            keep[kt] = True
            vis = special | (keep[tile_idx] & ~special)
            om = ~keep
            lg = np.concatenate([(K[vis] @ q) * inv, (kbar[om] @ q) * inv + logn[om],
                                 [] if keep[t] else [q @ K[i] * inv]])
            keys = np.concatenate([K[vis], kbar[om]] + ([] if keep[t] else [K[i][None, :]]))
            vals = np.concatenate([V[vis], vbar[om]] + ([] if keep[t] else [V[i][None, :]]))
        w = np.exp(lg - lg.max())
        P = w / w.sum()
        dP = vals @ do
        ds = P * (dP - (P * dP).sum())
        out[r] = ds @ keys * inv
    return out
