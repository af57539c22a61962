"""Linear global attention with a channel-softmax feature map and the
centred affine output correction (oracle side, float64).

Sources (Zebra3D pages):
  * "Global attention dominates runtime as views grow": linear attention
    aggregates global context at linear cost;
  * "Speedup scales with the number of input views": the linear stages
    apply Q/K normalisation, positional rotation and a channel-softmax
    feature map;
  * "A closed-form fit avoids retraining from scratch": a centred affine
    correction is applied to the linear output of each converted stage.

Readings where the pages are silent:
  * normalisation: per-head RMSNorm over the d channels,
    x / sqrt(mean(x^2) + eps) * g, eps = 1e-6, gain g (default ones);
  * rotation: 2D rotary on (patch row, patch col); channels [0, d/2) turn by
    the row and [d/2, d) by the column; within each half, channel j pairs
    with j + d/4 (j < d/4) and turns by the angle p * base^(-j/(d/4)),
    base = 100; special tokens sit at (0, 0); patch coordinates are 0-based;
  * feature map: softmax over the d channels, temperature 1;
  * every token is both a key and a query (non-causal);
  * output o_i = sum_j phi(q_i).phi(k_j) v_j / sum_j phi(q_i).phi(k_j);
  * affine correction y = mu + W (o - mu) + b with W acting on column
    vectors: y_a = mu_a + b_a + sum_c W[a][c] (o_c - mu_c); mu is an input
    (the calibration mean of the uncorrected output).
"""
from __future__ import annotations

import numpy as np

from .layout import TileMap


def rms_norm(x: np.ndarray, gain=None, eps: float = 1e-6) -> np.ndarray:
    """RMSNorm over the last axis, float64."""
    x = np.asarray(x, dtype=np.float64)
    r = np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    y = x / r
    return y if gain is None else y * np.asarray(gain, dtype=np.float64)


def positions(tm: TileMap):
    """(row, col) rotary position of every token; specials at (0, 0)."""
    loc = np.arange(tm.N) % tm.tpf
    p = np.maximum(loc - tm.S, 0)
    spec = loc < tm.S
    return np.where(spec, 0, p // tm.C), np.where(spec, 0, p % tm.C)


def rope2d(x: np.ndarray, prow: np.ndarray, pcol: np.ndarray, base: float = 100.0) -> np.ndarray:
    """2D rotary embedding of x [n][d] at positions (prow[n], pcol[n])."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h, q = d // 2, d // 4
    freq = base ** (-np.arange(q, dtype=np.float64) / q)
    out = np.empty_like(x)
    for half, p in ((0, prow), (1, pcol)):
        a = np.asarray(p, dtype=np.float64)[:, None] * freq[None, :]
        c, s = np.cos(a), np.sin(a)
        lo = x[:, half * h: half * h + q]
        hi = x[:, half * h + q: half * h + h]
        out[:, half * h: half * h + q] = lo * c - hi * s
        out[:, half * h + q: half * h + h] = hi * c + lo * s
    return out


def feature_map(x: np.ndarray) -> np.ndarray:
    """Softmax over the channel axis (max-subtracted), float64."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def featurize(x_h: np.ndarray, tm: TileMap, gain=None, eps=1e-6, base=100.0) -> np.ndarray:
    """phi(RoPE2D(RMSNorm(x))) for all N tokens of one head."""
    pr, pc = positions(tm)
    return feature_map(rope2d(rms_norm(x_h, gain, eps), pr, pc, base))


def kv_state(phik: np.ndarray, V_h: np.ndarray):
    """KV state S = sum_j phi(k_j) v_j^T  [d][d] and normaliser
    z = sum_j phi(k_j) [d]."""
    V = np.asarray(V_h, dtype=np.float64)
    return phik.T @ V, phik.sum(axis=0)


def apply_state(phiq: np.ndarray, S: np.ndarray, z: np.ndarray) -> np.ndarray:
    """o_i = phi(q_i)^T S / phi(q_i)^T z."""
    return (phiq @ S) / (phiq @ z)[:, None]


def affine(o: np.ndarray, W=None, b=None, mu=None) -> np.ndarray:
    """Centred affine correction y = mu + W (o - mu) + b (per head);
    None means identity W, zero b, zero mu."""
    o = np.asarray(o, dtype=np.float64)
    d = o.shape[-1]
    W = np.eye(d) if W is None else np.asarray(W, dtype=np.float64)
    b = np.zeros(d) if b is None else np.asarray(b, dtype=np.float64)
    mu = np.zeros(d) if mu is None else np.asarray(mu, dtype=np.float64)
    return mu + (o - mu) @ W.T + b


def linear_head(Q_h, K_h, V_h, tm: TileMap, toks=None, W=None, b=None, mu=None,
                gq=None, gk=None, eps=1e-6, base=100.0):
    """Linear-attention output (with the affine correction) of one head at
    the query tokens `toks` (default all). Returns [r][d] float64."""
    phik = featurize(K_h, tm, gk, eps, base)
    S, z = kv_state(phik, V_h)
    if toks is None:
        phiq = featurize(Q_h, tm, gq, eps, base)
    else:
        toks = np.asarray(toks, dtype=np.int64)
        pr, pc = positions(tm)
        phiq = feature_map(rope2d(rms_norm(Q_h[toks], gq, eps), pr[toks], pc[toks], base))
    return affine(apply_state(phiq, S, z), W, b, mu)


def mean_output(Q_h, K_h, V_h, tm: TileMap, gq=None, gk=None, eps=1e-6, base=100.0):
    """Mean over all tokens of the uncorrected linear output of one head:
    the calibration statistic mu of the centred correction."""
    return linear_head(Q_h, K_h, V_h, tm, None, None, None, None, gq, gk, eps, base).mean(axis=0)


def linear_attention(Q, K, V, tm: TileMap, W=None, b=None, mu=None,
                     gq=None, gk=None, eps=1e-6, base=100.0):
    """Full linear stage, all heads: [N][H][d] float64. W [H][d][d],
    b, mu, gq, gk [H][d] (None: identity / zero / ones)."""
    N, H, d = Q.shape
    O = np.empty((N, H, d))
    pick = lambda a, h: None if a is None else np.asarray(a)[h]  # noqa: E731
    for h in range(H):
        O[:, h] = linear_head(Q[:, h], K[:, h], V[:, h], tm, None, pick(W, h), pick(b, h),
                              pick(mu, h), pick(gq, h), pick(gk, h), eps, base)
    return O


def linear_rows(Q, K, V, tm: TileMap, rows, W=None, b=None, mu=None,
                gq=None, gk=None, eps=1e-6, base=100.0):
    """Linear output at sampled (head, token) rows [R][2]; the state still
    sums over all N tokens. Returns [R][d] float64."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), Q.shape[2]))
    pick = lambda a, h: None if a is None else np.asarray(a)[h]  # noqa: E731
    for h in np.unique(rows[:, 0]):
        idx = np.nonzero(rows[:, 0] == h)[0]
        out[idx] = linear_head(Q[:, h], K[:, h], V[:, h], tm, rows[idx, 1], pick(W, h),
                               pick(b, h), pick(mu, h), pick(gq, h), pick(gk, h), eps, base)
    return out
