"""Attention-mass coverage of a tile-sparse stage (oracle side, float64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: Zebra3D pages, "Sensitive stages also concentrate their attention":
stages are profiled by how concentrated their attention mass is, and the
stages that need faithful softmax interactions are those where sparse
selection can cover most of the relevant attention mass; "Linear-centered
stages plus tile-sparse stages" for the kept tiles and the mean-K/V
landmarks of the omitted ones.

Readings (the pages name the diagnostics but give no formula):
  * coverage of a patch query row i: the share of its DENSE softmax mass
    (over all N keys, logits q_i . k_j / sqrt(d)) that falls on the tokens
    of the key tiles its query tile kept; special keys and the omitted
    tiles' tokens are not covered;
  * landmark error of row i: how much of the omitted tiles' exact mass the
    landmarks miss, 1 - L_i / E_i, with E_i = sum over omitted tiles u and
    their tokens j of exp(q_i . k_j / sqrt(d)) and L_i = sum over omitted u
    of n_u exp(q_i . kbar_u / sqrt(d)) (the landmark logit carries ln n_u);
    0 when no tile is omitted. By Jensen's inequality L_i <= E_i, so the
    error lies in [0, 1) and is 0 exactly when every omitted tile's logits
    are equal (e.g. identical keys);
  * both are reported per (head, query tile) as the mean over the tile's
    rows.
"""
from __future__ import annotations

import math

import numpy as np

from .layout import TileMap, keep_count
from . import sparse as osp


def row_coverage(Q_h, K_h, tm: TileMap, t: int, kept: np.ndarray, kbar: np.ndarray):
    """Coverage and landmark error of every row of query tile t (one head).
    kept: the tile's kept key tiles. Returns (coverage [n_t], lm_error [n_t])."""
    d = Q_h.shape[1]
    inv = 1.0 / math.sqrt(d)
    K = np.asarray(K_h, dtype=np.float64)
    q = np.asarray(Q_h[tm.tokens[t]], dtype=np.float64)
    logits = q @ K.T * inv                      # [n_t][N], every key
    m = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - m)
    is_kept = np.zeros(tm.T, dtype=bool)
    is_kept[kept] = True
    tile = tm.tile_of                            # -1 for special tokens
    in_kept = np.zeros(tm.N, dtype=bool)
    in_omit = np.zeros(tm.N, dtype=bool)
    patch = tile >= 0
    in_kept[patch] = is_kept[tile[patch]]
    in_omit[patch] = ~is_kept[tile[patch]]
    total = w.sum(axis=1)
    coverage = w[:, in_kept].sum(axis=1) / total
    E = w[:, in_omit].sum(axis=1)
    omitted = np.nonzero(~is_kept)[0]
    lm_logit = q @ kbar[omitted].T * inv + np.log(tm.n[omitted].astype(np.float64))[None, :]
    L = np.exp(lm_logit - m).sum(axis=1)
    err = np.where(E > 0, 1.0 - L / np.where(E > 0, E, 1.0), 0.0)
    return coverage, err


def coverage_head(Q_h, K_h, tm: TileMap, y: float, query_tiles=None):
    """Per-query-tile coverage and landmark error of one head at sparsity y
    (selection as in oracle.sparse). Returns (coverage [len], lm_error [len])."""
    kbar, _, _ = osp.landmarks(K_h, K_h, tm)
    qt = np.arange(tm.T) if query_tiles is None else np.asarray(query_tiles)
    sel, _, _ = osp.select_tiles(Q_h, kbar, tm, y, query_tiles=qt)
    cov = np.empty(len(qt))
    err = np.empty(len(qt))
    for i, t in enumerate(qt):
        c, e = row_coverage(Q_h, K_h, tm, int(t), sel[i], kbar)
        cov[i], err[i] = c.mean(), e.mean()
    return cov, err


def coverage(Q, K, tm: TileMap, y: float):
    """All heads: (coverage [H][T], lm_error [H][T])."""
    H = Q.shape[1]
    out = [coverage_head(Q[:, h], K[:, h], tm, y) for h in range(H)]
    return np.stack([c for c, _ in out]), np.stack([e for _, e in out])


__all__ = ["row_coverage", "coverage_head", "coverage", "keep_count"]
