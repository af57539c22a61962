"""Tile-sparse softmax attention with mean-K/V landmarks, and dense softmax
attention (oracle side, float64).

Source: Zebra3D pages, "Linear-centered stages plus tile-sparse stages":
  * the selector keeps a key-tile fraction 1 - y for each query tile;
  * selected tiles keep full softmax interactions;
  * omitted tiles are summarised as mean key/value landmarks;
  * special-token keys stay visible;
  * special-token query rows keep dense attention;
  * every patch query keeps its own self key.
"Global attention dominates runtime as views grow" for dense global
attention over all views' tokens.

Readings where the pages are silent:
  * tile score for query tile t and key tile u: mean of the patch queries of
    t dotted with the mean key of u, divided by sqrt(d); per head; over all
    tiles of all frames, the query's own frame and own tile included;
  * ties in the top-k go to the lower tile index; the kept list is output in
    ascending tile order;
  * a landmark's logit is q . kbar_u / sqrt(d) + ln(n_u), so it weighs as
    n_u copies of (kbar_u, vbar_u); its value is vbar_u;
  * the landmark is the mean over all n_u tokens of the tile;
  * the self key (logit q_i . k_i / sqrt(d), value v_i) is added only when
    the query's own tile is not selected, so y = 0 is exactly dense
    attention;
  * special rows attend to all N keys; sparse stages apply no norm or
    rotation to Q and K.

The visible key set of a patch row is written as a mask over all tokens and
all landmarks (logit -inf where not visible); this is the definition above,
evaluated for a batch of rows at once.
"""
from __future__ import annotations

import math

import numpy as np

from .layout import TileMap, keep_count

ROW_BLOCK = 256


def tile_means(X_h: np.ndarray, tm: TileMap) -> np.ndarray:
    """Mean over each tile's tokens, [T][d] float64 (X_h is [N][d]).
    bf16 inputs sum exactly in float64; one rounding for the division."""
    out = np.empty((tm.T, X_h.shape[1]), dtype=np.float64)
    for u in range(tm.T):
        out[u] = X_h[tm.tokens[u]].astype(np.float64).sum(axis=0) / tm.n[u]
    return out


def landmarks(K_h: np.ndarray, V_h: np.ndarray, tm: TileMap):
    """Mean-K/V landmark of every tile of one head: (kbar [T][d],
    vbar [T][d], ln n [T])."""
    return tile_means(K_h, tm), tile_means(V_h, tm), np.log(tm.n.astype(np.float64))


def select_one(scores: np.ndarray, k: int):
    """Top-k key tiles of one query tile by (score descending, tile index
    ascending).

    Returns (kept tile ids ascending, near_tie flag, relative gap), where the
    gap compares the k-th and (k+1)-th ranked scores,
        |s_(k) - s_(k+1)| / max(|s_(k)|, |s_(k+1)|, 1e-300),
    and near_tie is gap < 1e-6: there two correct float64 implementations
    may keep a different last tile."""
    T = scores.shape[0]
    order = np.lexsort((np.arange(T), -scores))
    kept = np.sort(order[:k])
    if 0 < k < T:
        a, b = scores[order[k - 1]], scores[order[k]]
        gap = abs(a - b) / max(abs(a), abs(b), 1e-300)
    else:
        gap = math.inf
    return kept.astype(np.int64), bool(gap < 1e-6), float(gap)


def select_tiles(Q_h: np.ndarray, kbar: np.ndarray, tm: TileMap, y: float,
                 query_tiles=None):
    """Tile selection for one head.

    For each query tile t: qbar_t = mean of its patch queries, score
    s_{t,u} = qbar_t . kbar_u / sqrt(d) for every key tile u, keep the top
    k = keep_count(y, T). Returns (sel [len(query_tiles)][k] int64 ascending,
    near_tie bool array, gap array)."""
    k = keep_count(y, tm.T)
    d = kbar.shape[1]
    qt = range(tm.T) if query_tiles is None else query_tiles
    sel, tie, gap = [], [], []
    for t in qt:
        qbar = Q_h[tm.tokens[t]].astype(np.float64).sum(axis=0) / tm.n[t]
        s, nt, g = select_one((kbar @ qbar) / math.sqrt(d), k)
        sel.append(s)
        tie.append(nt)
        gap.append(g)
    sel = np.array(sel, dtype=np.int64).reshape(len(sel), k)
    return sel, np.array(tie, dtype=bool), np.array(gap)


def sparse_patch_rows(Q_h, K_h, V_h, tm: TileMap, toks, selected, kbar, vbar, logn):
    """Tile-sparse attention output for patch query rows of one head.

    toks      [r] patch token indices
    selected  [r][T] bool: row i's query tile kept key tile u
    Returns [r][d] float64. For row i in query tile t the logits (all scaled
    by 1/sqrt(d)) are
      q_i . k_j            for every token j of every kept tile
      q_i . kbar_u + ln n_u  (value vbar_u) for every tile u not kept
      q_i . k_s            for every special token s of every frame
      q_i . k_i            (value v_i) only if tile t itself is not kept
    """
    d = Q_h.shape[1]
    inv = 1.0 / math.sqrt(d)
    toks = np.asarray(toks, dtype=np.int64)
    K = K_h.astype(np.float64)
    V = V_h.astype(np.float64)
    q = Q_h[toks].astype(np.float64)
    special = tm.tile_of < 0
    tile_idx = np.where(special, 0, tm.tile_of)
    visible = special[None, :] | (selected[:, tile_idx] & ~special[None, :])
    l_tok = np.where(visible, q @ K.T * inv, -np.inf)
    l_lm = np.where(selected, -np.inf, q @ kbar.T * inv + logn[None, :])
    own = selected[np.arange(len(toks)), tm.tile_of[toks]]
    l_self = np.where(own, -np.inf, (q * K[toks]).sum(axis=1) * inv)
    m = np.maximum(np.maximum(l_tok.max(axis=1), l_lm.max(axis=1)), l_self)
    w_tok = np.exp(l_tok - m[:, None])
    w_lm = np.exp(l_lm - m[:, None])
    w_self = np.exp(l_self - m)
    num = w_tok @ V + w_lm @ vbar + w_self[:, None] * V[toks]
    den = w_tok.sum(axis=1) + w_lm.sum(axis=1) + w_self
    return num / den[:, None]


def dense_rows(Q_h, K_h, V_h, toks) -> np.ndarray:
    """Dense softmax attention of the given query tokens over all N keys
    (one head), 1/sqrt(d) scaling. Returns [len(toks)][d] float64."""
    d = Q_h.shape[1]
    toks = np.asarray(toks, dtype=np.int64)
    K = K_h.astype(np.float64)
    V = V_h.astype(np.float64)
    out = np.empty((len(toks), d))
    for i in range(0, len(toks), ROW_BLOCK):
        q = Q_h[toks[i:i + ROW_BLOCK]].astype(np.float64)
        lg = q @ K.T / math.sqrt(d)
        w = np.exp(lg - lg.max(axis=1, keepdims=True))
        out[i:i + ROW_BLOCK] = (w @ V) / w.sum(axis=1, keepdims=True)
    return out


def _sel_mask(sel_rows: np.ndarray, T: int) -> np.ndarray:
    m = np.zeros((sel_rows.shape[0], T), dtype=bool)
    if sel_rows.shape[1]:
        np.put_along_axis(m, sel_rows, True, axis=1)
    return m


def sparse_head(Q_h, K_h, V_h, tm: TileMap, y: float, toks, lm=None):
    """Tile-sparse output of one head at the given query tokens (patch or
    special). Returns (out [r][d], near_tie [r], sel of each patch row's
    tile or None for special rows)."""
    toks = np.asarray(toks, dtype=np.int64)
    kbar, vbar, logn = lm if lm is not None else landmarks(K_h, V_h, tm)
    out = np.empty((len(toks), Q_h.shape[1]))
    tie = np.zeros(len(toks), dtype=bool)
    spec = tm.tile_of[toks] < 0
    if spec.any():
        out[spec] = dense_rows(Q_h, K_h, V_h, toks[spec])
    pidx = np.nonzero(~spec)[0]
    if len(pidx):
        tiles, inv_idx = np.unique(tm.tile_of[toks[pidx]], return_inverse=True)
        sel, ties, _ = select_tiles(Q_h, kbar, tm, y, query_tiles=tiles)
        masks = _sel_mask(sel, tm.T)
        for i in range(0, len(pidx), ROW_BLOCK):
            blk = pidx[i:i + ROW_BLOCK]
            out[blk] = sparse_patch_rows(Q_h, K_h, V_h, tm, toks[blk],
                                         masks[inv_idx[i:i + ROW_BLOCK]], kbar, vbar, logn)
        tie[pidx] = ties[inv_idx]
    return out, tie


def sparse_attention(Q, K, V, tm: TileMap, y: float):
    """Full tile-sparse stage for all heads and tokens.
    Q, K, V: [N][H][d]. Returns (O [N][H][d] float64, sel [H][T][k] int64,
    near_tie [H][T] bool)."""
    N, H, d = Q.shape
    O = np.empty((N, H, d))
    k = keep_count(y, tm.T)
    sel_all = np.empty((H, tm.T, k), dtype=np.int64)
    tie_all = np.empty((H, tm.T), dtype=bool)
    for h in range(H):
        Qh, Kh, Vh = Q[:, h, :], K[:, h, :], V[:, h, :]
        lm = landmarks(Kh, Vh, tm)
        O[:, h], _ = sparse_head(Qh, Kh, Vh, tm, y, np.arange(N), lm=lm)
        sel_all[h], tie_all[h], _ = select_tiles(Qh, lm[0], tm, y)
    return O, sel_all, tie_all


def sparse_rows(Q, K, V, tm: TileMap, y: float, rows):
    """Tile-sparse output at sampled (head, token) rows. rows: [R][2] int.
    Returns ([R][d] float64, near_tie [R])."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), Q.shape[2]))
    tie = np.zeros(len(rows), dtype=bool)
    for h in np.unique(rows[:, 0]):
        idx = np.nonzero(rows[:, 0] == h)[0]
        out[idx], tie[idx] = sparse_head(Q[:, h], K[:, h], V[:, h], tm, y, rows[idx, 1])
    return out, tie


def dense_attention(Q, K, V):
    """Dense softmax attention for all heads and tokens, [N][H][d] float64."""
    N, H, d = Q.shape
    O = np.empty((N, H, d))
    for h in range(H):
        O[:, h] = dense_rows(Q[:, h], K[:, h], V[:, h], np.arange(N))
    return O
