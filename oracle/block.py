"""The attention steps either side of a global stage (oracle side, float64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (Zebra3D pages):
  * "Global attention dominates runtime as views grow": the backbones
    alternate frame-wise attention with global attention, so each image
    draws on the other views only in the global stages;
  * "Linear-centered stages plus tile-sparse stages": conversion keeps the
    normalisation layers and the positional encoding, so a sparse stage's
    queries and keys pass through the same per-head normalisation and 2D
    rotary as the linear stage's before the attention.

Readings (the pages give no formula):
  * frame-wise attention: every token of a frame (its special tokens and
    its patches) attends densely to all tokens of the same frame and no
    other, softmax of q.k / sqrt(d);
  * the query/key prologue is RoPE2D(RMSNorm(x)) exactly as in the linear
    stage (oracle.linear: per-head RMSNorm with gain and eps, channels
    [0, d/2) turned by the patch row and [d/2, d) by the column, specials
    at (0, 0)), applied to Q and K; its output is what the sparse stage
    (and a frame-wise stage) then attends with.
"""
from __future__ import annotations

import math

import numpy as np

from .layout import TileMap
from . import linear as olin


def qk_prologue(x_h, tm: TileMap, gain=None, eps: float = 1e-6, base: float = 100.0) -> np.ndarray:
    """RoPE2D(RMSNorm(x)) of every token of one head, [N][d] float64."""
    pr, pc = olin.positions(tm)
    return olin.rope2d(olin.rms_norm(x_h, gain, eps), pr, pc, base)


def round_bf16(x) -> np.ndarray:
    """Rounds to the nearest bfloat16 (ties to even) through float32, and
    widens back to float64: the precision in which a stage hands its
    prologue outputs to the next step (the selector decides from them)."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def frame_attention_head(Q_h, K_h, V_h, tm: TileMap) -> np.ndarray:
    """Frame-wise softmax attention of one head, [N][d] float64: the tokens
    of frame f (a contiguous range of tm.tpf tokens) attend to that range."""
    d = Q_h.shape[1]
    out = np.empty((tm.N, d))
    for f in range(tm.F):
        r = slice(f * tm.tpf, (f + 1) * tm.tpf)
        q = np.asarray(Q_h[r], dtype=np.float64)
        k = np.asarray(K_h[r], dtype=np.float64)
        v = np.asarray(V_h[r], dtype=np.float64)
        lg = q @ k.T / math.sqrt(d)
        w = np.exp(lg - lg.max(axis=1, keepdims=True))
        out[r] = (w @ v) / w.sum(axis=1, keepdims=True)
    return out


def frame_attention(Q, K, V, tm: TileMap) -> np.ndarray:
    """All heads: [N][H][d] float64."""
    H = Q.shape[1]
    return np.stack([frame_attention_head(Q[:, h], K[:, h], V[:, h], tm) for h in range(H)], axis=1)


def prologue(X, tm: TileMap, gain=None, eps: float = 1e-6, base: float = 100.0) -> np.ndarray:
    """qk_prologue of every head of X [N][H][d]; gain [H][d] or None."""
    H = X.shape[1]
    return np.stack([qk_prologue(X[:, h], tm, None if gain is None else np.asarray(gain)[h], eps, base)
                     for h in range(H)], axis=1)
