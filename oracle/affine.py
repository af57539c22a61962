"""Closed-form centred affine fit of a linear stage (oracle side, float64).

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use this module; the library never does.

Source (Zebra3D pages, "A closed-form fit avoids retraining from scratch"):
for each linear stage the dense model's softmax outputs (the teacher) and
the converted linear outputs are accumulated over scenes, tokens, heads and
views, and a centred affine correction is fitted by a regularised
least-squares solve in float64, with no gradient steps.

Readings where the pages are silent:
  * one fit per stage, pooled over tokens and heads (and calls), shared by
    all heads;
  * the model is the correction that oracle.linear applies,
    y = mu + W (o - mu) + b, with mu the mean of the linear outputs o;
  * the intercept is not regularised, so mu + b = mean of the teacher t;
  * ridge on W: minimise sum |(t - mean t) - W (o - mu)|^2 + lambda |W|_F^2
    with lambda = lambda_rel * trace(G) / d, G the centred Gram of o
    (lambda_rel is a parameter: the pages give no value).
"""
from __future__ import annotations

import numpy as np


def affine_stats(O: np.ndarray, T: np.ndarray) -> np.ndarray:
    """The accumulated statistics, flat in the library's order:
    [n, sum o (d), sum t (d), sum o o^T (d x d), sum o t^T (d x d)].
    O, T: arrays [..., d] of the same shape (every leading index a sample)."""
    d = O.shape[-1]
    X = np.asarray(O, dtype=np.float64).reshape(-1, d)
    Y = np.asarray(T, dtype=np.float64).reshape(-1, d)
    return np.concatenate([[float(X.shape[0])], X.sum(axis=0), Y.sum(axis=0),
                           (X.T @ X).ravel(), (X.T @ Y).ravel()])


def affine_fit(stats: np.ndarray, lambda_rel: float, d: int = 64):
    """(W [d][d], b [d], mu [d]) from the statistics, by the normal
    equations of the ridge problem: W^T = (G + lambda I)^-1 C with
    G = sum (o - mu)(o - mu)^T and C = sum (o - mu)(t - mean t)^T."""
    n = stats[0]
    so, st = stats[1:1 + d], stats[1 + d:1 + 2 * d]
    oo = stats[1 + 2 * d:1 + 2 * d + d * d].reshape(d, d)
    ot = stats[1 + 2 * d + d * d:].reshape(d, d)
    mu, tb = so / n, st / n
    G = oo - n * np.outer(mu, mu)
    C = ot - n * np.outer(mu, tb)
    lam = lambda_rel * np.trace(G) / d
    W = np.linalg.solve(G + lam * np.eye(d), C).T
    return W, tb - mu, mu


def affine_fit_direct(O: np.ndarray, T: np.ndarray, lambda_rel: float):
    """The same fit from the data: centre o and t, then least squares on
    the augmented system [Xc; sqrt(lambda) I] W^T = [Yc; 0] (the ridge
    problem written as an ordinary one)."""
    d = O.shape[-1]
    X = np.asarray(O, dtype=np.float64).reshape(-1, d)
    Y = np.asarray(T, dtype=np.float64).reshape(-1, d)
    mu, tb = X.mean(axis=0), Y.mean(axis=0)
    Xc, Yc = X - mu, Y - tb
    lam = lambda_rel * float((Xc * Xc).sum()) / d
    A = np.vstack([Xc, np.sqrt(lam) * np.eye(d)])
    B = np.vstack([Yc, np.zeros((d, d))])
    Wt, *_ = np.linalg.lstsq(A, B, rcond=None)
    return Wt.T, tb - mu, mu


def apply_affine(O: np.ndarray, W: np.ndarray, b: np.ndarray, mu: np.ndarray) -> np.ndarray:
    """y = mu + W (o - mu) + b on the last axis."""
    O = np.asarray(O, dtype=np.float64)
    return mu + (O - mu) @ W.T + b
