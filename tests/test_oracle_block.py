"""Pins of the oracle's frame-wise attention and query/key prologue
(Zebra3D pages, "Global attention dominates runtime as views grow" and
"Linear-centered stages plus tile-sparse stages"): scipy's softmax per
frame, a scalar brute force, one frame equalling dense attention, frame
permutation equivariance, and the prologue's row norms, its identity at
position (0, 0) and its agreement with the linear stage's steps."""
import math

import numpy as np
from scipy.special import softmax

from oracle import block as ob
from oracle import linear as olin
from oracle import sparse as osp
from oracle.layout import TileMap


def _qkv(tm, H, seed):
    g = np.random.default_rng(seed)
    return tuple(g.standard_normal((tm.N, H, 64)) * s for s in (1.5, 1.5, 1.0))


def test_frame_attention_matches_scipy_per_frame():
    tm = TileMap(3, 2, 7, 9)
    Q, K, V = _qkv(tm, 2, 0)
    O = ob.frame_attention(Q, K, V, tm)
    for h in range(2):
        for f in range(3):
            idx = np.arange(f * tm.tpf, (f + 1) * tm.tpf)
            want = softmax(Q[idx, h] @ K[idx, h].T / 8.0, axis=1) @ V[idx, h]
            assert np.abs(O[idx, h] - want).max() < 1e-13


def test_frame_attention_scalar_brute_force():
    tm = TileMap(2, 1, 3, 4)
    Q, K, V = _qkv(tm, 1, 1)
    O = ob.frame_attention_head(Q[:, 0], K[:, 0], V[:, 0], tm)
    for i in range(tm.N):
        f = i // tm.tpf
        keys = range(f * tm.tpf, (f + 1) * tm.tpf)
        lg = [sum(Q[i, 0, c] * K[j, 0, c] for c in range(64)) / 8.0 for j in keys]
        m = max(lg)
        w = [math.exp(x - m) for x in lg]
        want = [sum(wj * V[j, 0, c] for wj, j in zip(w, keys)) / sum(w) for c in range(64)]
        assert np.abs(O[i] - np.array(want)).max() < 1e-12


def test_one_frame_is_dense_attention_and_frames_permute():
    tm1 = TileMap(1, 3, 8, 8)
    Q, K, V = _qkv(tm1, 2, 2)
    assert np.abs(ob.frame_attention(Q, K, V, tm1) - osp.dense_attention(Q, K, V)).max() < 1e-13
    tm = TileMap(3, 2, 5, 6)
    Q, K, V = _qkv(tm, 1, 3)
    perm = [2, 0, 1]
    P = np.concatenate([np.arange(f * tm.tpf, (f + 1) * tm.tpf) for f in perm])
    O = ob.frame_attention(Q, K, V, tm)
    Op = ob.frame_attention(Q[P], K[P], V[P], tm)
    assert np.abs(Op - O[P]).max() < 1e-13


def test_prologue_norms_origin_and_linear_steps():
    tm = TileMap(2, 3, 6, 7)
    g = np.random.default_rng(4)
    X = g.standard_normal((tm.N, 2, 64)) * 3
    Y = ob.prologue(X, tm, eps=0.0)
    # RMSNorm then a rotation: every row has norm sqrt(64) = 8
    assert np.allclose(np.linalg.norm(Y, axis=2), 8.0, atol=1e-12)
    # specials and the top-left patch sit at (0, 0): only the norm acts
    spec = tm.specials
    assert np.allclose(Y[spec], olin.rms_norm(X[spec], eps=0.0), atol=1e-14)
    gain = 0.5 + g.random((2, 64))
    Yg = ob.prologue(X, tm, gain, 1e-3, 1000.0)
    pr, pc = olin.positions(tm)
    for h in range(2):
        want = olin.rope2d(olin.rms_norm(X[:, h], gain[h], 1e-3), pr, pc, 1000.0)
        assert np.abs(Yg[:, h] - want).max() < 1e-14
    # the relative-position property survives the prologue: the dot product
    # of two tokens' prologue outputs is unchanged when both move by the
    # same patch offset (same frame, same normalised content)
    tm2 = TileMap(1, 0, 6, 6)
    a, b = g.standard_normal((2, 64))
    Xp = np.zeros((tm2.N, 1, 64))
    Xp[0 * 6 + 1, 0], Xp[2 * 6 + 3, 0] = a, b   # tokens at (0,1) and (2,3)
    Xp[1 * 6 + 2, 0], Xp[3 * 6 + 4, 0] = a, b   # the same pair moved by (1,1)
    Yp = ob.prologue(Xp, tm2)[:, 0]
    assert abs(Yp[1] @ Yp[15] - Yp[8] @ Yp[22]) < 1e-12


def test_round_bf16_to_nearest_even():
    # bf16 keeps 7 mantissa bits: spacing 2^-7 above 1; ties go to even
    x = np.array([1.0, 1.0 + 2 ** -7, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8, -2.5, 0.0,
                  1.0 + 2 ** -8 + 2 ** -20, 3.0e38, -7.0e-3])
    got = ob.round_bf16(x)
    assert got[:7].tolist() == [1.0, 1.0 + 2 ** -7, 1.0 + 2 ** -6, 1.0, -2.5, 0.0, 1.0 + 2 ** -7]
    # every result is a bf16 value within half a bf16 ulp of its input
    m, e = np.frexp(np.abs(x[7:]))
    assert np.all(np.abs(got[7:] - x[7:]) <= 2.0 ** (e - 9))
    assert np.array_equal(ob.round_bf16(got), got)
