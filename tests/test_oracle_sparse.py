"""Pins of the oracle's landmarks, tile selection, tile-sparse attention and
dense attention against things other than the oracle itself: hand-derived
golden values, closed forms, textbook/library softmax, brute force and
invariances. Zebra3D pages, "Linear-centered stages plus tile-sparse
stages" defines the operator; the readings are listed in oracle/sparse.py."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import softmax

from oracle import sparse as osp
from oracle.layout import TileMap, keep_count

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand_qkv(N, H, d, seed):
    g = np.random.default_rng(seed)
    return (g.standard_normal((N, H, d)), g.standard_normal((N, H, d)),
            g.standard_normal((N, H, d)))


# ---------------------------------------------------------------- golden
def test_golden_q0_example():
    fx = json.load(open(os.path.join(GOLD, "sparse_q0_example.json")))
    L = fx["layout"]
    tm = TileMap(L["F"], L["S"], L["R"], L["C"])
    assert tm.N == 129 and tm.T == 2
    N, d = tm.N, L["d"]
    Q = np.zeros((N, 1, d))
    K = np.random.default_rng(3).standard_normal((N, 1, d))
    V = np.zeros((N, 1, d))
    V[0, 0, 0] = 1.0
    V[:, 0, 1] = 1.0
    V[fx["marked_token"], 0, 2] = 1.0
    assert tm.tile_of[fx["marked_token"]] == 1
    O, sel, _ = osp.sparse_attention(Q, K, V, tm, fx["y"])
    assert sel.tolist() == [[[0], [0]]]
    for e in fx["expected"]:
        for ch in range(3):
            want = float(Fraction(e[f"ch{ch}"]))
            assert O[e["token"], 0, ch] == pytest.approx(want, abs=1e-14), (e, ch)


def test_layout_counts_golden():
    fx = json.load(open(os.path.join(GOLD, "layout_counts.json")))
    for name, c in fx["configs"].items():
        if c["F"] > 512:
            continue  # the 1,024-view map is checked by closed form below
        tm = TileMap(c["F"], c["S"], c["R"], c["C"])
        assert tm.N == c["N"] and tm.T == c["T"], name
        sizes, counts = np.unique(tm.n[: tm.tiles_per_frame], return_counts=True)
        assert {str(s): int(n) for s, n in zip(sizes, counts)} == c["sizes"], name
        assert sorted(np.concatenate(tm.tokens).tolist() + tm.specials.tolist()) == list(range(tm.N))
        if "y" in c:
            assert keep_count(c["y"], c["T"]) == c["k"], name
    big = fx["configs"]["1024views"]
    assert big["F"] * (big["S"] + big["R"] * big["C"]) == big["N"]
    assert keep_count(big["y"], big["T"]) == big["k"]


def test_keep_count_rounds_not_floors():
    # (1 - 0.8) * 800 = 159.99999999999997 in double; the kept count is 160.
    assert math.floor((1 - 0.8) * 800) == 159
    assert keep_count(0.8, 800) == 160
    assert keep_count(0.0, 7) == 7 and keep_count(1.0, 7) == 0
    with pytest.raises(ValueError):
        keep_count(1.5, 10)


def test_tile_map_partial_tiles_and_order():
    tm = TileMap(2, 3, 11, 9)  # 2x2 tiles: 8x8, 8x1, 3x8, 3x1
    assert tm.T == 8
    assert tm.n[:4].tolist() == [64, 8, 24, 3]
    # tile 1 of frame 1 = rows 0..7, col 8
    base = 1 * (3 + 99) + 3
    assert tm.tokens[5].tolist() == [base + r * 9 + 8 for r in range(8)]
    assert tm.specials.tolist() == [0, 1, 2, 102, 103, 104]


# ---------------------------------------------------------------- landmarks
def test_landmark_of_identical_tile_is_that_tile():
    tm = TileMap(1, 2, 8, 11)
    N, d = tm.N, 64
    g = np.random.default_rng(0)
    # bf16-representable values (as every real input is): n equal values
    # then sum exactly and the division by n returns the value itself
    K = np.round(g.standard_normal((N, d)) * 64) / 64
    V = np.round(g.standard_normal((N, d)) * 64) / 64
    for u in range(tm.T):
        K[tm.tokens[u]] = K[tm.tokens[u][0]]
        V[tm.tokens[u]] = V[tm.tokens[u][0]]
    kbar, vbar, logn = osp.landmarks(K, V, tm)
    for u in range(tm.T):
        assert np.array_equal(kbar[u], K[tm.tokens[u][0]])
        assert np.array_equal(vbar[u], V[tm.tokens[u][0]])
    assert np.allclose(np.exp(logn), tm.n)


# ---------------------------------------------------------------- selection
def _brute_select(Q, K, tm, y):
    """Top-k by sorting explicit (-score, index) tuples with Python sorted."""
    d = Q.shape[1]
    k = keep_count(y, tm.T)
    out = []
    for t in range(tm.T):
        qb = [sum(Q[j, c] for j in tm.tokens[t]) / tm.n[t] for c in range(d)]
        sc = []
        for u in range(tm.T):
            kb = [sum(K[j, c] for j in tm.tokens[u]) / tm.n[u] for c in range(d)]
            sc.append((-sum(a * b for a, b in zip(qb, kb)) / math.sqrt(d), u))
        out.append(sorted(u for _, u in sorted(sc)[:k]))
    return out


@pytest.mark.parametrize("y", [0.0, 0.3, 0.5, 0.75, 1.0])
def test_selection_brute_force(y):
    tm = TileMap(2, 1, 10, 17, )  # 2x3 tiles per frame, partial
    Q, K, _ = _rand_qkv(tm.N, 1, 16, 5)
    kbar, _, _ = osp.landmarks(K[:, 0], K[:, 0], tm)
    sel, _, _ = osp.select_tiles(Q[:, 0], kbar, tm, y)
    assert sel.tolist() == _brute_select(Q[:, 0], K[:, 0], tm, y)


def test_selection_ties_go_to_lower_index_and_near_ties_flagged():
    s = np.array([1.0, 2.0, 2.0, 0.5, 2.0])
    kept, tie, gap = osp.select_one(s, 2)
    assert kept.tolist() == [1, 2] and tie and gap == 0.0
    kept, tie, _ = osp.select_one(np.array([3.0, 1.0, 2.0, 2.0 + 1e-9]), 2)
    assert kept.tolist() == [0, 3] and tie
    kept, tie, _ = osp.select_one(np.array([3.0, 1.0, 2.0, 2.5]), 2)
    assert kept.tolist() == [0, 3] and not tie


def test_selection_invariant_to_key_shift_and_equivariant_to_frame_perm():
    tm = TileMap(4, 2, 9, 9)
    Q, K, _ = _rand_qkv(tm.N, 1, 8, 7)
    Q, K = Q[:, 0], K[:, 0]
    kbar, _, _ = osp.landmarks(K, K, tm)
    sel, _, _ = osp.select_tiles(Q, kbar, tm, 0.5)
    # every score of a query tile moves by the same qbar . c / sqrt(d)
    c = np.random.default_rng(1).standard_normal(8) * 3
    kbar2, _, _ = osp.landmarks(K + c, K + c, tm)
    sel2, _, _ = osp.select_tiles(Q, kbar2, tm, 0.5)
    assert np.array_equal(sel, sel2)
    # permuting whole frames permutes query and key tiles alike
    perm = [2, 0, 3, 1]
    tpf = tm.tpf
    tok = np.concatenate([np.arange(f * tpf, (f + 1) * tpf) for f in perm])
    kb3, _, _ = osp.landmarks(K[tok], K[tok], tm)
    sel3, _, _ = osp.select_tiles(Q[tok], kb3, tm, 0.5)
    tpf_t = tm.tiles_per_frame
    old_of_new = np.concatenate([np.arange(f * tpf_t, (f + 1) * tpf_t) for f in perm])
    for t_new in range(tm.T):
        got = sorted(old_of_new[sel3[t_new]].tolist())
        assert got == sel[old_of_new[t_new]].tolist()


# ---------------------------------------------------------------- attention
def _scipy_dense(Q, K, V):
    d = Q.shape[1]
    return softmax(Q @ K.T / math.sqrt(d), axis=1) @ V


def test_dense_matches_scipy_softmax():
    Q, K, V = _rand_qkv(70, 1, 64, 11)
    got = osp.dense_rows(Q[:, 0], K[:, 0], V[:, 0], np.arange(70))
    assert np.allclose(got, _scipy_dense(Q[:, 0], K[:, 0], V[:, 0]), atol=1e-13)


def test_dense_attention_two_heads_match_scipy_per_head():
    """The all-heads wrapper (the reference of the dense GPU tests): each
    head's output equals scipy's softmax attention on that head's own
    Q, K, V. 300 rows cross the wrapper's 256-row blocks; head 1's inputs
    are scaled so that a head mix-up cannot go unnoticed."""
    Q, K, V = _rand_qkv(300, 2, 64, 21)
    Q[:, 1] *= 2.5
    V[:, 1] += 3.0
    got = osp.dense_attention(Q, K, V)
    assert got.shape == (300, 2, 64)
    for h in range(2):
        want = _scipy_dense(Q[:, h], K[:, h], V[:, h])
        assert np.abs(got[:, h] - want).max() < 1e-12, h
    other = _scipy_dense(Q[:, 0], K[:, 0], V[:, 0])
    assert np.abs(got[:, 1] - other).max() > 1.0


@pytest.mark.parametrize("shape", [(2, 5, 16, 16), (3, 2, 11, 13)])
def test_y0_is_dense(shape):
    tm = TileMap(*shape)
    Q, K, V = _rand_qkv(tm.N, 2, 64, 2)
    O, sel, _ = osp.sparse_attention(Q, K, V, tm, 0.0)
    assert sel.shape[2] == tm.T
    for h in range(2):
        ref = _scipy_dense(Q[:, h], K[:, h], V[:, h])
        assert np.abs(O[:, h] - ref).max() < 1e-12


@pytest.mark.parametrize("y", [0.25, 0.5, 1.0])
def test_special_rows_are_dense(y):
    tm = TileMap(3, 4, 9, 12)
    Q, K, V = _rand_qkv(tm.N, 1, 64, 4)
    O, _, _ = osp.sparse_attention(Q, K, V, tm, y)
    ref = _scipy_dense(Q[:, 0], K[:, 0], V[:, 0])
    assert np.abs(O[tm.specials, 0] - ref[tm.specials]).max() < 1e-12


@pytest.mark.parametrize("y", [0.0, 0.4, 0.75, 1.0])
def test_piecewise_constant_tiles_closed_form(y):
    """Tiles whose tokens share one key and one value: an omitted tile's
    landmark (weight n_u * exp(q.k_u)) is exactly that tile's dense
    contribution, so the sparse output is dense attention, plus one extra
    copy of the row's own key/value when its own tile was not kept."""
    tm = TileMap(2, 3, 12, 10)
    Q, K, V = _rand_qkv(tm.N, 1, 64, 9)
    Q, K, V = Q[:, 0], K[:, 0], V[:, 0]
    for u in range(tm.T):
        K[tm.tokens[u]] = K[tm.tokens[u][0]]
        V[tm.tokens[u]] = V[tm.tokens[u][0]]
    O, sel, _ = osp.sparse_attention(Q[:, None], K[:, None], V[:, None], tm, y)
    d = 64
    for t in range(tm.T):
        kept = t in set(sel[0, t].tolist())
        for i in tm.tokens[t]:
            keys, vals = K, V
            if not kept:
                keys = np.vstack([K, K[i]])
                vals = np.vstack([V, V[i]])
            want = softmax(keys @ Q[i] / math.sqrt(d)) @ vals
            assert np.abs(O[i, 0] - want).max() < 1e-12, (t, i, kept)


def test_shift_invariances():
    tm = TileMap(2, 2, 9, 16)
    Q, K, V = _rand_qkv(tm.N, 1, 64, 21)
    O, _, _ = osp.sparse_attention(Q, K, V, tm, 0.5)
    c = np.random.default_rng(2).standard_normal(64)
    O_k, _, _ = osp.sparse_attention(Q, K + c, V, tm, 0.5)
    O_v, _, _ = osp.sparse_attention(Q, K, V + c, tm, 0.5)
    assert np.abs(O_k - O).max() < 1e-11
    assert np.abs(O_v - (O + c)).max() < 1e-11


def test_k0_only_landmarks_specials_and_self():
    tm = TileMap(2, 2, 9, 9)
    Q, K, V = _rand_qkv(tm.N, 1, 64, 13)
    Q, K, V = Q[:, 0], K[:, 0], V[:, 0]
    O, sel, _ = osp.sparse_attention(Q[:, None], K[:, None], V[:, None], tm, 1.0)
    assert sel.shape == (1, tm.T, 0)
    for u in range(tm.T):
        for i in tm.tokens[u]:
            keys = [K[tm.tokens[w]].mean(axis=0) for w in range(tm.T)]
            vals = [V[tm.tokens[w]].mean(axis=0) for w in range(tm.T)]
            bias = [math.log(tm.n[w]) for w in range(tm.T)]
            for s in tm.specials:
                keys.append(K[s]); vals.append(V[s]); bias.append(0.0)
            keys.append(K[i]); vals.append(V[i]); bias.append(0.0)
            lg = np.array(keys) @ Q[i] / 8.0 + np.array(bias)
            assert np.abs(O[i, 0] - softmax(lg) @ np.array(vals)).max() < 1e-12


def _brute_row(Q, K, V, tm, sel_t, t, i):
    """Explicit key list of one patch row, built from the definition."""
    keys, vals = [], []
    kept = set(int(u) for u in sel_t)
    for u in range(tm.T):
        if u in kept:
            for j in tm.tokens[u]:
                keys.append(float(Q[i] @ K[j]) / 8.0)
                vals.append(V[j])
        else:
            kb = K[tm.tokens[u]].mean(axis=0)
            keys.append(float(Q[i] @ kb) / 8.0 + math.log(tm.n[u]))
            vals.append(V[tm.tokens[u]].mean(axis=0))
    for s in tm.specials:
        keys.append(float(Q[i] @ K[s]) / 8.0)
        vals.append(V[s])
    if t not in kept:
        keys.append(float(Q[i] @ K[i]) / 8.0)
        vals.append(V[i])
    return softmax(np.array(keys)) @ np.array(vals)


def test_rows_match_explicit_key_lists_and_sampled_rows():
    tm = TileMap(3, 5, 16, 13)
    Q, K, V = _rand_qkv(tm.N, 2, 64, 17)
    O, sel, _ = osp.sparse_attention(Q, K, V, tm, 0.6)
    g = np.random.default_rng(0)
    for h in range(2):
        for i in g.choice(tm.N, 25, replace=False):
            t = tm.tile_of[i]
            if t < 0:
                want = softmax(K[:, h] @ Q[i, h] / 8.0) @ V[:, h]
            else:
                want = _brute_row(Q[:, h], K[:, h], V[:, h], tm, sel[h, t], t, i)
            assert np.abs(O[i, h] - want).max() < 1e-12
    rows = np.array([[h, i] for h in range(2) for i in range(0, tm.N, 37)])
    got, _ = osp.sparse_rows(Q, K, V, tm, 0.6, rows)
    assert np.abs(got - O[rows[:, 1], rows[:, 0]]).max() < 1e-13


# ---------------------------------------------------------------- planted mistakes
def test_pins_catch_planted_mistakes(monkeypatch):
    """Plant plausible mistakes in the oracle (CPU only) and check that the
    pins above fail on them."""
    tm = TileMap(2, 3, 12, 10)
    Q, K, V = _rand_qkv(tm.N, 1, 64, 9)
    good, _, _ = osp.sparse_attention(Q, K, V, tm, 0.5)
    real_landmarks = osp.landmarks

    # (1) landmark weight ln n dropped
    monkeypatch.setattr(osp, "landmarks", lambda K_h, V_h, tm_: real_landmarks(K_h, V_h, tm_)[:2]
                        + (np.zeros(tm_.T),))
    bad, _, _ = osp.sparse_attention(Q, K, V, tm, 0.5)
    assert np.abs(bad - good).max() > 1e-3
    monkeypatch.setattr(osp, "landmarks", real_landmarks)

    # (2) selection order flipped (keeps the lowest scores)
    real_sel = osp.select_one
    monkeypatch.setattr(osp, "select_one", lambda s, k: real_sel(-s, k))
    kbar, _, _ = osp.landmarks(K[:, 0], K[:, 0], tm)
    sel_bad, _, _ = osp.select_tiles(Q[:, 0], kbar, tm, 0.5)
    monkeypatch.setattr(osp, "select_one", real_sel)
    sel_ok, _, _ = osp.select_tiles(Q[:, 0], kbar, tm, 0.5)
    assert sel_bad.tolist() != sel_ok.tolist()
    assert sel_ok.tolist() == _brute_select(Q[:, 0], K[:, 0], tm, 0.5)
