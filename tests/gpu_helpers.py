"""Helpers of the GPU parity tests: move seeded inputs to the device, run
the library through its C ABI, bring results back, compare with tolerances.

Tolerances (bf16 inputs and outputs, fp32 accumulation): max-abs 2e-2 and
mean-abs 2e-3 over the compared outputs."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import linear_global_attention_amd as zb
import zebra_synth as zs

MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda")


def dev_f32(a) -> torch.Tensor | None:
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda")


def bf16_host(t: torch.Tensor) -> np.ndarray:
    return zs.bf16_to_f32(t.cpu().numpy().view(np.uint16)).astype(np.float64)


def widen(a: np.ndarray) -> np.ndarray:
    return zs.bf16_to_f32(a).astype(np.float64)


def close(got: np.ndarray, want: np.ndarray, what: str) -> dict:
    err = np.abs(got - want)
    r = dict(max_abs=float(err.max()), mean_abs=float(err.mean()), n=int(err.size))
    log(f"{what}: max_abs={r['max_abs']:.3e} mean_abs={r['mean_abs']:.3e} over {r['n']} values")
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert r["max_abs"] <= MAX_ABS, f"{what}: max-abs {r['max_abs']:.3e} > {MAX_ABS}"
    assert r["mean_abs"] <= MEAN_ABS, f"{what}: mean-abs {r['mean_abs']:.3e} > {MEAN_ABS}"
    return r


class Stage:
    """Device copies of one stage's Q/K/V plus buffers and an output."""

    def __init__(self, L: zs.Layout, q, k, v, y: float, sparse: bool = True):
        self.L, self.y = L, y
        self.zL = zb.Layout(L.frames, L.specials, L.rows, L.cols, L.heads)
        self.q, self.k, self.v = dev(q), dev(k), dev(v)
        self.out = torch.empty_like(self.q)
        self.bufs = zb.StageBuffers(self.zL, y, sparse=sparse)

    def args(self, **kw) -> zb.Args:
        return zb.make_args(self.zL, self.q, self.k, self.v, self.out, self.bufs, self.y, **kw)

    def sparse(self):
        a = self.args()
        zb.sparse_stage(a)
        torch.cuda.synchronize()
        return self.out

    def select(self):
        """Pack, landmarks and tile selection only."""
        a = self.args()
        zb.pack_tiles(a)
        zb.landmarks(a)
        zb.select_tiles(a)
        torch.cuda.synchronize()
        return self.bufs.sel().cpu().numpy()

    def dense(self):
        zb.dense_attn(self.args())
        torch.cuda.synchronize()
        return self.out

    def linear(self, W=None, b=None, mu=None, gq=None, gk=None, eps=1e-6, base=100.0):
        Wd, bd, md = dev_f32(W), dev_f32(b), dev_f32(mu)
        gqd, gkd = dev_f32(gq), dev_f32(gk)
        zb.linear_attn(self.args(W=Wd, b=bd, mu=md, gq=gqd, gk=gkd, rms_eps=eps, rope_base=base))
        torch.cuda.synchronize()
        return self.out

    def rows(self, rows: np.ndarray) -> np.ndarray:
        """Output at (head, token) rows, float64 [R][64]."""
        r = torch.from_numpy(rows).to("cuda")
        o = self.out.view(self.L.tokens, self.L.heads, 64)[r[:, 1], r[:, 0]]
        return bf16_host(o)


NEAR_TIE = 1e-6


def valid_near_tie_list(kept: np.ndarray, scores: np.ndarray, k: int) -> None:
    """Checks a kept-tile list of a near-tie row, where several lists are
    correct. With a = the k-th and b = the (k+1)-th ranked oracle score and
    band = [b - delta, a + delta], delta = 1e-6 max(|a|, |b|): the list holds
    exactly k distinct tiles in ascending order, keeps every tile scoring
    above the band and none scoring below it."""
    kept = np.asarray(kept, dtype=np.int64)
    T = scores.shape[0]
    assert kept.shape == (k,), kept.shape
    assert np.all(np.diff(kept) > 0), "not strictly ascending"
    assert kept.min() >= 0 and kept.max() < T
    order = np.lexsort((np.arange(T), -scores))
    a, b = scores[order[k - 1]], scores[order[k]]
    delta = NEAR_TIE * max(abs(a), abs(b), 1e-300)
    must = np.flatnonzero(scores > a + delta)
    never = np.flatnonzero(scores < b - delta)
    assert np.isin(must, kept).all(), "a tile above the near-tie band was dropped"
    assert not np.isin(never, kept).any(), "a tile below the near-tie band was kept"


def compare_selection(sel_gpu: np.ndarray, sel_ref: np.ndarray, tie_ref: np.ndarray, what: str,
                      scores=None):
    """Bit-exact kept-tile lists except on near-tie rows, which are counted
    and, given scores(h, t) -> the oracle's fp64 scores of that row, checked
    for validity (valid_near_tie_list)."""
    assert sel_gpu.shape == sel_ref.shape, (sel_gpu.shape, sel_ref.shape)
    diff = np.any(sel_gpu != sel_ref, axis=-1)
    n_tie = int(tie_ref.sum())
    bad = diff & ~tie_ref
    log(f"{what}: {diff.sum()} of {diff.size} rows differ, {n_tie} near-tie rows, "
        f"{bad.sum()} differing non-tie rows")
    assert not bad.any(), f"{what}: selection differs on {bad.sum()} non-tie rows"
    if scores is not None:
        for h, t in np.argwhere(tie_ref):
            valid_near_tie_list(sel_gpu[h, t], scores(int(h), int(t)), sel_gpu.shape[-1])
        log(f"{what}: {n_tie} near-tie rows valid")
    return dict(rows=int(diff.size), near_tie=n_tie, differ=int(diff.sum()))


def oracle_scores(Q, K, tm, osp):
    """scores(h, t): the oracle's fp64 tile scores qbar_t . kbar_u / 8 of
    query tile t in head h (landmarks cached per head)."""
    cache = {}

    def f(h, t):
        if h not in cache:
            cache[h] = osp.landmarks(K[:, h], K[:, h], tm)[0]
        qbar = Q[tm.tokens[t], h].sum(axis=0) / tm.n[t]
        return cache[h] @ qbar / 8.0
    return f
