"""Seeded synthetic inputs for the global multi-view attention stage.

This module only draws inputs. It holds none of the attention arithmetic:
no landmarks, no selection, no softmax, no feature map. Both the fp64
oracle (through the tests) and the HIP library (through the tests and the
benchmark) take their inputs from here, byte for byte.

Sequence layout (the multi-view token sequence of a VGGT-style backbone):
each of F frames contributes S special tokens followed by an R x C patch
grid in row-major order, so token n of frame f sits at f*(S+R*C)+local.
Q, K and V are stored as [N][H][d] arrays of bfloat16 bit patterns
(numpy uint16), d = 64.

Value model ("tile-centroid" model). The pages describe video-like captures
in which attention concentrates on a few neighbouring frames (Zebra3D pages,
"Wide baselines punish the 0.7L setting"). To reproduce that structure each
(frame, 8x8 patch block, head) gets a centroid c ~ N(0, I_d):
  patch key    k = c[f][blk] + 0.5 * e_k
  patch query  q = 0.75 * (c[f-1][blk] + c[f+1][blk]) + 0.5 * e_q   (frames cyclic)
  patch value  v = e_v
  special q, k, v = e_q, e_k, e_v
with e ~ N(0, I) drawn per token and head. For two frames f-1 and f+1 are the
same frame, so q = 1.5 * c[other frame][blk] + 0.5 * e_q.

Randomness: every draw comes from a PCG64 stream keyed by
SeedSequence([seed, stage, tensor_id, chunk]), chunk = a fixed block of
2048 tokens (or one frame for the centroids). Values are drawn in float32,
combined in float32 and rounded to bfloat16 with round-to-nearest-even.
The bytes therefore do not depend on the thread count.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

__all__ = [
    "Layout", "CONFIGS", "stage_inputs", "stage_inputs_device", "affine_params", "calib_mean",
    "sample_rows", "bf16_to_f32", "f32_to_bf16", "draw_threads",
]

TOKEN_CHUNK = 2048
_T_CENTROID, _T_Q, _T_K, _T_V, _T_W, _T_B, _T_ROWS, _T_MU = range(8)


@dataclass(frozen=True)
class Layout:
    frames: int
    specials: int
    rows: int
    cols: int
    heads: int = 16
    head_dim: int = 64

    @property
    def tokens_per_frame(self) -> int:
        return self.specials + self.rows * self.cols

    @property
    def tokens(self) -> int:
        return self.frames * self.tokens_per_frame


# Synthetic multi-view shapes: a 2-frame 16x16 toy stage, and VGGT-like
# 37x37-patch frames with 5 special tokens at 32, 128, 512 and 1,024 views.
CONFIGS = {
    "2views_16x16": Layout(2, 5, 16, 16, heads=1),
    "32views": Layout(32, 5, 37, 37),
    "128views": Layout(128, 5, 37, 37),
    "512views": Layout(512, 5, 37, 37),
    "1024views": Layout(1024, 5, 37, 37),
}


def draw_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _rng(seed: int, stage: int, tensor: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([int(seed), int(stage), int(tensor), int(chunk)])))


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 bit patterns, round-to-nearest-even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _block_of_patch(L: Layout) -> np.ndarray:
    """Index of the 8x8 patch block that each patch of a frame falls in
    (row-major blocks). This is the data model's centroid assignment."""
    bc = -(-L.cols // 8)
    r = np.arange(L.rows)[:, None] // 8
    c = np.arange(L.cols)[None, :] // 8
    return (r * bc + c).reshape(-1)


def stage_inputs(L: Layout, seed: int = 0, stage: int = 0, threads: int | None = None):
    """Draw Q, K, V for one global stage. Returns (q, k, v) as uint16
    bf16 bit arrays of shape [N][H][d]."""
    H, d, F, S = L.heads, L.head_dim, L.frames, L.specials
    blocks = -(-L.rows // 8) * -(-L.cols // 8)
    cen = np.empty((F, blocks, H, d), np.float32)
    for f in range(F):
        _rng(seed, stage, _T_CENTROID, f).standard_normal(out=cen[f], dtype=np.float32)
    nb = (cen[(np.arange(F) - 1) % F] + cen[(np.arange(F) + 1) % F]) * np.float32(0.75)
    blk = _block_of_patch(L)
    tpf = L.tokens_per_frame
    N = L.tokens
    q = np.empty((N, H, d), np.uint16)
    k = np.empty((N, H, d), np.uint16)
    v = np.empty((N, H, d), np.uint16)
    nchunks = -(-N // TOKEN_CHUNK)

    def work(ci: int) -> None:
        n0, n1 = ci * TOKEN_CHUNK, min(N, (ci + 1) * TOKEN_CHUNK)
        n = np.arange(n0, n1)
        f = n // tpf
        loc = n % tpf
        patch = loc >= S
        pf, pb = f[patch], blk[loc[patch] - S]
        half = np.float32(0.5)
        for tid, out in ((_T_Q, q), (_T_K, k), (_T_V, v)):
            e = np.empty((n1 - n0, H, d), np.float32)
            _rng(seed, stage, tid, ci).standard_normal(out=e, dtype=np.float32)
            if tid != _T_V:
                e[patch] *= half
                e[patch] += (nb if tid == _T_Q else cen)[pf, pb]
            out[n0:n1] = f32_to_bf16(e)

    with ThreadPoolExecutor(threads or draw_threads()) as ex:
        list(ex.map(work, range(nchunks)))
    return q, k, v


def stage_inputs_device(L: Layout, seed: int = 0, stage: int = 0, device="cuda"):
    """The same tile-centroid model drawn with torch's generator on `device`
    (fast enough to give every stage of a long schedule fresh inputs). The
    stream is torch's, keyed by (seed, stage, tensor), so the values differ
    from stage_inputs'; anything checked against the oracle reads these
    tensors' own bytes back. Returns (q, k, v) as int16 tensors [N][H][d]
    holding bfloat16 bit patterns (round to nearest even)."""
    import torch
    H, d, F, S = L.heads, L.head_dim, L.frames, L.specials
    blocks = -(-L.rows // 8) * -(-L.cols // 8)

    def gen(tensor: int):
        g = torch.Generator(device=device)
        g.manual_seed((int(seed) * 1_000_003 + int(stage)) * 16 + tensor)
        return g

    cen = torch.randn((F, blocks, H, d), generator=gen(_T_CENTROID), device=device, dtype=torch.float32)
    idx = torch.arange(F, device=device)
    nb = (cen[(idx - 1) % F] + cen[(idx + 1) % F]) * 0.75
    blk = torch.from_numpy(_block_of_patch(L)).to(device)
    out = []
    for tid in (_T_Q, _T_K, _T_V):
        e = torch.randn((F, L.tokens_per_frame, H, d), generator=gen(tid), device=device, dtype=torch.float32)
        if tid != _T_V:
            e[:, S:] *= 0.5
            e[:, S:] += (nb if tid == _T_Q else cen)[:, blk]
        out.append(e.reshape(L.tokens, H, d).to(torch.bfloat16).view(torch.int16))
        del e
    return tuple(out)


def calib_mean(L: Layout, seed: int = 0, stage: int = 0):
    """A seeded stand-in for the calibration mean mu of the centred affine
    correction, 0.01 * N(0, I) per head (float32 [H][d])."""
    return (_rng(seed, stage, _T_MU, 0).standard_normal((L.heads, L.head_dim), dtype=np.float32)
            * np.float32(0.01))


def affine_params(L: Layout, seed: int = 0, stage: int = 0):
    """Per-head affine output parameters W = I + 0.05*G/8, b = 0.01*N(0, I)
    (float32, W as [H][d][d] acting on column vectors, b as [H][d])."""
    H, d = L.heads, L.head_dim
    g = _rng(seed, stage, _T_W, 0).standard_normal((H, d, d), dtype=np.float32)
    W = np.eye(d, dtype=np.float32)[None] + g * np.float32(0.05 / 8)
    b = _rng(seed, stage, _T_B, 0).standard_normal((H, d), dtype=np.float32) * np.float32(0.01)
    return W.astype(np.float32), b.astype(np.float32)


def sample_rows(L: Layout, n_rows: int, seed: int = 0, stage: int = 0,
                special_frames: int = 0) -> np.ndarray:
    """Seeded (head, token) query rows: every special-token row of
    `special_frames` distinct seed-chosen frames (all heads), then uniform
    rows over all (head, token) pairs until n_rows rows are drawn (no
    repeats). Returns int64 [n_rows][2], sorted by (head, token)."""
    g = _rng(seed, stage, _T_ROWS, 0)
    H, S, tpf = L.heads, L.specials, L.tokens_per_frame
    rows = set()
    if special_frames:
        frames = g.choice(L.frames, size=special_frames, replace=False)
        for f in frames:
            for s in range(S):
                for h in range(H):
                    rows.add((h, int(f) * tpf + s))
    if len(rows) > n_rows:
        raise ValueError("n_rows smaller than the special rows requested")
    while len(rows) < n_rows:
        h = int(g.integers(H))
        t = int(g.integers(L.tokens))
        rows.add((h, t))
    return np.array(sorted(rows), dtype=np.int64).reshape(-1, 2)
