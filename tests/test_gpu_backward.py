"""GPU parity of the backward passes (zebra_linear_attn_bwd) against the fp64
oracle (oracle/backward.py, pinned by finite differences in
test_oracle_backward.py), through the C ABI, on seeded synthetic inputs.

Bar of the linear stage, per element of dq, dk and dv: |gpu - oracle| <= one
bf16 step of the oracle value + 2^-12 x the largest |oracle| value of that
(token, head) row. The first term is the single rounding of the output to bf16. The
second bounds the fp32 arithmetic before it: products with the state and its
gradient carry about 16 significant bits (bf16 high/low splits), and the
softmax and RMSNorm backward subtract a row mean from every channel, which
can cancel most of a channel's value; 2^-12 leaves a factor of 16 over the
2^-16 of the products for that cancellation. The tile-sparse stage's bar is
derived beside SPARSE_ROW_REL below."""
import numpy as np
import pytest
import torch

import linear_global_attention_amd as zb
import zebra_synth as zs
from oracle import backward as obw
from oracle.layout import TileMap

from gpu_helpers import bf16_host, dev, dev_f32, log, widen

pytestmark = pytest.mark.gpu

ROW_REL = 2.0 ** -12
# The tile-sparse backward feeds P and the logit gradients dS to MFMA as
# bf16 (one rounding, 2^-9 relative, per term); where a row's sum of terms
# cancels to a fraction of its largest term, that grows to about 2^-6 of the
# row's largest gradient value. A row whose softmax puts almost all its mass
# on one key has a vanishing gradient (dS = P (dP - D) with dP - D ~ 1e-7
# from O(1) terms): there fp32 itself leaves an absolute error of a few
# 2^-24 |dP| |k|, which no per-row relative bound holds, so the bar adds
# 2^-12 of the largest gradient value of the head.
SPARSE_ROW_REL = 2.0 ** -6
SPARSE_HEAD_REL = 2.0 ** -12


def grad_close(got: np.ndarray, ref: np.ndarray, what: str, row_rel: float = ROW_REL,
               head_rel: float = 0.0) -> int:
    """got, ref [N][H][64]: |got - ref| <= one bf16 step of ref + row_rel x the
    row's largest |ref| + head_rel x the head's largest |ref|, per element.
    Returns the number of values beyond the bound (after logging the
    figures)."""
    assert np.isfinite(got).all(), f"{what}: non-finite gradient"
    step = 2.0 ** (np.frexp(np.maximum(np.abs(ref), 1e-300))[1] - 8)
    rowmax = np.abs(ref).max(axis=-1, keepdims=True)
    headmax = np.abs(ref).max(axis=(0, 2), keepdims=True)
    err = np.abs(got - ref)
    bound = step + row_rel * rowmax + head_rel * headmax
    rel = err / np.maximum(rowmax, 1e-300)
    log(f"{what}: max |err| / row max {rel.max():.2e}, mean {rel.mean():.2e}, "
        f"{int((err > step).sum())} of {err.size} values beyond one bf16 step, worst err / bound "
        f"{(err / bound).max():.3f}")
    nbad = int((err > bound).sum())
    if nbad:
        rows = np.argwhere((err > bound).any(axis=-1))
        log(f"{what}: {len(rows)} rows beyond the bound, first (token, head): {rows[:12].tolist()}")
    return nbad


def grads_close(got, ref, what: str, row_rel: float = ROW_REL, head_rel: float = 0.0) -> None:
    bad = {nm: grad_close(a, b, f"{what} {nm}", row_rel, head_rel) for nm, a, b in zip(("dq", "dk", "dv"), got, ref)}
    assert not any(bad.values()), f"{what}: values beyond the bound {bad}"


def _dy(L, seed):
    g = np.random.default_rng(seed)
    return zs.f32_to_bf16(g.standard_normal((L.tokens, L.heads, 64)).astype(np.float32))


def _linear_bwd_gpu(L, q, k, v, dy, W=None, gq=None, gk=None, eps=1e-6, base=100.0, fused=False):
    """dq, dk, dv of zebra_linear_attn_bwd as float64 [N][H][64]. fused: q,
    k, v (and dq, dk, dv) as slices of [N][3][H][64] buffers and dout as a
    slice of an [N][2][H][64] buffer."""
    zL = zb.Layout(L.frames, L.specials, L.rows, L.cols, L.heads)
    bufs = zb.StageBuffers(zL, 0.0, sparse=False)
    if fused:
        qkv = torch.stack([dev(q), dev(k), dev(v)], dim=1)
        qd, kd, vd = qkv[:, 0], qkv[:, 1], qkv[:, 2]
        dqkv = torch.zeros_like(qkv)
        gq_, gk_, gv_ = dqkv[:, 0], dqkv[:, 1], dqkv[:, 2]
        dout2 = torch.zeros((L.tokens, 2, L.heads, 64), dtype=torch.int16, device="cuda")
        dout2[:, 1] = dev(dy)
        dout = dout2[:, 1]
        out = dout2[:, 0]   # only its strides matter: the backward does not read out
    else:
        qd, kd, vd = dev(q), dev(k), dev(v)
        gq_, gk_, gv_ = (torch.zeros_like(qd) for _ in range(3))
        dout = dev(dy)
        out = torch.empty_like(dout)
    a = zb.make_args(zL, qd, kd, vd, out, bufs, 0.0, W=dev_f32(W), gq=dev_f32(gq), gk=dev_f32(gk),
                     rms_eps=eps, rope_base=base)
    zb.linear_attn_bwd(a, dout, gq_, gk_, gv_)
    torch.cuda.synchronize()
    res = tuple(bf16_host(t.contiguous()).reshape(L.tokens, L.heads, 64) for t in (gq_, gk_, gv_))
    if fused:
        assert torch.equal(qkv[:, 0], dev(q)) and torch.equal(qkv[:, 2], dev(v))
    return res


def _affine(L, seed):
    g = np.random.default_rng(seed)
    W = (np.eye(64)[None] + 0.2 * g.standard_normal((L.heads, 64, 64))).astype(np.float32)
    gq = (0.5 + g.random((L.heads, 64))).astype(np.float32)
    gk = (0.5 + g.random((L.heads, 64))).astype(np.float32)
    return W, gq, gk


CASES = [("partial", zs.Layout(3, 2, 11, 13, heads=2), False, False),
         ("partial-affine-gains", zs.Layout(3, 2, 11, 13, heads=2), True, False),
         ("vggt-2view-affine", zs.Layout(2, 5, 37, 37, heads=3), True, False),
         ("no-specials-fused", zs.Layout(3, 0, 9, 9, heads=2), True, True),
         ("vggt-2view-fused", zs.Layout(2, 5, 37, 37, heads=3), False, True),
         ("tiny-frames-affine-gains", zs.Layout(40, 1, 3, 4, heads=2), True, False)]


@pytest.mark.parametrize("name,L,affine,fused", CASES, ids=[c[0] for c in CASES])
def test_linear_bwd_full(name, L, affine, fused):
    """Every element of dq, dk and dv against the oracle, with and without
    the affine weight, RMSNorm gains, eps 1e-3 and rotary base 1e4, and with
    q, k, v, dq, dk, dv inside fused buffers and dout strided."""
    q, k, v = zs.stage_inputs(L, seed=31)
    dy = _dy(L, 31)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    W = gq = gk = None
    eps, base = 1e-6, 100.0
    if affine:
        W, gq, gk = _affine(L, 31)
        eps, base = 1e-3, 10000.0
    got = _linear_bwd_gpu(L, q, k, v, dy, W, gq, gk, eps, base, fused)
    ref = obw.linear_backward(widen(q), widen(k), widen(v), widen(dy), tm, W, gq, gk, eps, base)
    grads_close(got, ref, f"{name} linear backward")


def test_linear_bwd_32views():
    """32 views of 37x37 patches, 16 heads (44k tokens, a hundred
    workgroups per head): every element against the oracle."""
    L = zs.CONFIGS["32views"]
    q, k, v = zs.stage_inputs(L, seed=32)
    dy = _dy(L, 32)
    W, gq, gk = _affine(L, 32)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    got = _linear_bwd_gpu(L, q, k, v, dy, W, gq, gk)
    ref = obw.linear_backward(widen(q), widen(k), widen(v), widen(dy), tm, W, gq, gk)
    grads_close(got, ref, "32 views linear backward")


def test_linear_bwd_rejects_bad_arguments():
    L = zs.Layout(2, 1, 8, 8, heads=2)
    zL = zb.Layout(L.frames, L.specials, L.rows, L.cols, L.heads)
    q, k, v = (dev(x) for x in zs.stage_inputs(L, seed=1))
    bufs = zb.StageBuffers(zL, 0.0, sparse=False)
    a = zb.make_args(zL, q, k, v, torch.empty_like(q), bufs, 0.0)
    dq = torch.empty_like(q)
    with pytest.raises(ValueError):
        zb.linear_attn_bwd(a, torch.empty((L.tokens, L.heads, 32), dtype=torch.int16, device="cuda"), dq, dq, dq)
    st = zb.lib.zebra_linear_attn_bwd(__import__("ctypes").byref(a), None, zb._ptr(dq), zb._ptr(dq), zb._ptr(dq),
                                      zb._stream(None))
    assert st == 1 and "non-NULL" in zb.lib.zebra_last_error().decode()
    a.workspace_bytes = 16
    with pytest.raises(zb.ZebraError):
        zb.linear_attn_bwd(a, torch.empty_like(q), dq, dq, dq)


# ---------------------------------------------------------------- tile-sparse stage

def _sparse_bwd_gpu(L, q, k, v, dy, y, fused=False):
    """dq, dk, dv of zebra_sparse_attn_bwd (after pack with landmarks and
    selection on the same inputs) as float64 [N][H][64], and the kept tiles
    [H][T][k] the forward selected."""
    zL = zb.Layout(L.frames, L.specials, L.rows, L.cols, L.heads)
    bufs = zb.StageBuffers(zL, y, backward=True)
    if fused:
        qkv = torch.stack([dev(q), dev(k), dev(v)], dim=1)
        qd, kd, vd = qkv[:, 0], qkv[:, 1], qkv[:, 2]
        dqkv = torch.zeros_like(qkv)
        gq_, gk_, gv_ = dqkv[:, 0], dqkv[:, 1], dqkv[:, 2]
        dout2 = torch.zeros((L.tokens, 2, L.heads, 64), dtype=torch.int16, device="cuda")
        dout2[:, 1] = dev(dy)
        dout, out = dout2[:, 1], dout2[:, 0]
    else:
        qd, kd, vd = dev(q), dev(k), dev(v)
        gq_, gk_, gv_ = (torch.zeros_like(qd) for _ in range(3))
        dout = dev(dy)
        out = torch.empty_like(dout)
    a = zb.make_args(zL, qd, kd, vd, out, bufs, y)
    zb.pack_tiles(a)
    zb.select_tiles(a)
    zb.sparse_attn_bwd(a, dout, gq_, gk_, gv_)
    torch.cuda.synchronize()
    res = tuple(bf16_host(t.contiguous()).reshape(L.tokens, L.heads, 64) for t in (gq_, gk_, gv_))
    return res, bufs.sel().cpu().numpy().astype(np.int64)


SPARSE = [("partial-y0.5", zs.Layout(3, 2, 11, 13, heads=2), 0.5, False),
          ("no-specials-y0.3", zs.Layout(3, 0, 9, 9, heads=2), 0.3, False),
          ("dense-y0", zs.Layout(2, 3, 10, 7, heads=2), 0.0, False),
          ("landmarks-only-y1", zs.Layout(2, 2, 9, 11, heads=2), 1.0, False),
          ("vggt-2view-y0.8", zs.Layout(2, 5, 37, 37, heads=3), 0.8, False),
          ("fused-y0.6", zs.Layout(3, 40, 12, 10, heads=2), 0.6, True)]


@pytest.mark.parametrize("name,L,y,fused", SPARSE, ids=[c[0] for c in SPARSE])
def test_sparse_bwd_full(name, L, y, fused):
    """Every element of dq, dk and dv against the oracle's backward on the
    kept tiles the forward selected: partial tiles, no specials, y = 0
    (dense), y = 1 (landmarks only), 37x37 two-view, and fused QKV / dQKV
    buffers with a strided dout and 40 specials per frame (two special
    blocks)."""
    q, k, v = zs.stage_inputs(L, seed=41)
    dy = _dy(L, 41)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    got, sel = _sparse_bwd_gpu(L, q, k, v, dy, y, fused)
    ref = obw.sparse_backward(widen(q), widen(k), widen(v), widen(dy), tm, y, sel=sel)
    grads_close(got, ref, f"{name} sparse backward", SPARSE_ROW_REL, SPARSE_HEAD_REL)


def test_sparse_bwd_32views_rows_and_invariants():
    """32 views of 37x37 patches, 16 heads, y = 0.8: sampled dq rows (patch
    and special rows of 4 heads) against the oracle's row gradient on the
    forward's kept tiles, and over every key of every head the two exact
    invariants of softmax attention with mean landmarks: the value
    gradients sum to the output gradients, the key gradients sum to zero
    (within 2^-7 of the sum of their magnitudes: every term is rounded to
    bf16 once)."""
    L = zs.CONFIGS["32views"]
    y = 0.8
    q, k, v = zs.stage_inputs(L, seed=42)
    dy = _dy(L, 42)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    (dq, dk, dv), sel = _sparse_bwd_gpu(L, q, k, v, dy, y)
    dO = widen(dy)
    for nm, G, want in (("dv", dv, dO.sum(axis=0)), ("dk", dk, np.zeros((L.heads, 64)))):
        s = G.sum(axis=0)
        err = np.abs(s - want).max()
        scale = np.abs(G).sum(axis=0).max()
        log(f"32 views sparse backward: sum of {nm} over the keys within {err:.3e} of the invariant "
            f"(sum of magnitudes {scale:.3e})")
        assert err <= 2.0 ** -7 * scale
    Q, K, V = widen(q), widen(k), widen(v)
    rows = zs.sample_rows(L, 768, seed=42, special_frames=2)
    for h in range(4):
        toks = rows[rows[:, 0] == h, 1]
        ref = obw.sparse_dq_rows(Q[:, h], K[:, h], V[:, h], dO[:, h], tm, y, toks, sel=sel[h])
        got = dq[toks, h]
        n = grad_close(got[:, None, :], ref[:, None, :], f"32 views sparse backward dq rows, head {h}",
                       SPARSE_ROW_REL, SPARSE_HEAD_REL)
        assert n == 0


def test_sparse_bwd_128views_checkpoints():
    """128 views of 37x37 patches (3,200 key tiles, so the query-major
    passes' patch units meet at a checkpoint), 2 heads, y = 0.8: the exact
    invariants over every key, and sampled dq rows (patch and special rows
    of both heads) against the oracle's row gradient on the forward's kept
    tiles."""
    L = zs.Layout(128, 5, 37, 37, heads=2)
    y = 0.8
    q, k, v = zs.stage_inputs(L, seed=43)
    dy = _dy(L, 43)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    assert tm.T > 2048
    (dq, dk, dv), sel = _sparse_bwd_gpu(L, q, k, v, dy, y)
    dO = widen(dy)
    for nm, G, want in (("dv", dv, dO.sum(axis=0)), ("dk", dk, np.zeros((L.heads, 64)))):
        s = G.sum(axis=0)
        err = np.abs(s - want).max()
        scale = np.abs(G).sum(axis=0).max()
        log(f"128 views sparse backward: sum of {nm} over the keys within {err:.3e} of the invariant "
            f"(sum of magnitudes {scale:.3e})")
        assert err <= 2.0 ** -7 * scale
    Q, K, V = widen(q), widen(k), widen(v)
    rows = zs.sample_rows(L, 256, seed=43, special_frames=2)
    for h in range(L.heads):
        toks = rows[rows[:, 0] == h, 1]
        ref = obw.sparse_dq_rows(Q[:, h], K[:, h], V[:, h], dO[:, h], tm, y, toks, sel=sel[h])
        got = dq[toks, h]
        n = grad_close(got[:, None, :], ref[:, None, :], f"128 views sparse backward dq rows, head {h}",
                       SPARSE_ROW_REL, SPARSE_HEAD_REL)
        assert n == 0
