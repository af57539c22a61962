"""GPU parity of every hot-path entry point against the fp64 oracle, through
the C ABI, on seeded synthetic inputs (tile-centroid model).

Bars: packing, landmark means and tile selection bit-exact (selection except
rows whose k-th/(k+1)-th score gap is below 1e-6 relative, which are
counted and reported); attention outputs within max-abs 2e-2 and mean-abs
2e-3 of the oracle."""
import numpy as np
import pytest
import torch

import linear_global_attention_amd as zb
import zebra_synth as zs
from oracle import linear as olin
from oracle import sparse as osp
from oracle.layout import TileMap, keep_count

from gpu_helpers import Stage, bf16_host, close, compare_selection, dev_f32, log, oracle_scores, widen

pytestmark = pytest.mark.gpu


def _inputs(L, seed=0, stage=0):
    q, k, v = zs.stage_inputs(L, seed=seed, stage=stage)
    return q, k, v


def _sel_ref(Q, K, tm, y):
    H = Q.shape[1]
    sels, ties = [], []
    for h in range(H):
        kbar, _, _ = osp.landmarks(K[:, h], K[:, h], tm)
        s, t, _ = osp.select_tiles(Q[:, h], kbar, tm, y)
        sels.append(s)
        ties.append(t)
    return np.stack(sels), np.stack(ties)


# ------------------------------------------------------------- small, full
EDGE = [
    ("2views_16x16", zs.CONFIGS["2views_16x16"], 0.5),
    ("partial-no-specials", zs.Layout(3, 0, 11, 13, heads=2), 0.3),
    ("partial-y0", zs.Layout(2, 3, 9, 17, heads=2), 0.0),
    ("partial-y1", zs.Layout(2, 3, 9, 17, heads=2), 1.0),
    ("one-tile", zs.Layout(1, 2, 8, 8, heads=1), 0.5),
    ("one-small-tile", zs.Layout(1, 1, 3, 5, heads=1), 0.7),
    ("vggt-2view", zs.Layout(2, 5, 37, 37, heads=2), 0.8),
    # 13 frames: the attention groups query tiles of one tile position in
    # frames of one parity, five at a time (frames 0, 2, .., 8 | 1, 3, .., 9 |
    # 10, 12 | 11), so the last groups are short
    ("partial-13frames", zs.Layout(13, 2, 9, 11, heads=2), 0.6),
]


@pytest.mark.parametrize("name,L,y", EDGE, ids=[e[0] for e in EDGE])
def test_sparse_stage_full(name, L, y):
    log(f"sparse full {name} {L} y={y}")
    q, k, v = _inputs(L, seed=1)
    Q, K, V = widen(q), widen(k), widen(v)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    st = Stage(L, q, k, v, y)
    out = bf16_host(st.sparse()).reshape(L.tokens, L.heads, 64)
    O_ref, sel_ref, tie_ref = osp.sparse_attention(Q, K, V, tm, y)
    kk = keep_count(y, tm.T)
    if kk > 0:
        sel = st.bufs.sel().cpu().numpy()
        compare_selection(sel, sel_ref, tie_ref, f"{name} selection", oracle_scores(Q, K, tm, osp))
        # the bitmap agrees with the lists
        mask = st.bufs.selmask().cpu().numpy().view(np.uint32)
        for h in range(L.heads):
            for t in range(tm.T):
                bits = [u for u in range(tm.T) if (mask[h, t, u // 32] >> (u % 32)) & 1]
                assert bits == sel[h, t].tolist()
    close(out, O_ref, f"{name} sparse output")


@pytest.mark.parametrize("name,L,y", EDGE[:3] + EDGE[4:5], ids=[e[0] for e in EDGE[:3] + EDGE[4:5]])
def test_pack_and_landmarks_exact(name, L, y):
    q, k, v = _inputs(L, seed=2)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    st = Stage(L, q, k, v, y)
    st.sparse()
    H = L.heads
    kt = st.bufs.t["KT"].cpu().numpy().view(np.uint16)
    vt = st.bufs.t["VT"].cpu().numpy().view(np.uint16)
    slots = []
    off = 0
    for u in range(tm.T):
        slots.append(off)
        off += -(-int(tm.n[u]) // 32) * 32
    kt = kt[: H * off * 64].reshape(H, off, 64)
    vt = vt[: H * off * 64].reshape(H, off // 32, 64, 32)
    for u in range(tm.T):
        toks = tm.tokens[u]
        s0 = slots[u]
        n = len(toks)
        assert np.array_equal(kt[:, s0:s0 + n, :], k[toks].transpose(1, 0, 2)), u
        pad = -(-n // 32) * 32
        assert not kt[:, s0 + n:s0 + pad].any()
        for j, tok in enumerate(toks):
            blk, kk = (s0 + j) // 32, (s0 + j) % 32
            col = ((kk & 15) >> 2) * 8 + (kk >> 4) * 4 + (kk & 3)  # keys permuted per block
            assert np.array_equal(vt[:, blk, :, col], v[tok]), (u, j)
    kbar = st.bufs.kbar().cpu().numpy()
    for h in range(H):
        kb, _, _ = osp.landmarks(widen(k)[:, h], widen(v)[:, h], tm)
        assert np.array_equal(kbar[h], kb), h  # exact fp64 sums, one rounding
    # the landmarks written by the pack pass equal zebra_landmarks' from the
    # packed buffers, byte for byte (landmark table and its padding included)
    names = ("KBAR", "VBAR", "LOGN", "LM")
    fused = {n: st.bufs.t[n].clone() for n in names}
    for n in names:
        st.bufs.t[n].fill_(0x7F)
    zb.landmarks(st.args())
    torch.cuda.synchronize()
    for n in names:
        nb = zb.buffer_bytes(st.zL, y, n)
        assert torch.equal(st.bufs.t[n][:nb], fused[n][:nb]), n


def test_landmark_of_identical_tile_equals_tile():
    L = zs.Layout(2, 2, 11, 9, heads=2)
    q, k, v = _inputs(L, seed=3)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    for u in range(tm.T):
        k[tm.tokens[u]] = k[tm.tokens[u][0]]
        v[tm.tokens[u]] = v[tm.tokens[u][0]]
    st = Stage(L, q, k, v, 0.5)
    st.sparse()
    kbar = st.bufs.kbar().cpu().numpy()
    vbar = st.bufs.t["VBAR"][: L.heads * tm.T * 64 * 4].view(torch.float32).cpu().numpy()
    vbar = vbar.reshape(L.heads, tm.T, 64)
    for u in range(tm.T):
        assert np.array_equal(kbar[:, u], widen(k[tm.tokens[u][0]]))
        assert np.array_equal(vbar[:, u], widen(v[tm.tokens[u][0]]).astype(np.float32))


@pytest.mark.parametrize("name,L", [("2views_16x16", zs.CONFIGS["2views_16x16"]), ("partial", zs.Layout(3, 2, 11, 13, heads=2)),
                                    ("vggt-2view", zs.Layout(2, 5, 37, 37, heads=2))])
def test_dense_full(name, L):
    q, k, v = _inputs(L, seed=4)
    st = Stage(L, q, k, v, 0.0)
    out = bf16_host(st.dense()).reshape(L.tokens, L.heads, 64)
    ref = osp.dense_attention(widen(q), widen(k), widen(v))
    close(out, ref, f"{name} dense")


def test_y0_sparse_equals_dense_on_gpu():
    L = zs.Layout(2, 5, 16, 24, heads=2)
    q, k, v = _inputs(L, seed=5)
    st = Stage(L, q, k, v, 0.0)
    a = bf16_host(st.sparse())
    b = bf16_host(st.dense())
    close(a, b, "y=0 sparse vs dense (GPU)")


LIN = [("2views_16x16-identity", zs.CONFIGS["2views_16x16"], False),
       ("partial-affine", zs.Layout(3, 2, 11, 13, heads=2), True),
       ("vggt-2view-affine", zs.Layout(2, 5, 37, 37, heads=3), True),
       # 13 tokens per frame: a wave's next 16-token group lies several
       # frames on, so the stepped frame positions wrap more than once
       ("tiny-frames-affine", zs.Layout(40, 1, 3, 4, heads=2), True)]


@pytest.mark.parametrize("name,L,affine", LIN, ids=[x[0] for x in LIN])
def test_linear_full(name, L, affine):
    q, k, v = _inputs(L, seed=6)
    Q, K, V = widen(q), widen(k), widen(v)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    W = b = mu = None
    if affine:
        W, b = zs.affine_params(L, seed=6)
        mu = np.stack([olin.mean_output(Q[:, h], K[:, h], V[:, h], tm)
                       for h in range(L.heads)]).astype(np.float32)
    st = Stage(L, q, k, v, 0.0, sparse=False)
    out = bf16_host(st.linear(W, b, mu)).reshape(L.tokens, L.heads, 64)
    ref = olin.linear_attention(Q, K, V, tm, W, b, mu)
    close(out, ref, f"{name} linear")


GAINS = [("partial-gains", zs.Layout(3, 2, 11, 13, heads=2)),
         ("vggt-2view-gains", zs.Layout(2, 5, 37, 37, heads=3))]


@pytest.mark.parametrize("name,L", GAINS, ids=[x[0] for x in GAINS])
def test_linear_gains_eps_base(name, L):
    """zebra_linear_attn with per-head RMSNorm gains on Q and K (random, in
    [0.5, 1.5)), eps = 1e-3 and rotary base 10,000, plus the per-head affine
    correction: every row against the oracle at the same settings."""
    q, k, v = _inputs(L, seed=17)
    Q, K, V = widen(q), widen(k), widen(v)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    g = np.random.default_rng(17)
    gq = (0.5 + g.random((L.heads, 64))).astype(np.float32)
    gk = (0.5 + g.random((L.heads, 64))).astype(np.float32)
    eps, base = 1e-3, 10000.0
    W, b = zs.affine_params(L, seed=17)
    mu = np.stack([olin.mean_output(Q[:, h], K[:, h], V[:, h], tm, gq[h], gk[h], eps, base)
                   for h in range(L.heads)]).astype(np.float32)
    st = Stage(L, q, k, v, 0.0, sparse=False)
    out = bf16_host(st.linear(W, b, mu, gq, gk, eps, base)).reshape(L.tokens, L.heads, 64)
    ref = olin.linear_attention(Q, K, V, tm, W, b, mu, gq, gk, eps, base)
    close(out, ref, f"{name} linear with gains, eps {eps}, base {base}")
    # the settings matter at this tolerance: defaults give another output
    plain = olin.linear_attention(Q, K, V, tm, W, b, mu)
    assert np.abs(plain - ref).max() > 5e-2


def test_32views_linear_gains_rows():
    L = zs.CONFIGS["32views"]
    q, k, v = _inputs(L, seed=18)
    Q, K, V = widen(q), widen(k), widen(v)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    g = np.random.default_rng(18)
    gq = (0.5 + g.random((L.heads, 64))).astype(np.float32)
    gk = (0.5 + g.random((L.heads, 64))).astype(np.float32)
    W, b = zs.affine_params(L, seed=18)
    mu = (0.01 * g.standard_normal((L.heads, 64))).astype(np.float32)
    rows = zs.sample_rows(L, 512, seed=18, special_frames=2)
    st = Stage(L, q, k, v, 0.0, sparse=False)
    st.linear(W, b, mu, gq, gk, 1e-3, 10000.0)
    ref = olin.linear_rows(Q, K, V, tm, rows, W, b, mu, gq, gk, 1e-3, 10000.0)
    close(st.rows(rows), ref, "32 views: linear rows with gains, eps 1e-3, base 1e4")


def test_fused_qkv_and_strided_output():
    """Q, K and V as views of one fused projection output [N][3][H][64]
    (token stride 3*H*64) and the output as every other 64-channel row of a
    wider buffer (head stride 128): every entry point reads and writes
    through the strides. Results equal the contiguous run's bit for bit (the
    same kernels over the same values), the rows between the output views
    stay untouched, and the sparse output is within tolerance of the oracle."""
    from gpu_helpers import dev
    L = zs.Layout(3, 2, 11, 13, heads=2)
    y = 0.5
    q, k, v = _inputs(L, seed=19)
    N, H = L.tokens, L.heads
    zL = zb.Layout(L.frames, L.specials, L.rows, L.cols, H)
    W, b = zs.affine_params(L, seed=19)
    mu = zs.calib_mean(L, seed=19)
    Wd, bd, mud = (torch.from_numpy(x).cuda() for x in (W, b, mu))
    st = Stage(L, q, k, v, y)
    want_sparse = st.sparse().clone()
    zb.linear_attn(st.args(W=Wd, b=bd, mu=mud))
    torch.cuda.synchronize()
    want_linear = st.out.clone()
    want_dense = st.dense().clone()
    stats_c = torch.zeros(zb.AFFINE_STATS, dtype=torch.float64, device="cuda")
    st.out.copy_(want_linear)
    zb.affine_stats(st.args(), st.v, stats_c)

    qkv = torch.stack([dev(q), dev(k), dev(v)], dim=1)  # [N][3][H][64]
    qv, kv, vv = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    wide = torch.full((N, H, 2, 64), 0x1234, dtype=torch.int16, device="cuda")
    ov = wide[:, :, 1]
    bufs = zb.StageBuffers(zL, y)
    a = zb.make_args(zL, qv, kv, vv, ov, bufs, y)
    assert (a.L.tok_stride, a.L.head_stride, a.L.out_tok_stride, a.L.out_head_stride) == (3 * H * 64, 64, H * 128, 128)
    zb.sparse_stage(a)
    torch.cuda.synchronize()
    assert torch.equal(ov, want_sparse), "strided sparse stage differs from the contiguous one"
    out = bf16_host(ov.contiguous()).reshape(N, H, 64)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    O_ref, _, _ = osp.sparse_attention(widen(q), widen(k), widen(v), tm, y)
    close(out, O_ref, "fused-QKV strided sparse output")
    zb.linear_attn(zb.make_args(zL, qv, kv, vv, ov, bufs, y, W=Wd, b=bd, mu=mud))
    torch.cuda.synchronize()
    assert torch.equal(ov, want_linear), "strided linear stage differs"
    an = zb.make_args(zL, qv, kv, vv, ov, bufs, y, W=Wd, b=bd, mu=mud)
    an.workspace, an.workspace_bytes = None, 0
    ov.fill_(0)
    zb.linear_attn_noalloc(an)
    torch.cuda.synchronize()
    assert torch.equal(ov, want_linear), "strided no-alloc linear stage differs"
    stats_s = torch.zeros(zb.AFFINE_STATS, dtype=torch.float64, device="cuda")
    zb.affine_stats(zb.make_args(zL, qv, kv, vv, ov, bufs, y), vv, stats_s)
    torch.cuda.synchronize()
    assert torch.equal(stats_s, stats_c), "affine statistics through strides differ"
    zb.dense_attn(zb.make_args(zL, qv, kv, vv, ov, bufs, y))
    torch.cuda.synchronize()
    assert torch.equal(ov, want_dense), "strided dense attention differs"
    assert bool((wide[:, :, 0] == 0x1234).all()), "rows between the output views were written"
    log("fused QKV / strided output: sparse, linear, no-alloc linear, affine statistics, dense bit-equal")


COV = [("2views_16x16", zs.CONFIGS["2views_16x16"], 0.5), ("partial", zs.Layout(3, 2, 11, 13, heads=2), 0.3),
       ("partial-y0", zs.Layout(2, 3, 9, 17, heads=2), 0.0), ("partial-y1", zs.Layout(2, 3, 9, 17, heads=2), 1.0),
       ("vggt-2view", zs.Layout(2, 5, 37, 37, heads=2), 0.8)]
COV_TOL = 1e-4     # coverage: fp32 sums of exactly computed logits
# Landmark error: the kernel's landmark keys are kbar rounded to bf16 (as the
# sparse kernel uses them), the oracle's are fp64 means. Rounding moves each
# element by at most 2^-9 of itself, so a landmark logit moves by at most
# b = |q| |kbar| 2^-9 / 8 (Cauchy-Schwarz) and the landmark mass by a factor
# within e^(+-b); the error 1 - L/E then moves by at most e^b - 1 (L <= E).
# Each tile is held to that bound (b from its largest |q| and the head's
# largest |kbar|), and the mean deviation to 5e-3.
LMERR_MEAN = 5e-3


def _lm_bound(Q_h, K_h, tm, tiles):
    """e^b - 1 per query tile, b = max |q| * max |kbar| * 2^-9 / 8."""
    kb = np.array([K_h[tm.tokens[u]].mean(axis=0) for u in range(tm.T)])
    kmax = np.linalg.norm(kb, axis=1).max()
    qn = np.array([np.linalg.norm(Q_h[tm.tokens[t]], axis=1).max() for t in tiles])
    return np.expm1(qn * kmax * 2.0 ** -9 / 8.0)


def _coverage_gpu(st):
    a = st.args()
    zb.pack_tiles(a)
    zb.select_tiles(a)
    H, T = st.L.heads, st.bufs.T
    cov = torch.empty(H * T, dtype=torch.float32, device="cuda")
    err = torch.empty_like(cov)
    zb.coverage(a, cov, err)
    torch.cuda.synchronize()
    return cov.view(H, T).cpu().numpy().astype(np.float64), err.view(H, T).cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name,L,y", COV, ids=[c[0] for c in COV])
def test_coverage_full(name, L, y):
    """zebra_coverage against the oracle on every (head, query tile)."""
    from oracle import coverage as ocov
    q, k, v = _inputs(L, seed=20)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    cov, err = _coverage_gpu(Stage(L, q, k, v, y))
    rc, re = ocov.coverage(widen(q), widen(k), tm, y)
    dc, de = np.abs(cov - rc), np.abs(err - re)
    bound = np.stack([_lm_bound(widen(q[:, h]), widen(k[:, h]), tm, range(tm.T)) for h in range(L.heads)])
    log(f"{name} coverage: max |gpu - oracle| {dc.max():.2e}; landmark error: max {de.max():.2e}, "
        f"mean {de.mean():.2e}, largest share of its bound {(de / bound).max():.2f} "
        f"(coverage mean {rc.mean():.3f}, landmark error mean {re.mean():.3f})")
    assert dc.max() <= COV_TOL and np.all(de <= bound) and de.mean() <= LMERR_MEAN
    if y == 1.0:
        assert np.all(cov == 0.0)
    if y == 0.0:
        assert np.all(err == 0.0)


def test_32views_coverage_sampled_tiles():
    from oracle import coverage as ocov
    L = zs.CONFIGS["32views"]
    y = 0.8
    q, k, v = _inputs(L, seed=21)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    cov, err = _coverage_gpu(Stage(L, q, k, v, y))
    g = np.random.default_rng(21)
    worst_c = worst_e = 0.0
    de = []
    for h in (0, 7, 15):
        tiles = np.sort(g.choice(tm.T, 12, replace=False))
        rc, re = ocov.coverage_head(widen(q[:, h]), widen(k[:, h]), tm, y, query_tiles=tiles)
        worst_c = max(worst_c, float(np.abs(cov[h, tiles] - rc).max()))
        d = np.abs(err[h, tiles] - re)
        assert np.all(d <= _lm_bound(widen(q[:, h]), widen(k[:, h]), tm, tiles)), h
        de.append(d)
    de = np.concatenate(de)
    log(f"32 views coverage (36 sampled tiles): max |gpu - oracle| {worst_c:.2e}, landmark error max {de.max():.2e} "
        f"mean {de.mean():.2e}; mean coverage {cov.mean():.3f}, mean landmark error {err.mean():.3f}")
    assert worst_c <= COV_TOL and de.mean() <= LMERR_MEAN
    assert np.all((cov > 0) & (cov < 1)) and np.all(err > -1e-4) and np.all(err < 1)


PRO = [("partial-defaults", zs.Layout(3, 2, 11, 13, heads=2), None, 1e-6, 100.0),
       ("partial-gains", zs.Layout(3, 2, 11, 13, heads=2), 17, 1e-3, 1000.0),
       ("vggt-2view", zs.Layout(2, 5, 37, 37, heads=3), 18, 1e-6, 100.0)]


@pytest.mark.parametrize("name,L,gseed,eps,base", PRO, ids=[p[0] for p in PRO])
def test_qk_prologue(name, L, gseed, eps, base):
    """zebra_qk_prologue against the oracle's RoPE2D(RMSNorm(.)) rounded to
    bf16: every element within one bf16 step (fp32 on the GPU against fp64
    before the same rounding), and in place into a fused QKV buffer."""
    from gpu_helpers import dev
    from oracle import block as ob
    q, k, v = _inputs(L, seed=22)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    gq = gk = None
    if gseed is not None:
        g = np.random.default_rng(gseed)
        gq = (0.5 + g.random((L.heads, 64))).astype(np.float32)
        gk = (0.5 + g.random((L.heads, 64))).astype(np.float32)
    st = Stage(L, q, k, v, 0.0, sparse=False)
    a = st.args(gq=dev_f32(gq), gk=dev_f32(gk), rms_eps=eps, rope_base=base)
    qo, ko = torch.empty_like(st.q), torch.empty_like(st.k)
    zb.qk_prologue(a, qo, ko)
    torch.cuda.synchronize()
    for got, x, gain, nm in ((qo, q, gq, "q"), (ko, k, gk, "k")):
        ref = ob.round_bf16(ob.prologue(widen(x), tm, gain, eps, base))
        got = bf16_host(got).reshape(ref.shape)
        # One bf16 step of the result, but at least 2^-18: a rotated pair
        # lo*c - hi*s can cancel to a value far below its O(1) products
        # (the normalised rows have RMS 1, times gains < 1.5), and the fp32
        # rounding of those products and of the fp32 cos/sin table (a few
        # 2^-24 each) then exceeds a bf16 step of the small result.
        ulp = 2.0 ** (np.frexp(np.maximum(np.abs(ref), 1e-30))[1] - 8)
        err = np.abs(got - ref)
        bad = err > np.maximum(ulp, 2.0 ** -18)
        log(f"{name} prologue {nm}: {int((got != ref).sum())} of {got.size} values differ from the rounded oracle, "
            f"{int((err > ulp).sum())} by more than one bf16 step, largest such error {float(err[err > ulp].max(initial=0)):.2e}")
        assert not bad.any()
    # in place, inside a fused [N][3][H][64] buffer
    qkv = torch.stack([dev(q), dev(k), dev(v)], dim=1)
    zL = zb.Layout(L.frames, L.specials, L.rows, L.cols, L.heads)
    af = zb.make_args(zL, qkv[:, 0], qkv[:, 1], qkv[:, 2], None, None, 0.0, gq=dev_f32(gq), gk=dev_f32(gk),
                      rms_eps=eps, rope_base=base)
    zb.qk_prologue(af, qkv[:, 0], qkv[:, 1])
    torch.cuda.synchronize()
    assert torch.equal(qkv[:, 0], qo) and torch.equal(qkv[:, 1], ko) and torch.equal(qkv[:, 2], dev(v))


FRAME = [("2views_16x16", zs.CONFIGS["2views_16x16"]), ("partial", zs.Layout(3, 2, 11, 13, heads=2)),
         ("no-specials", zs.Layout(3, 0, 9, 9, heads=2)), ("vggt-2view", zs.Layout(2, 5, 37, 37, heads=2)),
         ("40-specials", zs.Layout(2, 40, 5, 7, heads=1))]


@pytest.mark.parametrize("name,L", FRAME, ids=[f[0] for f in FRAME])
def test_frame_attn_full(name, L):
    from oracle import block as ob
    q, k, v = _inputs(L, seed=23)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    st = Stage(L, q, k, v, 0.0, sparse=False)
    zb.frame_attn(st.args())
    torch.cuda.synchronize()
    out = bf16_host(st.out).reshape(L.tokens, L.heads, 64)
    close(out, ob.frame_attention(widen(q), widen(k), widen(v), tm), f"{name} frame-wise attention")


def test_alternating_block_32views():
    """One frame-wise stage, then a tile-sparse global stage (y = 0.8) whose
    queries and keys first pass the prologue, on 32 views: sampled rows of
    each step against the oracle taking the same steps (the prologue output
    rounded to bf16, where the selector decides from it)."""
    from oracle import block as ob
    L = zs.CONFIGS["32views"]
    y = 0.8
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    rows = zs.sample_rows(L, 384, seed=24, special_frames=1)
    q, k, v = _inputs(L, seed=24, stage=0)
    st = Stage(L, q, k, v, y)
    zb.frame_attn(st.args())
    torch.cuda.synchronize()
    Q, K, V = widen(q), widen(k), widen(v)
    ref = np.stack([ob.frame_attention_head(Q[:, h], K[:, h], V[:, h], tm)[t] for h, t in rows])
    close(st.rows(rows), ref, "32 views: frame-wise stage (sampled rows)")
    q2, k2, v2 = _inputs(L, seed=24, stage=1)
    st2 = Stage(L, q2, k2, v2, y)
    zb.qk_prologue(st2.args(), st2.q, st2.k)  # in place
    st2.sparse()
    Qp = ob.round_bf16(ob.prologue(widen(q2), tm))
    Kp = ob.round_bf16(ob.prologue(widen(k2), tm))
    ref2, _ = osp.sparse_rows(Qp, Kp, widen(v2), tm, y, rows)
    close(st2.rows(rows), ref2, "32 views: prologue + sparse global stage (sampled rows)")


# ------------------------------------------------------------- 32 views
def test_32views_sparse_selection_and_rows():
    L = zs.CONFIGS["32views"]
    y = 0.8
    log("32 views: drawing inputs")
    q, k, v = _inputs(L, seed=0)
    Q, K, V = widen(q), widen(k), widen(v)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    st = Stage(L, q, k, v, y)
    log("32 views: GPU sparse stage")
    st.sparse()
    sel = st.bufs.sel().cpu().numpy()
    sel_ref, tie_ref = _sel_ref(Q, K, tm, y)
    compare_selection(sel, sel_ref, tie_ref, "32 views: selection (all 16x800 query tiles)",
                      oracle_scores(Q, K, tm, osp))
    # every row of 40 seeded (head, query tile) pairs plus all special rows of 2 heads
    g = np.random.default_rng(0)
    rows = []
    for h, t in zip(g.integers(0, 16, 40), g.integers(0, tm.T, 40)):
        rows += [(int(h), int(tok)) for tok in tm.tokens[t]]
    rows += [(h, int(s)) for h in (0, 9) for s in tm.specials]
    rows = np.array(sorted(set(rows)), dtype=np.int64)
    log(f"32 views: oracle on {len(rows)} rows")
    ref, _ = osp.sparse_rows(Q, K, V, tm, y, rows)
    close(st.rows(rows), ref, "32 views: sparse rows")


def test_32views_dense_and_linear_rows():
    L = zs.CONFIGS["32views"]
    q, k, v = _inputs(L, seed=0)
    Q, K, V = widen(q), widen(k), widen(v)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    rows = zs.sample_rows(L, 512, seed=0, special_frames=2)
    st = Stage(L, q, k, v, 0.0)
    st.dense()
    ref = np.stack([osp.dense_rows(Q[:, h], K[:, h], V[:, h], [t])[0] for h, t in rows])
    close(st.rows(rows), ref, "32 views: dense rows")
    W, b = zs.affine_params(L, seed=0)
    mu = (0.01 * np.random.default_rng(1).standard_normal((L.heads, 64))).astype(np.float32)
    st.linear(W, b, mu)
    ref = olin.linear_rows(Q, K, V, tm, rows, W, b, mu)
    close(st.rows(rows), ref, "32 views: linear rows")


def test_128views_linear_full():
    L = zs.CONFIGS["128views"]
    log("128 views: drawing inputs")
    q, k, v = _inputs(L, seed=0)
    Q, K, V = widen(q), widen(k), widen(v)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    W, b = zs.affine_params(L, seed=0)
    log("128 views: oracle mean output")
    mu = np.stack([olin.mean_output(Q[:, h], K[:, h], V[:, h], tm)
                   for h in range(L.heads)]).astype(np.float32)
    st = Stage(L, q, k, v, 0.0, sparse=False)
    out = bf16_host(st.linear(W, b, mu)).reshape(L.tokens, L.heads, 64)
    log("128 views: oracle linear stage")
    ref = olin.linear_attention(Q, K, V, tm, W, b, mu)
    close(out, ref, "128 views: linear (all 175,872 x 16 rows)")


@pytest.mark.parametrize("y", [0.6, 0.8, 0.95])
def test_32views_special_rows_in_key_segments(y):
    """Special query rows see every key. The main kernel splits each special
    item's keys into about T/k segments (3, 5 and 8 at these y) and adds
    their partial sums afterwards. Every special row of two heads matches the
    oracle's dense rows, and sampled patch rows its sparse rows."""
    L = zs.CONFIGS["32views"]
    q, k, v = _inputs(L, seed=7)
    Q, K, V = widen(q), widen(k), widen(v)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    log(f"32 views: sparse stage y={y}")
    st = Stage(L, q, k, v, y)
    st.sparse()
    heads = (3, 12)
    spec = np.array([(h, int(t)) for h in heads for t in tm.specials], dtype=np.int64)
    ref = np.concatenate([osp.dense_rows(Q[:, h], K[:, h], V[:, h], list(tm.specials)) for h in heads])
    close(st.rows(spec), ref, f"32 views y={y}: special rows ({len(spec)})")
    rows = zs.sample_rows(L, 256, seed=7, special_frames=0)
    ref, _ = osp.sparse_rows(Q, K, V, tm, y, rows)
    close(st.rows(rows), ref, f"32 views y={y}: sparse rows")


def test_exact_fallback_rows():
    """Rows whose cheap logit bound lies far above their own logit are
    recomputed by the exact online-softmax kernel. Scaling the queries of a
    few query tiles and of one frame's special rows by 40 makes their
    |q| r_u term dominate the bound, so those groups are flagged; every
    output, flagged or not, matches the oracle."""
    L = zs.Layout(3, 2, 16, 24, heads=2)
    y = 0.5
    q, k, v = _inputs(L, seed=9)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    Qf = zs.bf16_to_f32(q).copy()
    for t in (0, 7, 13):
        Qf[tm.tokens[t], 1] *= 40.0
    Qf[tm.specials[L.specials:2 * L.specials], 0] *= 40.0
    q = zs.f32_to_bf16(Qf)
    Q, K, V = widen(q), widen(k), widen(v)
    st = Stage(L, q, k, v, y)
    out = bf16_host(st.sparse()).reshape(L.tokens, L.heads, 64)
    # white-box check that the fallback ran: the attention workspace starts
    # with one int flag per (head, query group), groups being the T query
    # tiles then the special groups of 64 rows
    gph = tm.T + (L.frames * L.specials + 63) // 64
    flags = st.bufs.t["WORKSPACE"][: 4 * L.heads * gph].view(torch.int32).view(L.heads, gph).cpu().numpy()
    assert all(flags[1, t] for t in (0, 7, 13)) and flags[0, tm.T], flags
    O_ref, _, _ = osp.sparse_attention(Q, K, V, tm, y)
    close(out, O_ref, "exact-fallback sparse (all rows)")
    st2 = Stage(L, q, k, v, 0.0)
    out = bf16_host(st2.dense()).reshape(L.tokens, L.heads, 64)
    close(out, osp.dense_attention(Q, K, V), "exact-fallback dense (all rows)")


# ------------------------------------------------------------- selector
def test_selection_exact_ties():
    """Equal scores are ranked by lower tile index. Every frame holds the same
    keys, so each of a frame's 9 tile means repeats in all 6 frames and every
    score occurs 6 times; k = 27 splits one such class. Query tiles 5 and 20
    are all-zero, so all 54 of their scores tie and tiles 0..26 are kept.
    Expected lists are built here from the 9 class scores; rows whose class
    scores lie within 1e-9 of each other are skipped."""
    L = zs.Layout(6, 2, 24, 24, heads=2)
    y = 0.5
    q, k, v = _inputs(L, seed=11)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    tok_pf = L.specials + L.rows * L.cols
    Kf = zs.bf16_to_f32(k).copy()
    for f in range(1, L.frames):
        Kf[f * tok_pf:(f + 1) * tok_pf] = Kf[:tok_pf]
    k = zs.f32_to_bf16(Kf)
    zero_tiles = (5, 20)
    Qf = zs.bf16_to_f32(q).copy()
    for t in zero_tiles:
        Qf[tm.tokens[t]] = 0.0
    q = zs.f32_to_bf16(Qf)
    Q, K = widen(q), widen(k)
    kk = keep_count(y, tm.T)
    tpf = tm.T // L.frames
    assert kk % L.frames != 0
    sel = Stage(L, q, k, v, y).select()
    sel_ref, _ = _sel_ref(Q, K, tm, y)
    checked = 0
    for h in range(L.heads):
        kbar, _, _ = osp.landmarks(K[:, h], K[:, h], tm)
        assert all(np.array_equal(kbar[u], kbar[u % tpf]) for u in range(tm.T))
        for t in range(tm.T):
            if t in zero_tiles:
                expect = np.arange(kk)
            else:
                qbar = Q[tm.tokens[t], h].sum(axis=0) / tm.n[t]
                cls = kbar[:tpf] @ qbar
                cs = np.sort(cls)
                if np.min(np.diff(cs)) <= 1e-9 * np.max(np.abs(cs)):
                    continue
                order = sorted(range(tm.T), key=lambda u: (-cls[u % tpf], u))
                expect = np.sort(np.array(order[:kk]))
            assert np.array_equal(sel[h, t], expect), (h, t, sel[h, t], expect)
            assert np.array_equal(sel_ref[h, t], expect), (h, t)
            checked += 1
    log(f"exact ties: {checked} of {L.heads * tm.T} rows checked")
    assert checked >= L.heads * tm.T // 2


def test_selection_gap():
    """The reported gap between the k-th and (k+1)-th ranked scores. Where
    the two round to different fp32 values it comes from those fp32 values,
    each within 2^-24 of its fp64 score, so it is within 2.5e-7 of the fp64
    gap; where they round to the same value both are recomputed in fp64
    (here: all-zero query tiles, whose scores all tie, gap 0)."""
    L = zs.Layout(8, 1, 40, 40, heads=2)
    y = 0.8
    q, k, v = _inputs(L, seed=14)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    Qf = zs.bf16_to_f32(q).copy()
    zero_tiles = (3, 77)
    for t in zero_tiles:
        Qf[tm.tokens[t]] = 0.0
    q = zs.f32_to_bf16(Qf)
    Q, K = widen(q), widen(k)
    st = Stage(L, q, k, v, y)
    st.select()
    gap = st.bufs.gap().cpu().numpy()
    worst = 0.0
    for h in range(L.heads):
        kbar, _, _ = osp.landmarks(K[:, h], K[:, h], tm)
        _, _, gref = osp.select_tiles(Q[:, h], kbar, tm, y)
        assert np.all(gap[h, list(zero_tiles)] == 0.0), gap[h, list(zero_tiles)]
        err = np.abs(gap[h] - gref)
        worst = max(worst, float(err.max()))
        assert err.max() <= 2.5e-7, (h, int(err.argmax()), gap[h, err.argmax()], gref[err.argmax()])
    log(f"gap: max |gpu - oracle| = {worst:.2e} over {L.heads * tm.T} rows")


@pytest.mark.parametrize("frames,heads", [(8, 2), (88, 1)], ids=["T200", "T2200"])
def test_selection_fp32_tie_ranked_in_fp64(frames, heads):
    """Every key token holds the same vector except channel 5, which is 0
    but for the first token of tiles u < 256, set to a distinct small bf16
    value eps_u = (1 + j/128) 2^-(20+e) (u = 128 e + j), and query channel 5
    is 1 on every token. All tile scores then
    round to one fp32 value (on most rows) while the perturbed ones differ in
    fp64 by about 1e-12 relative (far above fp64 rounding) and the others tie
    exactly, so the kept set is decided by the fp64 re-ranking of a tie group
    that straddles the cut, ties cut by tile index; it must equal the
    oracle's exactly on every row (no near-tie allowance). With 2,200 tiles
    the group is ranked in two LDS chunks."""
    L = zs.Layout(frames, 1, 40, 40, heads=heads)
    y = 0.8
    q, k, v = _inputs(L, seed=15)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    Kf = zs.bf16_to_f32(k).copy()
    base = Kf[0].copy()  # [H][64]
    base[:, 5] = 0.0
    Kf[:] = base
    for u in range(min(tm.T, 256)):
        j, e = u % 128, u // 128
        Kf[tm.tokens[u][0], :, 5] = (1.0 + j / 128.0) * 2.0 ** -(20 + e)
    k = zs.f32_to_bf16(Kf)
    assert np.array_equal(zs.bf16_to_f32(k), Kf)  # every value exact in bf16
    # query channel 5 = 1 on every token: the perturbations weigh the same
    # on every row (spacing >= 2^-28 / 512 between perturbed scores)
    Qf = zs.bf16_to_f32(q).copy()
    Qf[:, :, 5] = 1.0
    q = zs.f32_to_bf16(Qf)
    Q, K = widen(q), widen(k)
    sel = Stage(L, q, k, v, y).select()
    sel_ref, _ = _sel_ref(Q, K, tm, y)
    diff = np.any(sel != sel_ref, axis=-1)
    log(f"fp32 tie ranked in fp64: {int(diff.sum())} of {diff.size} rows differ")
    assert not diff.any(), np.argwhere(diff)[:5]


def test_selection_with_outlier_tiles():
    """A few key tiles scaled by 1e4 put their scores far outside the rest,
    so nearly all scores fall into one bin of the first score-uniform
    histogram and the selector must narrow by key bits over several levels.
    Lists match the oracle except on near-tie rows."""
    L = zs.Layout(16, 1, 64, 64, heads=1)
    y = 0.7
    q, k, v = _inputs(L, seed=12)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    Kf = zs.bf16_to_f32(k).copy()
    for u, f in ((100, 1e4), (517, -1e4), (1000, 3e3)):
        Kf[tm.tokens[u]] *= f
    k = zs.f32_to_bf16(Kf)
    Q, K = widen(q), widen(k)
    sel = Stage(L, q, k, v, y).select()
    sel_ref, tie_ref = _sel_ref(Q, K, tm, y)
    r = compare_selection(sel, sel_ref, tie_ref, "outlier tiles selection", oracle_scores(Q, K, tm, osp))
    assert r["near_tie"] < r["rows"] // 10


def test_selection_tie_group_after_narrowing():
    """600 of 1,024 key tiles are all-zero, so every query scores them 0
    exactly, and the cut at k = 307 falls inside that group on most rows. The
    first histogram level puts the whole group into one bin of more than 256
    keys, which narrows to a single score value; the tie is then cut by tile
    index. Expected lists: every tile scoring above 0, then the lowest-index
    zero tiles up to k (rows whose cut is elsewhere, or with a score within
    1e-9 of 0, are skipped)."""
    L = zs.Layout(16, 1, 64, 64, heads=1)
    y = 0.7
    q, k, v = _inputs(L, seed=13)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    zero = np.arange(200, 800)
    Kf = zs.bf16_to_f32(k).copy()
    for u in zero:
        Kf[tm.tokens[u]] = 0.0
    k = zs.f32_to_bf16(Kf)
    Q, K = widen(q), widen(k)
    kk = keep_count(y, tm.T)
    sel = Stage(L, q, k, v, y).select()
    kbar, _, _ = osp.landmarks(K[:, 0], K[:, 0], tm)
    assert not kbar[zero].any()
    checked = 0
    for t in range(tm.T):
        qbar = Q[tm.tokens[t], 0].sum(axis=0) / tm.n[t]
        s = kbar @ qbar
        nz = np.abs(s[s != 0])
        if nz.size and nz.min() <= 1e-9 * nz.max():
            continue
        pos = np.flatnonzero(s > 0)
        if not (len(pos) < kk <= len(pos) + len(zero)):
            continue
        expect = np.sort(np.concatenate([pos, zero[:kk - len(pos)]]))
        assert np.array_equal(sel[0, t], expect), (t, len(pos))
        checked += 1
    log(f"tie group: {checked} of {tm.T} rows checked")
    assert checked >= tm.T // 2


# ------------------------------------------------------------- affine fit
def test_affine_stats_and_fit():
    """zebra_affine_stats against the oracle's statistics (pooled over all
    N x H rows; 3,468 tokens leave a ragged last group), accumulation over
    two calls, and the fit from the GPU statistics against the oracle's fit:
    the corrected outputs agree to the stage tolerance."""
    from gpu_helpers import dev
    from oracle import affine as oaf
    L = zs.Layout(6, 2, 24, 24, heads=2)
    q, k, v = _inputs(L, seed=16)
    o, t = q, k  # any two bf16 tensors of the output layout
    st = Stage(L, q, k, v, 0.0)
    st.out.copy_(dev(o))
    teacher = dev(t)
    stats = torch.zeros(zb.AFFINE_STATS, dtype=torch.float64, device="cuda")
    zb.affine_stats(st.args(), teacher, stats)
    torch.cuda.synchronize()
    got = stats.cpu().numpy()
    O, T = widen(o), widen(t)
    ref = oaf.affine_stats(O, T)
    assert got[0] == ref[0] == L.tokens * L.heads
    err = np.abs(got - ref)
    scale = np.abs(ref).max()
    log(f"affine stats: max |gpu - oracle| = {err.max():.3e} (largest sum {scale:.3e})")
    assert err.max() <= 1e-6 * scale + 1e-6, err.max()
    zb.affine_stats(st.args(), teacher, stats)  # a second scene adds
    torch.cuda.synchronize()
    assert np.allclose(stats.cpu().numpy(), 2 * got, rtol=1e-12, atol=1e-9)
    for lam in (0.0, 1e-3):
        W, b, mu = zb.affine_solve(got, lam)
        Wr, br, mur = oaf.affine_fit(ref, lam)
        Y = oaf.apply_affine(O, W.astype(np.float64), b.astype(np.float64), mu.astype(np.float64))
        Yr = oaf.apply_affine(O, Wr, br, mur)
        close(Y, Yr, f"affine-corrected outputs (lambda_rel {lam})")
