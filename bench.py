"""Benchmark of the global multi-view attention stage on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--config 1024views]

Workload (default): 1,024 views of a VGGT-like backbone, 5 special tokens and
37x37 patches per frame, 1,406,976 tokens, 16 heads, d = 64, bf16, seeded
synthetic tile-centroid Q/K/V already resident in HBM. One step is one pass of
the whole hot path over that batch:
  a 0.8S tile-sparse stage  zebra_pack_tiles (landmarks in the same pass),
                            zebra_select_tiles, zebra_sparse_attn
  a linear stage            zebra_linear_attn (centred affine correction)
value = tokens / step time. Each entry point is timed with HIP events on the
stream it runs on (torch's current stream). Also reported: the attention
kernel's roofline (algorithmic flops counted exactly from the kept-tile
lists), the linear stage's HBM roofline, our dense attention on the same
inputs, and the fp64 oracle timed on a bounded sample on the host cores.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "global-attn tokens/s at 1,024 views (0.8S / linear); % MFMA peak & % HBM BW"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=3)
    p.add_argument("--warmup", type=int, default=1)
    p.add_argument("--config", default="1024views")
    p.add_argument("--y", type=float, default=0.8)
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-dense", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-schedule", action="store_true")
    p.add_argument("--no-backward", action="store_true")
    p.add_argument("--no-full-small", action="store_true",
                   help="skip the full oracle runs on the 2-view and 32-view workloads")
    p.add_argument("--dense-reps", type=int, default=5)
    p.add_argument("--rows-per-stage", type=int, default=32)
    p.add_argument("--calib-copy-gb", type=float, default=0.0,
                   help="also run a plain device copy of this many GB (counter calibration)")
    return p.parse_args()


def count_visible(zb, L, bufs, torch):
    """Exact (query row, visible key) pairs of the sparse stage, from the
    kept-tile lists: for a patch row of query tile t, the tokens of its kept
    tiles + the omitted tiles' landmarks + all special keys + its self key
    when t is not kept; special rows see all N keys."""
    from zebra_synth import Layout  # noqa: F401
    T, k, H = bufs.T, bufs.k, L.heads
    tr, tc = -(-L.rows // 8), -(-L.cols // 8)
    n_pf = torch.tensor([min(8, L.rows - 8 * a) * min(8, L.cols - 8 * b)
                         for a in range(tr) for b in range(tc)], dtype=torch.int64, device="cuda")
    n = n_pf.repeat(L.frames)
    nspec = L.frames * L.specials
    sel = bufs.sel()
    mask = bufs.selmask()
    t_idx = torch.arange(T, device="cuda")
    total = 0
    kept_tok_pairs = 0
    for h in range(H):
        kept_tok = n[sel[h].long()].sum(dim=1) if k > 0 else torch.zeros(T, dtype=torch.int64,
                                                                          device="cuda")
        words = mask[h][t_idx, t_idx // 32].long() & 0xFFFFFFFF
        own = (words >> (t_idx % 32)) & 1
        vis = kept_tok + (T - k) + nspec + (1 - own)
        total += int((n * vis).sum())
        kept_tok_pairs += int((n * kept_tok).sum())
    total += H * nspec * L.tokens
    return total, kept_tok_pairs


def _recorded(name: str, key: str):
    """A counter-measured figure from a committed rocprofv3 summary under
    profiles/ (a ```json block holding `key`, the kernel sources it was
    measured on and their SHA-256), or None when the file is missing or the
    sources changed since the counters were taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), flags=re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    h = hashlib.sha256()
    for src in rec["kernel_sources"]:
        h.update(open(os.path.join(ROOT, src), "rb").read())
    return rec[key] if h.hexdigest() == rec["sources_sha256"] else None


def recorded_traffic(config: str, y: float):
    """HBM-side bytes of one zebra_sparse_attn call (FETCH_SIZE and
    WRITE_SIZE, each scaled by a plain device copy) at 1,024 views, y = 0.8."""
    if config != "1024views" or abs(y - 0.8) > 1e-12:
        return None
    return _recorded("attn_traffic_1024views.md", "traffic_bytes_per_call")


def recorded_linear_traffic(config: str):
    """HBM-side bytes of one zebra_linear_attn call at 1,024 views, from the
    same kind of counter summary."""
    if config != "1024views":
        return None
    return _recorded("linear_traffic_1024views.md", "traffic_bytes_per_call")


def recorded_linear_bwd_traffic(config: str):
    """HBM-side bytes of one zebra_linear_attn_bwd call at 1,024 views."""
    if config != "1024views":
        return None
    return _recorded("linear_bwd_1024views.md", "traffic_bytes_per_call")


# ----------------------------------------------------------------- oracle pool
# The oracle runs in worker processes, one BLAS thread each, started from a
# fork server before the GPU is initialised. Large arrays reach the workers
# through shared memory.

def _pool_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass


def start_pool():
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    cores = len(os.sched_getaffinity(0))
    workers = max(1, min(16, cores))
    ctx = mp.get_context("forkserver")
    pool = ProcessPoolExecutor(workers, mp_context=ctx, initializer=_pool_init)
    list(pool.map(abs, range(workers)))  # start every worker now
    return pool, workers


class Shared:
    """Host arrays handed to the pool workers as .npy files in a private
    temporary directory (a full disk raises here, in the caller)."""

    def __init__(self, **arrays):
        import tempfile
        self.dir = tempfile.mkdtemp(prefix="zebra_bench_")
        self.meta = {}
        for name, a in arrays.items():
            path = os.path.join(self.dir, name + ".npy")
            np.save(path, np.ascontiguousarray(a))
            self.meta[name] = path

    def close(self):
        import shutil
        shutil.rmtree(self.dir, ignore_errors=True)


def _attach(meta):
    return {name: np.array(np.load(path, mmap_mode="r")) for name, path in meta.items()}


def _widen(a):
    import zebra_synth as zs
    return zs.bf16_to_f32(a).astype(np.float64)


def _job_landmarks(layout, meta):
    from oracle import sparse as osp
    from oracle.layout import TileMap
    d = _attach(meta)
    tm = TileMap(*layout)
    t0 = time.perf_counter()
    lm = osp.landmarks(_widen(d["k"]), _widen(d["v"]), tm)
    return time.perf_counter() - t0, lm


def _job_sparse_rows(layout, meta, y, toks, lm):
    from oracle import sparse as osp
    from oracle.layout import TileMap
    d = _attach(meta)
    tm = TileMap(*layout)
    t0 = time.perf_counter()
    out, _ = osp.sparse_head(_widen(d["q"]), _widen(d["k"]), _widen(d["v"]), tm, y, toks, lm=lm)
    return time.perf_counter() - t0, out


def _job_linear_state(layout, meta):
    from oracle import linear as olin
    from oracle.layout import TileMap
    d = _attach(meta)
    tm = TileMap(*layout)
    t0 = time.perf_counter()
    S, z = olin.kv_state(olin.featurize(_widen(d["k"]), tm), _widen(d["v"]))
    return time.perf_counter() - t0, (S, z)


def _job_linear_rows(layout, meta, toks, S, z, W=None, b=None, mu=None):
    from oracle import linear as olin
    from oracle.layout import TileMap
    d = _attach(meta)
    tm = TileMap(*layout)
    t0 = time.perf_counter()
    toks = np.asarray(toks, dtype=np.int64)
    pr, pc = olin.positions(tm)
    phiq = olin.feature_map(olin.rope2d(olin.rms_norm(_widen(d["q"])[toks]), pr[toks], pc[toks]))
    out = olin.affine(olin.apply_state(phiq, S, z), W, b, mu)
    return time.perf_counter() - t0, out


def _job_stage_check(layout, meta, kind, y, toks, W=None, b=None, mu=None):
    """The oracle's rows of one head of one schedule stage."""
    if kind == "sparse":
        _, lm = _job_landmarks(layout, meta)
        return _job_sparse_rows(layout, meta, y, toks, lm)[1]
    _, (S, z) = _job_linear_state(layout, meta)
    return _job_linear_rows(layout, meta, toks, S, z, W, b, mu)[1]


def _job_full_head(layout, meta, y):
    """The oracle on every row of one head: the tile-sparse stage at y (patch
    and special rows) and the linear stage (no affine correction)."""
    from oracle import linear as olin
    from oracle import sparse as osp
    from oracle.layout import TileMap
    d = _attach(meta)
    tm = TileMap(*layout)
    Q, K, V = (_widen(d[n])[:, None] for n in ("q", "k", "v"))
    t0 = time.perf_counter()
    out_s, sel, _ = osp.sparse_attention(Q, K, V, tm, y)
    t1 = time.perf_counter()
    out_l = olin.linear_attention(Q, K, V, tm)
    t2 = time.perf_counter()
    return t1 - t0, t2 - t1, out_s[:, 0], sel[0] if sel.ndim == 3 else sel, out_l[:, 0]


def full_small(pool, workers, zb, zs, torch, seed):
    """The fp64 oracle run in full (every row of every head) on the two small
    workloads, 2 views of 16x16 patches (1 head, y = 0.5) and 32 views of
    37x37 patches (16 heads, y = 0.8), one head per worker process, and the
    GPU's outputs of the same stages compared with it on every row (rows of
    query tiles whose kept-tile list differs from the oracle's, near-ties,
    are counted and left out)."""
    res = {}
    for name, y in (("2views_16x16", 0.5), ("32views", 0.8)):
        L = zs.CONFIGS[name]
        N, H = L.tokens, L.heads
        q, k, v = zs.stage_inputs(L, seed=seed)
        zL = zb.Layout(L.frames, L.specials, L.rows, L.cols, H)
        dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to("cuda")  # noqa: E731
        qd, kd, vd = dev(q), dev(k), dev(v)
        out_s, out_l = torch.empty_like(qd), torch.empty_like(qd)
        bufs = zb.StageBuffers(zL, y)
        zb.sparse_stage(zb.make_args(zL, qd, kd, vd, out_s, bufs, y))
        zb.linear_attn(zb.make_args(zL, qd, kd, vd, out_l, bufs, y))
        torch.cuda.synchronize()
        got_s = zs.bf16_to_f32(out_s.cpu().numpy().view(np.uint16)).reshape(N, H, 64).astype(np.float64)
        got_l = zs.bf16_to_f32(out_l.cpu().numpy().view(np.uint16)).reshape(N, H, 64).astype(np.float64)
        sel_gpu = bufs.sel().cpu().numpy()
        layout = (L.frames, L.specials, L.rows, L.cols)
        shs = [Shared(q=q[:, h], k=k[:, h], v=v[:, h]) for h in range(H)]
        try:
            t0 = time.perf_counter()
            futs = [pool.submit(_job_full_head, layout, sh.meta, y) for sh in shs]
            rs = [f.result() for f in futs]
            wall = time.perf_counter() - t0
        finally:
            for sh in shs:
                sh.close()
        from oracle.layout import TileMap
        tm = TileMap(*layout)
        es, el, skipped = [], [], 0
        for h, (_, _, ref_s, sel_ref, ref_l) in enumerate(rs):
            ok_tile = np.array([np.array_equal(sel_gpu[h, t], sel_ref[t]) for t in range(tm.T)])
            rows = np.ones(N, dtype=bool)
            rows[tm.tile_of >= 0] = ok_tile[tm.tile_of[tm.tile_of >= 0]]
            skipped += int((~rows).sum())
            es.append(np.abs(got_s[rows, h] - ref_s[rows]))
            el.append(np.abs(got_l[:, h] - ref_l))
        es, el = np.concatenate(es), np.concatenate(el)
        cpu_s = sum(r[0] + r[1] for r in rs)
        res[name] = {"tokens": N, "heads": H, "y": y, "oracle_wall_s": wall, "processes": workers,
                     "oracle_cpu_s": cpu_s, "oracle_tokens_per_s": N / wall,
                     "sparse_max_abs": float(es.max()), "sparse_mean_abs": float(es.mean()),
                     "sparse_rows_checked": int(es.shape[0]), "sparse_rows_near_tie": skipped,
                     "linear_max_abs": float(el.max()), "linear_mean_abs": float(el.mean())}
        del qd, kd, vd, out_s, out_l, bufs
        torch.cuda.empty_cache()
    return res


def cpu_baseline(pool, workers, L, q, k, v, y, seed):
    """The fp64 oracle on a bounded sample of the same batch (head 0), run
    over `workers` processes of one BLAS thread each and extrapolated to a
    full sparse + linear stage on that many cores."""
    from oracle.layout import TileMap
    R = 1024
    g = np.random.default_rng(seed)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    patch = np.nonzero(tm.tile_of >= 0)[0]
    f = int(g.integers(L.frames))
    spec = tm.specials[f * L.specials:(f + 1) * L.specials]
    toks = np.sort(np.concatenate([g.choice(patch, R - len(spec), replace=False), spec]))
    layout = (L.frames, L.specials, L.rows, L.cols)
    sh = Shared(q=q[:, 0], k=k[:, 0], v=v[:, 0])
    try:
        t0 = time.perf_counter()
        f_lm = pool.submit(_job_landmarks, layout, sh.meta)
        f_st = pool.submit(_job_linear_state, layout, sh.meta)
        t_lm, lm = f_lm.result()
        chunks = np.array_split(toks, workers)
        f_rows = [pool.submit(_job_sparse_rows, layout, sh.meta, y, c, lm) for c in chunks if len(c)]
        t_st, (S, z) = f_st.result()
        f_lin = [pool.submit(_job_linear_rows, layout, sh.meta, c, S, z) for c in chunks if len(c)]
        rows_s = [fu.result() for fu in f_rows]
        rows_l = [fu.result() for fu in f_lin]
        wall = time.perf_counter() - t0
    finally:
        sh.close()
    t_rows = sum(t for t, _ in rows_s)  # CPU seconds over all sampled rows
    t_apply = sum(t for t, _ in rows_l)
    out_s = np.concatenate([o for _, o in rows_s])
    out_l = np.concatenate([o for _, o in rows_l])
    H, N = L.heads, L.tokens
    # one core: every head's landmarks and rows (state and rows for linear);
    # `workers` cores share that work
    sparse_s = H * (t_lm + N * t_rows / len(toks)) / workers
    linear_s = H * (t_st + N * t_apply / len(toks)) / workers
    return dict(
        value=N / (sparse_s + linear_s), unit="tokens/s", cores=int(workers), kind="oracle",
        sample=(f"head 0 of the same batch: landmarks of all {tm.T} tiles + {len(toks)} rows "
                f"({len(spec)} special rows of frame {f}, the rest uniform patch rows) of the tile-sparse "
                f"y={y} stage; KV state over all {N} tokens + the same rows of the linear stage; "
                f"{wall:.1f} s wall on {workers} processes; extrapolated to all {N} tokens x {H} heads "
                f"on the same {workers} cores"),
        sparse_stage_s=sparse_s, linear_stage_s=linear_s, wall_s=wall,
        host_cores=len(os.sched_getaffinity(0)),
        threads_note="one process per core, one BLAS thread per process",
    ), (toks, out_s, out_l)


# ----------------------------------------------------------------- schedule
LINEAR_STAGES = 17
SPARSE_STAGES = 7


def schedule(zb, zs, torch, pool, L, zL, bufs, seed, y, rows_per_stage, log_fn):
    """The pages' 0.7L/0.8S global-attention schedule: 24 stages, stages
    0-16 linear and 17-23 tile-sparse at sparsity y, each on fresh
    tile-centroid inputs drawn on the device from seed + stage. Each stage is
    bracketed by HIP events on the stream it runs on; the draws happen
    between the brackets. After each stage a few (head, token) rows of one
    head are copied out with that head's inputs and checked by the fp64
    oracle in the pool."""
    N, H = L.tokens, L.heads
    layout = (L.frames, L.specials, L.rows, L.cols)
    stage_ms, checks, pending = [], [], []
    max_pending = 8
    out = torch.empty((N, H, 64), dtype=torch.int16, device="cuda")

    def _finish(job):
        st, kind, h, toks, got, sh, fu = job
        try:
            ref = fu.result()
        finally:
            sh.close()
        err = np.abs(_widen(got) - ref)
        return dict(stage=st, kind=kind, head=int(h), rows=int(len(toks)),
                    max_abs=float(err.max()), mean_abs=float(err.mean()))

    tpf = L.tokens_per_frame
    for st in range(LINEAR_STAGES + SPARSE_STAGES):
        linear = st < LINEAR_STAGES
        q, k, v = zs.stage_inputs_device(L, seed=seed, stage=st)
        kw = {}
        if linear:
            W, b = zs.affine_params(L, seed=seed, stage=st)
            mu = zs.calib_mean(L, seed=seed, stage=st)
            kw = dict(W=torch.from_numpy(W).cuda(), b=torch.from_numpy(b).cuda(), mu=torch.from_numpy(mu).cuda())
        args = zb.make_args(zL, q, k, v, out, bufs, y, **kw)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        if linear:
            zb.linear_attn(args)
        else:
            zb.sparse_stage(args)
        e1.record()
        torch.cuda.synchronize()
        stage_ms.append(e0.elapsed_time(e1))
        # sampled rows of head st % H: uniform tokens, plus the special rows
        # of one frame for a sparse stage
        h = st % H
        g = np.random.default_rng([seed, st, 7])
        toks = g.choice(N, rows_per_stage, replace=False)
        if not linear:
            f = int(g.integers(L.frames))
            toks = np.concatenate([toks, f * tpf + np.arange(L.specials)])
        toks = np.unique(toks)
        got = out[torch.from_numpy(toks).cuda(), h].cpu().numpy().view(np.uint16)
        host = lambda t: t[:, h].contiguous().cpu().numpy().view(np.uint16)  # noqa: E731
        while len(pending) >= max_pending:  # bound the files on disk
            checks.append(_finish(pending.pop(0)))
        sh = Shared(q=host(q), k=host(k), v=host(v))
        aff = (W[h].astype(np.float64), b[h].astype(np.float64), mu[h].astype(np.float64)) if linear else ()
        fu = pool.submit(_job_stage_check, layout, sh.meta, "linear" if linear else "sparse", y, toks, *aff)
        pending.append((st, "linear" if linear else "sparse", h, toks, got, sh, fu))
        del q, k, v, args
        log_fn(f"schedule stage {st} ({'linear' if linear else 'sparse'}): {stage_ms[-1]:.3f} ms")
    while pending:
        checks.append(_finish(pending.pop(0)))
    return stage_ms, checks


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU per process here; --gpus must be 1"}))
        sys.exit(2)
    # the oracle's worker processes start before the GPU is initialised
    pool, workers = (None, 0) if (a.no_cpu and a.no_schedule) else start_pool()
    import torch
    import linear_global_attention_amd as zb
    import zebra_synth as zs

    L = zs.CONFIGS[a.config]
    N, H = L.tokens, L.heads
    zL = zb.Layout(L.frames, L.specials, L.rows, L.cols, H)
    log(f"drawing inputs {L} ({N} tokens)")
    t0 = time.time()
    q, k, v = zs.stage_inputs(L, seed=a.seed, stage=0)
    W, b = zs.affine_params(L, seed=a.seed, stage=0)
    log(f"drew inputs in {time.time() - t0:.1f}s")
    dev = lambda x: torch.from_numpy(x.view(np.int16)).to("cuda")  # noqa: E731
    qd, kd, vd = dev(q), dev(k), dev(v)
    out = torch.empty_like(qd)
    out_lin = torch.empty_like(qd)
    bufs = zb.StageBuffers(zL, a.y)
    Wd = torch.from_numpy(W).to("cuda")
    bd = torch.from_numpy(b).to("cuda")
    # calibration mean of the uncorrected linear output (set-up, untimed)
    zb.linear_attn(zb.make_args(zL, qd, kd, vd, out_lin, bufs, a.y))
    mud = out_lin.view(torch.bfloat16).view(N, H, 64).float().mean(dim=0).contiguous()
    args_s = zb.make_args(zL, qd, kd, vd, out, bufs, a.y)
    args_l = zb.make_args(zL, qd, kd, vd, out_lin, bufs, a.y, W=Wd, b=bd, mu=mud)
    torch.cuda.synchronize()

    parts = ["pack_landmarks", "select", "sparse_attn", "linear"]
    fns = [zb.pack_tiles, zb.select_tiles, zb.sparse_attn]

    def step(ev=None):
        for i, fn in enumerate(fns):
            if ev:
                ev[i][0].record()
            fn(args_s)
            if ev:
                ev[i][1].record()
        if ev:
            ev[3][0].record()
        zb.linear_attn(args_l)
        if ev:
            ev[3][1].record()

    for i in range(a.warmup):
        log(f"warmup step {i}")
        step()
    torch.cuda.synchronize()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in parts] for _ in range(a.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for s in range(a.steps):
        step(evs[s])
    stop.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(stop) / a.steps
    per = {p: float(np.mean([evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(a.steps)]))
           for i, p in enumerate(parts)}
    log(f"step {ms_step:.2f} ms; " + ", ".join(f"{p} {t:.3f} ms" for p, t in per.items()))

    # exact algorithmic work of the attention launch
    pairs, kept_pairs = count_visible(zb, L, bufs, torch)
    flops = 4 * 64 * pairs
    att_ms = per["sparse_attn"]
    achieved = flops / (att_ms * 1e-3) / 1e12
    lin_bytes = 4 * N * H * 64 * 2  # read Q, K, V once, write O once
    lin_gbs = lin_bytes / (per["linear"] * 1e-3) / 1e9
    sparse_ms = per["pack_landmarks"] + per["select"] + per["sparse_attn"]
    # pack + landmarks: read K and V once, write the packed keys/values and
    # the landmark buffers once
    pack_bytes = 2 * N * H * 64 * 2 + sum(bufs.t[n].numel() * bufs.t[n].element_size()
                                          for n in ("KT", "VT", "KS", "VS", "KBAR", "VBAR", "LOGN", "LM"))
    pack_gbs = pack_bytes / (per["pack_landmarks"] * 1e-3) / 1e9

    result = {
        "metric": METRIC, "value": N / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": (f"{L.frames}-view global stage pair: one {a.y}S tile-sparse stage "
                                f"+ one linear stage on the same batch"),
                   "frames": L.frames, "specials_per_frame": L.specials,
                   "patch_grid": [L.rows, L.cols], "tokens": N, "heads": H, "head_dim": 64,
                   "y": a.y, "kept_tiles": bufs.k, "tiles": bufs.T, "parallelism": "single GPU"},
        "roofline": {"kernel": "attn_kernel (zebra_sparse_attn)", "bound": "mfma",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": recorded_traffic(a.config, a.y),
                     "traffic_unit": "bytes per zebra_sparse_attn call (L2-to-fabric reads + writes)",
                     "algorithmic_flops": flops, "kept_tile_flops": 4 * 64 * kept_pairs,
                     "kept_tile_frac": 4 * 64 * kept_pairs / (att_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                     "avg_launch_ms": att_ms},
        "roofline_linear": {"kernels": "linear_state + linear_reduce + linear_apply",
                            "bound": "hbm", "achieved": lin_gbs, "peak": PEAK_HBM_GBS,
                            "unit": "GB/s", "frac": lin_gbs / PEAK_HBM_GBS,
                            "algorithmic_bytes": lin_bytes, "avg_launch_ms": per["linear"],
                            "traffic": recorded_linear_traffic(a.config)},
        "roofline_pack": {"kernels": "pack_kernel (zebra_pack_tiles, landmarks fused)", "bound": "hbm",
                          "achieved": pack_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": pack_gbs / PEAK_HBM_GBS, "algorithmic_bytes": pack_bytes,
                          "avg_launch_ms": per["pack_landmarks"]},
        "stage_ms": per,
        "sparse_stage": {"ms": sparse_ms, "tokens_per_s": N / (sparse_ms * 1e-3)},
        "linear_stage": {"ms": per["linear"], "tokens_per_s": N / (per["linear"] * 1e-3)},
        "wall_s_timed_region": t_wall,
    }

    # closed-form affine fit statistics (calibration, outside the step): the
    # uncorrected linear output against the sparse stage's output as teacher,
    # timed over 3 calls after one warm-up call; reads o and t once each
    out_plain = torch.empty_like(qd)
    zb.linear_attn(zb.make_args(zL, qd, kd, vd, out_plain, bufs, a.y))
    stats = torch.zeros(zb.AFFINE_STATS, dtype=torch.float64, device="cuda")
    args_f = zb.make_args(zL, qd, kd, vd, out_plain, bufs, a.y)
    zb.affine_stats(args_f, out, stats)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        zb.affine_stats(args_f, out, stats)
    e1.record()
    torch.cuda.synchronize()
    aff_ms = e0.elapsed_time(e1) / 3
    aff_bytes = 2 * N * H * 64 * 2
    result["roofline_affine_stats"] = {
        "kernels": "affine_stats_kernel + affine_sum_kernel (zebra_affine_stats)", "bound": "hbm",
        "achieved": aff_bytes / (aff_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
        "frac": aff_bytes / (aff_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "algorithmic_bytes": aff_bytes,
        "avg_launch_ms": aff_ms}
    del out_plain, stats

    if not a.no_backward:
        # backward of the linear stage (gradients of q, k, v for a training
        # stage after conversion): a seeded synthetic bf16 output gradient,
        # 3 calls after one warm-up call. Algorithmic bytes: read q, k, v and
        # dout once, write dq, dk, dv once.
        log("linear-stage backward (3 calls)")
        dyd = zs.stage_inputs_device(L, seed=a.seed + 1, stage=0)[0]
        gq_, gk_, gv_ = (torch.empty_like(qd) for _ in range(3))
        args_b = zb.make_args(zL, qd, kd, vd, out_lin, bufs, a.y, W=Wd)
        zb.linear_attn_bwd(args_b, dyd, gq_, gk_, gv_)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            zb.linear_attn_bwd(args_b, dyd, gq_, gk_, gv_)
        e1.record()
        torch.cuda.synchronize()
        bwd_ms = e0.elapsed_time(e1) / 3
        bwd_bytes = 7 * N * H * 64 * 2
        result["roofline_linear_bwd"] = {
            "kernels": ("linear_bwd_state + linear_bwd_query + linear_bwd_key, with two fp64 sums and "
                        "two operand folds (zebra_linear_attn_bwd)"), "bound": "hbm",
            "achieved": bwd_bytes / (bwd_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": bwd_bytes / (bwd_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "algorithmic_bytes": bwd_bytes,
            "avg_launch_ms": bwd_ms, "traffic": recorded_linear_bwd_traffic(a.config)}
        del args_b
        # backward of the tile-sparse stage on the step's kept tiles and
        # landmarks (the stage buffers still hold them), with a workspace
        # sized for it; one call. Algorithmic work: 10 x 64 flops per
        # visible (row, key) pair (the logits, dP, dV, dK and dQ products),
        # 2.5 times the forward's 4 x 64.
        log("tile-sparse backward (1 call)")
        ws = torch.empty(zb.buffer_bytes(zL, a.y, "BWD_WORKSPACE"), dtype=torch.uint8, device="cuda")
        args_sb = zb.make_args(zL, qd, kd, vd, out, bufs, a.y)
        args_sb.workspace = ctypes.c_void_p(ws.data_ptr())
        args_sb.workspace_bytes = ws.numel()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        zb.sparse_attn_bwd(args_sb, dyd, gq_, gk_, gv_)
        e1.record()
        torch.cuda.synchronize()
        sb_ms = e0.elapsed_time(e1)
        sb_flops = 10 * 64 * pairs
        result["roofline_sparse_bwd"] = {
            "kernels": ("sbwd_rows (statistics, dq), sbwd_transpose, sbwd_keys (special keys, landmarks, kept "
                        "tiles), sbwd_reduce (zebra_sparse_attn_bwd)"), "bound": "mfma",
            "achieved": sb_flops / (sb_ms * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": sb_flops / (sb_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "algorithmic_flops": sb_flops,
            "avg_launch_ms": sb_ms, "vs_forward_sparse_attn": sb_ms / att_ms}
        del dyd, gq_, gk_, gv_, args_sb, ws

    dms = None
    if not a.no_dense:
        log(f"dense baseline ({a.dense_reps} calls, median)")
        args_d = zb.make_args(zL, qd, kd, vd, out, bufs, a.y)
        times = []
        for _ in range(a.dense_reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            zb.dense_attn(args_d)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        dms = float(np.median(times))
        dflops = 4 * 64 * N * N * H
        result["dense_stage"] = {"ms": dms, "ms_calls": times, "tflops": dflops / (dms * 1e-3) / 1e12,
                                 "mfma_frac": dflops / (dms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        result["speedup_vs_dense"] = {"sparse_stage": dms / sparse_ms,
                                      "linear_stage": dms / per["linear"]}
        result["context"] = ("the pages report 6.2x / 5.5x / 7.1x END-TO-END model speedups at "
                             "1,024 views on unstated hardware; not comparable to these "
                             "attention-only figures")
        # dense overwrote `out` and the packed buffers; rerun the sparse stage
        # for the sample check
        for fn in fns:
            fn(args_s)
        torch.cuda.synchronize()

    if a.calib_copy_gb > 0:
        nb = int(a.calib_copy_gb * 1e9)
        src = torch.empty(nb, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        result["calib_copy_bytes"] = nb
        del src, dst

    if not a.no_cpu:
        log(f"cpu baseline (oracle on a bounded sample, {workers} processes)")
        cb, (toks, ref_s, ref_l) = cpu_baseline(pool, workers, L, q, k, v, a.y, a.seed)
        result["cpu_baseline"] = cb
        tk = torch.from_numpy(toks).to("cuda")
        got_s = out.view(torch.bfloat16).view(N, H, 64)[tk, 0].double().cpu().numpy()
        zb.linear_attn(zb.make_args(zL, qd, kd, vd, out_lin, bufs, a.y))  # uncorrected
        torch.cuda.synchronize()
        got_l = out_lin.view(torch.bfloat16).view(N, H, 64)[tk, 0].double().cpu().numpy()
        es, el = np.abs(got_s - ref_s), np.abs(got_l - ref_l)
        result["sample_check"] = {"rows": int(len(toks)), "head": 0,
                                  "sparse_max_abs": float(es.max()), "sparse_mean_abs": float(es.mean()),
                                  "linear_max_abs": float(el.max()), "linear_mean_abs": float(el.mean())}

    if not a.no_schedule:
        log("24-stage 0.7L/0.8S schedule on fresh per-stage inputs")
        del qd, kd, vd, out, out_lin, args_s, args_l
        torch.cuda.empty_cache()
        stage_ms, checks = schedule(zb, zs, torch, pool, L, zL, bufs, a.seed, a.y, a.rows_per_stage, log)
        total = float(sum(stage_ms))
        sch = {"stages": len(stage_ms), "linear_stages": LINEAR_STAGES, "sparse_stages": SPARSE_STAGES,
               "y_sparse": a.y, "ms": total, "tokens_per_s": N / (total * 1e-3),
               "linear_ms_mean": float(np.mean(stage_ms[:LINEAR_STAGES])),
               "sparse_ms_mean": float(np.mean(stage_ms[LINEAR_STAGES:])),
               "stage_ms": stage_ms,
               "inputs": ("fresh tile-centroid Q/K/V per stage, drawn on the device from seed + stage "
                          "between the stages' event brackets; affine W, b and a seeded calibration mean "
                          "per linear stage"),
               "check": checks,
               "check_max_abs": max(c["max_abs"] for c in checks),
               "check_mean_abs_max": max(c["mean_abs"] for c in checks)}
        if dms is not None:
            sch["dense_stage_ms"] = dms
            sch["speedup_vs_dense"] = 24 * dms / total
            result["speedup_vs_dense"]["schedule_0.7L/0.8S_24_stages"] = 24 * dms / total
        result["schedule"] = sch
    if not a.no_cpu and not a.no_full_small:
        log(f"oracle in full on the 2-view and 32-view workloads ({workers} processes)")
        result["oracle_full_small"] = full_small(pool, workers, zb, zs, torch, a.seed)
    if pool is not None:
        pool.shutdown()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
