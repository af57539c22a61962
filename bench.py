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


def recorded_traffic(config: str, y: float):
    """HBM-side bytes of one zebra_sparse_attn call, from the committed
    rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE, each scaled by a
    plain device copy), or None when that summary is for another workload or
    the kernel sources changed since the counters were taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", "attn_traffic_1024views.md")
    if config != "1024views" or abs(y - 0.8) > 1e-12 or not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), flags=re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    h = hashlib.sha256()
    for src in rec["kernel_sources"]:
        h.update(open(os.path.join(ROOT, src), "rb").read())
    return rec["traffic_bytes_per_call"] if h.hexdigest() == rec["sources_sha256"] else None


def cpu_baseline(L, q, k, v, y, seed):
    """The fp64 oracle on a bounded sample of the same batch (head 0), timed
    on the host and extrapolated to a full sparse + linear stage."""
    from oracle import linear as olin
    from oracle import sparse as osp
    from oracle.layout import TileMap
    import zebra_synth as zs
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    R = 640
    g = np.random.default_rng(seed)
    tm = TileMap(L.frames, L.specials, L.rows, L.cols)
    patch = np.nonzero(tm.tile_of >= 0)[0]
    toks = np.sort(g.choice(patch, R, replace=False))
    Qh = zs.bf16_to_f32(q[:, 0]).astype(np.float64)
    Kh = zs.bf16_to_f32(k[:, 0]).astype(np.float64)
    Vh = zs.bf16_to_f32(v[:, 0]).astype(np.float64)
    t0 = time.perf_counter()
    lm = osp.landmarks(Kh, Vh, tm)
    t_lm = time.perf_counter() - t0
    t0 = time.perf_counter()
    out_s, _ = osp.sparse_head(Qh, Kh, Vh, tm, y, toks, lm=lm)
    t_rows = time.perf_counter() - t0
    t0 = time.perf_counter()
    phik = olin.featurize(Kh, tm)
    S, z = olin.kv_state(phik, Vh)
    t_state = time.perf_counter() - t0
    t0 = time.perf_counter()
    pr, pc = olin.positions(tm)
    phiq = olin.feature_map(olin.rope2d(olin.rms_norm(Qh[toks]), pr[toks], pc[toks]))
    out_l = olin.apply_state(phiq, S, z)
    t_apply = time.perf_counter() - t0
    H, N = L.heads, L.tokens
    sparse_s = H * (t_lm + N * t_rows / R)
    linear_s = H * (t_state + N * t_apply / R)
    wall = t_lm + t_rows + t_state + t_apply
    return dict(
        value=N / (sparse_s + linear_s), unit="tokens/s", cores=int(blas), kind="oracle",
        sample=(f"head 0 of the same batch: landmarks of all {tm.T} tiles + {R} sampled patch rows "
                f"(tile-sparse y={y}); KV state over all {N} tokens + the same {R} rows (linear); "
                f"{wall:.1f} s of CPU, extrapolated to all {N} tokens x {H} heads"),
        sparse_stage_s=sparse_s, linear_stage_s=linear_s, wall_s=wall,
        threads_note="numpy element-wise work runs on one thread; BLAS calls use `cores` threads",
    ), (toks, out_s, out_l)


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU per process here; --gpus must be 1"}))
        sys.exit(2)
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
                            "algorithmic_bytes": lin_bytes, "avg_launch_ms": per["linear"]},
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

    if not a.no_dense:
        log("dense baseline (one call)")
        args_d = zb.make_args(zL, qd, kd, vd, out, bufs, a.y)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        zb.dense_attn(args_d)
        e1.record()
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1)
        dflops = 4 * 64 * N * N * H
        result["dense_stage"] = {"ms": dms, "tflops": dflops / (dms * 1e-3) / 1e12,
                                 "mfma_frac": dflops / (dms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        result["speedup_vs_dense"] = {"sparse_stage": dms / sparse_ms,
                                      "linear_stage": dms / per["linear"],
                                      "schedule_0.7L/0.8S_24_stages":
                                          24 * dms / (7 * sparse_ms + 17 * per["linear"])}
        result["context"] = ("the pages report 6.2x / 5.5x / 7.1x END-TO-END model speedups at "
                             "1,024 views on unstated hardware; not comparable to this "
                             "attention-only figure")
        # dense overwrote `out`; rerun the sparse stage for the sample check
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

    if not a.no_cpu:
        log("cpu baseline (oracle on a bounded sample)")
        cb, (toks, ref_s, ref_l) = cpu_baseline(L, q, k, v, a.y, a.seed)
        result["cpu_baseline"] = cb
        tk = torch.from_numpy(toks).to("cuda")
        got_s = out.view(torch.bfloat16).view(N, H, 64)[tk, 0].double().cpu().numpy()
        zb.linear_attn(zb.make_args(zL, qd, kd, vd, out_lin, bufs, a.y))  # uncorrected
        torch.cuda.synchronize()
        got_l = out_lin.view(torch.bfloat16).view(N, H, 64)[tk, 0].double().cpu().numpy()
        result["sample_check"] = {"rows": int(len(toks)),
                                  "sparse_max_abs": float(np.abs(got_s - ref_s).max()),
                                  "linear_max_abs": float(np.abs(got_l - ref_l).max())}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
