"""Python binding of libzebra, the MI355X (gfx950) global multi-view
attention stage of a Zebra3D-style hybrid model.

Argument marshalling only: every step runs in the HIP kernels behind the C
ABI of include/zebra.h. PyTorch provides device memory and streams. The
library must have been built (python linear_global_attention_amd/build.py);
importing the binding raises if libzebra.so is missing, and every call
raises ZebraError on a non-zero status. There is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

__all__ = [
    "ZebraError", "lib", "Layout", "Args", "StageBuffers", "keep_count", "num_tiles",
    "buffer_bytes", "pack_tiles", "landmarks", "select_tiles", "sparse_attn", "linear_attn",
    "dense_attn", "sparse_stage", "validate", "EXPORTS", "linear_attn_noalloc",
    "BUF", "OP",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzebra.so")

from .abi import (AFFINE_STATS, BUF, EXPORTS, NOALLOC_SCRATCH_BYTES, OP, STATUS, Args,  # noqa: E402,F401
                  CLayout, declare as _declare)

_Layout = CLayout


class ZebraError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python linear_global_attention_amd/build.py`")
    # One HIP runtime per process: the torch wheel bundles its own
    # libamdhip64 (same soname as /opt/rocm's). Loading torch first makes
    # libzebra bind to that copy; loaded the other way round, the process
    # would hold two runtimes and the second one sees no device.
    import torch  # noqa: F401
    return _declare(ctypes.CDLL(LIB_PATH))


lib = _load()


@dataclass(frozen=True)
class Layout:
    frames: int
    specials: int
    rows: int
    cols: int
    heads: int = 16
    head_dim: int = 64

    def c(self) -> _Layout:
        return _Layout(self.frames, self.specials, self.rows, self.cols, self.heads, self.head_dim)

    @property
    def tokens(self) -> int:
        return self.frames * (self.specials + self.rows * self.cols)


def _as_layout(L) -> Layout:
    if isinstance(L, Layout):
        return L
    return Layout(L.frames, L.specials, L.rows, L.cols, L.heads, L.head_dim)


def keep_count(L, y: float) -> int:
    return int(lib.zebra_keep_count(ctypes.byref(_as_layout(L).c()), float(y)))


def num_tiles(L) -> int:
    return int(lib.zebra_num_tiles(ctypes.byref(_as_layout(L).c())))


def buffer_bytes(L, y: float, which: str) -> int:
    return int(lib.zebra_buffer_bytes(ctypes.byref(_as_layout(L).c()), float(y), BUF[which]))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class StageBuffers:
    """Device buffers of one stage shape (torch uint8 tensors sized by
    zebra_buffer_bytes). `gap` is allocated only if asked for."""

    def __init__(self, L, y: float, device="cuda", with_gap: bool = True, sparse: bool = True,
                 backward: bool = False):
        import torch
        self.L, self.y = _as_layout(L), float(y)
        names = ["KT", "VT", "KS", "VS", "WORKSPACE"]
        if sparse:
            names += ["KBAR", "VBAR", "LOGN", "LM", "SEL", "SELMASK"] + (["GAP"] if with_gap else [])
        self.t = {}
        for n in names:
            # backward: a workspace large enough for zebra_sparse_attn_bwd too
            nb = buffer_bytes(self.L, self.y, "BWD_WORKSPACE" if (n == "WORKSPACE" and backward) else n)
            self.t[n] = torch.empty(max(nb, 256), dtype=torch.uint8, device=device)
        self.k = keep_count(self.L, self.y)
        self.T = num_tiles(self.L)

    def view(self, name, dtype, shape):
        import torch  # noqa: F401
        t = self.t[name]
        n = 1
        for s in shape:
            n *= s
        return t[: n * _itemsize(dtype)].view(dtype).view(*shape)

    def sel(self):
        import torch
        return self.view("SEL", torch.int32, (self.L.heads, self.T, self.k))

    def selmask(self):
        import torch
        return self.view("SELMASK", torch.int32, (self.L.heads, self.T, (self.T + 31) // 32))

    def gap(self):
        import torch
        return self.view("GAP", torch.float64, (self.L.heads, self.T)) if "GAP" in self.t else None

    def kbar(self):
        import torch
        return self.view("KBAR", torch.float64, (self.L.heads, self.T, 64))


def _itemsize(dtype) -> int:
    import torch
    return torch.empty((), dtype=dtype).element_size()


def _rows_view(name, t, L: Layout):
    """Checks a bf16 [N][H][64] tensor argument (int16 or bfloat16 storage,
    on the GPU, 64 contiguous channels per row, 16-byte aligned) and returns
    its (token, head) element strides."""
    import torch
    if t.dtype not in (torch.int16, torch.bfloat16):
        raise ValueError(f"{name}: bf16 data expected (int16 or bfloat16 storage), got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: device tensor expected, got {t.device}")
    if tuple(t.shape) != (L.tokens, L.heads, L.head_dim):
        raise ValueError(f"{name}: shape {tuple(t.shape)} is not [N][H][64] = "
                         f"{(L.tokens, L.heads, L.head_dim)}")
    if t.stride(2) != 1:
        raise ValueError(f"{name}: the 64 channels of a row must be contiguous")
    if t.data_ptr() % 16:
        raise ValueError(f"{name}: data must be 16-byte aligned")
    return t.stride(0), t.stride(1)


def _f32(name, t, n):
    import torch
    if t is None:
        return None
    if t.dtype != torch.float32 or t.device.type != "cuda" or not t.is_contiguous() or t.numel() < n:
        raise ValueError(f"{name}: contiguous float32 device tensor of at least {n} elements expected")
    return t


def make_args(L, q=None, k=None, v=None, out=None, bufs: StageBuffers | None = None, y=0.0,
              W=None, b=None, mu=None, gq=None, gk=None, rms_eps=1e-6, rope_base=100.0) -> Args:
    """Fills zebra_args from torch tensors after checking them: q, k, v and
    out bf16 [N][H][64] (views with other token and head strides allowed,
    e.g. slices of a fused QKV projection; q, k and v must share their
    strides), W [H][64][64], b, mu, gq, gk [H][64] float32."""
    Lp = _as_layout(L)
    a = Args()
    a.L = Lp.c()
    strides = [(n, _rows_view(n, t, Lp)) for n, t in (("q", q), ("k", k), ("v", v)) if t is not None]
    if strides:
        if len({st for _, st in strides}) != 1:
            raise ValueError("q, k and v must have the same token and head strides: "
                             + ", ".join(f"{n} {st}" for n, st in strides))
        a.L.tok_stride, a.L.head_stride = strides[0][1]
    if out is not None:
        a.L.out_tok_stride, a.L.out_head_stride = _rows_view("out", out, Lp)
    H = Lp.heads
    W, b, mu = _f32("W", W, H * 64 * 64), _f32("b", b, H * 64), _f32("mu", mu, H * 64)
    gq, gk = _f32("gq", gq, H * 64), _f32("gk", gk, H * 64)
    a.y = float(y)
    a.q, a.k, a.v, a.out = _ptr(q), _ptr(k), _ptr(v), _ptr(out)
    a.W, a.b, a.mu, a.gq, a.gk = _ptr(W), _ptr(b), _ptr(mu), _ptr(gq), _ptr(gk)
    a.rms_eps, a.rope_base = float(rms_eps), float(rope_base)
    # The struct holds bare device addresses: keep the tensors they point
    # into alive for as long as the struct, so that a temporary passed here
    # is not freed (and its memory handed to the next allocation) before
    # the kernels that read it have run.
    a._keep = (q, k, v, out, W, b, mu, gq, gk, bufs)
    if bufs is not None:
        t = bufs.t
        g = lambda n: _ptr(t[n]) if n in t else None  # noqa: E731
        a.kt, a.vt, a.ks, a.vs = g("KT"), g("VT"), g("KS"), g("VS")
        a.kbar, a.vbar, a.logn, a.lm = g("KBAR"), g("VBAR"), g("LOGN"), g("LM")
        a.sel, a.selmask, a.gap = g("SEL"), g("SELMASK"), g("GAP")
        a.workspace = g("WORKSPACE")
        a.workspace_bytes = t["WORKSPACE"].numel() if "WORKSPACE" in t else 0
    return a


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)


def _call(fn, args: Args, stream):
    st = fn(ctypes.byref(args), _stream(stream))
    if st != 0:
        raise ZebraError(st, lib.zebra_last_error().decode())


def validate(args: Args, op: str) -> int:
    return int(lib.zebra_validate(ctypes.byref(args), OP[op]))


def last_error() -> str:
    return lib.zebra_last_error().decode()


def pack_tiles(args: Args, stream=None):
    _call(lib.zebra_pack_tiles, args, stream)


def landmarks(args: Args, stream=None):
    _call(lib.zebra_landmarks, args, stream)


def select_tiles(args: Args, stream=None):
    _call(lib.zebra_select_tiles, args, stream)


def sparse_attn(args: Args, stream=None):
    _call(lib.zebra_sparse_attn, args, stream)


def linear_attn(args: Args, stream=None):
    _call(lib.zebra_linear_attn, args, stream)


def linear_attn_noalloc(args: Args, stream=None):
    """zebra_linear_attn with the library's static device scratch in place
    of args.workspace (for callers that cannot allocate)."""
    _call(lib.zebra_linear_attn_noalloc, args, stream)



def dense_attn(args: Args, stream=None):
    _call(lib.zebra_dense_attn, args, stream)


def affine_stats(args: Args, teacher, stats, stream=None):
    """Adds the affine-fit statistics of o = args.out against `teacher`
    (bf16 [N][H][64], a device tensor with the token and head strides of
    args' q, k, v) into `stats` (fp64 device tensor of AFFINE_STATS
    elements, zeroed by the caller before the first call)."""
    import torch
    Lp = Layout(args.L.frames, args.L.specials, args.L.rows, args.L.cols, args.L.heads, args.L.head_dim)
    ts, hs = _rows_view("teacher", teacher, Lp)
    if (args.L.tok_stride or Lp.heads * 64, args.L.head_stride or 64) != (ts, hs):
        raise ValueError("teacher must have the token and head strides of q, k and v")
    if stats.dtype != torch.float64 or stats.device.type != "cuda" or stats.numel() < AFFINE_STATS:
        raise ValueError(f"stats: float64 device tensor of {AFFINE_STATS} elements expected")
    st = lib.zebra_affine_stats(ctypes.byref(args), _ptr(teacher), _ptr(stats), _stream(stream))
    if st != 0:
        raise ZebraError(st, lib.zebra_last_error().decode())


def frame_attn(args: Args, stream=None):
    """Frame-wise softmax attention of args.q over the keys of each token's
    own frame, into args.out (packs K/V into args' buffers first)."""
    _call(lib.zebra_frame_attn, args, stream)


def qk_prologue(args: Args, q_out, k_out, stream=None):
    """RoPE2D(RMSNorm(.)) of args.q and args.k (gains args.gq, args.gk,
    args.rms_eps, args.rope_base) into q_out and k_out: bf16 device tensors
    with the token and head strides of args' q, k and v (they may be q and k
    themselves)."""
    Lp = Layout(args.L.frames, args.L.specials, args.L.rows, args.L.cols, args.L.heads, args.L.head_dim)
    want = (args.L.tok_stride or Lp.heads * 64, args.L.head_stride or 64)
    for name, t in (("q_out", q_out), ("k_out", k_out)):
        if _rows_view(name, t, Lp) != want:
            raise ValueError(f"{name} must have the token and head strides of q, k and v {want}")
    st = lib.zebra_qk_prologue(ctypes.byref(args), _ptr(q_out), _ptr(k_out), _stream(stream))
    if st != 0:
        raise ZebraError(st, lib.zebra_last_error().decode())


def linear_attn_bwd(args: Args, dout, dq, dk, dv, stream=None):
    """Gradients of sum(dout * out) for the linear stage of args (q, k, v,
    W, gq, gk, rms_eps, rope_base; b and mu do not enter) into dq, dk, dv.
    dout: bf16 device tensor with the strides of args' out; dq, dk, dv: bf16
    device tensors with the strides of args' q, k and v."""
    Lp = Layout(args.L.frames, args.L.specials, args.L.rows, args.L.cols, args.L.heads, args.L.head_dim)
    want_in = (args.L.tok_stride or Lp.heads * 64, args.L.head_stride or 64)
    want_out = (args.L.out_tok_stride or Lp.heads * 64, args.L.out_head_stride or 64)
    if _rows_view("dout", dout, Lp) != want_out:
        raise ValueError(f"dout must have the token and head strides of out {want_out}")
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if _rows_view(name, t, Lp) != want_in:
            raise ValueError(f"{name} must have the token and head strides of q, k and v {want_in}")
    st = lib.zebra_linear_attn_bwd(ctypes.byref(args), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _stream(stream))
    if st != 0:
        raise ZebraError(st, lib.zebra_last_error().decode())


def sparse_attn_bwd(args: Args, dout, dq, dk, dv, stream=None):
    """Gradients of sum(dout * out) for the tile-sparse stage of args (the
    kept tiles and landmarks of args' buffers, from pack_tiles and
    select_tiles on the same inputs) into dq, dk, dv. dout: bf16 device
    tensor with the strides of args' out; dq, dk, dv: bf16 device tensors
    with the strides of args' q, k and v. args' workspace must be sized for
    the backward (StageBuffers(..., backward=True))."""
    Lp = Layout(args.L.frames, args.L.specials, args.L.rows, args.L.cols, args.L.heads, args.L.head_dim)
    want_in = (args.L.tok_stride or Lp.heads * 64, args.L.head_stride or 64)
    want_out = (args.L.out_tok_stride or Lp.heads * 64, args.L.out_head_stride or 64)
    if _rows_view("dout", dout, Lp) != want_out:
        raise ValueError(f"dout must have the token and head strides of out {want_out}")
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if _rows_view(name, t, Lp) != want_in:
            raise ValueError(f"{name} must have the token and head strides of q, k and v {want_in}")
    st = lib.zebra_sparse_attn_bwd(ctypes.byref(args), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _stream(stream))
    if st != 0:
        raise ZebraError(st, lib.zebra_last_error().decode())


def coverage(args: Args, cov, lm_error, stream=None):
    """Attention-mass coverage of the kept tiles and landmark error of the
    omitted ones per (head, query tile), into float32 device tensors
    cov, lm_error of H*T elements. Needs the packed keys, landmarks and the
    kept-tile bitmap of args' stage (pack_tiles and select_tiles first)."""
    import torch
    n = args.L.heads * num_tiles(Layout(args.L.frames, args.L.specials, args.L.rows, args.L.cols, args.L.heads))
    for name, t in (("cov", cov), ("lm_error", lm_error)):
        if t.dtype != torch.float32 or t.device.type != "cuda" or not t.is_contiguous() or t.numel() < n:
            raise ValueError(f"{name}: contiguous float32 device tensor of {n} elements expected")
    st = lib.zebra_coverage(ctypes.byref(args), _ptr(cov), _ptr(lm_error), _stream(stream))
    if st != 0:
        raise ZebraError(st, lib.zebra_last_error().decode())


def affine_solve(stats, lambda_rel: float):
    """fp64 host solve of the centred affine fit from the statistics (a
    host float64 array of AFFINE_STATS elements): returns W [64][64], b [64],
    mu [64] as float32 numpy arrays (one fit for all heads)."""
    import numpy as np
    s = np.ascontiguousarray(stats, dtype=np.float64)
    assert s.shape == (AFFINE_STATS,), s.shape
    W = np.zeros((64, 64), np.float32)
    b = np.zeros(64, np.float32)
    mu = np.zeros(64, np.float32)
    st = lib.zebra_affine_solve(s.ctypes.data, float(lambda_rel), W.ctypes.data, b.ctypes.data, mu.ctypes.data)
    if st != 0:
        raise ZebraError(st, lib.zebra_last_error().decode())
    return W, b, mu


def sparse_stage(args: Args, stream=None):
    """One tile-sparse global stage: pack (with the landmarks in the same
    pass), select, attention."""
    pack_tiles(args, stream)
    select_tiles(args, stream)
    sparse_attn(args, stream)
