"""Python binding of libzebra, the MI355X (gfx950) global multi-view
attention stage of a Zebra3D-style hybrid model.

Argument marshalling only: every step runs in the HIP kernels behind the C
ABI of include/zebra.h. PyTorch provides device memory and streams. The
library must have been built (python -m linear_global_attention_amd.build);
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
    "dense_attn", "sparse_stage", "validate", "EXPORTS",
    "BUF", "OP",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzebra.so")

BUF = dict(KT=0, VT=1, KS=2, VS=3, KBAR=4, VBAR=5, LOGN=6, LM=7, SEL=8, SELMASK=9, GAP=10,
           WORKSPACE=11)
OP = dict(PACK=0, LANDMARKS=1, SELECT=2, SPARSE=3, LINEAR=4, DENSE=5, AFFINE_STATS=6)
AFFINE_STATS = 1 + 2 * 64 + 2 * 64 * 64  # doubles of the affine-fit statistics
STATUS = {0: "ZEBRA_OK", 1: "ZEBRA_ERR_INVALID_ARG", 2: "ZEBRA_ERR_UNSUPPORTED",
          3: "ZEBRA_ERR_WORKSPACE", 4: "ZEBRA_ERR_HIP"}
EXPORTS = ["zebra_pack_tiles", "zebra_landmarks", "zebra_select_tiles", "zebra_sparse_attn",
           "zebra_linear_attn", "zebra_dense_attn", "zebra_validate", "zebra_buffer_bytes",
           "zebra_keep_count", "zebra_num_tiles", "zebra_last_error", "zebra_version",
           "zebra_affine_stats", "zebra_affine_solve"]


class ZebraError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class _Layout(ctypes.Structure):
    _fields_ = [("frames", ctypes.c_int32), ("specials", ctypes.c_int32),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


_vp = ctypes.c_void_p


class Args(ctypes.Structure):
    """Mirror of zebra_args."""
    _fields_ = [("L", _Layout), ("y", ctypes.c_double),
                ("q", _vp), ("k", _vp), ("v", _vp), ("out", _vp),
                ("W", _vp), ("b", _vp), ("mu", _vp), ("gq", _vp), ("gk", _vp),
                ("rms_eps", ctypes.c_float), ("rope_base", ctypes.c_float),
                ("kt", _vp), ("vt", _vp), ("ks", _vp), ("vs", _vp),
                ("kbar", _vp), ("vbar", _vp), ("logn", _vp), ("lm", _vp),
                ("sel", _vp), ("selmask", _vp), ("gap", _vp),
                ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m linear_global_attention_amd.build`")
    # One HIP runtime per process: the torch wheel bundles its own
    # libamdhip64 (same soname as /opt/rocm's). Loading torch first makes
    # libzebra bind to that copy; loaded the other way round, the process
    # would hold two runtimes and the second one sees no device.
    import torch  # noqa: F401
    so = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    for name in ("zebra_pack_tiles", "zebra_landmarks", "zebra_select_tiles",
                 "zebra_sparse_attn", "zebra_linear_attn", "zebra_dense_attn"):
        f = getattr(so, name)
        f.argtypes = [P(Args), _vp]
        f.restype = ctypes.c_int
    so.zebra_validate.argtypes = [P(Args), ctypes.c_int]
    so.zebra_validate.restype = ctypes.c_int
    so.zebra_buffer_bytes.argtypes = [P(_Layout), ctypes.c_double, ctypes.c_int]
    so.zebra_buffer_bytes.restype = ctypes.c_size_t
    so.zebra_keep_count.argtypes = [P(_Layout), ctypes.c_double]
    so.zebra_keep_count.restype = ctypes.c_int64
    so.zebra_num_tiles.argtypes = [P(_Layout)]
    so.zebra_num_tiles.restype = ctypes.c_int64
    so.zebra_last_error.argtypes = []
    so.zebra_last_error.restype = ctypes.c_char_p
    so.zebra_version.argtypes = []
    so.zebra_version.restype = ctypes.c_char_p
    so.zebra_affine_stats.argtypes = [P(Args), _vp, _vp, _vp]
    so.zebra_affine_stats.restype = ctypes.c_int
    so.zebra_affine_solve.argtypes = [_vp, ctypes.c_double, _vp, _vp, _vp]
    so.zebra_affine_solve.restype = ctypes.c_int
    return so


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

    def __init__(self, L, y: float, device="cuda", with_gap: bool = True, sparse: bool = True):
        import torch
        self.L, self.y = _as_layout(L), float(y)
        names = ["KT", "VT", "KS", "VS", "WORKSPACE"]
        if sparse:
            names += ["KBAR", "VBAR", "LOGN", "LM", "SEL", "SELMASK"] + (["GAP"] if with_gap else [])
        self.t = {}
        for n in names:
            nb = buffer_bytes(self.L, self.y, n)
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


def make_args(L, q=None, k=None, v=None, out=None, bufs: StageBuffers | None = None, y=0.0,
              W=None, b=None, mu=None, gq=None, gk=None, rms_eps=1e-6, rope_base=100.0) -> Args:
    a = Args()
    a.L = _as_layout(L).c()
    a.y = float(y)
    a.q, a.k, a.v, a.out = _ptr(q), _ptr(k), _ptr(v), _ptr(out)
    a.W, a.b, a.mu, a.gq, a.gk = _ptr(W), _ptr(b), _ptr(mu), _ptr(gq), _ptr(gk)
    a.rms_eps, a.rope_base = float(rms_eps), float(rope_base)
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


def dense_attn(args: Args, stream=None):
    _call(lib.zebra_dense_attn, args, stream)


def affine_stats(args: Args, teacher, stats, stream=None):
    """Adds the affine-fit statistics of o = args.out against `teacher`
    (bf16 [N][H][64], a device tensor) into `stats` (fp64 device tensor of
    AFFINE_STATS elements, zeroed by the caller before the first call)."""
    st = lib.zebra_affine_stats(ctypes.byref(args), _ptr(teacher), _ptr(stats), _stream(stream))
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
