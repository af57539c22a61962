"""The C ABI of libzebra (include/zebra.h) as ctypes declarations: the
argument structs, status and buffer codes, and the argument and result
types of every export. Pure ctypes: importing it loads no library and no
torch, so a host-only check can declare the exports of any build of the
library (python -c 'import importlib.util ...' by path, or through the
package binding)."""
from __future__ import annotations

import ctypes

BUF = dict(KT=0, VT=1, KS=2, VS=3, KBAR=4, VBAR=5, LOGN=6, LM=7, SEL=8, SELMASK=9, GAP=10,
           WORKSPACE=11, BWD_WORKSPACE=12)
OP = dict(PACK=0, LANDMARKS=1, SELECT=2, SPARSE=3, LINEAR=4, DENSE=5, AFFINE_STATS=6, COVERAGE=7, PROLOGUE=8, FRAME=9,
          LINEAR_BWD=10, SPARSE_BWD=11)
AFFINE_STATS = 1 + 2 * 64 + 2 * 64 * 64  # doubles of the affine-fit statistics
NOALLOC_SCRATCH_BYTES = 64 << 20
STATUS = {0: "ZEBRA_OK", 1: "ZEBRA_ERR_INVALID_ARG", 2: "ZEBRA_ERR_UNSUPPORTED",
          3: "ZEBRA_ERR_WORKSPACE", 4: "ZEBRA_ERR_HIP"}
EXPORTS = ["zebra_pack_tiles", "zebra_landmarks", "zebra_select_tiles", "zebra_sparse_attn",
           "zebra_linear_attn", "zebra_dense_attn", "zebra_validate", "zebra_buffer_bytes",
           "zebra_keep_count", "zebra_num_tiles", "zebra_last_error", "zebra_version",
           "zebra_affine_stats", "zebra_affine_solve", "zebra_linear_attn_noalloc", "zebra_coverage",
           "zebra_qk_prologue", "zebra_frame_attn", "zebra_linear_attn_bwd",
           "zebra_sparse_attn_bwd"]
STAGE_CALLS = ("zebra_pack_tiles", "zebra_landmarks", "zebra_select_tiles", "zebra_sparse_attn",
               "zebra_linear_attn", "zebra_dense_attn", "zebra_linear_attn_noalloc",
               "zebra_frame_attn")


class CLayout(ctypes.Structure):
    _fields_ = [("frames", ctypes.c_int32), ("specials", ctypes.c_int32),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("tok_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64),
                ("out_tok_stride", ctypes.c_int64), ("out_head_stride", ctypes.c_int64)]


_vp = ctypes.c_void_p


class Args(ctypes.Structure):
    """Mirror of zebra_args."""
    _fields_ = [("L", CLayout), ("y", ctypes.c_double),
                ("q", _vp), ("k", _vp), ("v", _vp), ("out", _vp),
                ("W", _vp), ("b", _vp), ("mu", _vp), ("gq", _vp), ("gk", _vp),
                ("rms_eps", ctypes.c_float), ("rope_base", ctypes.c_float),
                ("kt", _vp), ("vt", _vp), ("ks", _vp), ("vs", _vp),
                ("kbar", _vp), ("vbar", _vp), ("logn", _vp), ("lm", _vp),
                ("sel", _vp), ("selmask", _vp), ("gap", _vp),
                ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t)]


def declare(so: ctypes.CDLL) -> ctypes.CDLL:
    """Sets the argument and result types of every export of `so`."""
    P = ctypes.POINTER
    for name in STAGE_CALLS:
        f = getattr(so, name)
        f.argtypes = [P(Args), _vp]
        f.restype = ctypes.c_int
    so.zebra_validate.argtypes = [P(Args), ctypes.c_int]
    so.zebra_validate.restype = ctypes.c_int
    so.zebra_buffer_bytes.argtypes = [P(CLayout), ctypes.c_double, ctypes.c_int]
    so.zebra_buffer_bytes.restype = ctypes.c_size_t
    so.zebra_keep_count.argtypes = [P(CLayout), ctypes.c_double]
    so.zebra_keep_count.restype = ctypes.c_int64
    so.zebra_num_tiles.argtypes = [P(CLayout)]
    so.zebra_num_tiles.restype = ctypes.c_int64
    so.zebra_last_error.argtypes = []
    so.zebra_last_error.restype = ctypes.c_char_p
    so.zebra_version.argtypes = []
    so.zebra_version.restype = ctypes.c_char_p
    so.zebra_affine_stats.argtypes = [P(Args), _vp, _vp, _vp]
    so.zebra_affine_stats.restype = ctypes.c_int
    so.zebra_qk_prologue.argtypes = [P(Args), _vp, _vp, _vp]
    so.zebra_qk_prologue.restype = ctypes.c_int
    so.zebra_linear_attn_bwd.argtypes = [P(Args), _vp, _vp, _vp, _vp, _vp]
    so.zebra_linear_attn_bwd.restype = ctypes.c_int
    so.zebra_sparse_attn_bwd.argtypes = [P(Args), _vp, _vp, _vp, _vp, _vp]
    so.zebra_sparse_attn_bwd.restype = ctypes.c_int
    so.zebra_coverage.argtypes = [P(Args), _vp, _vp, _vp]
    so.zebra_coverage.restype = ctypes.c_int
    so.zebra_affine_solve.argtypes = [_vp, ctypes.c_double, _vp, _vp, _vp]
    so.zebra_affine_solve.restype = ctypes.c_int
    return so
