"""The C ABI library loads without a GPU, exports every symbol declared in
include/zebra.h, sizes its buffers and rejects bad arguments on the host
(zebra_validate makes no GPU call)."""
import ctypes
import os
import re

import pytest

import linear_global_attention_amd as zb
from oracle.layout import TileMap, keep_count as oracle_keep

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zebra.h")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*[\w\s\*]*?\b(zebra_\w+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 12
    so = ctypes.CDLL(zb.LIB_PATH)
    for n in names:
        assert hasattr(so, n), n
    assert set(zb.EXPORTS) == set(names)
    assert b"gfx950" in zb.lib.zebra_version()


@pytest.mark.parametrize("cfg,y", [((2, 5, 16, 16, 1), 0.5), ((32, 5, 37, 37, 16), 0.8),
                                   ((512, 5, 37, 37, 16), 0.6), ((1024, 5, 37, 37, 16), 0.8),
                                   ((3, 0, 11, 13, 2), 0.3)])
def test_counts_match_the_oracle_tile_map(cfg, y):
    F, S, R, C, H = cfg
    L = zb.Layout(F, S, R, C, H)
    assert zb.num_tiles(L) == F * -(-R // 8) * -(-C // 8)
    assert zb.keep_count(L, y) == oracle_keep(y, zb.num_tiles(L))
    if F <= 32:
        tm = TileMap(F, S, R, C)
        assert zb.num_tiles(L) == tm.T
        # packed slots: every tile padded to a multiple of 32
        slots = sum(-(-int(n) // 32) * 32 for n in tm.n)
        assert zb.buffer_bytes(L, y, "KT") == H * slots * 64 * 2
    T = zb.num_tiles(L)
    k = zb.keep_count(L, y)
    assert zb.buffer_bytes(L, y, "SEL") == H * T * max(k, 1) * 4
    assert zb.buffer_bytes(L, y, "SELMASK") == H * T * ((T + 31) // 32) * 4
    assert zb.buffer_bytes(L, y, "KBAR") == H * T * 64 * 8
    assert zb.buffer_bytes(L, y, "WORKSPACE") > 0


def test_keep_count_edge_cases():
    L = zb.Layout(32, 5, 37, 37)
    assert zb.keep_count(L, 0.8) == 160  # round, not floor
    assert zb.keep_count(L, 0.0) == 800 and zb.keep_count(L, 1.0) == 0
    assert zb.keep_count(L, -0.1) == -1 and zb.keep_count(L, 1.5) == -1
    assert zb.keep_count(L, float("nan")) == -1


def _fake(n=1):
    return ctypes.c_void_p(0x1000 * n)


def _full_args(L, y):
    a = zb.Args()
    a.L = L.c()
    a.y = y
    for i, f in enumerate(["q", "k", "v", "out", "kt", "vt", "ks", "vs", "kbar", "vbar", "logn",
                           "lm", "sel", "selmask", "workspace"]):
        setattr(a, f, _fake(i + 1))
    a.workspace_bytes = zb.buffer_bytes(L, y, "BWD_WORKSPACE")
    return a


def test_validate_accepts_and_rejects_on_host():
    L = zb.Layout(4, 5, 37, 37, 2)
    for op in zb.OP:
        assert zb.validate(_full_args(L, 0.5), op) == 0, op
    a = _full_args(L, 0.5)
    a.q = None
    assert zb.validate(a, "SPARSE") == 1 and "q" in zb.last_error()
    assert zb.validate(a, "PACK") == 0  # pack does not read q
    a = _full_args(L, 1.5)
    assert zb.validate(a, "SELECT") == 1
    a = _full_args(L, 0.5)
    a.workspace_bytes = 16
    assert zb.validate(a, "SELECT") == 3 and zb.validate(a, "LINEAR") == 3
    a = _full_args(zb.Layout(4, 5, 37, 37, 2, head_dim=128), 0.5)
    assert zb.validate(a, "LINEAR") == 2
    a = _full_args(zb.Layout(4, 5, 200, 37, 2), 0.5)
    assert zb.validate(a, "PACK") == 2
    a = _full_args(zb.Layout(0, 5, 37, 37, 2), 0.5)
    assert zb.validate(a, "PACK") == 1
    assert zb.lib.zebra_validate(None, 0) == 1
    assert zb.validate(_full_args(L, 0.5), "PACK") == 0 and zb.last_error() == ""


def test_entry_points_fail_before_any_launch():
    # invalid arguments return an error status without touching the GPU
    L = zb.Layout(4, 5, 37, 37, 2)
    a = _full_args(L, 0.5)
    a.kt = None
    for fn in (zb.lib.zebra_pack_tiles, zb.lib.zebra_landmarks, zb.lib.zebra_sparse_attn,
               zb.lib.zebra_dense_attn):
        assert fn(ctypes.byref(a), None) == 1
    with pytest.raises(zb.ZebraError, match="INVALID_ARG"):
        zb.pack_tiles(a, stream=0)


def test_affine_entry_points_reject_on_host():
    """zebra_affine_stats checks its arguments before any launch; the host
    solve needs no GPU at all."""
    L = zb.Layout(4, 5, 37, 37, 2)
    a = _full_args(L, 0.5)
    buf = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    f = zb.lib.zebra_affine_stats
    assert f(ctypes.byref(a), None, buf, None) == 1 and "teacher" in zb.last_error()
    assert f(ctypes.byref(a), buf, None, None) == 1 and "stats" in zb.last_error()
    a.out = None
    assert f(ctypes.byref(a), buf, buf, None) == 1 and "out" in zb.last_error()
    a = _full_args(L, 0.5)
    a.workspace_bytes = 16
    assert f(ctypes.byref(a), buf, buf, None) == 3
    assert zb.lib.zebra_affine_solve(None, 0.0, None, None, None) == 1


def test_noalloc_linear_rejects_on_host():
    """zebra_linear_attn_noalloc checks its pointers and that the layout's
    scratch fits the library's static array before any GPU call."""
    f = zb.lib.zebra_linear_attn_noalloc
    big = zb.Layout(2048, 5, 37, 37, 16)  # about 100 MB of partial states
    a = _full_args(big, 0.0)
    assert f(ctypes.byref(a), None) == 3 and "scratch" in zb.last_error()
    a = _full_args(zb.Layout(4, 5, 37, 37, 2), 0.0)
    a.k = None
    assert f(ctypes.byref(a), None) == 1 and "k" in zb.last_error()
    a = _full_args(zb.Layout(4, 5, 37, 37, 2, head_dim=32), 0.0)
    assert f(ctypes.byref(a), None) == 2
    assert zb.NOALLOC_SCRATCH_BYTES == 64 << 20


def test_strides_and_alignment_checked_on_host():
    """Token/head strides of q, k, v and out: 0 (contiguous) or positive
    multiples of 8 elements, at least 64; tensor pointers 16-byte aligned."""
    L = zb.Layout(4, 5, 37, 37, 2)
    a = _full_args(L, 0.5)
    a.L.tok_stride, a.L.head_stride = 3 * 2 * 64, 64  # a fused QKV projection
    a.L.out_tok_stride, a.L.out_head_stride = 2 * 128, 128
    for op in zb.OP:
        assert zb.validate(a, op) == 0, op
    for field, bad in (("tok_stride", 60), ("head_stride", 12), ("out_tok_stride", 100), ("out_head_stride", -64)):
        b = _full_args(L, 0.5)
        setattr(b.L, field, bad)
        assert zb.validate(b, "LINEAR") == 1 and "stride" in zb.last_error(), field
    b = _full_args(L, 0.5)
    b.q = ctypes.c_void_p(0x1008)
    assert zb.validate(b, "SPARSE") == 1 and "aligned" in zb.last_error()
    # buffer sizes do not depend on the strides
    Ls = zb.CLayout(4, 5, 37, 37, 2, 64, 384, 64, 256, 128) if hasattr(zb, "CLayout") else None
    if Ls is not None:
        assert zb.lib.zebra_buffer_bytes(ctypes.byref(Ls), 0.5, zb.BUF["KT"]) == zb.buffer_bytes(L, 0.5, "KT")


def test_sparse_bwd_rejects_wide_row_spans():
    """The tile-sparse backward addresses a key tile's rows by 32-bit element
    offsets from its first row, so it rejects layouts whose 8 patch rows of
    q/k/v (or of dout, which has out's strides) span 2^31 or more elements;
    the forward entry points accept them (their validation does not touch
    memory)."""
    L = zb.Layout(4, 5, 37, 37, 2)
    a = _full_args(L, 0.5)
    assert zb.validate(a, "SPARSE_BWD") == 0
    for field in ("tok_stride", "out_tok_stride"):
        b = _full_args(L, 0.5)
        setattr(b.L, field, 1 << 23)  # 8 rows x 37 columns x 2^23 > 2^31
        assert zb.validate(b, "SPARSE_BWD") == 2 and "2^31" in zb.last_error(), field
        assert zb.validate(b, "SPARSE") == 0, field
    b = _full_args(L, 0.5)
    b.L.tok_stride = (1 << 31) // (8 * 37) // 8 * 8  # just below the bound
    assert zb.validate(b, "SPARSE_BWD") == 0


def test_make_args_rejects_wrong_tensors():
    import torch
    L = zb.Layout(2, 1, 3, 5, 1)
    x = torch.zeros((L.tokens, 1, 64), dtype=torch.float32)
    with pytest.raises(ValueError, match="bf16"):
        zb.make_args(L, q=x)
    with pytest.raises(ValueError, match="device"):
        zb.make_args(L, q=x.to(torch.int16))
    with pytest.raises(ValueError, match="float32"):
        zb.make_args(L, W=torch.zeros(64 * 64, dtype=torch.float64))
