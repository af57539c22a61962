"""Host-only exercise of the sanitized build of libzebra (run by
tests/test_sanitized_host.py in a child process with the AddressSanitizer
runtime preloaded): argument validation of every operation, tile geometry
and buffer sizing over many layouts, the keep count, error paths of every
entry point (all before any GPU call) and the fp64 affine solve. Exits
non-zero on a failed check; the sanitizers abort on any report."""
import ctypes
import importlib.util
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
spec = importlib.util.spec_from_file_location(
    "zebra_abi", os.path.join(ROOT, "linear_global_attention_amd", "abi.py"))
abi = importlib.util.module_from_spec(spec)
spec.loader.exec_module(abi)

so = abi.declare(ctypes.CDLL(sys.argv[1]))


def layout(F, S, R, C, H, d=64, st=(0, 0, 0, 0)):
    return abi.CLayout(F, S, R, C, H, d, *st)


def args(L, y, fill=True):
    a = abi.Args()
    a.L = L
    a.y = y
    if fill:
        for i, f in enumerate(["q", "k", "v", "out", "kt", "vt", "ks", "vs", "kbar", "vbar", "logn",
                               "lm", "sel", "selmask", "workspace"]):
            setattr(a, f, ctypes.c_void_p(0x1000 * (i + 1)))
        a.workspace_bytes = so.zebra_buffer_bytes(ctypes.byref(L), y, abi.BUF["BWD_WORKSPACE"])
    return a


checks = 0


def check(cond, what):
    global checks
    checks += 1
    if not cond:
        print("FAILED:", what, so.zebra_last_error().decode())
        sys.exit(1)


g = np.random.default_rng(0)
# geometry and sizing over many layouts, including edge and invalid ones
for F, S, R, C, H in [(1, 0, 1, 1, 1), (2, 5, 16, 16, 1), (3, 2, 11, 13, 2), (1024, 5, 37, 37, 16),
                      (7, 1, 128, 128, 3), (1, 0, 129, 8, 1), (0, 1, 8, 8, 1), (2, -1, 8, 8, 1),
                      (5, 3, 8, 127, 65535), (1, 0, 8, 8, 65536)]:
    L = layout(F, S, R, C, H)
    T = so.zebra_num_tiles(ctypes.byref(L))
    ok = F >= 1 and S >= 0 and 1 <= R <= 128 and 1 <= C <= 128 and 1 <= H <= 65535
    check((T > 0) == ok, f"num_tiles {F},{S},{R},{C},{H} -> {T}")
    if ok:
        check(T == F * -(-R // 8) * -(-C // 8), "tile count")
        for y in (0.0, 0.2, 0.5, 0.8, 1.0, 0.3333):
            k = so.zebra_keep_count(ctypes.byref(L), y)
            check(k == max(0, min(T, round((1 - y) * T))), f"keep count {y}")
            for w in range(len(abi.BUF)):
                so.zebra_buffer_bytes(ctypes.byref(L), y, w)
        check(so.zebra_keep_count(ctypes.byref(L), 1.5) == -1, "y > 1")
        check(so.zebra_buffer_bytes(ctypes.byref(L), 0.5, 99) == 0, "unknown buffer")
# validation of every operation, good and bad arguments
L = layout(4, 5, 37, 37, 2)
for op in sorted(abi.OP.values()):
    check(so.zebra_validate(ctypes.byref(args(L, 0.5)), op) == 0, f"op {op} accepts")
    check(so.zebra_validate(ctypes.byref(args(L, 0.5, fill=False)), op) == 1, f"op {op} rejects NULLs")
check(so.zebra_validate(ctypes.byref(args(L, 0.5)), 42) == 1, "unknown op")
check(so.zebra_validate(None, 0) == 1, "NULL args")
for st in [(384, 64, 256, 128), (72, 8, 0, 0), (0, 0, 60, 64), (-8, 64, 0, 0), (1 << 41, 64, 0, 0)]:
    a = args(layout(4, 5, 37, 37, 2, st=st), 0.5)
    good = all(s == 0 or (s >= 64 and s % 8 == 0 and s <= 1 << 40) for s in st)
    check((so.zebra_validate(ctypes.byref(a), 4) == 0) == good, f"strides {st}")
a = args(L, 0.5)
a.q = ctypes.c_void_p(0x1004)
check(so.zebra_validate(ctypes.byref(a), 3) == 1, "misaligned q")
a = args(L, 0.5)
a.workspace_bytes = 1
for op in (2, 3, 4, 5, 6, abi.OP["LINEAR_BWD"], abi.OP["SPARSE_BWD"]):
    check(so.zebra_validate(ctypes.byref(a), op) == 3, f"small workspace op {op}")
# every entry point fails on the host before any launch
a = args(L, 0.5, fill=False)
for name in abi.STAGE_CALLS:
    check(getattr(so, name)(ctypes.byref(a), None) == 1, name)
big = args(layout(4096, 5, 37, 37, 16), 0.0)
check(so.zebra_linear_attn_noalloc(ctypes.byref(big), None) == 3, "no-alloc scratch limit")
check(so.zebra_affine_stats(ctypes.byref(args(L, 0.5)), None, None, None) == 1, "affine stats NULLs")
g4 = [ctypes.c_void_p(0x9000 + 0x100 * i) for i in range(4)]
check(so.zebra_linear_attn_bwd(ctypes.byref(args(L, 0.5)), None, g4[1], g4[2], g4[3], None) == 1, "bwd NULL dout")
check(so.zebra_linear_attn_bwd(ctypes.byref(args(L, 0.5)), g4[0], g4[1], ctypes.c_void_p(0x9208), g4[3], None) == 1,
      "bwd misaligned dk")
check(so.zebra_linear_attn_bwd(ctypes.byref(args(L, 0.5, fill=False)), *g4, None) == 1, "bwd NULL q")
check(so.zebra_sparse_attn_bwd(ctypes.byref(args(L, 0.5)), None, g4[1], g4[2], g4[3], None) == 1, "sparse bwd NULL dout")
check(so.zebra_sparse_attn_bwd(ctypes.byref(args(L, 1.5)), *g4, None) == 1, "sparse bwd y > 1")
check(so.zebra_buffer_bytes(ctypes.byref(L), 0.5, abi.BUF["BWD_WORKSPACE"]) >=
      so.zebra_buffer_bytes(ctypes.byref(L), 0.5, abi.BUF["WORKSPACE"]), "backward workspace covers the forward's")
# fp64 affine solve: recovers a planted map from exact statistics
n, d = 5000, 64
o = g.standard_normal((n, d))
Wt = np.eye(d) + 0.1 * g.standard_normal((d, d))
bt = 0.3 * g.standard_normal(d)
t = o @ Wt.T + bt
stats = np.concatenate([[n], o.sum(0), t.sum(0), (o.T @ o).ravel(), (o.T @ t).ravel()])
W = np.zeros((d, d), np.float32)
b = np.zeros(d, np.float32)
mu = np.zeros(d, np.float32)
rc = so.zebra_affine_solve(stats.ctypes.data, 0.0, W.ctypes.data, b.ctypes.data, mu.ctypes.data)
check(rc == 0, "affine solve")
check(np.abs(W - Wt).max() < 1e-4, "solved W")
check(np.abs((mu + b) - (Wt @ o.mean(0) + bt)).max() < 1e-4, "solved intercept")
bad = stats.copy()
bad[0] = 0
check(so.zebra_affine_solve(bad.ctypes.data, 0.0, W.ctypes.data, b.ctypes.data, mu.ctypes.data) == 1, "n = 0")
check(so.zebra_affine_solve(stats.ctypes.data, -1.0, W.ctypes.data, b.ctypes.data, mu.ctypes.data) == 1,
      "negative ridge")
check(so.zebra_affine_solve(None, 0.0, None, None, None) == 1, "NULL solve")
check(b"gfx950" in so.zebra_version(), "version")
print(f"sanitized host checks passed: {checks}")
