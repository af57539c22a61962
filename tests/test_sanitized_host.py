"""The library's host code (argument validation, tile geometry, buffer
sizing, the fp64 affine solve) built with AddressSanitizer and
UndefinedBehaviorSanitizer and exercised on the CPU in a child process
(tests/sanitized_host_check.py) with the sanitizer runtime preloaded. Any
sanitizer report aborts the child."""
import glob
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location("_zebra_build", os.path.join(ROOT, "linear_global_attention_amd",
                                                                                 "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    return b


def _runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_host_code_under_asan_and_ubsan():
    rt = _runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in this ROCm installation")
    b = _build_module()
    lib = b.SAN_LIB
    srcs = [os.path.join(b.CSRC, f) for f in b.SOURCES]
    if not os.path.exists(lib) or os.path.getmtime(lib) < max(os.path.getmtime(s) for s in srcs):
        b.build_sanitized()
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitized_host_check.py"), lib],
                       env=env, capture_output=True, text=True, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "sanitized host checks passed" in r.stdout
