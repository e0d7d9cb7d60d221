"""The debug and sanitizer builds of the library (CPU).

* libzha_debug.so (built by __graft_entry__.build()) compiles the device invariant checks
  into the same kernels and exports the same functions; the release library compiles none.
* libzha_asan.so: the host side built with AddressSanitizer and UndefinedBehaviorSanitizer;
  the host-validation tests (tests/test_abi.py, no GPU work) run against it in a child
  process with the sanitizer runtime preloaded, and must pass with no report.
"""
from __future__ import annotations

import ctypes
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "tests"))

from test_abi import declared_functions  # noqa: E402


def _lib(variant):
    """The variant's library, built again when any source or header is newer than it."""
    from hierarchical_tree_indexed_03_amd import build_lib
    path = build_lib.VARIANTS[variant]["out"]
    srcs = glob.glob(os.path.join(ROOT, "hierarchical_tree_indexed_03_amd", "csrc", "*.*")) + \
        glob.glob(os.path.join(ROOT, "include", "*.h"))
    if not os.path.exists(path) or os.path.getmtime(path) < max(os.path.getmtime(f) for f in srcs):
        build_lib.build(variant=variant)
    return path


def test_debug_library_has_checks_and_exports():
    lib = ctypes.CDLL(_lib("debug"))
    lib.zha_debug_checks_compiled.restype = ctypes.c_int32
    assert lib.zha_debug_checks_compiled() == 1
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} missing from the debug library"


def test_release_library_has_no_checks():
    lib = ctypes.CDLL(_lib("release"))
    lib.zha_debug_checks_compiled.restype = ctypes.c_int32
    assert lib.zha_debug_checks_compiled() == 0


def _asan_runtime():
    cands = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return cands[-1] if cands else None


def test_host_validation_under_asan_ubsan():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in the toolchain")
    path = _lib("asan")
    env = dict(os.environ)
    env.update(ZHA_LIB_PATH=path, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-3000:]
