"""The host layer (argument checks, workspace sizes, split planning, status
strings) under AddressSanitizer and UndefinedBehaviorSanitizer: the boundary
tests run in a child process against libqsa_san.so, a build of the same
sources with host-side sanitizers, with the ASan runtime preloaded.  CPU only:
every case returns before any HIP call."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_boundary_tests_clean_under_asan_ubsan():
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-only sanitizer run (the boundary cases use fake device addresses)")
    from top_indexed_sparse_qsa_amd import build as B
    rt = B.asan_runtime()
    if not rt:
        pytest.skip("no shared ASan runtime in this ROCm install")
    lib = B.build(sanitize=True)
    env = dict(os.environ, LIBQSA_PATH=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_boundary.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
