"""The library's host code under AddressSanitizer (no GPU): a copy of libspecache built with the
host pass instrumented (build.py --asan), loaded through SPECACHE_LIB into a Python process that
preloads the sanitizer's runtime, runs the host-side test files -- exports, argument validation
before any HIP call, workspace sizing, the binding's shape checks.  A heap or stack overrun in
the validation paths aborts that process."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from decode_attention_bit_kivi_amd import build  # noqa: E402

HOST_TESTS = ["tests/test_library_host.py", "tests/test_binding_host.py"]


def test_host_code_is_clean_under_address_sanitizer(tmp_path):
    try:
        build.hipcc()
        runtime = build.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = str(tmp_path / "libspecache_asan.so")
    build.build(jobs=8, verbose=False, out=lib, build_dir=str(tmp_path / "obj"), asan=True)
    env = dict(os.environ, LD_PRELOAD=runtime, SPECACHE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *HOST_TESTS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "AddressSanitizer" not in r.stderr
    shutil.rmtree(tmp_path / "obj", ignore_errors=True)
