"""The C ABI's host code (validation, planning, aliasing checks, dispatch up to the
launch) under AddressSanitizer and UndefinedBehaviorSanitizer: the CPU boundary tests
run in a child process against a copy of libfar.so built with host-only sanitizers, and
must pass with no sanitizer report."""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_CHILD = """
import os, sys
sys.path.insert(0, {root!r}); sys.path.insert(0, os.path.join({root!r}, "tests"))
from residual_add_rmsnorm_fp32_amd import binding as B
B.load_library({lib!r})
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", os.path.join({root!r}, "tests", "test_boundary_cpu.py")]))
"""


def test_boundary_checks_under_asan_and_ubsan(tmp_path):
    from residual_add_rmsnorm_fp32_amd import build as bld
    if not os.path.exists(bld.LIB_PATH):
        pytest.skip("libfar.so not built")
    try:
        lib, runtime = bld.build_sanitized()
    except (RuntimeError, OSError, subprocess.CalledProcessError) as e:
        pytest.skip(f"no sanitized build here: {e}")
    if not os.path.exists(runtime):
        pytest.skip("no ASan runtime")
    log = str(tmp_path / "san")
    env = dict(os.environ, LD_PRELOAD=runtime,
               ASAN_OPTIONS=f"detect_leaks=0:verify_asan_link_order=0:log_path={log}",
               UBSAN_OPTIONS=f"print_stacktrace=1:log_path={log}")
    res = subprocess.run([sys.executable, "-c", _CHILD.format(root=ROOT, lib=lib)], env=env,
                         capture_output=True, text=True, timeout=600)
    reports = [open(p).read() for p in glob.glob(log + "*")]
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-2000:]
    assert "passed" in res.stdout
    assert not reports, reports[0][:3000]
