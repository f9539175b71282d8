"""The C ABI's host paths under AddressSanitizer: tests/test_abi.py (argument checks,
configuration validation, workspace sizing, status strings, the static entry's refusals; no
GPU) run in a child process against the library built with host-side ASan, with clang's ASan
runtime preloaded.  Any invalid host memory access in those paths aborts the child."""

import os
import subprocess
import sys

from mla_tree_verify_mlaverify_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_host_asan():
    lib = build.ASAN_LIB_PATH
    if not os.path.exists(lib) or os.path.getmtime(lib) < max(
            os.path.getmtime(os.path.join(build.CSRC, f)) for f in build.SOURCES):
        build.build_asan()
    env = dict(os.environ, LD_PRELOAD=build.asan_runtime(), MLAVERIFY_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout
