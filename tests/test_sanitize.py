"""The host code of the library (argument checks, the planner, workspace
layout, tracing state) under AddressSanitizer and UndefinedBehaviorSanitizer:
cross_entropy_amd/build.py --sanitize builds the library with both on its
host compilation, and the host ABI tests (tests/test_abi.py, including its
planner sweep) run against that build in a child process with the ASan
runtime preloaded. Any report aborts the child, which fails this test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_abi_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from cross_entropy_amd import build as b
    try:
        path = b.build(sanitize=True)
    except RuntimeError as e:   # pragma: no cover
        pytest.fail(f"sanitizer build failed: {e}")
    env = b.sanitizer_env()
    probe = ("import sys; sys.path.insert(0, %r); from cross_entropy_amd import _native as n; n.load(); "
             "maps = open('/proc/self/maps').read(); "
             "assert %r in maps, 'sanitizer build not loaded'; assert 'libclang_rt.asan' in maps" % (ROOT, path))
    r = subprocess.run([sys.executable, "-c", probe], env=env, capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, capture_output=True, text=True, cwd=ROOT, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr
