"""The C ABI's host code under AddressSanitizer, on the CPU: a host-only
sanitizer build of the library (the gfx950 code is not instrumented) runs
every test of tests/test_abi.py (argument checks, the workspace arithmetic,
status strings, the exported symbols) in a child process with the
sanitizer runtime preloaded. Any invalid host memory access ends that
process with a sanitizer report."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import ctypes, sys
sys.path.insert(0, {root!r})
sys.path.insert(0, {tests!r})
import group_limited_routing_amd as gl
gl.LIB_PATH = {lib!r}
gl.lib()
# the sanitizer runtime is live in this process, and the instrumented
# library is the one loaded
assert hasattr(ctypes.CDLL(None), "__asan_report_load8")
assert any("libbeam_moe_asan.so" in line for line in open("/proc/self/maps"))
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", {abi!r}]))
"""


def test_abi_host_code_under_address_sanitizer():
    from group_limited_routing_amd import build
    rt = build.asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime next to hipcc's clang")
    lib = build.build(asan=True)
    env = dict(os.environ, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:exitcode=99")
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib,
                        abi=os.path.join(ROOT, "tests", "test_abi.py"))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=600, cwd=ROOT)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-2000:])
    assert "passed" in r.stdout
