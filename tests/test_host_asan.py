"""Host-side AddressSanitizer over the C ABI's host code.

The library's host code (spec validation, arena, workspace and cache-state sizing, argument
checks, the probe guards) is rebuilt with AddressSanitizer -- the device code is unchanged and
nothing here runs on a GPU -- and the host-only ABI tests (test_abi.py) run against it in a
child process with the sanitizer's runtime preloaded.  An invalid read or write, or a use after
free, in that code ends the child with a sanitizer report and fails this test.
"""
import os
import subprocess
import sys

import pytest

from cvr_ranking_model_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = """
import ctypes, sys
sys.path.insert(0, {root!r})
ctypes.CDLL(None)["__asan_init"]          # the sanitizer runtime is in this process
import cvr_ranking_model_amd.cvr as cv
cv.LIB_PATH = {lib!r}
assert cv.lib()._name == {lib!r}
import pytest
sys.exit(pytest.main(["-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider", {tests!r}]))
"""


def test_abi_host_code_under_address_sanitizer(tmp_path):
    try:
        runtime = build.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = build.build(asan=True, out_dir=str(tmp_path))
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms, "the library's host code is not instrumented"
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    code = CHILD.format(root=ROOT, lib=lib, tests=os.path.join(ROOT, "tests", "test_abi.py"))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "passed" in r.stdout
