"""The host side of the library (planner, offsets, argument validation of every
entry point) built as plain C++ under AddressSanitizer and
UndefinedBehaviorSanitizer, with the kernel launchers stubbed out, and the
CPU tests of that code run against it in a child process (CPU only)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = ["tests/test_abi.py", "tests/test_planner_cpp.py", "tests/test_host_fuzz.py"]


def _runtime(name):
    r = subprocess.run(["g++", "-print-file-name=" + name], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def hostcheck_lib():
    from jagged_flashattention_amd import hostcheck
    asan = _runtime("libasan.so")
    if asan is None or not hostcheck.available():
        pytest.skip("g++ with AddressSanitizer or the HIP headers not available")
    return hostcheck.build(), asan


def test_hostcheck_build_is_instrumented(hostcheck_lib):
    lib, _ = hostcheck_lib
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    # no device code in it: the launchers are the stubs
    assert "__hip_fatbin" not in syms


def test_host_tests_pass_under_sanitizers(hostcheck_lib):
    lib, asan = hostcheck_lib
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan, JFA_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *TESTS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
