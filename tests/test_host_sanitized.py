"""The host C++ under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The validator, the handle and ABI layer, and the safetensors/JSON header reader
(which parses untrusted headers up to 100 MB) are rebuilt with g++'s sanitizers
and the host test suites are run against that build in a child process with
the sanitizer runtimes preloaded: any invalid access, overflow or undefined
operation aborts the child and fails this test.
"""
import os
import subprocess
import sys

import pytest

import host_sanitize as H


def test_host_suites_pass_under_asan_and_ubsan():
    rt = H.runtimes()
    if rt is None:
        pytest.skip("g++ sanitizer runtimes are not installed")
    lib = H.build()
    nm = subprocess.run(["nm", os.path.join(H.OUT, "bsf8_inspect.o")], capture_output=True, text=True).stdout
    assert "__asan_report" in nm and "__ubsan_handle" in nm, "the host objects are not instrumented"
    env = dict(os.environ, LD_PRELOAD=":".join(rt), BSF8_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    suites = [os.path.join(H.ROOT, "tests", f) for f in
              ("test_abi_host.py", "test_inspect_safetensors.py", "test_oracle_validate.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu"] + suites,
                       cwd=H.ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
