"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
tests/sanitized_build.py builds the library with both sanitizers on the host
code and runs tests/test_abi_cpu.py against that build (argument validation,
error paths, the timer bookkeeping, the refusal of a stale build) with the
sanitizer runtime preloaded.  Any report aborts the child and fails here."""
import os
import subprocess

import pytest

import tests.sanitized_build as sb


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc not available")
def test_abi_host_code_is_sanitizer_clean():
    lib = sb.build()
    out = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_" in out and "__ubsan_handle" in out, "the build is not instrumented"
    r = sb.run_abi_tests()
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
