"""The C ABI's host runtime under AddressSanitizer and UndefinedBehaviorSanitizer
(host code only): plan lifecycle, workspace sizing and every argument check
before device work, run by the driver tests/abi_sanitize.cpp on fake device
pointers.  No GPU needed."""
import os
import shutil
import subprocess

import pytest


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_abi_host_paths_under_asan_and_ubsan():
    from autoregressive_normalizing_flow_amd import build
    exe = build.build_abi_sanitize_check()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    print(out[-2000:])
    assert r.returncode == 0, out[-4000:]
    assert "OK: 0 failed checks" in r.stdout
    assert "runtime error" not in out and "AddressSanitizer" not in out
