"""The boundary's CPU tests (argument validation, workspace sizing, error
paths, symbol exports) again, against a build of the library whose host code
carries AddressSanitizer and UndefinedBehaviorSanitizer: any invalid memory
access or undefined behaviour in the host side of the C ABI fails them. Device
code cannot run under ASan here, so only host code is covered."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_abi_under_host_sanitizers():
    from expert_routing_router_amd import build_sanitized as bs
    lib = bs.build()
    rt = bs.runtime_path()
    assert os.path.exists(rt), rt
    env = dict(os.environ, LD_PRELOAD=rt, MOE_ROCM_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi_cpu.py", "-q", "-x", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
