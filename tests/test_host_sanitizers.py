"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The C ABI is rebuilt with both sanitizers on its host code (argument validation, launch
planning, workspace carving; the device code is unchanged) and the host-only tests - every
host-detectable error path of test_abi.py and the workspace audit of every workload shape in
test_workspace_audit.py - run against that build in a child process with the sanitizer runtime
preloaded.  A heap overflow, a use after free or undefined behaviour in any of those host paths
aborts the child and fails this test.  No GPU is touched: none of these calls launches."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(600)
def test_host_paths_clean_under_asan_and_ubsan():
    if not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not available")
    from block_diffusion_drafter_states_amd import build as b
    lib = b.build_host_sanitized()
    env = dict(os.environ)
    env["DFLASH_LIB_PATH"] = lib
    env["LD_PRELOAD"] = b.sanitizer_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["PYTHONDONTWRITEBYTECODE"] = "1"
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py"),
                          os.path.join(ROOT, "tests", "test_workspace_audit.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=540)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
