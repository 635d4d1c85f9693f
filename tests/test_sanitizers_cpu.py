"""Host sanitizers over the C ABI and the planner (no GPU).

The library is rebuilt with AddressSanitizer and UndefinedBehaviorSanitizer on the host code
of the ABI (api.cpp) and the planner (plan.cpp); the CPU ABI tests then run against that build
in a child process that preloads the ASan runtime.  Any out-of-bounds access, use after free
or undefined behaviour on those paths aborts the child."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_abi_and_planner_under_asan_ubsan():
    from vlm_shared_prefix_amd import build as B
    lib = B.build_sanitized()
    rt = B.asan_runtime()
    assert os.path.exists(rt), rt
    env = dict(os.environ, LD_PRELOAD=rt, JEV_LIBRARY=lib, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    probe = subprocess.run([sys.executable, "-c", "from vlm_shared_prefix_amd import jev; print(jev.LIB_PATH)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stderr[-2000:]
    assert probe.stdout.strip() == lib
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi_cpu.py", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
