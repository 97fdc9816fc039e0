"""The host-logic tests again, against a build of the library whose host code carries
AddressSanitizer and UndefinedBehaviorSanitizer (``build.py --asan-host``; device code as
usual, never run here). Any invalid access, leak-free use-after-free, overflow or undefined
operation in the host core (slot assignment, view resolution, step plans, table packing)
aborts the child run. CPU only: no GPU is touched.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"


def _asan_runtime():
    try:
        out = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                             capture_output=True, text=True, timeout=60)
    except (OSError, subprocess.TimeoutExpired):
        return None
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.timeout(600)
def test_host_logic_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "libhogwild_asan.so")
    build = subprocess.run([sys.executable, "-m", "shared_kv_cache_amd.build", "--asan-host", lib],
                           cwd=ROOT, capture_output=True, text=True, timeout=400)
    assert build.returncode == 0, build.stdout[-2000:] + build.stderr[-2000:]
    env = dict(os.environ, HOGWILD_LIBRARY=lib, LD_PRELOAD=runtime,
               # the interpreter's own allocations are not the library's: no leak report;
               # any error report ends the run with a failure status
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_host_cpu.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=400)
    tail = (run.stdout[-3000:] + run.stderr[-3000:])
    assert run.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
    assert " passed" in run.stdout, tail
