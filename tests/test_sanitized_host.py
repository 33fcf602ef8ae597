"""The library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer: the C ABI's argument validation, the block
manager and the scheduler loop, exercised by the CPU test suites of the ABI,
the block manager, the scheduler, the waste figures and the binding's
checks, run in a child process against libpagedattn_san.so (built by
build(sanitize=True): host sources instrumented, device kernels unchanged)
with clang's ASan runtime preloaded.  Any sanitizer report fails the run."""
import os
import subprocess
import sys

import pytest

from paged_kv_cache_403_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUITES = ["tests/test_abi_cpu.py", "tests/test_scheduler.py", "tests/test_waste.py",
          "tests/test_binding_validation.py", "tests/test_oracle_block_manager.py"]


def test_host_code_runs_clean_under_asan_and_ubsan():
    if not os.path.exists(B.LIB_SAN):
        pytest.skip("libpagedattn_san.so not built (paged_kv_cache_403_amd.build.build(sanitize=True))")
    rt = B.asan_runtime()
    assert os.path.exists(rt), rt
    # the instrumentation is really there
    nm = subprocess.run(["nm", "-D", "--undefined-only", B.LIB_SAN], capture_output=True, text=True).stdout
    assert "__asan_report" in nm and "__ubsan_handle" in nm
    env = dict(os.environ, LD_PRELOAD=rt, PAGEDATTN_LIB=B.LIB_SAN,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", *SUITES, "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        "-x"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
