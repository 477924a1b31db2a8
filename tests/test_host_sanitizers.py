"""The boundary's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The argument checks, workspace planning and launch set-up of the C ABI
(ds_api.hip, host pass) and the CPU calibration are rebuilt with
-fsanitize=address,undefined and no recovery, linked with the ordinary kernel
objects, and the CPU boundary tests (every rejection path with fake device
pointers, workspace sizing, calibration against the oracle) run against that
build in a child process with the toolchain's ASan runtime preloaded.  Any
sanitizer report ends the child with a non-zero status.  No GPU is used."""
import os
import subprocess
import sys

from long_context_sparse_ds_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_boundary_tests_pass_under_host_sanitizers():
    lib = B.build_host_sanitized()
    env = dict(os.environ, DSPARSE_LIB=lib, LD_PRELOAD=B.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                          "tests/test_abi_cpu.py", "tests/test_host_logic.py"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (res.stdout[-3000:] + "\n" + res.stderr[-6000:])
    assert res.returncode == 0, tail
    assert "runtime error" not in res.stdout + res.stderr, tail
    assert "AddressSanitizer" not in res.stdout + res.stderr, tail
