"""The ABI and plan tests once more, against a build of the library whose host
code (plan builder, argument checks, workspace layout, uploads) carries
AddressSanitizer and UBSan checks; device code is unchanged. Runs on the CPU:
host-only plans need no GPU."""

import os
import subprocess
import sys

from paged_kv_attention_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_host_sanitizers():
    lib = B.build(verbose=False, sanitize=True)
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "host code is not instrumented"
    env = dict(os.environ, LD_PRELOAD=B.sanitizer_runtime(), FI_LIB_PATH=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider", os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=1200)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, out
    assert " passed" in r.stdout, out
