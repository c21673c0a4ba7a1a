"""The host side of libspec (argument validation, plan checks, workspace
layout, the error paths) under AddressSanitizer and UndefinedBehaviorSanitizer.

A second build of the library instruments only its host code (the device code
is unchanged: every sanitizer flag goes to the host compiler), and the
boundary tests run against it in a child process with the ASan runtime
preloaded.  No GPU is touched: those tests exercise the host checks only."""
import glob
import os
import subprocess
import sys

import pytest

from layer_speculative_decoding_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_LIB = os.path.join(ROOT, "_build", "libspec_san.so")
HOST_SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-shared-libsan"]


def _asan_runtime():
    cands = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return cands[-1] if cands else None


@pytest.mark.slow
def test_boundary_checks_clean_under_asan_and_ubsan():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no clang ASan runtime in this ROCm installation")
    build.build(extra_flags=HOST_SAN_FLAGS, lib=SAN_LIB)
    syms = subprocess.run(["nm", "-D", SAN_LIB], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle" in syms   # the host code is instrumented
    env = dict(os.environ, LD_PRELOAD=rt, SPEC_LIB_PATH=SAN_LIB,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = ("import sys, pytest, layer_speculative_decoding_amd as L; "
            "assert L.LIB_PATH == sys.argv[1], L.LIB_PATH; "
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', 'tests/test_boundary.py']))")
    r = subprocess.run([sys.executable, "-c", code, SAN_LIB], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
