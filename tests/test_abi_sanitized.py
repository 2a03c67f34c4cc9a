"""The C-ABI validation tests (test_abi.py) and the launch-plan sweep of the
SSM_DEBUG checks (test_debug_build.py) once more, on a build whose host side
(argument checks, workspace sizing, dispatch, plan checks) runs under
AddressSanitizer and UndefinedBehaviorSanitizer, in a subprocess that
preloads the sanitizer runtime.  CPU only: no kernel is launched."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_clean_under_host_sanitizers():
    from selective_state_space_03_amd import build as b
    from selective_state_space_03_amd import build_sanitized as bs

    if not os.path.exists(b.LIB_PATH) or not os.path.isdir(b.BUILD):
        b.build()
    try:
        lib = bs.build_host_sanitized()
    except RuntimeError:
        b.build()
        lib = bs.build_host_sanitized()
    env = dict(os.environ, SSM_MI355X_LIB=lib, SSM_MI355X_DEBUG_LIB=lib, LD_PRELOAD=bs.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_debug_build.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out, out[-2000:]
    # the library the subprocess loaded is the instrumented one
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_" in nm and "__ubsan_" in nm
