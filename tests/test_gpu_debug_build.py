"""The SSM_DEBUG build of the library on the GPU: the parity cases of
tests/debug_build_cases.py (scan with splits and without allocation, the blocked
single pass, chunked
scan with segments on both paths, backward) pass with the host-side launch-plan
checks in front of every launch, and the checks ran."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def test_debug_build_parity_and_checks():
    from selective_state_space_03_amd import build as b

    assert os.path.exists(b.DEBUG_LIB_PATH), "the debug build is made by build() with the regular one"
    env = dict(os.environ, SSM_MI355X_LIB=b.DEBUG_LIB_PATH, PYTHONUNBUFFERED="1")
    res = subprocess.run([sys.executable, os.path.join(HERE, "debug_build_cases.py")], env=env,
                         capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    checks = int(res.stdout.strip().splitlines()[-1])
    # 4 scans + 1 without allocation + 1 blocked + 2 chunked scans + 1 backward
    assert checks == 9, out[-2000:]
