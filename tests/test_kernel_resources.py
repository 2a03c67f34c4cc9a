"""Register, scratch and occupancy figures of the blocked scan kernel, from the
compiler's resource report (hipcc for gfx950; no GPU needed).  Its pipeline of
loads issued three blocks ahead only holds when no per-lane array falls back
to scratch memory (every scratch access would wait for all loads in flight),
and its grid (3.75 workgroups per CU at the bulk shape) is only resident at
once with four waves per SIMD."""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from selective_state_space_03_amd import build as b


def _report(src):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        cmd = [hipcc, *b.COMMON, *b.DEVICE_FLAGS, "--cuda-device-only", "-c", os.path.join(b.CSRC, src),
               "-o", os.path.join(d, "k.o"), "-Rpass-analysis=kernel-resource-usage"]
        res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-3000:]
    kernels, cur = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+)", line)
        if cur and m:
            kernels[cur][m.group(1).strip()] = int(m.group(2))
    return kernels


def test_blocked_scan_kernel_resources():
    ks = {k: v for k, v in _report("scan_blocked.hip").items() if "scan_blk_kernel" in k}
    assert len(ks) == 4, sorted(ks)  # y in bf16 / fp32, with and without the gate
    for name, r in ks.items():
        assert r["ScratchSize"] == 0, (name, r)
        assert r["VGPRs Spill"] == 0 and r["SGPRs Spill"] == 0, (name, r)
        assert r["Occupancy"] >= 4, (name, r)
