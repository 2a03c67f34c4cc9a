"""Parity cases run through the SSM_DEBUG build of the library (the binding
loads whatever SSM_MI355X_LIB names): scans with time splits (and the
no-allocation entry point), the blocked single pass, the chunked scan with segments on both of its
paths, and the backward, each against the float64 oracle.  Every launch is
preceded by the debug build's plan checks; the last line printed is the
number of plans they checked.  Run by tests/test_gpu_debug_build.py in a
process of its own."""
import os
import sys

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import selective_state_space_03_amd as ssm  # noqa: E402
import ssm_workloads as W  # noqa: E402
from gpu_util import (DEV, check, dev_tensor, np64, scan_bwd_gpu, scan_bwd_oracle, scan_gpu, scan_oracle,  # noqa: E402
                      ssd_gpu, ssd_oracle)


def main():
    assert os.path.samefile(ssm.LIB_PATH, os.environ["SSM_MI355X_LIB"]), ssm.LIB_PATH
    L = ssm.lib()
    assert L.ssm_debug_checks() == 0, "not the debug build"
    # scans: the layer recipe with ragged channels and tiles, split or not
    w = W.scan_prefill(batch=2, seqlen=300, dim=200, unsaturated=True)
    yo, ho, co = scan_oracle(w)
    for split in (0, 1, 3, 16):
        y, st, cc = scan_gpu(w, time_split=split)
        check(np64(y), yo, 2e-3, f"debug build scan split={split}")
        check(np64(st), ho, 2e-3, f"debug build scan state split={split}")
        assert np.array_equal(np64(cc), co)
    # the no-allocation entry point on the same call
    o = w.opts
    st = torch.empty((2, 200, 16), dtype=torch.float32, device=DEV)
    y = ssm.scan_fwd_noalloc(dev_tensor(w, "x"), dev_tensor(w, "A"), dev_tensor(w, "B"), dev_tensor(w, "C"),
                             dev_tensor(w, "dt"), D=dev_tensor(w, "D"), z=dev_tensor(w, "z"),
                             conv_w=dev_tensor(w, "conv_w"), dt_rank1=True, dt_w=dev_tensor(w, "dt_w"),
                             dt_bias=dev_tensor(w, "dt_bias"), dt_min=o["dt_min"], dt_max=o["dt_max"],
                             ssm_state_out=st, y_dtype=torch.float32, time_split=5)
    torch.cuda.synchronize()
    check(np64(y), yo, 2e-3, "debug build scan (no allocation)")
    # the blocked single pass (bulk recipe, ragged tail)
    w = W.scan_bulk(batch=2, seqlen=300, dim=128, unsaturated=True)
    yo, ho, _ = scan_oracle(w)
    y, st, _ = scan_gpu(w, time_split=ssm.SCAN_BLOCKED)
    check(np64(y), yo, 2e-3, "debug build blocked scan")
    check(np64(st), ho, 2e-3, "debug build blocked scan state")
    # chunked scan: the tuned kernel with segments and pieces, then a shape of the vector-ALU path
    w = W.ssd_long(batch=2, seqlen=2085, nheads=3, headdim=96, ngroups=1, gated=True, unsaturated=True)
    out, st = ssd_gpu(w, segments=3)
    oo, so = ssd_oracle(w)
    check(np64(out), oo, 2e-3, "debug build chunked scan (segments)")
    check(np64(st), so, 2e-3, "debug build chunked scan state")
    w = W.ssd_long(batch=2, seqlen=700, nheads=4, headdim=48, ngroups=2, d_state=64, chunk_size=64, unsaturated=True)
    out, st = ssd_gpu(w)
    oo, so = ssd_oracle(w)
    check(np64(out), oo, 2e-3, "debug build chunked scan (vector-ALU path)")
    # backward: runs of segments, ragged channels, conv and cache
    w = W.scan_prefill(batch=2, seqlen=129, dim=200, unsaturated=True)
    rng = np.random.Generator(np.random.PCG64(5))
    dy = rng.standard_normal((2, 129, 200)).astype(np.float32)
    cache = rng.standard_normal((2, 200, 3)).astype(np.float32)
    g = scan_bwd_gpu(w, dy, cache_in=cache)
    go = scan_bwd_oracle(w, dy, cache_in=cache)
    assert set(g) == set(go)
    for k in sorted(go):
        check(g[k], go[k], 1e-5, f"debug build backward d{k}")
    print(L.ssm_debug_checks(), flush=True)


if __name__ == "__main__":
    main()
