"""ssm_scan_fwd_noalloc (the scan entry point for callers that cannot
allocate device memory; its workspace is the library's own device scratch)
against ssm_scan_fwd on the same inputs, through the C ABI: two calls in a
row, the second on a smaller input, each equal to ssm_scan_fwd (same kernels,
same time split: bit for bit, and so within the 2e-3 max|y| bound of a
bf16-input workload), and a call past the scratch size refused."""
import numpy as np
import pytest
import torch

import selective_state_space_03_amd as ssm
import ssm_workloads as W
from gpu_util import DEV, check, dev_tensor, np64

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _args(w):
    o = w.opts
    pos = (dev_tensor(w, "x"), dev_tensor(w, "A"), dev_tensor(w, "B"), dev_tensor(w, "C"), dev_tensor(w, "dt"))
    kw = dict(D=dev_tensor(w, "D"), z=dev_tensor(w, "z"), conv_w=dev_tensor(w, "conv_w") if o["conv"] else None,
              dt_rank1=o["dt_rank1"], dt_w=dev_tensor(w, "dt_w"), dt_bias=dev_tensor(w, "dt_bias"),
              dt_softplus=o["dt_softplus"], dt_min=o["dt_min"], dt_max=o["dt_max"], y_dtype=torch.float32)
    return pos, kw


def _both(w, time_split=0, state_in=None, cache_in=None):
    """The same call through both entry points; returns (y, state, cache) of each."""
    pos, kw = _args(w)
    Bt, E = w.dims["batch"], w.dims["dim"]
    res = []
    for fn in (ssm.scan_fwd, ssm.scan_fwd_noalloc):
        st = torch.full((Bt, E, 16), float("nan"), device=DEV)
        cc = torch.full((Bt, E, 3), float("nan"), device=DEV) if w.opts["conv"] else None
        y = fn(*pos, **kw, ssm_state_in=state_in, ssm_state_out=st, conv_cache_in=cache_in, conv_cache_out=cc,
               time_split=time_split)
        torch.cuda.synchronize()
        res.append((y, st, cc))
    return res


def _same(ref, got, what):
    for a, b, name in zip(ref, got, ("y", "state", "cache")):
        if a is None:
            continue
        assert torch.isfinite(b).all(), f"{what} {name}: not every element written"
        check(np64(b), np64(a), TOL, f"{what} {name}")
        assert torch.equal(a, b), f"{what} {name}: differs from ssm_scan_fwd"


def test_noalloc_matches_scan_fwd_twice_second_smaller():
    # call 1: the layer-prefill recipe (conv, rank-1 dt, gate), several waves,
    # the library's own time split
    w1 = W.scan_prefill(batch=2, seqlen=700, dim=520, unsaturated=True)
    r1 = _both(w1)
    _same(r1[0], r1[1], "first call")
    # call 2, smaller, right after: the bulk recipe (E-wide bf16 dt, no conv),
    # a forced split of 3, from a given state; the scratch still holds call 1
    w2 = W.scan_bulk(batch=1, seqlen=300, dim=136)
    rng = np.random.Generator(np.random.PCG64(31))
    st_in = torch.from_numpy(rng.standard_normal((1, 136, 16)).astype(np.float32)).to(DEV)
    r2 = _both(w2, time_split=3, state_in=st_in)
    _same(r2[0], r2[1], "second call")


def test_noalloc_blocked_matches_scan_fwd():
    """The blocked single pass through both entry points (its table records in
    the scratch), twice, the second call smaller."""
    w1 = W.scan_bulk(batch=2, seqlen=333, dim=192)
    r1 = _both(w1, time_split=ssm.SCAN_BLOCKED)
    _same(r1[0], r1[1], "blocked, first call")
    w2 = W.scan_bulk(batch=1, seqlen=40, dim=64, unsaturated=True)
    r2 = _both(w2, time_split=ssm.SCAN_BLOCKED)
    _same(r2[0], r2[1], "blocked, second call")


def test_noalloc_refuses_past_its_scratch():
    w = W.scan_bulk(batch=64, seqlen=4096, dim=64)
    pos, kw = _args(w)
    with pytest.raises(ssm.SsmError) as e:
        ssm.scan_fwd_noalloc(*pos, **kw)
    assert e.value.status == 3 and "scratch" in str(e.value)
