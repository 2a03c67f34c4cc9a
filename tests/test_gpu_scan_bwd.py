"""GPU parity of ssm_scan_bwd (the scan stage's backward, with states
recomputed per 16-step segment) against the float64 oracle's reverse-mode
ssm_layer_scan_backward, through the C ABI.  Every gradient is fp32 computed
from exact inputs, so each gradient is held to the fp32 bound
max|err| <= 1e-5 max|grad| (measured: at most 7e-7 at full size, the sums
over time and channels taken in another order than the oracle's)."""
import numpy as np
import pytest
import torch

import ssm_workloads as W
from gpu_util import check, scan_bwd_gpu, scan_bwd_oracle

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _dy(w, seed=31):
    d = w.dims
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(
        (d["batch"], d["seqlen"], d["dim"])).astype(np.float32)


def _compare(w, **kw):
    dy = _dy(w)
    g = scan_bwd_gpu(w, dy, **kw)
    go = scan_bwd_oracle(w, dy, **kw)
    assert set(g) == set(go), (sorted(g), sorted(go))
    for k in sorted(go):
        check(g[k], go[k], TOL, f"{w.name} d{k}")


@pytest.mark.parametrize("unsat", [False, True])
def test_bwd_tiny_fp32(unsat):
    """batch 1, L 64, E 16, rank-1 dt, gate, D, no conv."""
    _compare(W.scan_tiny(unsaturated=unsat))


@pytest.mark.parametrize("seqlen", [1, 16, 37, 64, 65, 129, 300])
def test_bwd_prefill_recipe(seqlen):
    """bf16 x/z, conv + SiLU, rank-1 dt, bf16 B/C at batch 2, E 200 (a ragged
    channel group, and a last block of four groups with three spare waves),
    with an initial state, a conv cache and a gradient on the final state;
    ragged last segment, and runs of four segments that end exactly at the
    sequence end (64), one step past it (65) or part-way (129, 300)."""
    w = W.scan_prefill(batch=2, seqlen=seqlen, dim=200, unsaturated=True)
    rng = np.random.Generator(np.random.PCG64(5))
    _compare(w, state_in=rng.standard_normal((2, 200, 16)).astype(np.float32) * 0.5,
             cache_in=rng.standard_normal((2, 200, 3)).astype(np.float32),
             dstate_out=rng.standard_normal((2, 200, 16)).astype(np.float32))


def test_bwd_prefill_recipe_saturated_no_extras():
    """Most steps on the upper clip (no dt gradient there), zero initial state."""
    _compare(W.scan_prefill(batch=1, seqlen=200, dim=72))


@pytest.mark.parametrize("unsat", [False, True])
def test_bwd_bulk_recipe(unsat):
    """E-wide bf16 dt with bias and softplus, no conv, bf16 everything."""
    _compare(W.scan_bulk(batch=2, seqlen=100, dim=40, unsaturated=unsat))


def test_bwd_deterministic():
    w = W.scan_prefill(batch=2, seqlen=100, dim=64, unsaturated=True)
    dy = _dy(w)
    a = scan_bwd_gpu(w, dy)
    b = scan_bwd_gpu(w, dy)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_bwd_full_size():
    """The layer-prefill workload at full size (1 x 2048, E 7680)."""
    w = W.scan_prefill(unsaturated=True)
    _compare(w)
