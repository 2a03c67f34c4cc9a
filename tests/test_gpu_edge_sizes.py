"""GPU parity at degenerate sizes, through the C ABI: one channel, one short of
and one past a 64-channel group, one or two tokens, with and without a time
split; one head of the narrowest headdim in the chunked scan and its decode
step; one channel in the decode step and the backward; an empty batch.
Tolerances as in the per-entry-point tests: 1e-5 max|ref| for fp32 work,
2e-3 for bf16 inputs."""
import numpy as np
import pytest
import torch

import selective_state_space_03_amd as ssm
import ssm_workloads as W
from gpu_util import (DEV, check, dev_tensor, np64, scan_bwd_gpu, scan_bwd_oracle, scan_gpu, scan_oracle,
                      ssd_decode_gpu, ssd_gpu, ssd_oracle)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dim", [1, 63, 65])
@pytest.mark.parametrize("seqlen", [1, 2, 9, 40])
@pytest.mark.parametrize("split", [0, 1, 4])
def test_scan_edge_sizes_fp32(dim, seqlen, split):
    w = W.scan_tiny(batch=2, seqlen=seqlen, dim=dim, unsaturated=True)
    y, st, _ = scan_gpu(w, time_split=split)
    yo, ho, _ = scan_oracle(w)
    check(np64(y), yo, 1e-5, f"scan E={dim} L={seqlen} split={split}")
    check(np64(st), ho, 1e-5, f"scan state E={dim} L={seqlen} split={split}")


@pytest.mark.parametrize("dim", [1, 65])
@pytest.mark.parametrize("seqlen", [1, 3, 33])
def test_scan_edge_sizes_layer_recipe(dim, seqlen):
    """conv + rank-1 dt + gate at one channel or a group and one more."""
    w = W.scan_prefill(batch=1, seqlen=seqlen, dim=dim, unsaturated=True)
    y, st, cc = scan_gpu(w, time_split=2 if seqlen >= 16 else 0)
    yo, ho, co = scan_oracle(w)
    check(np64(y), yo, 2e-3, f"layer-recipe scan E={dim} L={seqlen}")
    check(np64(st), ho, 2e-3, f"layer-recipe state E={dim} L={seqlen}")
    assert np.array_equal(np64(cc), co)


def test_scan_empty_batch():
    w = W.scan_tiny(batch=1, seqlen=8, dim=16)
    t = {k: dev_tensor(w, k) for k in ("x", "A", "B", "C", "dt", "D", "z", "dt_w", "dt_bias")}
    empty = lambda a: a[:0]  # noqa: E731
    y = ssm.scan_fwd(empty(t["x"]), t["A"], empty(t["B"]), empty(t["C"]), empty(t["dt"]), D=t["D"], z=empty(t["z"]),
                     dt_rank1=True, dt_w=t["dt_w"], dt_bias=t["dt_bias"], dt_min=w.opts["dt_min"],
                     dt_max=w.opts["dt_max"])
    torch.cuda.synchronize()
    assert tuple(y.shape) == (0, 8, 16)


@pytest.mark.parametrize("dim", [1, 65])
def test_decode_edge_sizes(dim):
    """One decode step at batch 1 from a random state and cache."""
    w = W.decode_stream(batch=1, dim=dim, prefill=0, steps=1, unsaturated=True)
    from oracle import ssm_oracle as O

    rng = np.random.Generator(np.random.PCG64(31))
    st0 = rng.standard_normal((1, dim, 16)).astype(np.float32)
    cc0 = rng.standard_normal((1, dim, 3)).astype(np.float32)
    t = lambda k: torch.from_numpy(np.array(w.arrays[k], copy=True)).to(DEV)  # noqa: E731
    st = torch.from_numpy(st0.copy()).to(DEV)
    cc = torch.from_numpy(cc0.copy()).to(DEV)
    o = w.opts
    y = ssm.decode_step(t("x")[0], t("A"), t("B")[0], t("C")[0], t("dt")[0], st, conv_cache=cc, D=t("D"),
                        z=t("z")[0], conv_w=t("conv_w"), dt_rank1=True, dt_w=t("dt_w"), dt_bias=t("dt_bias"),
                        dt_min=o["dt_min"], dt_max=o["dt_max"])
    torch.cuda.synchronize()
    f = w.f64
    yo, co, ho = O.decode_step(f("x")[0], f("A"), f("B")[0], f("C")[0], conv_cache=cc0.astype(np.float64),
                               ssm_state=st0.astype(np.float64), D=f("D"), z_t=f("z")[0], conv_w=f("conv_w"),
                               dt_raw_t=f("dt")[0], dt_w=f("dt_w"), dt_bias=f("dt_bias"),
                               dt_min=float(o["dt_min"]), dt_max=float(o["dt_max"]))
    check(np64(y), yo, 1e-5, f"decode E={dim}")
    check(np64(st), ho, 1e-5, f"decode state E={dim}")
    assert np.array_equal(np64(cc), co)


@pytest.mark.parametrize("seqlen", [1, 129])
@pytest.mark.parametrize("headdim,d_state,chunk", [(16, 64, 128), (8, 16, 64)])
def test_ssd_one_head(seqlen, headdim, d_state, chunk):
    """One head of the narrowest headdim: the matrix-core kernel (16 x 64,
    chunk 128) and the vector-ALU path (8 x 16, chunk 64)."""
    w = W.ssd_long(batch=1, seqlen=seqlen, nheads=1, headdim=headdim, ngroups=1, d_state=d_state, chunk_size=chunk,
                   unsaturated=True)
    out, st = ssd_gpu(w)
    oo, so = ssd_oracle(w, sequential=True)
    check(np64(out), oo, 2e-3, f"ssd one head P={headdim} N={d_state} L={seqlen}")
    check(np64(st), so, 2e-3, f"ssd one head state P={headdim} N={d_state} L={seqlen}")


def test_ssd_decode_one_head():
    w = W.ssd_decode(batch=1, nheads=1, headdim=16, ngroups=1, d_state=64)
    st = torch.from_numpy(w.arrays["state0"].copy()).to(DEV)
    out = ssd_decode_gpu(w, st)
    torch.cuda.synchronize()
    oo, so = ssd_oracle(w, state_in=w.arrays["state0"], sequential=True)
    check(np64(out), oo[:, 0], 1e-5, "ssd decode one head")
    check(np64(st), so, 1e-5, "ssd decode one head state")


@pytest.mark.parametrize("dim", [1, 17])
@pytest.mark.parametrize("seqlen", [1, 2])
def test_bwd_edge_sizes(dim, seqlen):
    w = W.scan_prefill(batch=1, seqlen=seqlen, dim=dim, unsaturated=True)
    dy = np.random.Generator(np.random.PCG64(33)).standard_normal((1, seqlen, dim)).astype(np.float32)
    g = scan_bwd_gpu(w, dy)
    go = scan_bwd_oracle(w, dy)
    assert set(g) == set(go)
    for k in sorted(go):
        check(g[k], go[k], 1e-5, f"bwd E={dim} L={seqlen} d{k}")
