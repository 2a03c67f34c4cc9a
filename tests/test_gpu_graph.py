"""The entry points captured in a HIP graph: every replay (with eager work and
synchronisations between replays) must reproduce the eager call bit for bit.
The library records no memset or host-side work inside its launches, so a
captured call is just its kernels."""
import numpy as np
import pytest
import torch

import selective_state_space_03_amd as ssm
import ssm_workloads as W
from gpu_util import DEV, dev_tensor, scan_gpu

pytestmark = pytest.mark.gpu


def _capture(call, stream):
    stream.wait_stream(torch.cuda.current_stream())
    call.run()  # warm-up outside the graph
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        call.run()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("split", [0, 5])
def test_scan_graph_replays(split):
    w = W.scan_prefill(batch=2, seqlen=300, dim=200, unsaturated=True)
    y_ref, st_ref, cc_ref = scan_gpu(w, time_split=split)
    o, d = w.opts, w.dims
    stream = torch.cuda.Stream(DEV)
    y = torch.empty((2, 300, 200), dtype=torch.float32, device=DEV)
    st = torch.empty((2, 200, 16), dtype=torch.float32, device=DEV)
    cc = torch.empty((2, 200, 3), dtype=torch.float32, device=DEV)
    call = ssm.scan_fwd(dev_tensor(w, "x"), dev_tensor(w, "A"), dev_tensor(w, "B"), dev_tensor(w, "C"),
                        dev_tensor(w, "dt"), D=dev_tensor(w, "D"), z=dev_tensor(w, "z"),
                        conv_w=dev_tensor(w, "conv_w"), conv_cache_out=cc, dt_rank1=True,
                        dt_w=dev_tensor(w, "dt_w"), dt_bias=dev_tensor(w, "dt_bias"), dt_min=o["dt_min"],
                        dt_max=o["dt_max"], ssm_state_out=st, y=y, time_split=split, stream=stream, prepare=True)
    g = _capture(call, stream)
    for _ in range(3):
        for t in (y, st, cc):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(st, st_ref) and torch.equal(cc, cc_ref)


def test_blocked_scan_graph_replays():
    """The blocked single pass (table packing + scan) captured and replayed."""
    w = W.scan_bulk(batch=2, seqlen=300, dim=128)
    y_ref, st_ref, _ = scan_gpu(w, time_split=ssm.SCAN_BLOCKED)
    o = w.opts
    stream = torch.cuda.Stream(DEV)
    y = torch.empty((2, 300, 128), dtype=torch.float32, device=DEV)
    st = torch.empty((2, 128, 16), dtype=torch.float32, device=DEV)
    call = ssm.scan_fwd(dev_tensor(w, "x"), dev_tensor(w, "A"), dev_tensor(w, "B"), dev_tensor(w, "C"),
                        dev_tensor(w, "dt"), D=dev_tensor(w, "D"), z=dev_tensor(w, "z"),
                        dt_bias=dev_tensor(w, "dt_bias"), dt_min=o["dt_min"], dt_max=o["dt_max"],
                        ssm_state_out=st, y=y, time_split=ssm.SCAN_BLOCKED, stream=stream, prepare=True)
    g = _capture(call, stream)
    for _ in range(3):
        for t in (y, st):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(st, st_ref)


def test_decode_graph_replays():
    w = W.decode_stream(batch=8, dim=200, prefill=0, steps=1)
    t = lambda k: torch.from_numpy(np.ascontiguousarray(w.arrays[k])).to(DEV)
    X, Z, R, Bm, Cm = (t(k) for k in ("x", "z", "dt", "B", "C"))
    A, D, cw, dw, db = (t(k) for k in ("A", "D", "conv_w", "dt_w", "dt_bias"))
    rng = np.random.Generator(np.random.PCG64(12))
    st0 = torch.from_numpy(rng.standard_normal((8, 200, 16)).astype(np.float32)).to(DEV)
    cc0 = torch.from_numpy(rng.standard_normal((8, 200, 3)).astype(np.float32)).to(DEV)
    kw = dict(D=D, z=Z[0], conv_w=cw, dt_rank1=True, dt_w=dw, dt_bias=db, dt_min=1e-3, dt_max=0.1)
    st_ref, cc_ref = st0.clone(), cc0.clone()
    y_ref = ssm.decode_step(X[0], A, Bm[0], Cm[0], R[0], st_ref, conv_cache=cc_ref, **kw)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream(DEV)
    st, cc = st0.clone(), cc0.clone()
    y = torch.empty((8, 200), dtype=torch.float32, device=DEV)
    call = ssm.decode_step(X[0], A, Bm[0], Cm[0], R[0], st, conv_cache=cc, y=y, stream=stream, prepare=True, **kw)
    g = _capture(call, stream)
    for _ in range(3):
        st.copy_(st0)
        cc.copy_(cc0)
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(st, st_ref) and torch.equal(cc, cc_ref)


def test_chunk_scan_graph_replays():
    w = W.ssd_long(seqlen=512, nheads=4, headdim=32)
    o, d = w.opts, w.dims
    x, dtr, A, B, C, D, db = (dev_tensor(w, k) for k in ("x", "dt", "A", "B", "C", "D", "dt_bias"))
    kw = dict(chunk_size=128, D=D, dt_bias=db, dt_min=o["dt_min"], dt_max=o["dt_max"])
    st_ref = torch.empty((1, 4, 32, 64), dtype=torch.float32, device=DEV)
    out_ref = ssm.chunk_scan_fwd(x, dtr, A, B, C, state_out=st_ref, out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream(DEV)
    st = torch.empty_like(st_ref)
    out = torch.empty_like(out_ref)
    call = ssm.chunk_scan_fwd(x, dtr, A, B, C, state_out=st, out=out, stream=stream, prepare=True, **kw)
    g = _capture(call, stream)
    for _ in range(3):
        out.fill_(float("nan"))
        st.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, out_ref) and torch.equal(st, st_ref)


def test_chunk_scan_gated_ragged_graph_replays():
    w = W.ssd_long(seqlen=300, nheads=4, headdim=32, gated=True)
    o = w.opts
    x, dtr, A, B, C, D, db, z = (dev_tensor(w, k) for k in ("x", "dt", "A", "B", "C", "D", "dt_bias", "z"))
    kw = dict(chunk_size=128, D=D, dt_bias=db, dt_min=o["dt_min"], dt_max=o["dt_max"], z=z)
    st_ref = torch.empty((1, 4, 32, 64), dtype=torch.float32, device=DEV)
    out_ref = ssm.chunk_scan_fwd(x, dtr, A, B, C, state_out=st_ref, out_dtype=torch.bfloat16, **kw)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream(DEV)
    st = torch.empty_like(st_ref)
    out = torch.empty_like(out_ref)
    call = ssm.chunk_scan_fwd(x, dtr, A, B, C, state_out=st, out=out, stream=stream, prepare=True, **kw)
    g = _capture(call, stream)
    for _ in range(3):
        out.fill_(float("nan"))
        st.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, out_ref) and torch.equal(st, st_ref)


def test_chunk_decode_graph_replays():
    w = W.ssd_decode(batch=4, nheads=8, headdim=32, ngroups=2, d_state=64, gated=True)
    o = w.opts
    tok = lambda k: dev_tensor(w, k)[:, 0].contiguous()
    x, dtr, B, C, z = (tok(k) for k in ("x", "dt", "B", "C", "z"))
    A, D, db = (dev_tensor(w, k) for k in ("A", "D", "dt_bias"))
    st0 = torch.from_numpy(w.arrays["state0"]).to(DEV)
    kw = dict(D=D, dt_bias=db, dt_min=o["dt_min"], dt_max=o["dt_max"], z=z)
    st_ref = st0.clone()
    out_ref = ssm.chunk_decode_step(x, dtr, A, B, C, st_ref, out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream(DEV)
    st = st0.clone()
    out = torch.empty_like(out_ref)
    call = ssm.chunk_decode_step(x, dtr, A, B, C, st, out=out, stream=stream, prepare=True, **kw)
    g = _capture(call, stream)
    for _ in range(3):
        st.copy_(st0)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, out_ref) and torch.equal(st, st_ref)
