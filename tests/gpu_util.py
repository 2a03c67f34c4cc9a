"""Helpers shared by the GPU parity tests: move a seeded workload to the GPU,
call the HIP path through the binding, call the float64 oracle on the same
arrays (optionally on a sample of channels), and compare."""
from __future__ import annotations

import numpy as np
import torch

import selective_state_space_03_amd as ssm
import ssm_workloads as W
from oracle import ssm_oracle as O

DEV = torch.device("cuda:0")


def dev_tensor(w: W.Workload, key: str, device=DEV):
    a = w.arrays.get(key)
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if not a.flags.writeable:  # torch wants a writable source even for a copy to the device
        a = a.copy()
    if key in w.bf16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def check(got, want, tol, what, out_bf16=False):
    """max |got - want| <= tol * max|want| (+ 2^-8 |want_i| when the output was
    rounded to bf16, the rounding bound of the storage format itself)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values in the GPU result"
    if want.size == 0:
        return 0.0
    scale = float(np.max(np.abs(want)))
    err = np.abs(got - want)
    bound = tol * scale + (2.0 ** -8 * np.abs(want) if out_bf16 else 0.0)
    worst = float(np.max(err - bound))
    assert worst <= 0.0, (f"{what}: max|err| {float(np.max(err)):.3e} exceeds bound "
                          f"(tol {tol:g} * max|ref| {scale:.3e}); worst excess {worst:.3e}")
    return float(np.max(err)) / max(scale, 1e-300)


# ---------------------------------------------------------------------- scan

def scan_gpu(w: W.Workload, *, y_dtype=torch.float32, time_split=0, state_in=None, cache_in=None,
             want_state=True, want_cache=True, y_fill=None, discretization="euler"):
    o = w.opts
    d = w.dims
    Bt, E, N = d["batch"], d["dim"], d["d_state"]
    st = torch.empty((Bt, E, N), dtype=torch.float32, device=DEV) if want_state else None
    cc = torch.empty((Bt, E, 3), dtype=torch.float32, device=DEV) if (want_cache and o["conv"]) else None
    y = None
    if y_fill is not None:
        y = torch.full((Bt, d["seqlen"], E), y_fill, dtype=y_dtype, device=DEV)
    y = ssm.scan_fwd(
        dev_tensor(w, "x"), dev_tensor(w, "A"), dev_tensor(w, "B"), dev_tensor(w, "C"), dev_tensor(w, "dt"),
        D=dev_tensor(w, "D"), z=dev_tensor(w, "z"), conv_w=dev_tensor(w, "conv_w") if o["conv"] else None,
        conv_cache_in=cache_in, conv_cache_out=cc, dt_rank1=o["dt_rank1"], dt_w=dev_tensor(w, "dt_w"),
        dt_bias=dev_tensor(w, "dt_bias"), dt_softplus=o["dt_softplus"], dt_min=o["dt_min"], dt_max=o["dt_max"],
        ssm_state_in=state_in, ssm_state_out=st, y=y, y_dtype=y_dtype, time_split=time_split,
        discretization=discretization)
    torch.cuda.synchronize()
    return y, st, cc


def _sel(a, batches, channels, axis_e):
    if a is None:
        return None
    if batches is not None:
        a = a[batches]
    if channels is not None:
        a = np.take(a, channels, axis=axis_e)
    return a


def scan_oracle(w: W.Workload, *, state_in=None, cache_in=None, batches=None, channels=None,
                discretization="euler"):
    """Oracle on (a sample of) the workload: batches / channels index lists.
    Channels of the diagonal scan are independent, so a sample is exact."""
    o = w.opts
    f = w.f64
    x = _sel(f("x"), batches, channels, 2)
    z = _sel(f("z"), batches, channels, 2)
    B = _sel(f("B"), batches, None, 2)
    C = _sel(f("C"), batches, None, 2)
    ch = (lambda v: v if channels is None or v is None else v[channels])
    if o["dt_rank1"]:
        dt_kw = dict(dt_raw=_sel(f("dt"), batches, None, 1), dt_w=ch(f("dt_w")))
    else:
        dt_kw = dict(dt=_sel(f("dt"), batches, channels, 2))
    sti = _sel(state_in, batches, channels, 1) if state_in is not None else None
    cci = _sel(cache_in, batches, channels, 1) if cache_in is not None else None
    return O.ssm_layer_scan(
        x, ch(f("A")), B, C, D=ch(f("D")), z=z, conv_w=ch(f("conv_w")) if o["conv"] else None,
        conv_cache=cci, dt_bias=ch(f("dt_bias")), dt_softplus=o["dt_softplus"], dt_min=float(o["dt_min"]),
        dt_max=float(o["dt_max"]), ssm_state=sti, discretization=discretization, **dt_kw)


# ---------------------------------------------------------------------- SSD

def ssd_gpu(w: W.Workload, *, out_dtype=torch.float32, state_in=None, want_state=True, D_override=None,
            z_f32=False, segments=0):
    """The workload's gate z (when it has one) goes in as bf16, or as its fp32
    widening with z_f32."""
    d = w.dims
    o = w.opts
    st = (torch.empty((d["batch"], d["nheads"], d["headdim"], d["d_state"]), dtype=torch.float32, device=DEV)
          if want_state else None)
    D = dev_tensor(w, "D") if D_override is None else torch.from_numpy(D_override).to(DEV)
    z = None
    if "z" in w.arrays:
        z = dev_tensor(w, "z")
        if z_f32:
            z = z.float()
    out = ssm.chunk_scan_fwd(dev_tensor(w, "x"), dev_tensor(w, "dt"), dev_tensor(w, "A"), dev_tensor(w, "B"),
                             dev_tensor(w, "C"), chunk_size=d["chunk_size"], D=D, dt_bias=dev_tensor(w, "dt_bias"),
                             dt_softplus=o["dt_softplus"], dt_min=o["dt_min"], dt_max=o["dt_max"],
                             state_in=state_in, state_out=st, out_dtype=out_dtype, z=z, segments=segments)
    torch.cuda.synchronize()
    return out, st


def ssd_oracle(w: W.Workload, *, heads=None, state_in=None, D_override=None, sequential=False):
    """Oracle on (a sample of) the heads; heads are independent given B, C."""
    o = w.opts
    f = w.f64
    hs = slice(None) if heads is None else heads
    x = f("x")[:, :, hs]
    bias = f("dt_bias")
    dt = O.compute_dt(f("dt")[:, :, hs], None if bias is None else bias[hs], float(o["dt_min"]),
                      float(o["dt_max"]), use_softplus=o["dt_softplus"])
    A = f("A")[hs]
    D = (f("D") if D_override is None else np.asarray(D_override, np.float64))[hs]
    Bm, Cm = f("B"), f("C")
    H = w.dims["nheads"]
    G = w.dims["ngroups"]
    if heads is not None and G > 1:  # keep each sampled head's own group
        grp = np.asarray(heads) // (H // G)
        Bm, Cm = Bm[:, :, grp], Cm[:, :, grp]
    st = None if state_in is None else np.asarray(state_in, np.float64)[:, hs]
    z = f("z")[:, :, hs] if "z" in w.arrays else None
    if sequential:
        return O.ssd_scan_sequential(x, dt, A, Bm, Cm, D=D, state=st, z=z)
    return O.ssd_chunk_scan(x, dt, A, Bm, Cm, D=D, state=st, chunk_size=w.dims["chunk_size"], z=z)


# ---------------------------------------------------------------------- SSD decode

def ssd_decode_gpu(w: W.Workload, state, t=0, *, out_dtype=torch.float32, x_f32=False, bc_f32=False, z_f32=False,
                   D_override=None, stream=None):
    """One ssm_chunk_decode_step on token t of the workload; state (Bt, H, P, N)
    fp32 on the device is updated in place.  x / B, C / z go in as bf16 or
    widened to fp32."""
    o = w.opts

    def tok(key, f32):
        a = dev_tensor(w, key)
        if a is None:
            return None
        a = a[:, t].contiguous()
        return a.float() if f32 else a

    D = dev_tensor(w, "D") if D_override is None else torch.from_numpy(D_override).to(DEV)
    out = ssm.chunk_decode_step(tok("x", x_f32), tok("dt", False), dev_tensor(w, "A"), tok("B", bc_f32),
                                tok("C", bc_f32), state, D=D, dt_bias=dev_tensor(w, "dt_bias"),
                                dt_softplus=o["dt_softplus"], dt_min=o["dt_min"], dt_max=o["dt_max"],
                                z=tok("z", z_f32), out_dtype=out_dtype, stream=stream)
    return out


# ---------------------------------------------------------------------- layer

def layer_gpu(w: W.Workload, *, tokens=None, out_dtype=torch.float32, cache_in=None, state_in=None,
              want_state=True, want_cache=True):
    """ssm_layer_fwd on the workload's hidden states [:, tokens] (all when None)."""
    d = w.dims
    o = w.opts
    hidden = dev_tensor(w, "hidden")
    if tokens is not None:
        hidden = hidden[:, tokens].contiguous()
    Bt, E, N = d["batch"], d["dim"], d["d_state"]
    st = torch.empty((Bt, E, N), dtype=torch.float32, device=DEV) if want_state else None
    cc = torch.empty((Bt, E, 3), dtype=torch.float32, device=DEV) if want_cache else None
    out = ssm.layer_fwd(hidden, dev_tensor(w, "W_in"), dev_tensor(w, "conv_w"), dev_tensor(w, "W_x"),
                        dev_tensor(w, "dt_w"), dev_tensor(w, "A"), dev_tensor(w, "W_out"),
                        dt_bias=dev_tensor(w, "dt_bias"), D=dev_tensor(w, "D"), conv_cache_in=cache_in,
                        conv_cache_out=cc, ssm_state_in=state_in, ssm_state_out=st, dt_softplus=o["dt_softplus"],
                        dt_min=o["dt_min"], dt_max=o["dt_max"], out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, st, cc


def layer_oracle(w: W.Workload, *, tokens=None, cache_in=None, state_in=None):
    o = w.opts
    f = w.f64
    hidden = f("hidden")
    if tokens is not None:
        hidden = hidden[:, tokens]
    return O.ssm_layer_forward(hidden, f("W_in"), f("conv_w"), f("W_x"), f("dt_w"), f("dt_bias"), f("A"),
                               f("W_out"), D=f("D"), conv_cache=cache_in, ssm_state=state_in,
                               dt_softplus=o["dt_softplus"], dt_min=float(o["dt_min"]), dt_max=float(o["dt_max"]))


# ---------------------------------------------------------------------- scan backward

def scan_bwd_gpu(w: W.Workload, dy, *, state_in=None, cache_in=None, dstate_out=None):
    """ssm_scan_bwd on the workload with the upstream gradient dy (numpy, fp32)."""
    o = w.opts
    tt = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)  # noqa
    g = ssm.scan_bwd(
        dev_tensor(w, "x"), dev_tensor(w, "A"), dev_tensor(w, "B"), dev_tensor(w, "C"), dev_tensor(w, "dt"), tt(dy),
        D=dev_tensor(w, "D"), z=dev_tensor(w, "z"), conv_w=dev_tensor(w, "conv_w") if o["conv"] else None,
        conv_cache_in=tt(cache_in), dt_rank1=o["dt_rank1"], dt_w=dev_tensor(w, "dt_w"),
        dt_bias=dev_tensor(w, "dt_bias"), dt_softplus=o["dt_softplus"], dt_min=o["dt_min"], dt_max=o["dt_max"],
        ssm_state_in=tt(state_in), dstate_out=tt(dstate_out))
    torch.cuda.synchronize()
    return {k: np64(v) for k, v in g.items()}


def scan_bwd_oracle(w: W.Workload, dy, *, state_in=None, cache_in=None, dstate_out=None):
    o = w.opts
    f = w.f64
    kw = dict(D=f("D"), z=f("z"), conv_w=f("conv_w") if o["conv"] else None, conv_cache=cache_in,
              dt_bias=f("dt_bias"), dt_softplus=o["dt_softplus"], dt_min=float(o["dt_min"]),
              dt_max=float(o["dt_max"]), ssm_state=state_in, dstate_out=dstate_out)
    if o["dt_rank1"]:
        kw.update(dt_raw=f("dt"), dt_w=f("dt_w"))
    else:
        kw.update(dt=f("dt"))
    g = O.ssm_layer_scan_backward(f("x"), f("A"), f("B"), f("C"), np.asarray(dy, np.float64), **kw)
    # name the rank-1 input's gradient like the GPU side ("dt" is the input r there)
    if o["dt_rank1"]:
        g["dt"] = g.pop("dt_raw")
    return {k: v for k, v in g.items() if v is not None}
