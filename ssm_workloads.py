"""Seeded synthetic inputs for the selective-scan path.

This module only draws random numbers and stores them in the dtypes of the
workloads (fp32, or bf16 rounded to nearest-even and kept as uint16 bit
patterns).  It holds none of the method's arithmetic: no softplus, clip, conv,
decay or scan.  The tests and the benchmark call it; both the float64 oracle
and the HIP path then consume the very same arrays.

Recipes (one numpy Generator(PCG64(seed)) per workload, float32 normal draws,
drawn in the order listed in each function):

* scan_tiny          batch 1, L 64, E 16, N 16, fp32, rank-1 dt, no conv.
* scan_prefill       Bit-Axon layer prefill: batch 1, L 2048, E 7680, N 16,
                     bf16 x/z, conv1d k=4, rank-1 dt, bf16 B/C.
* scan_bulk          batch 8, L 4096, E 7680, N 16, bf16 u/dt/z (E-wide) and B/C.
* decode_stream      batch 64, E 7680, N 16, fp32, 256 prefill + 1024 decode tokens.
* ssd_long           batch 1, L 65536, 80 heads x 96, 1 group, N 64, chunk 128.

Every size can be overridden so the tests can run the same recipe at sizes the
oracle finishes in seconds.  `unsaturated=True` shifts the dt pre-activation
down (bias ~ N(-4, 1), raw values x2) so softplus and both clip edges are
exercised instead of nearly every dt sitting on the upper clip.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

DT_MIN = np.float32(1e-3)
DT_MAX = np.float32(0.1)
CONV_K = 4


def bf16_bits(a) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    """A named set of arrays.  Names in `bf16` hold uint16 bf16 bit patterns; all
    other arrays are float32.  `opts` carries the scalar settings (dt clip
    bounds, softplus on/off, chunk size, ...)."""
    name: str
    kind: str
    dims: dict
    arrays: dict
    bf16: set = field(default_factory=set)
    opts: dict = field(default_factory=dict)

    def f64(self, key):
        """The array widened to float64 (exact for fp32 and bf16)."""
        a = self.arrays.get(key)
        if a is None:
            return None
        if key in self.bf16:
            return bf16_to_f32(a).astype(np.float64)
        return np.asarray(a, dtype=np.float64)


def _normal(rng, shape, std=1.0, mean=0.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return x


def _diag_a(dim, d_state):
    """A for every channel: the diagonal -1 .. -d_state that A = -exp(A_log) takes
    at the A_log = log(1..d_state) initialisation, stored exactly in fp32."""
    row = -np.arange(1, d_state + 1, dtype=np.float32)
    return np.ascontiguousarray(np.broadcast_to(row, (dim, d_state)))


A_INITS = ("diag", "log_init", "random")


def _a_matrix(rng, dim, d_state, a_init):
    """A (dim, d_state) fp32 in one of three forms:
    diag      -1 .. -d_state stored exactly (the A_log = log(1..N) initialisation);
    log_init  the same initialisation as a model stores it: A_log = log(1..N) and
              A = -exp(A_log), both rounded to fp32 (several entries then differ
              from -(n+1) in the last bit, as a trained or loaded A does);
    random    A_log ~ U[0, ln 16] drawn per (channel, state), A = -exp(A_log) in
              fp32: no structure shared across channels or states.
    Only `random` draws from rng (after every other draw of the workload)."""
    if a_init == "diag":
        return _diag_a(dim, d_state)
    if a_init == "log_init":
        a_log = np.log(np.arange(1, d_state + 1, dtype=np.float32)).astype(np.float32)
        row = (-np.exp(a_log)).astype(np.float32)
        return np.ascontiguousarray(np.broadcast_to(row, (dim, d_state)))
    if a_init == "random":
        a_log = rng.uniform(0.0, np.log(16.0), (dim, d_state)).astype(np.float32)
        return (-np.exp(a_log)).astype(np.float32)
    raise ValueError(f"a_init must be one of {A_INITS}, got {a_init!r}")


def scan_tiny(batch=1, seqlen=64, dim=16, d_state=16, seed=1, unsaturated=False):
    """Tiny fp32 scan.  Draws: u, z, B, C ~ N(0,1); D ~ N(0,1); r ~ N(0,1) (batch, L);
    w_dt, b_dt ~ N(0, 0.5).  dt = clip(softplus(w_dt * r + b_dt), 1e-3, 0.1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    u = _normal(rng, (batch, seqlen, dim))
    z = _normal(rng, (batch, seqlen, dim))
    B = _normal(rng, (batch, seqlen, d_state))
    C = _normal(rng, (batch, seqlen, d_state))
    D = _normal(rng, (dim,))
    r = _normal(rng, (batch, seqlen))
    w_dt = _normal(rng, (dim,), 0.5)
    b_dt = _normal(rng, (dim,), 0.5)
    if unsaturated:
        r *= np.float32(2.0)
        b_dt = _normal(rng, (dim,), 1.0, -4.0)
    return Workload(
        "scan_tiny" + ("_unsat" if unsaturated else ""), "scan",
        dict(batch=batch, seqlen=seqlen, dim=dim, d_state=d_state),
        dict(x=u, z=z, B=B, C=C, D=D, dt=r, dt_w=w_dt, dt_bias=b_dt, A=_diag_a(dim, d_state)),
        set(), dict(dt_rank1=True, dt_softplus=True, dt_min=DT_MIN, dt_max=DT_MAX, conv=False))


def scan_prefill(batch=1, seqlen=2048, dim=7680, d_state=16, seed=2, unsaturated=False, a_init="diag"):
    """Bit-Axon SSM layer prefill.  Draws: x_branch, z ~ N(0,1) -> bf16 (batch, L, E);
    conv_w ~ N(0, 0.5) (E, 4) fp32, no bias; B, C ~ N(0,1) -> bf16 (batch, L, N);
    r ~ N(0,1) fp32 (batch, L); w_dt, b_dt ~ N(0, 0.5) (E); D ~ N(0,1) (E).
    Zero ssm_state and conv_cache in.  a_init: see _a_matrix."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = bf16_bits(_normal(rng, (batch, seqlen, dim)))
    z = bf16_bits(_normal(rng, (batch, seqlen, dim)))
    conv_w = _normal(rng, (dim, CONV_K), 0.5)
    B = bf16_bits(_normal(rng, (batch, seqlen, d_state)))
    C = bf16_bits(_normal(rng, (batch, seqlen, d_state)))
    r = _normal(rng, (batch, seqlen))
    w_dt = _normal(rng, (dim,), 0.5)
    b_dt = _normal(rng, (dim,), 0.5)
    D = _normal(rng, (dim,))
    if unsaturated:
        r *= np.float32(2.0)
        b_dt = _normal(rng, (dim,), 1.0, -4.0)
    A = _a_matrix(rng, dim, d_state, a_init)
    return Workload(
        "scan_prefill" + ("_unsat" if unsaturated else "") + ("" if a_init == "diag" else "_" + a_init), "scan",
        dict(batch=batch, seqlen=seqlen, dim=dim, d_state=d_state),
        dict(x=x, z=z, conv_w=conv_w, B=B, C=C, dt=r, dt_w=w_dt, dt_bias=b_dt, D=D, A=A),
        {"x", "z", "B", "C"},
        dict(dt_rank1=True, dt_softplus=True, dt_min=DT_MIN, dt_max=DT_MAX, conv=True))


def scan_bulk(batch=8, seqlen=4096, dim=7680, d_state=16, seed=3, unsaturated=False, a_init="diag"):
    """Bandwidth-bound bulk scan.  Draws: u, z ~ N(0,1) -> bf16 (batch, L, E);
    dt_raw ~ N(0, 0.5) -> bf16 (batch, L, E) (E-wide, the dt_proj output);
    dt_bias ~ N(0, 0.5) (E); B, C ~ N(0,1) -> bf16 (batch, L, N); D ~ N(0,1) (E).
    dt = clip(softplus(dt_raw + dt_bias), 1e-3, 0.1) is formed by the consumer.
    a_init: see _a_matrix."""
    rng = np.random.Generator(np.random.PCG64(seed))
    u = bf16_bits(_normal(rng, (batch, seqlen, dim)))
    z = bf16_bits(_normal(rng, (batch, seqlen, dim)))
    dt_scale = 1.0 if unsaturated else 0.5
    dt = bf16_bits(_normal(rng, (batch, seqlen, dim), dt_scale))
    b_dt = _normal(rng, (dim,), 0.5)
    B = bf16_bits(_normal(rng, (batch, seqlen, d_state)))
    C = bf16_bits(_normal(rng, (batch, seqlen, d_state)))
    D = _normal(rng, (dim,))
    if unsaturated:
        b_dt = _normal(rng, (dim,), 1.0, -4.0)
    A = _a_matrix(rng, dim, d_state, a_init)
    return Workload(
        "scan_bulk" + ("_unsat" if unsaturated else "") + ("" if a_init == "diag" else "_" + a_init), "scan",
        dict(batch=batch, seqlen=seqlen, dim=dim, d_state=d_state),
        dict(x=u, z=z, dt=dt, dt_bias=b_dt, B=B, C=C, D=D, A=A),
        {"x", "z", "dt", "B", "C"},
        dict(dt_rank1=False, dt_softplus=True, dt_min=DT_MIN, dt_max=DT_MAX, conv=False))


def decode_stream(batch=64, dim=7680, d_state=16, prefill=256, steps=1024, seed=4, unsaturated=False):
    """Batched decode.  Draws: conv_w ~ N(0, 0.5) (E, 4); w_dt, b_dt ~ N(0, 0.5) (E);
    D ~ N(0,1) (E); then per token t (prefill and decode alike): x_t, z_t ~ N(0,1)
    (batch, E); r_t ~ N(0,1) (batch); B_t, C_t ~ N(0,1) (batch, N).  All fp32.
    Arrays are stored token-major: x (T, batch, E), r (T, batch), B (T, batch, N)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    T = prefill + steps
    conv_w = _normal(rng, (dim, CONV_K), 0.5)
    w_dt = _normal(rng, (dim,), 0.5)
    b_dt = _normal(rng, (dim,), 0.5)
    D = _normal(rng, (dim,))
    if unsaturated:
        b_dt = _normal(rng, (dim,), 1.0, -4.0)
    x = np.empty((T, batch, dim), np.float32)
    z = np.empty((T, batch, dim), np.float32)
    r = np.empty((T, batch), np.float32)
    B = np.empty((T, batch, d_state), np.float32)
    C = np.empty((T, batch, d_state), np.float32)
    for t in range(T):
        x[t] = _normal(rng, (batch, dim))
        z[t] = _normal(rng, (batch, dim))
        r[t] = _normal(rng, (batch,), 2.0 if unsaturated else 1.0)
        B[t] = _normal(rng, (batch, d_state))
        C[t] = _normal(rng, (batch, d_state))
    return Workload(
        "decode_stream" + ("_unsat" if unsaturated else ""), "decode",
        dict(batch=batch, dim=dim, d_state=d_state, prefill=prefill, steps=steps),
        dict(x=x, z=z, dt=r, B=B, C=C, conv_w=conv_w, dt_w=w_dt, dt_bias=b_dt, D=D,
             A=_diag_a(dim, d_state)),
        set(),
        dict(dt_rank1=True, dt_softplus=True, dt_min=DT_MIN, dt_max=DT_MAX, conv=True,
             token_major=True))


def ssd_long(batch=1, seqlen=65536, nheads=80, headdim=96, ngroups=1, d_state=64, chunk_size=128,
             seed=5, unsaturated=False, gated=False):
    """Long-context chunked SSD.  Draws: x ~ N(0,1) -> bf16 (batch, L, H, P);
    B, C ~ N(0,1) -> bf16 (batch, L, G, N); A_log ~ U[0, ln 16] (H) with
    A = -exp(A_log) stored in fp32; dt_raw ~ N(0,1) fp32 (batch, L, H);
    dt_bias ~ N(0, 0.5) (H); D ~ N(0,1) (H); with gated, last, a gate
    z ~ N(0,1) -> bf16 (batch, L, H, P).  Zero initial state."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = bf16_bits(_normal(rng, (batch, seqlen, nheads, headdim)))
    B = bf16_bits(_normal(rng, (batch, seqlen, ngroups, d_state)))
    C = bf16_bits(_normal(rng, (batch, seqlen, ngroups, d_state)))
    A = (-np.exp(rng.uniform(0.0, np.log(16.0), nheads))).astype(np.float32)
    dt_raw = _normal(rng, (batch, seqlen, nheads), 2.0 if unsaturated else 1.0)
    b_dt = _normal(rng, (nheads,), 1.0, -4.0) if unsaturated else _normal(rng, (nheads,), 0.5)
    D = _normal(rng, (nheads,))
    arrays = dict(x=x, B=B, C=C, A=A, dt=dt_raw, dt_bias=b_dt, D=D)
    if gated:
        arrays["z"] = bf16_bits(_normal(rng, (batch, seqlen, nheads, headdim)))
    return Workload(
        "ssd_long" + ("_unsat" if unsaturated else "") + ("_gated" if gated else ""), "ssd",
        dict(batch=batch, seqlen=seqlen, nheads=nheads, headdim=headdim, ngroups=ngroups,
             d_state=d_state, chunk_size=chunk_size),
        arrays,
        {"x", "B", "C", "z"} if gated else {"x", "B", "C"},
        dict(dt_softplus=True, dt_min=DT_MIN, dt_max=DT_MAX))


def ssd_decode(batch=64, nheads=80, headdim=96, ngroups=1, d_state=64, steps=1, seed=9, gated=False,
               unsaturated=True):
    """Batched decode steps of the multi-head scan: the draws of ssd_long with
    L = steps tokens per sequence (x, B, C, z in bf16; dt_raw, dt_bias, A, D in
    fp32), plus a starting state state0 ~ N(0,1) fp32 (batch, H, P, N) from a
    generator of its own (seed + 1)."""
    w = ssd_long(batch=batch, seqlen=steps, nheads=nheads, headdim=headdim, ngroups=ngroups, d_state=d_state,
                 seed=seed, unsaturated=unsaturated, gated=gated)
    rng = np.random.Generator(np.random.PCG64(seed + 1))
    w.arrays["state0"] = _normal(rng, (batch, nheads, headdim, d_state))
    w.name = "ssd_decode" + ("_gated" if gated else "")
    return w


def layer_prefill(batch=1, seqlen=2048, d_model=2560, dim=7680, d_state=16, seed=11):
    """The whole Axon-SSM layer forward with random weights of the page's shapes
    (D 2560, E 7680, N 16).  Draws, in order: hidden ~ N(0,1) -> bf16
    (batch, L, D); W_in ~ N(0,1)/sqrt(D) -> bf16 (2E, D); conv_w ~ N(0,0.5)
    (E, 4); W_x ~ N(0,1)/sqrt(E) -> bf16 (2N+1, E); dt_w ~ N(0,0.5) (E);
    dt_bias ~ N(0,0.5) (E); D ~ N(0,1) (E); W_out ~ N(0,1)/sqrt(E) -> bf16
    (D, E).  A = -(1..N) per channel; zero state and conv cache."""
    rng = np.random.Generator(np.random.PCG64(seed))
    hidden = bf16_bits(_normal(rng, (batch, seqlen, d_model)))
    W_in = bf16_bits(_normal(rng, (2 * dim, d_model), 1.0 / np.sqrt(d_model)))
    conv_w = _normal(rng, (dim, 4), 0.5)
    W_x = bf16_bits(_normal(rng, (2 * d_state + 1, dim), 1.0 / np.sqrt(dim)))
    dt_w = _normal(rng, (dim,), 0.5)
    dt_bias = _normal(rng, (dim,), 0.5)
    D = _normal(rng, (dim,))
    W_out = bf16_bits(_normal(rng, (d_model, dim), 1.0 / np.sqrt(dim)))
    A = -np.tile(np.arange(1, d_state + 1, dtype=np.float32), (dim, 1))
    return Workload(
        "layer_prefill", "layer",
        dict(batch=batch, seqlen=seqlen, d_model=d_model, dim=dim, d_state=d_state),
        dict(hidden=hidden, W_in=W_in, conv_w=conv_w, W_x=W_x, dt_w=dt_w, dt_bias=dt_bias, D=D, W_out=W_out, A=A),
        {"hidden", "W_in", "W_x", "W_out"},
        dict(dt_softplus=True, dt_min=DT_MIN, dt_max=DT_MAX))
