"""Pins for the float64 oracle: checks against what the pages and the mathematics
fix, written independently of the oracle's own code paths.

Each `pin_*` takes the oracle module and raises AssertionError when the oracle
disagrees.  test_oracle_pins.py runs them on the real oracle;
test_oracle_mutations.py runs them on copies of the oracle with a planted
mistake and requires that some pin fails for every mistake.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"{what}: max|err| {err:.3e} > {tol:.1e} * {scale:.3e}"


def _sig(v):
    return 1.0 / (1.0 + math.exp(-v)) if v >= 0 else math.exp(v) / (1.0 + math.exp(v))


# ---------------------------------------------------------------------------
# Q1: brute-force unrolled product-sum (velog "Mamba computation")
# ---------------------------------------------------------------------------

def pin_unrolled_product_sum(orc):
    """h_t = (A_t...A_1) h_0 + sum_j (A_t...A_{j+1}) B_j x_j evaluated literally
    with explicit products in pure Python, then y_t = C_t . h_t + D u_t, gated."""
    rng = _rng(101)
    Bt, L, E, N = 2, 9, 3, 4
    u = rng.standard_normal((Bt, L, E))
    dt = rng.uniform(0.01, 0.5, (Bt, L, E))
    A = -rng.uniform(0.2, 3.0, (E, N))
    Bm = rng.standard_normal((Bt, L, N))
    Cm = rng.standard_normal((Bt, L, N))
    D = rng.standard_normal(E)
    z = rng.standard_normal((Bt, L, E))
    h0 = rng.standard_normal((Bt, E, N))
    y, hL = orc.selective_scan(u, dt, A, Bm, Cm, D=D, z=z, ssm_state=h0)
    for b in range(Bt):
        for e in range(E):
            for t in range(L):
                acc = 0.0
                hs = []
                for n in range(N):
                    prod0 = 1.0
                    for i in range(t + 1):
                        prod0 *= math.exp(dt[b, i, e] * A[e, n])
                    h = prod0 * h0[b, e, n]
                    for j in range(t + 1):
                        prod = 1.0
                        for i in range(j + 1, t + 1):
                            prod *= math.exp(dt[b, i, e] * A[e, n])
                        h += prod * dt[b, j, e] * Bm[b, j, n] * u[b, j, e]
                    hs.append(h)
                    acc += Cm[b, t, n] * h
                acc += D[e] * u[b, t, e]
                acc *= z[b, t, e] * _sig(z[b, t, e])
                assert abs(acc - y[b, t, e]) <= 1e-12 * max(1.0, abs(acc)), (b, t, e, acc, y[b, t, e])
                if t == L - 1:
                    for n in range(N):
                        assert abs(hs[n] - hL[b, e, n]) <= 1e-12 * max(1.0, abs(hs[n]))


# ---------------------------------------------------------------------------
# Q2: recurrence == convolution for a fixed SSM (ultralytics glossary, "How SSMs work")
# ---------------------------------------------------------------------------

def _lti_conv(x, A_bar, B_bar, C):
    L = len(x)
    K = np.array([float(np.dot(C, (A_bar ** k) * B_bar)) for k in range(L)])
    return np.array([float(np.dot(K[: t + 1][::-1], x[: t + 1])) for t in range(L)])


def pin_recurrence_equals_convolution(orc):
    g = _golden("p4_recurrence_vs_convolution.json")
    L, N, delta = g["seq_len"], g["d_state"], g["delta"]
    rng = _rng(102)
    x = rng.standard_normal(L)
    A = -(rng.uniform(0.0, 1.0, N) + 0.5)
    B = rng.standard_normal(N)
    C = rng.standard_normal(N)
    A_bar = np.exp(delta * A)
    u = x.reshape(1, L, 1)
    dt = np.full((1, L, 1), delta)
    Bs = np.broadcast_to(B, (1, L, N))
    Cs = np.broadcast_to(C, (1, L, N))
    # zero-order hold B_bar, the page's own setting; the page prints allclose(atol) == True
    y_rec, _ = orc.selective_scan(u, dt, A.reshape(1, N), Bs, Cs, discretization="zoh")
    y_conv = _lti_conv(x, A_bar, (A_bar - 1.0) / A * B, C)
    assert bool(np.allclose(y_rec[0, :, 0], y_conv, atol=g["atol"])) == g["printed_result"]
    _close(y_rec[0, :, 0], y_conv, 1e-12, "zoh recurrence vs convolution")
    # the Euler form of B used by the scan path: B_bar = delta * B
    y_rec_e, _ = orc.selective_scan(u, dt, A.reshape(1, N), Bs, Cs)
    _close(y_rec_e[0, :, 0], _lti_conv(x, A_bar, delta * B, C), 1e-12, "euler recurrence vs convolution")


# ---------------------------------------------------------------------------
# Q3: geometric-series closed form for constant input
# ---------------------------------------------------------------------------

def pin_constant_input_closed_form(orc):
    L, N = 40, 6
    dt, uval = 0.07, 1.3
    A = -np.arange(1, N + 1, dtype=np.float64) * 0.8
    B = np.linspace(-1.0, 2.0, N)
    C = np.linspace(0.5, -1.5, N)
    y, h = orc.selective_scan(np.full((1, L, 1), uval), np.full((1, L, 1), dt), A.reshape(1, N),
                              np.broadcast_to(B, (1, L, N)), np.broadcast_to(C, (1, L, N)))
    a = np.exp(dt * A)
    for t in range(L):
        ht = dt * B * uval * (1.0 - a ** (t + 1)) / (1.0 - a)
        _close(y[0, t, 0], np.dot(C, ht), 1e-12, f"closed form y_{t}")
    _close(h[0, 0], dt * B * uval * (1.0 - a ** L) / (1.0 - a), 1e-12, "closed form h_L")


# ---------------------------------------------------------------------------
# Q4: single step, with and without an initial state
# ---------------------------------------------------------------------------

def pin_single_step(orc):
    rng = _rng(104)
    Bt, E, N = 3, 5, 7
    u = rng.standard_normal((Bt, 1, E))
    dt = rng.uniform(0.001, 0.3, (Bt, 1, E))
    A = -rng.uniform(0.5, 8.0, (E, N))
    Bm = rng.standard_normal((Bt, 1, N))
    Cm = rng.standard_normal((Bt, 1, N))
    D = rng.standard_normal(E)
    z = rng.standard_normal((Bt, 1, E))
    gate = z[:, 0] / (1.0 + np.exp(-z[:, 0]))
    y, _ = orc.selective_scan(u, dt, A, Bm, Cm, D=D, z=z)
    want = (dt[:, 0] * u[:, 0] * np.sum(Cm[:, 0] * Bm[:, 0], axis=-1)[:, None] + D * u[:, 0]) * gate
    _close(y[:, 0], want, 1e-13, "single step from zero")
    h0 = rng.standard_normal((Bt, E, N))
    y2, h1 = orc.selective_scan(u, dt, A, Bm, Cm, D=D, z=z, ssm_state=h0)
    hwant = np.exp(dt[:, 0, :, None] * A) * h0 + dt[:, 0, :, None] * Bm[:, 0, None, :] * u[:, 0, :, None]
    _close(h1, hwant, 1e-13, "single step state")
    _close(y2[:, 0], (np.einsum("ben,bn->be", hwant, Cm[:, 0]) + D * u[:, 0]) * gate, 1e-13, "single step y")


# ---------------------------------------------------------------------------
# Q5: chunked == sequential (chunkscan; SSD chunk formula; SSD == scan on E = H*P)
# ---------------------------------------------------------------------------

def pin_chunked_equals_sequential(orc):
    rng = _rng(105)
    Bt, L, E, N = 2, 23, 4, 5
    u = rng.standard_normal((Bt, L, E))
    dt = rng.uniform(0.001, 0.4, (Bt, L, E))
    A = -rng.uniform(0.3, 6.0, (E, N))
    Bm = rng.standard_normal((Bt, L, N))
    Cm = rng.standard_normal((Bt, L, N))
    D = rng.standard_normal(E)
    z = rng.standard_normal((Bt, L, E))
    h0 = rng.standard_normal((Bt, E, N))
    y, h = orc.selective_scan(u, dt, A, Bm, Cm, D=D, z=z, ssm_state=h0)
    for chunk in (1, 2, 3, 5, 8, 16, 23, 40):
        yc, hc = orc.selective_scan_chunked(u, dt, A, Bm, Cm, D=D, z=z, ssm_state=h0, chunk=chunk)
        _close(yc, y, 1e-12, f"chunked y chunk={chunk}")
        _close(hc, h, 1e-12, f"chunked h chunk={chunk}")


def _ssd_inputs(seed, Bt=2, L=32, H=4, P=3, G=2, N=5):
    rng = _rng(seed)
    x = rng.standard_normal((Bt, L, H, P))
    dt = rng.uniform(0.001, 0.5, (Bt, L, H))
    A = -rng.uniform(0.2, 9.0, H)
    Bm = rng.standard_normal((Bt, L, G, N))
    Cm = rng.standard_normal((Bt, L, G, N))
    D = rng.standard_normal(H)
    S0 = rng.standard_normal((Bt, H, P, N))
    return x, dt, A, Bm, Cm, D, S0


def pin_ssd_chunked_equals_sequential(orc):
    x, dt, A, Bm, Cm, D, S0 = _ssd_inputs(106)
    L = x.shape[1]
    out, S = orc.ssd_scan_sequential(x, dt, A, Bm, Cm, D=D, state=S0)
    for Q in (1, 2, 4, 8, 16, L):  # Q = L is the single quadratic (masked) form
        oc, Sc = orc.ssd_chunk_scan(x, dt, A, Bm, Cm, D=D, state=S0, chunk_size=Q)
        _close(oc, out, 1e-11, f"ssd chunked out Q={Q}")
        _close(Sc, S, 1e-11, f"ssd chunked state Q={Q}")


def pin_ssd_ragged_chunks(orc):
    """A sequence that is not a whole number of chunks (its last chunk shorter)
    gives the plain recurrence too, for lengths below, at and across chunk
    boundaries."""
    x, dt, A, Bm, Cm, D, S0 = _ssd_inputs(108, L=45)
    for L in (1, 7, 16, 17, 45):
        args = (x[:, :L], dt[:, :L], A, Bm[:, :L], Cm[:, :L])
        out, S = orc.ssd_scan_sequential(*args, D=D, state=S0)
        for Q in (4, 16, 32):
            oc, Sc = orc.ssd_chunk_scan(*args, D=D, state=S0, chunk_size=Q)
            _close(oc, out, 1e-11, f"ssd ragged out L={L} Q={Q}")
            _close(Sc, S, 1e-11, f"ssd ragged state L={L} Q={Q}")


def pin_ssd_gate(orc):
    """The gate multiplies the ungated output (D included) by SiLU(z) = z
    sigmoid(z), sigmoid from scipy's expit where available; z = 0 zeroes the
    output; the gate leaves the state alone; both forms agree."""
    x, dt, A, Bm, Cm, D, S0 = _ssd_inputs(109, L=20)
    z = _rng(110).standard_normal(x.shape) * 3.0
    try:
        from scipy.special import expit
    except ImportError:  # pragma: no cover
        expit = lambda v: 0.5 * (1.0 + np.tanh(0.5 * v))
    o0, S0s = orc.ssd_scan_sequential(x, dt, A, Bm, Cm, D=D, state=S0)
    og, Sg = orc.ssd_scan_sequential(x, dt, A, Bm, Cm, D=D, state=S0, z=z)
    _close(og, o0 * z * expit(z), 1e-12, "ssd gate = SiLU(z) factor")
    _close(Sg, S0s, 0.0, "ssd gate leaves the state")
    oz, _ = orc.ssd_scan_sequential(x, dt, A, Bm, Cm, D=D, state=S0, z=np.zeros_like(z))
    assert np.all(oz == 0.0), "z = 0 must zero the gated output"
    oc, _ = orc.ssd_chunk_scan(x, dt, A, Bm, Cm, D=D, state=S0, chunk_size=8, z=z)
    _close(oc, og, 1e-11, "ssd gate chunked vs sequential")


def pin_ssd_prefill_then_decode(orc):
    """Chunked prefill of the first T0 tokens, then one-token steps from the
    returned state, equal one pass over all tokens (outputs and final state)."""
    x, dt, A, Bm, Cm, D, S0 = _ssd_inputs(111, L=23)
    z = _rng(112).standard_normal(x.shape)
    full, Sf = orc.ssd_chunk_scan(x, dt, A, Bm, Cm, D=D, state=S0, chunk_size=8, z=z)
    T0 = 11
    o1, S = orc.ssd_chunk_scan(x[:, :T0], dt[:, :T0], A, Bm[:, :T0], Cm[:, :T0], D=D, state=S0, chunk_size=8,
                               z=z[:, :T0])
    outs = [o1]
    for t in range(T0, x.shape[1]):
        ot, S = orc.ssd_scan_sequential(x[:, t:t + 1], dt[:, t:t + 1], A, Bm[:, t:t + 1], Cm[:, t:t + 1], D=D,
                                        state=S, z=z[:, t:t + 1])
        outs.append(ot)
    _close(np.concatenate(outs, axis=1), full, 1e-11, "ssd prefill + decode out")
    _close(S, Sf, 1e-11, "ssd prefill + decode state")


def pin_ssd_equals_channel_scan(orc):
    """The multi-head scan is the diagonal scan on E = H*P channels whose
    d_state entries all decay with the head's scalar A and whose B, C are the
    head's group's."""
    x, dt, A, Bm, Cm, D, S0 = _ssd_inputs(107)
    Bt, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    out, S = orc.ssd_scan_sequential(x, dt, A, Bm, Cm, D=D, state=S0)
    hpg = H // G
    for h in range(H):
        g = h // hpg
        u = x[:, :, h, :]  # (Bt, L, P) -> P channels
        dth = np.repeat(dt[:, :, h, None], P, axis=2)
        Ah = np.full((P, N), A[h])
        yh, sh = orc.selective_scan(u, dth, Ah, Bm[:, :, g, :], Cm[:, :, g, :], D=np.full(P, D[h]),
                                    ssm_state=S0[:, h])
        _close(out[:, :, h, :], yh, 1e-12, f"ssd head {h} vs channel scan")
        _close(S[:, h], sh, 1e-12, f"ssd head {h} state vs channel scan")


# ---------------------------------------------------------------------------
# Q6: prefill + decode == prefill (Axon-SSM "Autoregressive decoding")
# ---------------------------------------------------------------------------

def _layer_inputs(seed, Bt=2, T=14, E=5, N=4, K=4):
    rng = _rng(seed)
    return dict(
        x=rng.standard_normal((Bt, T, E)), z=rng.standard_normal((Bt, T, E)),
        B=rng.standard_normal((Bt, T, N)), C=rng.standard_normal((Bt, T, N)),
        r=rng.standard_normal((Bt, T)), conv_w=rng.standard_normal((E, K)) * 0.5,
        conv_b=rng.standard_normal(E) * 0.1, dt_w=rng.standard_normal(E) * 0.5,
        dt_bias=rng.standard_normal(E) * 0.5 - 2.0, D=rng.standard_normal(E),
        A=-rng.uniform(0.5, 5.0, (E, N)))


def pin_prefill_then_decode(orc):
    p = _layer_inputs(108)
    T = p["x"].shape[1]
    common = dict(D=p["D"], conv_w=p["conv_w"], conv_b=p["conv_b"], dt_w=p["dt_w"],
                  dt_bias=p["dt_bias"], dt_softplus=True, dt_min=1e-3, dt_max=0.1)
    y_all, h_all, c_all = orc.ssm_layer_scan(p["x"], p["A"], p["B"], p["C"], z=p["z"], dt_raw=p["r"], **common)
    for L0 in (0, 1, 2, 5):
        y0, h, cache = orc.ssm_layer_scan(p["x"][:, :L0], p["A"], p["B"][:, :L0], p["C"][:, :L0],
                                          z=p["z"][:, :L0], dt_raw=p["r"][:, :L0], **common)
        _close(y0, y_all[:, :L0], 1e-13, f"prefill part L0={L0}")
        for t in range(L0, T):
            yt, cache, h = orc.decode_step(p["x"][:, t], p["A"], p["B"][:, t], p["C"][:, t], conv_cache=cache,
                                           ssm_state=h, z_t=p["z"][:, t], dt_raw_t=p["r"][:, t], **common)
            _close(yt, y_all[:, t], 1e-12, f"decode y t={t} after L0={L0}")
        _close(h, h_all, 1e-12, f"decode final state L0={L0}")
        _close(cache, c_all, 0.0, f"decode final conv cache L0={L0}")
    # split prefill: state and cache of the first part continue the second
    for L1 in (1, 3, 7):
        ya, ha, ca = orc.ssm_layer_scan(p["x"][:, :L1], p["A"], p["B"][:, :L1], p["C"][:, :L1],
                                        z=p["z"][:, :L1], dt_raw=p["r"][:, :L1], **common)
        yb, hb, cb = orc.ssm_layer_scan(p["x"][:, L1:], p["A"], p["B"][:, L1:], p["C"][:, L1:],
                                        z=p["z"][:, L1:], dt_raw=p["r"][:, L1:], conv_cache=ca, ssm_state=ha,
                                        **common)
        _close(np.concatenate([ya, yb], axis=1), y_all, 1e-12, f"split prefill y L1={L1}")
        _close(hb, h_all, 1e-12, f"split prefill state L1={L1}")
        _close(cb, c_all, 0.0, f"split prefill cache L1={L1}")


def pin_conv_cache_contents(orc):
    """conv_cache after a prefill holds the last K-1 raw inputs, oldest first; for
    a prompt shorter than K-1 the zero padding is included."""
    p = _layer_inputs(109, T=6)
    x = p["x"]
    _, cache = orc.causal_depthwise_conv1d(x, p["conv_w"])
    assert np.array_equal(cache, np.transpose(x[:, -3:, :], (0, 2, 1)))
    _, cache2 = orc.causal_depthwise_conv1d(x[:, :2], p["conv_w"])
    want = np.concatenate([np.zeros((x.shape[0], x.shape[2], 1)), np.transpose(x[:, :2], (0, 2, 1))], axis=2)
    assert np.array_equal(cache2, want)


# ---------------------------------------------------------------------------
# Q7: library special cases
# ---------------------------------------------------------------------------

def pin_library_special_cases(orc):
    rng = _rng(110)
    Bt, L, E, K = 2, 17, 3, 4
    x = rng.standard_normal((Bt, L, E))
    w = rng.standard_normal((E, K))
    bias = rng.standard_normal(E)
    xc, _ = orc.causal_depthwise_conv1d(x, w, bias)
    for b in range(Bt):
        for e in range(E):
            ref = np.convolve(x[b, :, e], w[e, ::-1])[:L] + bias[e]
            _close(xc[b, :, e], ref, 1e-14, "conv vs np.convolve")
    v = np.linspace(-30.0, 30.0, 601)
    _close(orc.softplus(v), np.log1p(np.exp(v)), 1e-14, "softplus")
    try:
        from scipy.special import expit
        _close(orc.sigmoid(v), expit(v), 1e-15, "sigmoid vs expit")
        _close(orc.silu(v), v * expit(v), 1e-14, "silu")
    except ImportError:  # scipy absent: compare with the textbook form away from overflow
        _close(orc.sigmoid(v), 1.0 / (1.0 + np.exp(-v)), 1e-15, "sigmoid")
    # compute_dt: bias, softplus, inclusive clip; rank-1 dt_proj is an outer product
    raw = np.linspace(-12.0, 3.0, 151)
    bias_v = 0.25
    got = orc.compute_dt(raw, bias_v, 1e-3, 0.1)
    _close(got, np.clip(np.log1p(np.exp(raw + bias_v)), 1e-3, 0.1), 1e-15, "compute_dt")
    _close(orc.compute_dt(raw, None, None, None, use_softplus=False), raw, 0.0, "compute_dt identity")
    r = rng.standard_normal((2, 3))
    wv = rng.standard_normal(4)
    _close(orc.dt_proj_rank1(r, wv), np.einsum("bt,e->bte", r, wv), 1e-15, "rank-1 dt_proj")


# ---------------------------------------------------------------------------
# Q8: causality
# ---------------------------------------------------------------------------

def pin_causality(orc):
    p = _layer_inputs(111, T=12)
    common = dict(D=p["D"], conv_w=p["conv_w"], dt_w=p["dt_w"], dt_bias=p["dt_bias"],
                  dt_softplus=True, dt_min=1e-3, dt_max=0.1)
    y, _, _ = orc.ssm_layer_scan(p["x"], p["A"], p["B"], p["C"], z=p["z"], dt_raw=p["r"], **common)
    t0 = 6
    for key in ("x", "z", "B", "C", "r"):
        q = {k: v.copy() for k, v in p.items()}
        q[key][:, t0] += 3.0
        y2, _, _ = orc.ssm_layer_scan(q["x"], q["A"], q["B"], q["C"], z=q["z"], dt_raw=q["r"], **common)
        assert np.array_equal(y2[:, :t0], y[:, :t0]), f"output before t0 changed when {key} changed at t0"
        assert not np.array_equal(y2[:, t0], y[:, t0]), f"output at t0 ignored {key}"


# ---------------------------------------------------------------------------
# Q9: A initialisation (Axon-SSM "State initialization")
# ---------------------------------------------------------------------------

def pin_a_init(orc):
    g = _golden("a_init_diagonal.json")
    n = np.arange(1, g["d_state"] + 1, dtype=np.float64)
    A = orc.a_from_log(np.log(n))
    want = np.array(g["A"], np.float64)
    assert np.all(np.abs(A - want) <= 2 * np.spacing(np.abs(want))), (A, want)


# ---------------------------------------------------------------------------
# Q10: linearity and the B/C scaling invariance of the pure scan
# ---------------------------------------------------------------------------

def pin_linearity(orc):
    rng = _rng(112)
    Bt, L, E, N = 2, 11, 3, 4
    dt = rng.uniform(0.01, 0.3, (Bt, L, E))
    A = -rng.uniform(0.5, 4.0, (E, N))
    Bm = rng.standard_normal((Bt, L, N))
    Cm = rng.standard_normal((Bt, L, N))
    D = rng.standard_normal(E)
    u1, u2 = rng.standard_normal((2, Bt, L, E))
    h1, h2 = rng.standard_normal((2, Bt, E, N))
    al, be = 1.7, -0.6
    ya, sa = orc.selective_scan(u1, dt, A, Bm, Cm, D=D, ssm_state=h1)
    yb, sb = orc.selective_scan(u2, dt, A, Bm, Cm, D=D, ssm_state=h2)
    yc, sc = orc.selective_scan(al * u1 + be * u2, dt, A, Bm, Cm, D=D, ssm_state=al * h1 + be * h2)
    _close(yc, al * ya + be * yb, 1e-12, "linearity y")
    _close(sc, al * sa + be * sb, 1e-12, "linearity state")
    y0, _ = orc.selective_scan(u1, dt, A, Bm, Cm)
    ys, _ = orc.selective_scan(u1, dt, A, 2.5 * Bm, Cm / 2.5)
    _close(ys, y0, 1e-12, "B*a, C/a invariance")


# ---------------------------------------------------------------------------
# Q11: zero cases of the skip and the gate
# ---------------------------------------------------------------------------

def pin_zero_cases(orc):
    rng = _rng(113)
    Bt, L, E, N = 2, 9, 3, 4
    u = rng.standard_normal((Bt, L, E))
    dt = rng.uniform(0.01, 0.3, (Bt, L, E))
    A = -rng.uniform(0.5, 4.0, (E, N))
    Bm = rng.standard_normal((Bt, L, N))
    Cm = rng.standard_normal((Bt, L, N))
    D = rng.standard_normal(E)
    z = rng.standard_normal((Bt, L, E))
    gate = z / (1.0 + np.exp(-z))
    y, _ = orc.selective_scan(u, dt, A, np.zeros_like(Bm), Cm, D=D, z=z)
    _close(y, D * u * gate, 1e-15, "B = 0")
    y, _ = orc.selective_scan(u, dt, A, Bm, np.zeros_like(Cm), D=D, z=z)
    _close(y, D * u * gate, 1e-15, "C = 0")
    yg, _ = orc.selective_scan(u, dt, A, Bm, Cm, D=D, z=np.full_like(z, 40.0))
    yn, _ = orc.selective_scan(u, dt, A, Bm, Cm, D=D)
    _close(yg / 40.0, yn, 1e-15, "saturated gate is the identity times z")


# ---------------------------------------------------------------------------
# Q13: affine-map monoid and the Blelloch scan
# ---------------------------------------------------------------------------

def pin_affine_monoid_and_blelloch(orc):
    rng = _rng(114)
    maps = [(rng.uniform(-1.5, 1.5), rng.standard_normal()) for _ in range(13)]
    ident = (1.0, 0.0)

    def apply(m, h):
        return m[0] * h + m[1]

    for i in range(len(maps) - 2):
        p, q, r = maps[i], maps[i + 1], maps[i + 2]
        l = orc.affine_compose(orc.affine_compose(p, q), r)
        rr = orc.affine_compose(p, orc.affine_compose(q, r))
        assert abs(l[0] - rr[0]) < 1e-12 and abs(l[1] - rr[1]) < 1e-12
        for h in (0.3, -2.0):
            assert abs(apply(orc.affine_compose(p, q), h) - apply(q, apply(p, h))) < 1e-12
        assert orc.affine_compose(p, ident) == (p[0] * 1.0, 1.0 * p[1] + 0.0)
        assert orc.affine_compose(ident, p) == (1.0 * p[0], p[0] * 0.0 + p[1])
    # Blelloch exclusive scan vs the sequential exclusive fold, every length
    for n in range(0, 14):
        got = orc.blelloch_exclusive_scan(maps[:n], orc.affine_compose, ident)
        acc = ident
        for k in range(n):
            assert abs(got[k][0] - acc[0]) < 1e-12 and abs(got[k][1] - acc[1]) < 1e-12, (n, k)
            acc = (acc[0] * maps[k][0], maps[k][0] * acc[1] + maps[k][1])
    # the textbook example: exclusive prefix sums of 1..8 are k(k-1)/2
    got = orc.blelloch_exclusive_scan(list(range(1, 9)), lambda a, b: a + b, 0)
    assert got == [k * (k - 1) // 2 for k in range(1, 9)]


# ---------------------------------------------------------------------------
# SSD: closed forms of the chunk formula's terms
# ---------------------------------------------------------------------------

def pin_ssd_terms(orc):
    """With B = 0 only the previous-state and D terms remain:
    out[l] = e^{dA[l]} C[l] S0 + D x[l] and S decays by e^{dA[Q-1]}; with C = 0
    and D absent the output is zero; a one-token chunk is the single step."""
    x, dt, A, Bm, Cm, D, S0 = _ssd_inputs(115, L=8, G=1)
    Bt, L, H, P = x.shape
    out, S = orc.ssd_chunk_scan(x, dt, A, np.zeros_like(Bm), Cm, D=D, state=S0, chunk_size=8)
    dA = np.cumsum(dt * A[None, None, :], axis=1)  # (Bt, L, H)
    want = np.exp(dA)[..., None] * np.einsum("bln,bhpn->blhp", Cm[:, :, 0], S0) + x * D[None, None, :, None]
    _close(out, want, 1e-13, "ssd B=0")
    _close(S, np.exp(dA[:, -1])[:, :, None, None] * S0, 1e-13, "ssd B=0 state")
    out0, _ = orc.ssd_chunk_scan(x, dt, A, Bm, np.zeros_like(Cm), D=None, state=S0, chunk_size=4)
    _close(out0, np.zeros_like(out0), 0.0, "ssd C=0")
    o1, S1 = orc.ssd_chunk_scan(x[:, :1], dt[:, :1], A, Bm[:, :1], Cm[:, :1], D=D, state=S0, chunk_size=1)
    a = np.exp(dt[:, 0] * A[None])  # (Bt, H)
    Sw = a[:, :, None, None] * S0 + (dt[:, 0, :, None] * x[:, 0])[..., None] * Bm[:, 0, 0][:, None, None, :]
    _close(S1, Sw, 1e-13, "ssd one-token state")
    _close(o1[:, 0], np.einsum("bhpn,bn->bhp", Sw, Cm[:, 0, 0]) + x[:, 0] * D[None, :, None], 1e-13,
           "ssd one-token out")



def pin_linear_brute_force(orc):
    """linear(x, W) is the sum over the input index of x times W[out, in], by loops."""
    rng = _rng(71)
    x = rng.standard_normal((2, 3, 5))
    W = rng.standard_normal((4, 5))
    want = np.zeros((2, 3, 4))
    for b in range(2):
        for t in range(3):
            for o in range(4):
                acc = 0.0
                for i in range(5):
                    acc += x[b, t, i] * W[o, i]
                want[b, t, o] = acc
    _close(orc.linear(x, W), want, 1e-13, "linear")


def _layer_weights(rng, Dm, E, N, K=4):
    return dict(W_in=rng.standard_normal((2 * E, Dm)) * 0.3, conv_w=rng.standard_normal((E, K)) * 0.5,
                W_x=rng.standard_normal((2 * N + 1, E)) * 0.3, dt_w=rng.standard_normal(E) * 0.5,
                dt_bias=rng.standard_normal(E) * 0.5, A=-np.tile(np.arange(1, N + 1, dtype=np.float64), (E, 1)),
                W_out=rng.standard_normal((Dm, E)) * 0.3, D=rng.standard_normal(E))


def pin_layer_wiring(orc):
    """The layer with structured weights reduces to pieces computed here by hand:
    in_proj = [I; 2I] makes x_branch = hidden and z = 2 hidden, out_proj = I
    returns y, and x_proj rows that are unit vectors pick B, C and dt_raw out of
    the post-conv activation u = SiLU(conv(x_branch)) (B first, then C, then
    dt_raw, as the dataflow lists them).  The scan is then the plain
    recurrence, written out here."""
    rng = _rng(72)
    Bt, L, E, N = 2, 9, 6, 2
    hidden = rng.standard_normal((Bt, L, E))
    conv_w = rng.standard_normal((E, 4)) * 0.5
    W_in = np.concatenate([np.eye(E), 2.0 * np.eye(E)])
    pick = [4, 1, 0, 5, 3]  # B from channels 4, 1; C from 0, 5; dt_raw from 3
    W_x = np.zeros((2 * N + 1, E))
    for j, e in enumerate(pick):
        W_x[j, e] = 1.0
    dt_w = rng.uniform(0.5, 1.5, E)
    dt_bias = rng.standard_normal(E) * 0.3
    A = -np.tile(np.arange(1, N + 1, dtype=np.float64), (E, 1))
    D = rng.standard_normal(E)
    out, h_end, cache = orc.ssm_layer_forward(hidden, W_in, conv_w, W_x, dt_w, dt_bias, A, np.eye(E), D=D,
                                              dt_min=1e-3, dt_max=0.5)
    # by hand: conv (cross-correlation, zero history), SiLU, the picks, the scan
    u = np.zeros((Bt, L, E))
    for b in range(Bt):
        for t in range(L):
            for e in range(E):
                acc = 0.0
                for k in range(4):
                    tt = t - 3 + k
                    if tt >= 0:
                        acc += conv_w[e, k] * hidden[b, tt, e]
                u[b, t, e] = acc * _sig(acc)
    y = np.zeros((Bt, L, E))
    h = np.zeros((Bt, E, N))
    for b in range(Bt):
        for t in range(L):
            Bv = [u[b, t, pick[0]], u[b, t, pick[1]]]
            Cv = [u[b, t, pick[2]], u[b, t, pick[3]]]
            r = u[b, t, pick[4]]
            for e in range(E):
                pre = dt_w[e] * r + dt_bias[e]
                dt = min(max(math.log1p(math.exp(pre)), 1e-3), 0.5)
                acc = 0.0
                for n in range(N):
                    h[b, e, n] = math.exp(dt * A[e, n]) * h[b, e, n] + dt * Bv[n] * u[b, t, e]
                    acc += Cv[n] * h[b, e, n]
                zz = 2.0 * hidden[b, t, e]
                y[b, t, e] = (acc + D[e] * u[b, t, e]) * zz * _sig(zz)
    _close(out, y, 1e-12, "layer wiring: out")
    _close(h_end, h, 1e-12, "layer wiring: state")
    _close(cache, np.transpose(hidden[:, L - 3:, :], (0, 2, 1)), 0.0, "layer wiring: conv cache")


def pin_layer_prefill_split(orc):
    """A layer over L tokens equals the layer over the first L1 tokens followed by
    the layer over the rest from the returned ssm_state and conv_cache."""
    rng = _rng(73)
    Bt, L, L1, Dm, E, N = 2, 11, 4, 5, 6, 3
    wts = _layer_weights(rng, Dm, E, N)
    hidden = rng.standard_normal((Bt, L, Dm))
    kw = dict(D=wts["D"], dt_min=1e-3, dt_max=0.3)
    args = [wts[k] for k in ("W_in", "conv_w", "W_x", "dt_w", "dt_bias", "A", "W_out")]
    o_all, h_all, c_all = orc.ssm_layer_forward(hidden, *args, **kw)
    o1, h1, c1 = orc.ssm_layer_forward(hidden[:, :L1], *args, **kw)
    o2, h2, c2 = orc.ssm_layer_forward(hidden[:, L1:], *args, conv_cache=c1, ssm_state=h1, **kw)
    _close(np.concatenate([o1, o2], axis=1), o_all, 1e-12, "layer split: out")
    _close(h2, h_all, 1e-12, "layer split: state")
    _close(c2, c_all, 0.0, "layer split: cache")


def pin_layer_projections_linear(orc):
    """out_proj is linear in its weight (2 W_out doubles the output), a zero
    hidden input from a zero state gives a zero output, and the output of a
    single token depends on nothing after it."""
    rng = _rng(74)
    Bt, L, Dm, E, N = 1, 6, 4, 5, 2
    wts = _layer_weights(rng, Dm, E, N)
    hidden = rng.standard_normal((Bt, L, Dm))
    args = lambda W_out: [wts[k] for k in ("W_in", "conv_w", "W_x", "dt_w", "dt_bias", "A")] + [W_out]
    o1, _, _ = orc.ssm_layer_forward(hidden, *args(wts["W_out"]), D=wts["D"], dt_min=1e-3, dt_max=0.3)
    o2, _, _ = orc.ssm_layer_forward(hidden, *args(2.0 * wts["W_out"]), D=wts["D"], dt_min=1e-3, dt_max=0.3)
    _close(o2, 2.0 * o1, 1e-12, "layer: out_proj linear")
    o0, h0, _ = orc.ssm_layer_forward(np.zeros_like(hidden), *args(wts["W_out"]), D=wts["D"], dt_min=1e-3,
                                      dt_max=0.3)
    assert np.all(o0 == 0.0) and np.all(h0 == 0.0), "layer: zero input must give zero output and state"
    h2 = hidden.copy()
    h2[:, 3:] += 1.0
    o3, _, _ = orc.ssm_layer_forward(h2, *args(wts["W_out"]), D=wts["D"], dt_min=1e-3, dt_max=0.3)
    _close(o3[:, :3], o1[:, :3], 0.0, "layer: causal")


def pin_zoh_steady_state(orc):
    """Zero-order hold keeps the continuous system's fixed point: with constant
    u and B, x' = A x + B u settles at -B u / A, and the ZOH recurrence
    h <- e^{dt A} h + ((e^{dt A} - 1) / A) B u has exactly that fixed point for
    any dt (Euler's, dt B u / (1 - e^{dt A}), does not).  After enough steps
    the state matches it; the one-step coefficient is checked against expm1."""
    Bt, L, E, N = 1, 1000, 3, 4  # slowest mode: e^{-0.05 * 1000} of the initial gap left
    A = -np.array([[0.5, 1.0, 2.0, 4.0]] * E)
    u = np.full((Bt, L, E), 0.7)
    Bv = np.array([0.3, -1.2, 2.0, 0.9])
    B = np.tile(Bv, (Bt, L, 1))
    C = np.ones((Bt, L, N))
    dt = np.full((Bt, L, E), 0.1)
    _, h = orc.selective_scan(u, dt, A, B, C, discretization="zoh")
    want = -Bv[None, :] * 0.7 / A  # (E, N)
    _close(h[0], want, 1e-7, "zoh steady state")
    _, h_e = orc.selective_scan(u, dt, A, B, C, discretization="euler")
    assert np.max(np.abs(h_e[0] - want)) > 1e-3, "euler must not share the zoh fixed point"
    # one step from zero: h_1 = (e^{dt A} - 1) / A * B u
    _, h1 = orc.selective_scan(u[:, :1], dt[:, :1], A, B[:, :1], C[:, :1], discretization="zoh")
    _close(h1[0], np.expm1(0.1 * A) / A * Bv[None, :] * 0.7, 1e-14, "zoh one step")
    # and the layer scan / decode step pass the choice through
    y_l, h_l, _ = orc.ssm_layer_scan(u[:, :5], A, B[:, :5], C[:, :5], dt=dt[:, :5], dt_softplus=False,
                                     discretization="zoh")
    y_s, h_s = orc.selective_scan(u[:, :5], dt[:, :5], A, B[:, :5], C[:, :5], discretization="zoh")
    _close(y_l, y_s, 0.0, "layer scan zoh")
    y_d, _, h_d = orc.decode_step(u[:, 0], A, B[:, 0], C[:, 0], conv_cache=None, ssm_state=None, dt_t=dt[:, 0],
                                  dt_softplus=False, discretization="zoh")
    _close(h_d, h1, 0.0, "decode step zoh")


def _fd_check(orc, fwd_kwargs, grads, keys, rng, what, eps=1e-6, tol=1e-6):
    """Central differences of L = sum(dy * y) + sum(dstate_out * h_L) against the
    backward's gradients, for every element of every input in `keys`."""
    dy = fwd_kwargs.pop("_dy")
    dso = fwd_kwargs.pop("_dstate_out")

    def loss(kw):
        y, h, _ = orc.ssm_layer_scan(**kw)
        val = float(np.sum(dy * y))
        if dso is not None:
            val += float(np.sum(dso * h))
        return val

    for key in keys:
        base = np.array(fwd_kwargs[key], dtype=np.float64)
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            for sgn in (1.0, -1.0):
                pert = base.copy()
                pert[idx] += sgn * eps
                kw = dict(fwd_kwargs)
                kw[key] = pert
                num[idx] += sgn * loss(kw)
        num /= 2 * eps
        g = grads[key]
        scale = max(1.0, float(np.max(np.abs(num))))
        err = float(np.max(np.abs(g - num)))
        assert err <= tol * scale, f"{what}: d/d{key} max|err| {err:.3e} > {tol:.1e} * {scale:.3e}"
    fwd_kwargs["_dy"], fwd_kwargs["_dstate_out"] = dy, dso


def pin_backward_finite_differences(orc):
    """The scan-stage backward against central finite differences of the
    forward, for every input: (1) conv, rank-1 dt with softplus, gate, D,
    initial state, conv cache and a gradient on the final state, clip bounds
    out of reach; (2) E-wide dt without softplus and with some steps clipped
    at either bound, no conv, gate or D."""
    rng = _rng(81)
    Bt, L, E, N = 2, 5, 3, 4
    kw = dict(x=rng.standard_normal((Bt, L, E)), A=-rng.uniform(0.5, 3.0, (E, N)),
              B=rng.standard_normal((Bt, L, N)), C=rng.standard_normal((Bt, L, N)), D=rng.standard_normal(E),
              z=rng.standard_normal((Bt, L, E)), conv_w=rng.standard_normal((E, 4)) * 0.5,
              conv_b=rng.standard_normal(E) * 0.2, conv_cache=rng.standard_normal((Bt, E, 3)),
              dt_raw=rng.standard_normal((Bt, L)), dt_w=rng.standard_normal(E) * 0.5,
              dt_bias=rng.standard_normal(E) * 0.5 - 1.0, dt_min=1e-4, dt_max=50.0,
              ssm_state=rng.standard_normal((Bt, E, N)))
    kw["_dy"] = rng.standard_normal((Bt, L, E))
    kw["_dstate_out"] = rng.standard_normal((Bt, E, N))
    fwd = {k: v for k, v in kw.items() if not k.startswith("_")}
    g = orc.ssm_layer_scan_backward(dy=kw["_dy"], dstate_out=kw["_dstate_out"], **fwd)
    names = {"x": "x", "A": "A", "B": "B", "C": "C", "D": "D", "z": "z", "conv_w": "conv_w", "conv_b": "conv_b",
             "conv_cache": "conv_cache", "dt_raw": "dt_raw", "dt_w": "dt_w", "dt_bias": "dt_bias",
             "ssm_state": "ssm_state"}
    _fd_check(orc, kw, {k: g[v] for k, v in names.items()}, list(names), rng, "backward (conv, rank-1 dt)")

    Bt, L, E, N = 1, 6, 2, 3
    dt_e = rng.uniform(0.02, 0.4, (Bt, L, E))
    dt_e[0, 1, 0] = 0.005   # below dt_min: clipped, no gradient
    dt_e[0, 4, 1] = 0.9     # above dt_max
    kw = dict(x=rng.standard_normal((Bt, L, E)), A=-rng.uniform(0.5, 3.0, (E, N)),
              B=rng.standard_normal((Bt, L, N)), C=rng.standard_normal((Bt, L, N)), dt=dt_e,
              dt_bias=np.zeros(E), dt_softplus=False, dt_min=0.01, dt_max=0.5)
    kw["_dy"] = rng.standard_normal((Bt, L, E))
    kw["_dstate_out"] = None
    fwd = {k: v for k, v in kw.items() if not k.startswith("_")}
    g = orc.ssm_layer_scan_backward(dy=kw["_dy"], **fwd)
    assert g["dt"][0, 1, 0] == 0.0 and g["dt"][0, 4, 1] == 0.0, "clipped steps carry no dt gradient"
    _fd_check(orc, kw, {k: g[k] for k in ("x", "A", "B", "C", "dt", "dt_bias")}, ["x", "A", "B", "C", "dt", "dt_bias"],
              rng, "backward (E-wide dt, clipped)")

ALL_PINS = [
    pin_unrolled_product_sum,
    pin_recurrence_equals_convolution,
    pin_constant_input_closed_form,
    pin_single_step,
    pin_chunked_equals_sequential,
    pin_ssd_chunked_equals_sequential,
    pin_ssd_ragged_chunks,
    pin_ssd_gate,
    pin_ssd_prefill_then_decode,
    pin_ssd_equals_channel_scan,
    pin_prefill_then_decode,
    pin_conv_cache_contents,
    pin_library_special_cases,
    pin_causality,
    pin_a_init,
    pin_linearity,
    pin_zero_cases,
    pin_affine_monoid_and_blelloch,
    pin_ssd_terms,
    pin_linear_brute_force,
    pin_layer_wiring,
    pin_layer_prefill_split,
    pin_layer_projections_linear,
    pin_zoh_steady_state,
    pin_backward_finite_differences,
]
