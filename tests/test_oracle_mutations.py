"""Plant a mistake in a copy of the oracle (on the CPU) and require that some
pin catches it.  This shows the pins are sensitive to the plausible errors: a
dropped term, a wrong sign, index or operand order."""
import importlib.util
import os

import pytest

import oracle_pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "ssm_oracle.py")

MUTATIONS = {
    "update_sign": ("h = dA * h + dB * u[:, t, :, None]", "h = dA * h - dB * u[:, t, :, None]"),
    "decay_sign": ("dA = np.exp(dtt * A[None, :, :])", "dA = np.exp(-dtt * A[None, :, :])"),
    "readout_wrong_t": ("yt = np.sum(C[:, t, None, :] * h, axis=-1)",
                        "yt = np.sum(C[:, max(t - 1, 0), None, :] * h, axis=-1)"),
    "drop_D": ("            yt = yt + _f64(D)[None, :] * u[:, t, :]\n        y[:, t, :] = yt\n    if z",
               "            yt = yt\n        y[:, t, :] = yt\n    if z"),
    "gate_sigmoid": ("    if z is not None:\n        y = y * silu(z)\n    return y, h\n",
                     "    if z is not None:\n        y = y * sigmoid(z)\n    return y, h\n"),
    "conv_taps_reversed": ("xc += w[None, None, :, k] * xpad[:, k:k + L, :]",
                           "xc += w[None, None, :, K - 1 - k] * xpad[:, k:k + L, :]"),
    "conv_cache_shifted": ("xpad[:, L:L + K - 1, :]", "xpad[:, L - 1:L + K - 2, :]"),
    "softplus_sign": ("return np.logaddexp(0.0, _f64(x))", "return np.logaddexp(0.0, -_f64(x))"),
    "no_upper_clip": ("s = np.minimum(s, float(hi))", "s = s"),
    "rank1_sum": ("_f64(dt_raw)[..., None] * _f64(w)[None, None, :]", "_f64(dt_raw)[..., None] + _f64(w)[None, None, :]"),
    "zoh_wrong": ("dB = (dA - 1.0) / A[None, :, :] * B[:, t, None, :]", "dB = (dA - 1.0) * A[None, :, :] * B[:, t, None, :]"),
    "decode_drops_cache": ("conv_cache=conv_cache if conv_w is not None else None", "conv_cache=None"),
    "blelloch_order": ("tree[i] = op(tree[i], left)", "tree[i] = op(left, tree[i])"),
    "compose_order": ("return (a1 * a2, a2 * b1 + b2)", "return (a1 * a2, a1 * b2 + b1)"),
    "chunk_prod_reset": ("prod = prod * dA", "prod = dA"),
    "ssd_exclusive_cumsum": ("dA = np.cumsum(dtc * A[None, None, :], axis=1)",
                             "dA = np.cumsum(dtc * A[None, None, :], axis=1) - dtc * A[None, None, :]"),
    "ssd_strict_mask": ("causal = ls[None, :] <= ls[:, None]", "causal = ls[None, :] < ls[:, None]"),
    "ssd_state_drops_dt": ("wgt = np.exp(last[:, None, :] - dA) * dtc", "wgt = np.exp(last[:, None, :] - dA)"),
    "ssd_state_no_decay": ("S = np.exp(last)[:, :, None, None] * S + np.einsum", "S = S + np.einsum"),
    "ssd_prev_no_decay": ("o += np.exp(dA)[..., None] * np.einsum", "o += np.einsum"),
    "ssd_group_map": ("return np.arange(H) // (H // G)", "return np.arange(H) % G"),
    "ssd_cb_transposed": ('cb = np.einsum("blhn,bshn->bhls", Ch, Bh)', 'cb = np.einsum("blhn,bshn->bhsl", Ch, Bh)'),
    "ssd_seq_dt_dropped": ("S = a[:, :, None, None] * S + (dt[:, t, :, None] * x[:, t])[..., None]",
                           "S = a[:, :, None, None] * S + (x[:, t])[..., None]"),
    "a_from_log_sign": ("return -np.exp(_f64(A_log))", "return np.exp(_f64(A_log))"),
    "ssd_ragged_tail_dropped": ("for c in range((L + Q - 1) // Q):", "for c in range(L // Q):"),
    "ssd_gate_sigmoid": ("    return out * silu(_f64(z))", "    return out * sigmoid(_f64(z))"),
    "layer_xz_swapped": ("x_branch, z = xz[..., :E], xz[..., E:]", "z, x_branch = xz[..., :E], xz[..., E:]"),
    "layer_xproj_on_x": ("dbc = linear(u, W_x)", "dbc = linear(x_branch, W_x)"),
    "layer_bc_swapped": ("B, C, dt_raw = dbc[..., :N], dbc[..., N:2 * N], dbc[..., 2 * N]",
                         "C, B, dt_raw = dbc[..., :N], dbc[..., N:2 * N], dbc[..., 2 * N]"),
    "layer_dt_from_first": ("B, C, dt_raw = dbc[..., :N], dbc[..., N:2 * N], dbc[..., 2 * N]",
                            "B, C, dt_raw = dbc[..., 1:N + 1], dbc[..., N + 1:2 * N + 1], dbc[..., 0]"),
    "layer_no_gate": ("y, h, cache = ssm_layer_scan(x_branch, A, B, C, D=D, z=z,",
                      "y, h, cache = ssm_layer_scan(x_branch, A, B, C, D=D, z=None,"),
    "layer_state_not_passed": ("dt_min=dt_min, dt_max=dt_max, ssm_state=ssm_state)\n    return linear(y, W_out)",
                               "dt_min=dt_min, dt_max=dt_max, ssm_state=None)\n    return linear(y, W_out)"),
    "linear_weight_transposed": ("return _f64(x) @ _f64(W).T", "return _f64(x) @ _f64(W)[:, ::-1].T"),
    "zoh_not_passed_by_layer": ("ssm_state=ssm_state, discretization=discretization)\n    return y, h, cache_out",
                                "ssm_state=ssm_state)\n    return y, h, cache_out"),
    "zoh_coef_uses_dt": ("dB = (dA - 1.0) / A[None, :, :] * B[:, t, None, :]", "dB = dtt * dA * B[:, t, None, :]"),
    "bwd_gate_derivative": ("out[\"z\"] = dy * yc * (sg * (1.0 + zf * (1.0 - sg)))", "out[\"z\"] = dy * yc * sg"),
    "bwd_no_decay_in_G": ("C[:, t, None, :] + a_next * G_next if t < L - 1", "C[:, t, None, :] + G_next if t < L - 1"),
    "bwd_dA_missing_decay": ("dA += np.sum(G * dtv[:, t, :, None] * a * h_prev, axis=0)",
                             "dA += np.sum(G * dtv[:, t, :, None] * h_prev, axis=0)"),
    "bwd_clip_ignored": ("inside = (sp > lo) & (sp < hi)", "inside = np.ones_like(sp, dtype=bool)"),
    "bwd_conv_taps_reversed": ("dxpad[:, k:k + L, :] += dxc * w[None, None, :, k]",
                               "dxpad[:, k:k + L, :] += dxc * w[None, None, :, K - 1 - k]"),
    "bwd_state_in_no_decay": ("out[\"ssm_state\"] = a_next * G_next if", "out[\"ssm_state\"] = G_next if"),
    "ssd_seq_gate_dropped": ("    return _gate(out, z), S\n\n\ndef ssd_chunk_scan",
                          "    return out, S\n\n\ndef ssd_chunk_scan"),
}


def _load_mutant(name, old, new):
    """The oracle's source with the first occurrence of `old` replaced by `new`."""
    with open(ORACLE_SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation {name}: pattern not found"
    spec = importlib.util.spec_from_loader(f"oracle_mutant_{name}", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(src.replace(old, new, 1), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_pin_catches_mutation(name):
    mod = _load_mutant(name, *MUTATIONS[name])
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as exc:  # a failing assertion or a crash both count
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin caught the planted mistake {name}"
