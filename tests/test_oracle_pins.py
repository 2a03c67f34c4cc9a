"""The float64 oracle against what the pages and the mathematics fix (CPU only)."""
import json
import os

import pytest

import oracle_pins
from oracle import ssm_oracle


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(ssm_oracle)


def test_bit_axon_shape_accounting():
    """Per-layer parameter count from the dataflow shapes, times 16 SSM layers,
    lands within 1.5 % of the "about 960M" the Axon-SSM page states; this fixes
    A_log as (E, d_state), x_proj as E -> 2*d_state+1 and dt_proj as 1 -> E."""
    with open(os.path.join(oracle_pins.GOLDEN, "bit_axon_ssm_shapes.json")) as f:
        g = json.load(f)
    Dm, E, N, K = g["hidden_dim"], g["expand_dim"], g["d_state"], g["conv_kernel"]
    per_layer = (Dm * 2 * E          # in_proj
                 + E * K + E         # depthwise conv weight + bias
                 + E * (2 * N + 1)   # x_proj
                 + E + E             # dt_proj weight (1 -> E) + dt_bias
                 + E * N             # A_log
                 + E                 # D
                 + E * Dm)           # out_proj
    total = per_layer * g["ssm_layers"] / 1e6
    assert abs(total - g["stated_total_millions"]) / g["stated_total_millions"] < 0.015, total
    assert total < g["stated_model_billions"] * 1e3


# Q13 as properties: the affine maps (a, b) of the segment scan form a monoid
# under composition (associative, identity (1, 0)), composition applies the
# first map then the second, and the Blelloch exclusive scan equals the
# sequential exclusive fold for any list of maps.  Examples are drawn by
# hypothesis from a fixed seed (derandomize), so the run is repeatable.
from hypothesis import given, settings, strategies as st  # noqa: E402

_coef = st.floats(min_value=-1.5, max_value=1.5, allow_nan=False, allow_infinity=False)
_map = st.tuples(_coef, st.floats(min_value=-4.0, max_value=4.0, allow_nan=False, allow_infinity=False))


@settings(max_examples=300, derandomize=True, deadline=None)
@given(_map, _map, _map, st.floats(min_value=-3.0, max_value=3.0, allow_nan=False))
def test_affine_monoid_properties(p, q, r, h):
    O = ssm_oracle
    left = O.affine_compose(O.affine_compose(p, q), r)
    right = O.affine_compose(p, O.affine_compose(q, r))
    assert abs(left[0] - right[0]) <= 1e-12 and abs(left[1] - right[1]) <= 1e-12
    ident = (1.0, 0.0)
    assert O.affine_compose(p, ident) == (p[0], p[1]) and O.affine_compose(ident, p) == (p[0], p[1])
    pq = O.affine_compose(p, q)
    assert abs((pq[0] * h + pq[1]) - (q[0] * (p[0] * h + p[1]) + q[1])) <= 1e-12


@settings(max_examples=150, derandomize=True, deadline=None)
@given(st.lists(_map, min_size=0, max_size=40))
def test_blelloch_scan_equals_sequential_fold(maps):
    O = ssm_oracle
    got = O.blelloch_exclusive_scan(list(maps), O.affine_compose, (1.0, 0.0))
    acc = (1.0, 0.0)
    assert len(got) == len(maps)
    for k, m in enumerate(maps):
        scale = 1.0 + abs(acc[0]) + abs(acc[1])
        assert abs(got[k][0] - acc[0]) <= 1e-12 * scale and abs(got[k][1] - acc[1]) <= 1e-12 * scale, k
        acc = (acc[0] * m[0], m[0] * acc[1] + m[1])
