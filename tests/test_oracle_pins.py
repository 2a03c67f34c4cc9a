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
