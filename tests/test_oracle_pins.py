"""The CPU oracle against its pins (see tests/pins.py for what each pin is)."""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from tests import pins

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def O():
    return oracle.default()


@pytest.mark.parametrize("pin", pins.PINS, ids=lambda p: p.__name__)
def test_pin(O, pin):
    pin(O)


def test_workload_shapes_match_weight_budget():
    """P12: the full-size workloads reproduce the pages' weight budget (62 MoE
    layers; 256 experts per layer ~ 799 B parameters; latent projections ~ 4.2 B)."""
    with open(os.path.join(HERE, "golden", "weight_budget.json")) as f:
        g = json.load(f)
    w = synth.WORKLOADS["decode_bf16"]
    layers = g["layers"]["value"]
    experts = 3 * w.Dp * w.F * w.E * layers
    latent = 2 * w.D * w.Dp * layers
    assert abs(experts - g["experts_params"]["value"]) / g["experts_params"]["value"] < 0.001
    assert abs(latent - g["latent_projection_params"]["value"]) / g["latent_projection_params"][
        "value"] < 0.01
    assert (w.D, w.Dp) == tuple(g["pooler_shape"]["value"])
    assert w.E == g["experts_per_layer"]["value"]


def test_topk_gap_helper():
    l = np.array([[3.0, 1.0, 2.0, 2.0]], np.float32)
    assert oracle.topk_gap(l, 1)[0] == 1.0 and oracle.topk_gap(l, 2)[0] == 0.0
    assert np.isinf(oracle.topk_gap(l, 4)[0])
