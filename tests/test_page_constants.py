"""P-f: closed forms from the figures the pages print (tests/golden/page_constants.json).

These pin the layer shape used everywhere (hidden 5120, 256 experts of
three 5120 x 2560 matrices, 8 groups of 32, keep 4, top 8, scale 2.5): a
wrong shape constant would break one of the parameter sums the pages quote.
"""

import json
import os

import pytest

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")


@pytest.fixture(scope="module")
def page():
    with open(GOLDEN) as f:
        return {k: v for k, v in json.load(f).items() if not k.startswith("_")}


def test_workload_shape_matches_pages(page):
    B = workloads.BEAM
    assert B["hidden"] == page["hidden_size"]["value"]
    assert B["intermediate"] == page["moe_intermediate_size"]["value"]
    assert B["n_experts"] == page["n_experts"]["value"]
    assert B["n_group"] == page["n_group"]["value"]
    assert B["n_experts"] // B["n_group"] == page["group_size"]["value"]
    assert B["topk_group"] == page["topk_group"]["value"]
    assert B["top_k"] == page["top_k"]["value"]
    assert B["routed_scaling_factor"] == page["routed_scaling_factor"]["value"]
    assert page["moe_layers"]["value"] + page["dense_layers"]["value"] == page["n_layers"]["value"]


def test_parameter_arithmetic(page):
    H, I, E = 5120, 2560, 256
    per_expert = 3 * H * I
    assert per_expert == 39_321_600
    assert per_expert == pytest.approx(page["params_per_expert_approx"]["value"],
                                       rel=page["params_per_expert_approx"]["rel_tol"])
    L = page["moe_layers"]["value"]
    experts_total = L * E * per_expert
    replicated = page["replicated_params_B"]["value"] * 1e9
    total = experts_total + replicated
    assert total / 1e9 == pytest.approx(page["total_params_B"]["value"], abs=page["total_params_B"]["abs_tol"])
    share = 100.0 * experts_total / total
    assert share == pytest.approx(page["expert_share_of_params_pct"]["value"],
                                  abs=page["expert_share_of_params_pct"]["abs_tol"])
    active = L * page["top_k"]["value"] * per_expert + replicated
    assert active / 1e9 == pytest.approx(page["active_params_B"]["value"], abs=page["active_params_B"]["abs_tol"])
    # expert-parallel memory in BF16: expert bytes split over P devices plus the
    # replicated 16 GB on each
    for P, key in [(16, "ep16_h200_GB_per_gpu"), (8, "ep8_h200_GB_per_gpu")]:
        gb = (experts_total * 2 / P + replicated * 2) / 1e9
        assert gb == pytest.approx(page[key]["value"], abs=page[key]["abs_tol"])
    assert total * 2 / 1e12 == pytest.approx(page["bf16_checkpoint_TB"]["value"],
                                             abs=page["bf16_checkpoint_TB"]["abs_tol"])
