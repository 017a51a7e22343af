"""Pins of the packing density and workload shapes to the model facts the
pages print (tests/golden/maple_preview_facts.json, each fact with its
citation).  The pages give no worked example of the layer itself."""
import json
import os

import numpy as np

from ternary_weight_moe_amd import synth as S
from ternary_weight_moe_amd import _native as N

FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "maple_preview_facts.json")))["facts"]


def fact(name):
    return FACTS[name]["value"]


def test_stack_workload_has_the_printed_shape():
    for name in ("decode_stack", "batched_stack_zipf"):
        w = S.WORKLOADS[name]
        assert w.n_layers == fact("layers")
        assert w.n_experts == fact("experts")
        assert w.top_k == fact("top_k")
    for name in ("decode_layer", "prefill_4096", "prefill_16384"):
        w = S.WORKLOADS[name]
        assert (w.n_experts, w.top_k) == (fact("experts"), fact("top_k"))


def test_layout_stores_two_bits_per_weight():
    # the host packer turns rows x cols ternary values into rows*cols*bits/8 bytes
    rng = np.random.default_rng(7)
    rows, cols = 48, 256
    w = rng.integers(-1, 2, size=(rows, cols), dtype=np.int8)
    assert set(np.unique(w)) <= set(fact("weight_values"))
    packed = N.maple_ternary_pack_host(w)
    assert packed.nbytes * 8 == rows * cols * fact("weight_bits")


def test_expert_shapes_fit_the_printed_parameter_counts():
    w = S.WORKLOADS["decode_stack"]
    per_expert = 3 * w.hidden * w.inter             # gate, up, down
    total_expert = w.n_layers * w.n_experts * per_expert
    active_expert = w.n_layers * w.top_k * per_expert
    # expert weights are most, but not all, of the printed totals (attention,
    # embeddings and the head are the rest)
    assert 0.85 * fact("total_params") < total_expert < fact("total_params")
    assert active_expert < fact("active_params")
    # at 2 bits per weight, the whole printed model fits the printed checkpoint
    packed_model = fact("total_params") * fact("weight_bits") / 8
    assert packed_model < fact("checkpoint_bytes") < 1.1 * packed_model
    packed_experts = total_expert * fact("weight_bits") // 8
    assert packed_experts == w.n_layers * w.n_experts * 3 * w.hidden * w.inter // 4
