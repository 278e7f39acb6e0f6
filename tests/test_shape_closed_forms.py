"""The layer's shape against the sizes the pages print (tests/golden/beam_layer_shape.json).

A SwiGLU expert with gate, up and down projections and no biases has 3*H*I
parameters.  The pages' own parameter counts, the experts' share of the model,
the BF16 checkpoint size and the per-GPU expert-parallel memory all follow from
that count, which leaves no room for extra per-expert parameters (biases, a
shared expert) in the layer the oracle implements.
"""
import json
import os

from synth import gen

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "beam_layer_shape.json")))


def v(k):
    return G[k]["value"]


def test_real_shape_matches_pages():
    w = gen.workload("decode")
    assert (w.hidden, w.inter, w.n_experts) == (v("hidden"), v("inter"), v("experts_per_layer"))
    assert (w.n_groups, w.n_experts // w.n_groups, w.topk_groups, w.top_k, w.alpha) == (8, 32, 4, 8, 2.5)


def test_params_per_expert():
    p = 3 * v("hidden") * v("inter")
    assert p == 39_321_600
    assert abs(p - v("params_per_expert_approx")) / v("params_per_expert_approx") < G["params_per_expert_approx"]["rel_tol"]


def test_expert_share_of_model():
    experts = v("moe_layers") * v("experts_per_layer") * 3 * v("hidden") * v("inter")
    share = 100.0 * experts / v("total_params")
    assert abs(share - v("expert_share_percent")) < G["expert_share_percent"]["abs_tol"]


def test_active_params_close_the_budget():
    """8 routed experts per MoE layer plus the replicated 8B reproduce the 23.4B active count."""
    active = v("moe_layers") * 8 * 3 * v("hidden") * v("inter") + v("replicated_params")
    assert abs(active - v("active_params")) / v("active_params") < 0.01


def test_bf16_checkpoint_size():
    gb = 2 * v("total_params") / 1e9
    assert abs(gb - v("bf16_checkpoint_GB")) < G["bf16_checkpoint_GB"]["abs_tol"]


def test_expert_parallel_memory():
    experts_bytes = 2 * v("moe_layers") * v("experts_per_layer") * 3 * v("hidden") * v("inter")
    repl = 2 * v("replicated_params")
    for n, key in ((16, "ep_GB_per_gpu_16"), (8, "ep_GB_per_gpu_8")):
        gb = (experts_bytes / n + repl) / 1e9
        assert abs(gb - v(key)) < G[key]["abs_tol"], (n, gb)
