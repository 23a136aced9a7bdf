"""The full-size synthetic workload against the figures the pages print
(tests/golden/pages_model_figures.json, each value with its page and section)."""
import json
import os

import pytest

from block_diffusion_decoding_dg_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "pages_model_figures.json")


@pytest.fixture(scope="module")
def fig():
    with open(GOLDEN) as f:
        return {k: v["value"] for k, v in json.load(f).items() if not k.startswith("_")}


@pytest.mark.parametrize("name", ["full", "full_x8", "full_long"])
def test_full_workloads_have_the_pages_model_shape(fig, name):
    w = synth.WORKLOADS[name]
    assert w.n_experts == fig["experts"] and w.top_k == fig["routed_active"]
    assert w.canvas_len == fig["canvas_tokens"]
    # one shared expert: the step adds exactly one dense SwiGLU FFN per layer
    assert fig["shared_experts"] == 1 and w.shared_hidden > 0
    total = w.param_count() / 1e9
    active = w.active_param_count() / 1e9
    assert round(total, 1) == fig["total_params_billion"], total
    assert abs(active - fig["active_params_billion"]) < 0.1, active


def test_pages_step_arithmetic_is_coherent(fig):
    """The pages' own numbers agree with each other: throughput = tokens per pass
    / time per pass, and a 256-token canvas at ~20 tokens per pass takes ~12
    passes.  This is what the bench's output tok/s means (decode only)."""
    tok_per_step = fig["h100_tps_diffusion"] * fig["h100_ms_per_step"] / 1e3
    assert abs(tok_per_step - fig["tokens_per_pass"]) < 0.5
    assert abs(fig["canvas_tokens"] / tok_per_step - fig["mean_effective_steps"]) < 1.0
