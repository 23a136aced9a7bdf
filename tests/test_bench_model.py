"""The bench's algorithmic byte and FLOP model (host arithmetic only, no GPU):
the figures DESIGN's roofline rests on, recomputed from the model shape."""
import bench
from block_diffusion_decoding_dg_amd import synth


def test_full_step_bytes_and_roofline():
    w = synth.WORKLOADS["full"]
    d, hd, es = w.d_model, w.head_dim, 2
    touched = [58.0] * w.n_layers
    b = bench.step_bytes(w, 4096, 256, touched)
    dense = ((16 + 16) * hd * d + 16 * hd * d + 128 * d + 3 * d * 2112) * es
    expert = 3 * 704 * d * es
    kv = 30 * 2 * 8 * hd * es
    assert b == 30 * dense + 30 * 58 * expert + (4096 + 256) * kv + w.vocab * d * es
    # the KV-only part of a second request in the same step
    assert bench.step_bytes(w, 4096, 256, touched, weights=False) == (4096 + 256) * kv
    f = bench.step_flops(w, 4096, 256, 128)
    assert abs(max(b / 8e12, f / 2.5e15) * 1e3 - 3.31) < 0.02  # ms, HBM-bound
    # every expert touched: the bound quoted for uniform routing (about 6.4 ms)
    b128 = bench.step_bytes(w, 4096, 256, [128.0] * 30)
    assert 6.3 < b128 / 8e12 * 1e3 < 6.5


def test_self_cond_adds_its_bytes():
    w, ws = synth.WORKLOADS["full"], synth.WORKLOADS["full_sc"]
    t = [58.0] * w.n_layers
    extra = bench.step_bytes(ws, 4096, 256, t) - bench.step_bytes(w, 4096, 256, t)
    assert extra == w.vocab * w.d_model * 2 + 256 * w.vocab * 12 + 3 * w.d_model * 256 * 2


def test_expert_up_bytes_by_format():
    for name, per_weight in (("full", 2.0), ("full_fp8", 1.0), ("full_mxfp4", 0.5 + 1 / 32)):
        w = synth.WORKLOADS[name]
        m = bench.expert_matrix_bytes(w, w.expert_hidden, w.d_model)
        scale = 4 * w.expert_hidden if name == "full_fp8" else 0
        assert m == w.expert_hidden * w.d_model * per_weight + scale
