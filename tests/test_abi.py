"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, sizes workspaces and rejects bad arguments before touching the
device."""
import ctypes
import os
import re

import pytest

from block_diffusion_decoding_dg_amd import dg, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", fn)).read()
            names |= set(re.findall(r"^\s*(?:dg_status|void|int32_t|const char\*)\s+(dg_\w+)\s*\(", txt, re.M))
    return names


@pytest.fixture(scope="module")
def lib():
    return dg.load()


def test_every_declared_symbol_is_exported(lib):
    declared = _declared()
    assert {"dg_create", "dg_prefill", "dg_denoise_step", "dg_commit_block", "dg_generate"} <= declared
    for name in declared:
        assert hasattr(lib, name), name
    assert declared == set(dg.EXPORTS)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workspace_sizes(name):
    w = synth.WORKLOADS[name]
    kv, scratch = dg.dg_workspace_size(dg.model_config(w))
    es = 2 if w.dtype == "bf16" else 4
    assert kv == w.n_requests * w.n_layers * 2 * w.n_kv_heads * w.max_ctx * w.head_dim * es
    assert scratch > 0


def _cfg(**kw):
    c = dg.model_config(synth.WORKLOADS["tiny"])
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("bad", [dict(canvas_len=128), dict(head_dim=24), dict(vocab=500), dict(max_ctx=300),
                                 dict(n_q_heads=3), dict(top_k=17), dict(max_requests=17), dict(dtype=7),
                                 dict(d_model=0), dict(expert_hidden=100), dict(n_experts=300),
                                 # quantized experts need a bf16 model; 3 is no format
                                 dict(expert_format=1), dict(expert_format=2), dict(expert_format=3),
                                 # self-conditioning: bf16 models only, width a multiple of 64, at most 4096
                                 dict(self_cond_hidden=64), dict(self_cond_hidden=-64)])
def test_bad_configs_rejected(bad):
    with pytest.raises(dg.DgError) as e:
        dg.dg_workspace_size(_cfg(**bad))
    assert e.value.status == dg.DG_ERR_INVALID_ARG


def test_create_validates_before_device_work(lib):
    cfg = _cfg()
    scfg = dg.SamplerConfig(tau=0.5, max_steps=64)
    out = ctypes.c_void_p(123)
    # null weights
    st = lib.dg_create(ctypes.byref(cfg), ctypes.byref(scfg), None, None, 0, None, 0, None, ctypes.byref(out))
    assert st == dg.DG_ERR_INVALID_ARG and not out.value
    assert b"weights" in lib.dg_last_error(None)
    # weights present (dummy non-null pointers are never dereferenced before the size check)
    L = cfg.n_layers
    layers = (dg.LayerWeights * L)()
    for l in range(L):
        for n, _ in dg.LayerWeights._fields_:
            setattr(layers[l], n, 0x1000)
    w = dg.Weights(embed=0x1000, final_norm=0x1000, layers=layers)
    kv, sc = dg.dg_workspace_size(cfg)
    st = lib.dg_create(ctypes.byref(cfg), ctypes.byref(scfg), ctypes.byref(w), ctypes.c_void_p(0x1000), kv - 1,
                       ctypes.c_void_p(0x1000), sc, None, ctypes.byref(out))
    assert st == dg.DG_ERR_WORKSPACE
    bad = [dg.SamplerConfig(tau=-1.0, max_steps=64),
           dg.SamplerConfig(tau=0.5, max_steps=64, mode=2),
           dg.SamplerConfig(tau=0.5, max_steps=64, mode=1, budget=-0.1, stop_entropy=0.005),
           dg.SamplerConfig(tau=0.5, max_steps=64, mode=1, budget=float("nan"), stop_entropy=0.005),
           dg.SamplerConfig(tau=0.5, max_steps=64, mode=1, budget=0.1, stop_entropy=float("inf"))]
    for b in bad:
        st = lib.dg_create(ctypes.byref(cfg), ctypes.byref(b), ctypes.byref(w), ctypes.c_void_p(0x1000), kv,
                           ctypes.c_void_p(0x1000), sc, None, ctypes.byref(out))
        assert st == dg.DG_ERR_INVALID_ARG and not out.value, (b.mode, b.budget, b.stop_entropy)


def test_null_context_calls_fail_cleanly(lib):
    info = (dg.StepInfo * 1)()
    assert lib.dg_denoise_step(None, info) == dg.DG_ERR_INVALID_ARG
    assert lib.dg_kernel_timer_every(None, 1) == dg.DG_ERR_INVALID_ARG
    assert lib.dg_prefill(None, 0, None, 0, 0) == dg.DG_ERR_INVALID_ARG
    assert lib.dg_commit_block(None, 0, None) == dg.DG_ERR_INVALID_ARG
    assert lib.dg_philox_tokens(0, -1, 0, 4, 10, None, None) == dg.DG_ERR_INVALID_ARG
    lib.dg_destroy(None)


def test_every_launch_refusal_reaches_the_caller_as_a_status(lib):
    """Each launcher's refusal path (arguments its kernels do not implement):
    the launcher queues nothing and the entry point returns DG_ERR_UNSUPPORTED
    with the launch named, instead of stopping the process."""
    cases = dg.dg_debug_refusal_cases()
    assert len(cases) == 11
    names = ["bf16 streaming projection on a non-bf16 model", "bf16 streaming add projection on a non-bf16 model",
             "routed streaming projection on a non-bf16 model", "dense projection", "routed projection",
             "routed projection", "dense projection", "FFN norm", "combine and norm", "embedding transpose",
             "self-conditioning fold"]
    for (st, msg), name in zip(cases, names):
        assert st == dg.DG_ERR_UNSUPPORTED, (st, msg)
        assert msg == "launch refused: " + name
    buf = ctypes.create_string_buffer(8)
    assert lib.dg_debug_refusal_case(len(cases), buf, len(buf)) == dg.DG_ERR_INVALID_ARG
    assert lib.dg_debug_refusal_case(-1, None, 0) == dg.DG_ERR_INVALID_ARG


def test_self_cond_workspace():
    """Self-conditioning adds to the scratch exactly: the transposed embedding,
    the open rows' logits (fp32) and softmax (bf16), the split partial sums, the
    state, and the MLP's input and hidden rows (each carved on 256-byte
    boundaries); the KV cache is unchanged.  A width that is not a multiple of 64
    or above 4096 is rejected."""
    w, ws = synth.WORKLOADS["mid"], synth.WORKLOADS["mid_sc"]
    kv0, sc0 = dg.dg_workspace_size(dg.model_config(w))
    kv1, sc1 = dg.dg_workspace_size(dg.model_config(ws))
    assert kv1 == kv0
    rows, V, d, m = w.n_requests * w.canvas_len, w.vocab, w.d_model, ws.self_cond_hidden
    parts = [V * d * 2, rows * V * 4, rows * V * 2, 16 * rows * d * 4, rows * d * 4, rows * d * 2, rows * m * 2]
    assert sc1 - sc0 == sum((p + 255) // 256 * 256 for p in parts)
    for bad in (100, 8192):
        c = dg.model_config(ws)
        c.self_cond_hidden = bad
        with pytest.raises(dg.DgError) as e:
            dg.dg_workspace_size(c)
        assert e.value.status == dg.DG_ERR_INVALID_ARG
