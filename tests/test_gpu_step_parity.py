"""Whole denoising steps against the oracle, with distinct weights in every
layer, at the mid-size shape and at the three full-size workloads: one canvas
over a 4096-row prefix, eight canvases over 4096-row prefixes each, and one
canvas over a 131072-row prefix.

The committed prefixes are synth.make_prefix_kv rows written into both sides'
caches (a CPU prefill of 4096 or 131072 prompt tokens through the full-size
model is out of reach; the prefill itself is checked against the oracle at the
mid shape in full and at the full shape on sampled rows, test_gpu_mid.py and
test_gpu_full.py).  Each test runs one step on both sides from the same state
and applies both comparisons of tests/step_parity.py: the free-running step
(the library's dg_denoise_step with its per-layer taps) and the teacher-forced
layer-by-layer check (the library's attention and MoE halves on the oracle's
own layer inputs), where the 1e-3 routing band holds."""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_decoding_dg_amd import synth
from tests import helpers, step_parity as sp
from tests.gpu_common import log, make_decoder

pytestmark = pytest.mark.gpu


def _run(wname, P, n_req, spread=None, logit_rows=8):
    """One step of the workload on both sides.  spread: the free-running bands;
    None computes them on this step with a second, plain-arithmetic oracle run."""
    w = synth.WORKLOADS[wname]
    log("%s: generating the model on the GPU (%d requests, %d-row prefixes)" % (wname, n_req, P))
    tw = synth.make_weights(w, seed=0, device="cuda")
    torch.cuda.synchronize()
    dec = make_decoder(w, tw, max_requests=n_req, max_ctx=P + w.canvas_len)
    dec.enable_taps()
    seeds = list(range(n_req))  # request r draws with seed r
    for r in range(n_req):
        sp.fill_prefix(dec, w, r, P, prefix_seed=100 + r)
        dec.dg_set_committed(r, P, seeds[r])
    before = [dict(seed=seeds[r], block=0, step=0) for r in range(n_req)]
    infos = dec.dg_denoise_step()
    assert all(infos[r]["active"] and infos[r]["step"] == 1 for r in range(n_req))
    log("%s: GPU step done; oracle step (float64, bf16 model)" % wname)
    ocfg = helpers.oracle_config(w)
    scfg = oracle.SamplerConfig(tau=w.tau, max_steps=w.max_steps)
    ow = sp.oracle_weights(tw)
    prec = helpers.oracle_precision(w)
    states = [sp.oracle_request(w, P, 100 + r, seeds[r]) for r in range(n_req)]
    results = oracle.denoise_step_batch(states, ocfg, scfg, ow, prec, keep_logits=True)
    plain_results = None
    if spread is None:
        log("%s: plain-arithmetic oracle step" % wname)
        pst = [sp.oracle_request(w, P, 100 + r, seeds[r]) for r in range(n_req)]
        plain_results = oracle.denoise_step_batch(pst, ocfg, scfg, sp.oracle_weights(tw), oracle.Precision(False),
                                                  keep_logits=True)
        spread = sp.oracle_spread(results, plain_results, w.top_k)
        log("%s: oracle spread (bf16 model vs exact arithmetic): routing differences per layer %s, widest gap decided "
            "differently %s; logits rel L2 median %.2e max %.2e; entropy %.2e; argmax differences %d (widest gap overturned or moved %.1e)"
            % (wname, spread["router_flips"].tolist(), ["%.1e" % v for v in spread["router_gap"]], spread["logit_med"],
               spread["logit_max"], spread["entropy"], spread["argmax_flips"], spread["argmax_gap"]))
    stats = {}
    # the free-running comparison reads the step's own taps and canvas first; the
    # teacher-forced ops then overwrite the canvas rows' cache entries
    err = None
    try:
        sp.free_running(dec, w, list(range(n_req)), results, before, stats, spread, plain_results,
                        n_logit_rows=logit_rows)
    except AssertionError as e:  # report after the teacher-forced check has run too
        err = e
    log("%s: teacher-forced layers" % wname)
    sp.teacher_forced(dec, w, list(range(n_req)), results, [P] * n_req, stats)
    if err is not None:
        raise err
    dec.close()
    del tw
    torch.cuda.empty_cache()
    stats["spread"] = spread
    return stats


def test_mid_step_parity():
    """The mid-size model (8 layers, 32 experts top-4) over a 1024-row prefix."""
    st = _run("mid", 1024, 1)
    log("mid: %s" % {k: v for k, v in st.items() if k not in ("layer_err", "flip_gaps", "spread")})


@pytest.mark.timeout(900)
def test_full_step_parity_one_canvas():
    """The 4096-in workload: one canvas over a 4096-row prefix, all 30 layers."""
    st = _run("full", 4096, 1)
    log("full: %s" % {k: v for k, v in st.items() if k not in ("layer_err", "flip_gaps", "spread")})


@pytest.mark.timeout(1200)
def test_full_step_parity_eight_canvases():
    """The 8-request workload: eight canvases, each over its own 4096-row prefix,
    denoised in one step (2048 rows through every layer)."""
    st = _run("full_x8", 4096, 8, logit_rows=4)
    log("full_x8: %s" % {k: v for k, v in st.items() if k not in ("layer_err", "flip_gaps", "spread")})


@pytest.mark.timeout(1200)
def test_full_step_parity_long_prefix():
    """The long-context workload: one canvas over a 131072-row prefix."""
    st = _run("full_long", 131072, 1)
    log("full_long: %s" % {k: v for k, v in st.items() if k not in ("layer_err", "flip_gaps", "spread")})
