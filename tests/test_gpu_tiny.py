"""GPU parity on the tiny fp32 workload (vocab 512, d 64, 2 layers, 4/2 heads of
16, 8 experts top-2 + shared, 64-token prompt, one 256-token canvas, tau 0.5,
64-step cap), plus the crafted sampler and LM-head cases that random weights
never reach.  Every result is compared with the oracle on the same seeded
inputs."""
import numpy as np
import pytest
import torch

import oracle
from oracle import philox
from block_diffusion_decoding_dg_amd import dg, synth
from tests import helpers
from tests.gpu_common import (check_step, log, make_decoder, normwise, rel_l2, to_gpu)

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS["tiny"]


@pytest.fixture(scope="module")
def setup():
    tw = synth.make_weights(W, seed=0)
    return tw, to_gpu(tw), helpers.oracle_config(W), helpers.oracle_weights(W, tw)


@pytest.mark.parametrize("seed,block,step,n,vocab", [
    (0, 0, 0, 256, 512), (7, 3, 41, 256, 32768), (2 ** 63 + 5, 1, 255, 1000, 262144), (11, 0, 1, 37, 1000),
    (3, 9, 2, 1, 7)])
def test_philox_tokens_bit_exact(seed, block, step, n, vocab):
    log("philox", seed, block, step, n, vocab)
    out = torch.empty(n, dtype=torch.int32, device="cuda")
    dg.dg_philox_tokens(seed, block, step, n, vocab, out)
    ref = philox.draw_tokens(seed, block, step, np.arange(n), vocab)
    assert np.array_equal(out.cpu().numpy(), ref)


def _cache_check(dec, st, ocfg, P, tol, req=0):
    for l in range(ocfg.n_layers):
        k, vt = dec.kv_views(req, l)
        kg = k[:, :P, :].float().cpu().numpy().transpose(1, 0, 2)
        vg = vt[:, :, :P].float().cpu().numpy().transpose(2, 0, 1)
        assert normwise(kg.reshape(P, -1), st.cache_k[l][:P].reshape(P, -1)) < tol, ("K", l)
        assert normwise(vg.reshape(P, -1), st.cache_v[l][:P].reshape(P, -1)) < tol, ("V", l)


def test_tiny_full_block_free_running(setup):
    tw, twg, ocfg, ow = setup
    prompt = synth.make_prompt(W, seed=0)
    seed = 1234
    dec = make_decoder(W, twg)
    log("tiny: prefill")
    dec.dg_prefill(0, prompt, seed)
    st = oracle.new_request(ocfg, seed, W.max_ctx)
    oracle.prefill(st, prompt, ocfg, ow, oracle.Precision())
    _cache_check(dec, st, ocfg, len(prompt), 1e-4)
    scfg = oracle.SamplerConfig(W.tau, W.max_steps)
    n_resync = 0
    steps = 0
    while True:
        r, resync, info, _ = check_step(W, dec, st, ocfg, scfg, ow, oracle.Precision())
        n_resync += resync
        steps += 1
        assert info["n_open"] == r.n_open
        if r.done:
            break
    log("tiny: %d steps, %d resyncs" % (steps, n_resync))
    assert steps == W.max_steps
    ids_g = dec.dg_commit_block(0)
    ids_o = oracle.commit_block(st, ocfg, ow, oracle.Precision())
    assert np.array_equal(ids_g, ids_o)
    _cache_check(dec, st, ocfg, len(prompt) + 256, 1e-4)
    assert dec.dg_get_request(0)["committed"] == len(prompt) + 256


def test_tiny_generate_matches_oracle(setup):
    tw, twg, ocfg, ow = setup
    prompt = synth.make_prompt(W, seed=5, length=100)
    w2 = synth.Workload(**{**W.__dict__, "prompt_len": 100, "n_out": 300, "max_steps": 6})
    dec = make_decoder(w2, twg, max_ctx=640)
    outs, stats = dec.dg_generate([prompt], 300, [77])
    ref, steps, _ = oracle.generate(prompt, 300, 77, ocfg, oracle.SamplerConfig(w2.tau, 6), ow, oracle.Precision())
    log("tiny generate stats", stats)
    assert np.array_equal(outs[0], ref)
    assert stats["steps"] == sum(steps) and stats["tokens"] == 512


def test_tiny_prefill_chunked_and_empty_prompt(setup):
    tw, twg, ocfg, ow = setup
    prompt = synth.make_prompt(W, seed=9, length=250)
    dec = make_decoder(W, twg, max_ctx=576, prefill_chunk=48)   # 6 chunks, ragged tail of 10
    dec.dg_prefill(0, prompt, 1)
    st = oracle.new_request(ocfg, 1, 576)
    oracle.prefill(st, prompt, ocfg, ow, oracle.Precision())
    _cache_check(dec, st, ocfg, 250, 1e-4)
    # an empty prompt: the canvas attends only to itself
    dec.dg_prefill(0, np.zeros(0, np.int32), 3)
    st0 = oracle.new_request(ocfg, 3, 576)
    oracle.prefill(st0, np.zeros(0, np.int64), ocfg, ow, oracle.Precision())
    scfg = oracle.SamplerConfig(W.tau, W.max_steps)
    check_step(W, dec, st0, ocfg, scfg, ow, oracle.Precision())


@pytest.mark.parametrize("t,pos0,causal", [(256, 64, 0), (37, 300, 1), (5, 0, 0), (200, 17, 1)])
def test_tiny_attention_op(setup, t, pos0, causal):
    tw, twg, ocfg, ow = setup
    dec = make_decoder(W, twg, max_ctx=512)
    dec.dg_set_committed(0, 0, 0)
    rng = np.random.default_rng(t + pos0)
    # committed prefix: seeded K/V written straight into the caller-owned cache
    pk = rng.standard_normal((pos0, ocfg.n_kv_heads, ocfg.head_dim)).astype(np.float32)
    pv = rng.standard_normal((pos0, ocfg.n_kv_heads, ocfg.head_dim)).astype(np.float32)
    k, vt = dec.kv_views(0, 1)
    k[:, :pos0, :] = torch.from_numpy(pk.transpose(1, 0, 2)).cuda()
    vt[:, :, :pos0] = torch.from_numpy(pv.transpose(1, 2, 0)).cuda()
    x = synth.make_normal((t, ocfg.d_model), seed=t, std=1.0)
    xg = x.cuda().contiguous()
    dec.dg_op_attention(0, 1, xg, pos0, causal)
    lw = ow.layers[1]
    xo = x.numpy().astype(np.float64)
    mask = None
    if causal:
        mask = np.arange(pos0 + t)[None, :] <= (pos0 + np.arange(t))[:, None]
    ref, tr = _attn_half(xo, pos0 + np.arange(t), lw, ocfg, pk.astype(np.float64), pv.astype(np.float64), mask)
    assert normwise(xg.cpu().numpy(), ref) < 1e-4


def _attn_half(x, pos, lw, cfg, kpre, vpre, mask):
    """Attention half only: the oracle's layer with the FFN skipped."""
    y, tr = oracle.layer_forward(x, pos, lw, cfg, oracle.Precision(), kpre, vpre, mask=mask, skip_ffn=True)
    return y, tr


@pytest.mark.parametrize("t", [1, 23, 256, 300])
def test_tiny_moe_op(setup, t):
    tw, twg, ocfg, ow = setup
    dec = make_decoder(W, twg)
    x = synth.make_normal((t, ocfg.d_model), seed=100 + t, std=1.0)
    xg = x.cuda().contiguous()
    ids = torch.empty((t, ocfg.top_k), dtype=torch.int32, device="cuda")
    gates = torch.empty((t, ocfg.top_k), dtype=torch.float32, device="cuda")
    dec.dg_op_moe(0, xg, ids, gates)
    xo = x.numpy().astype(np.float64)
    b = oracle.rmsnorm(xo, ow.layers[0].ffn_norm, ocfg.rms_eps)
    f, r, oids, ogates = oracle.moe(b, ow.layers[0], ocfg, oracle.Precision())
    from tests.gpu_common import compare_router, topk_gap
    tr = oracle.model.LayerTrace(router_logits=r, ids=oids, gates=ogates)
    flips = compare_router(ids.cpu().numpy(), gates.cpu().numpy(), tr, ocfg.top_k, 1e-5)
    keep = np.setdiff1d(np.arange(t), flips)
    assert normwise(xg.cpu().numpy()[keep], (xo + f)[keep]) < 1e-4


def test_tiny_lm_head_crafted_rows(setup):
    """Crafted head: final-norm gain 60 and rows mixing E[t] with a random
    direction, so entropies span ~0 .. ln V; duplicated embedding rows give exact
    logit ties (argmax must take the lower id); zero rows give uniform logits."""
    tw, twg, ocfg, ow = setup
    rng = np.random.default_rng(4)
    emb = tw["embed"].clone()
    emb[300] = emb[17]
    emb[401] = emb[5]
    twc = dict(tw)
    twc["embed"] = emb
    twc["final_norm"] = torch.full_like(tw["final_norm"], 60.0)
    dec = make_decoder(W, to_gpu(twc))
    owc = helpers.oracle_weights(W, twc)
    n = 256
    toks = rng.integers(0, W.vocab, n)
    toks[:8] = 17
    toks[8:16] = 5
    mix = rng.uniform(0.0, 1.0, n) ** 2
    mix[:16] = 0.0  # the tie rows point exactly along E[17] / E[5]
    e = owc.embed[toks]
    e = e / np.linalg.norm(e, axis=1, keepdims=True)
    u = rng.standard_normal((n, ocfg.d_model))
    u -= np.sum(u * e, axis=1, keepdims=True) * e
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    h = (np.sqrt(1 - mix)[:, None] * e + np.sqrt(mix)[:, None] * u).astype(np.float32)
    h[250:] = 0.0  # uniform logits: H = ln V, argmax 0
    hg = torch.from_numpy(h).cuda()
    ent, lse, am = dec.dg_op_lm_head(hg)
    o = oracle.lm_head_stats(h.astype(np.float64), owc.embed, owc.final_norm, ocfg, oracle.Precision(),
                             keep_logits=True)
    eg = ent.cpu().numpy()
    assert np.all(np.abs(eg - o["entropy"]) <= 1e-4 * np.maximum(o["entropy"], 1.0)), np.abs(eg - o["entropy"]).max()
    assert np.all(np.abs(lse.cpu().numpy() - o["lse"]) <= 1e-4 * np.maximum(np.abs(o["lse"]), 1.0))
    from tests.gpu_common import topk_gap
    gap = topk_gap(o["logits"].astype(np.float32), 1)
    amg = am.cpu().numpy()
    for i in np.nonzero(amg != o["argmax"])[0]:
        assert gap[i] < 1e-3, (i, amg[i], o["argmax"][i], gap[i])
    assert np.all(amg[250:] == 0)
    assert np.all(o["argmax"][:8] == 17) and np.all(amg[:8] == 17)    # tie 17/300 -> 17
    assert np.all(o["argmax"][8:16] == 5) and np.all(amg[8:16] == 5)  # tie 5/401 -> 5
    assert o["entropy"].min() < 0.05 and (o["entropy"] < W.tau).sum() > 10
    log("lm head crafted: entropy range %.3g..%.3g, %d below tau" % (o["entropy"].min(), o["entropy"].max(),
                                                                   (o["entropy"] < W.tau).sum()))


@pytest.mark.parametrize("trial", range(6))
def test_tiny_sampler_crafted(setup, trial):
    """Threshold path, ties, values equal to tau, the cap: bit-exact with the oracle."""
    tw, twg, ocfg, ow = setup
    dec = make_decoder(W, twg)
    dec.dg_set_committed(0, 64, 99 + trial)
    rng = np.random.default_rng(trial)
    C = 256
    tau = W.tau
    H = np.round(rng.uniform(0.0, 1.2, C), 2).astype(np.float32)   # many ties, some == tau
    if trial == 1:
        H[:] = 0.7                                                   # all tied above tau
    am = rng.integers(0, W.vocab, C).astype(np.int32)
    acc = rng.random(C) < (0.0 if trial == 0 else 0.4)
    ids = rng.integers(0, W.vocab, C).astype(np.int32)
    step = [1, 5, 63, 64, 64, 30][trial]
    block = trial
    dec.dg_set_canvas(0, ids, acc, step - 1, block)
    info = dec.dg_op_sample(0, torch.from_numpy(H).cuda(), torch.from_numpy(am).cuda(), step)
    ids_g, acc_g = dec.dg_get_canvas(0)
    acc_e, acc_f = oracle.sampler_decide(H, am, acc, tau, step, W.max_steps)
    take = acc_e | acc_f
    ids_o = ids.copy()
    ids_o[take] = am[take]
    still = ~(acc | take)
    pos = np.nonzero(still)[0]
    ids_o[pos] = philox.draw_tokens(99 + trial, block, step, pos, W.vocab)
    assert np.array_equal(acc_g, acc | take)
    assert np.array_equal(ids_g, ids_o)
    assert info["n_accepted"] == acc_e.sum() and info["n_forced"] == acc_f.sum()
    assert info["n_open"] == still.sum() and info["done"] == int(still.sum() == 0)


# ------------------------------------------------ entropy-budget sampler ----

def _budget_ref(H, am, ids, acc, prev, step, seed, block, budget, stop, cap):
    """The oracle's budget rule applied to one call of the sampler op."""
    canvas = np.where(acc, ids, am)
    e, f, stopped = oracle.budget_decide(H, am, acc, canvas, prev, budget, stop, step, cap)
    take = e | f
    ids2 = ids.copy()
    ids2[take] = am[take]
    still = ~(acc | take)
    pos = np.nonzero(still)[0]
    ids2[pos] = philox.draw_tokens(seed, block, step, pos, W.vocab)
    return ids2, acc | take, e, f, still, canvas, stopped


@pytest.mark.parametrize("trial", range(8))
def test_tiny_sampler_budget_crafted(setup, trial):
    """Budget rule through the sampler op, three successive calls per case (the
    second and third see the previous argmax canvas): spread entropies, sums
    landing exactly on the budget, ties, zeros, NaN / inf / negative inputs, the
    cap and the early stop.  Bit-exact with the oracle."""
    tw, twg, ocfg, ow = setup
    rng = np.random.default_rng(100 + trial)
    C = 256
    budget, stop, cap = 0.1, 0.005, W.max_steps
    if trial == 1:
        budget = 0.125
        H = (rng.integers(0, 9, C) / 256.0).astype(np.float32)     # binary-exact; sums land on 0.125
    elif trial == 2:
        H = np.zeros(C, np.float32)
    elif trial == 3:
        H = np.full(C, 0.03, np.float32)
    elif trial == 4:
        H = rng.uniform(1, 5, C).astype(np.float32)
    elif trial == 5:
        H = rng.exponential(0.02, C).astype(np.float32)
        H[rng.choice(C, 12, replace=False)] = [np.nan, np.inf, -1e-7, -0.0, 0.0, 64.0, 65.0, 1e-30, np.nan,
                                               -np.inf, 3e-45, 0.1]
    elif trial in (6, 7):
        budget = 0.0
        H = rng.uniform(0, 0.008, C).astype(np.float32)             # mean below 0.005
    else:
        H = rng.exponential(0.01, C).astype(np.float32)
    seed = 500 + trial
    dec = make_decoder(W, twg, sampler="budget", budget=budget, stop_entropy=stop)
    dec.dg_set_committed(0, 64, seed)
    am = rng.integers(0, W.vocab, C).astype(np.int32)
    acc = rng.random(C) < (0.0 if trial in (2, 3, 6, 7) else 0.3)
    ids = rng.integers(0, W.vocab, C).astype(np.int32)
    block = trial
    step0 = cap - 2 if trial == 4 else 1
    dec.dg_set_canvas(0, ids, acc, step0 - 1, block)
    prev = None
    for call in range(3):
        step = step0 + call
        if trial == 7 and call == 1:
            am = am.copy()
            am[np.nonzero(~acc)[0][-1]] ^= 1                         # one open argmax moves: no stop yet
        info = dec.dg_op_sample(0, torch.from_numpy(H).cuda(), torch.from_numpy(am).cuda(), step)
        ids_g, acc_g = dec.dg_get_canvas(0)
        ids_o, acc_o, e, f, still, prev, stopped = _budget_ref(H, am, ids, acc, prev, step, seed, block, budget,
                                                               stop, cap)
        log("budget trial %d call %d: %d by budget, %d forced, %d open, stop %s"
            % (trial, call, e.sum(), f.sum(), still.sum(), stopped))
        assert np.array_equal(acc_g, acc_o), (trial, call)
        assert np.array_equal(ids_g, ids_o), (trial, call)
        assert info["n_accepted"] == e.sum() and info["n_forced"] == f.sum()
        assert info["n_open"] == still.sum() and info["done"] == int(still.sum() == 0)
        if trial == 6:
            assert stopped == (call == 1)
        if trial == 7:
            assert stopped == (call == 2)
        ids, acc = ids_o, acc_o
        if still.sum() == 0:
            break


def _scaled_embed(tw, scale):
    """Tiny weights with the embedding (and so the tied LM head) scaled, which
    sharpens the predictions into the range the budget sampler works in."""
    tws = dict(tw)
    tws["embed"] = tw["embed"] * scale
    return to_gpu(tws), helpers.oracle_weights(W, tws)


def test_tiny_budget_block_free_running(setup):
    tw, _, ocfg, _ = setup
    twg, ow = _scaled_embed(tw, 10.0)
    prompt = synth.make_prompt(W, seed=0)
    seed = 4321
    dec = make_decoder(W, twg, sampler="budget")
    dec.dg_prefill(0, prompt, seed)
    st = oracle.new_request(ocfg, seed, W.max_ctx)
    oracle.prefill(st, prompt, ocfg, ow, oracle.Precision())
    scfg = oracle.SamplerConfig(W.tau, W.max_steps, mode="budget")
    gstate, steps, n_resync, per_step = {}, 0, 0, []
    while True:
        r, resync, info, _ = check_step(W, dec, st, ocfg, scfg, ow, oracle.Precision(),
                                     gstate=gstate)
        steps += 1
        n_resync += resync
        per_step.append(int(r.accept_entropy.sum()))
        assert info["n_open"] == r.n_open
        if r.done:
            break
    log("tiny budget: %d steps, accepted per step %s, %d resyncs" % (steps, per_step, n_resync))
    assert 1 < steps < W.max_steps and max(per_step) > 1
    ids_g = dec.dg_commit_block(0)
    ids_o = oracle.commit_block(st, ocfg, ow, oracle.Precision())
    assert np.array_equal(ids_g, ids_o)


def test_tiny_budget_generate_matches_oracle(setup):
    tw, _, ocfg, _ = setup
    twg, ow = _scaled_embed(tw, 12.0)
    prompt = synth.make_prompt(W, seed=6, length=80)
    dec = make_decoder(W, twg, max_ctx=640, sampler="budget")
    outs, stats = dec.dg_generate([prompt], 400, [91])
    ref, steps, _ = oracle.generate(prompt, 400, 91, ocfg, oracle.SamplerConfig(W.tau, W.max_steps, mode="budget"),
                                    ow, oracle.Precision())
    log("tiny budget generate: steps %s, stats %s" % (steps, stats))
    assert np.array_equal(outs[0], ref)
    assert stats["steps"] == sum(steps) and sum(steps) < 2 * W.max_steps
