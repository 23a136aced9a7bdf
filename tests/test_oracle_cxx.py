"""Pins of the C++ oracle (oracle/cxx): against the numpy oracle, an
independent implementation that is itself pinned to closed forms and library
routines (tests/test_oracle_pins.py), and against numpy's own Philox4x64-10.
CPU only."""
import numpy as np
import pytest

import oracle
from oracle import cxx, philox
from block_diffusion_decoding_dg_amd import synth
from tests import helpers


@pytest.fixture(scope="module", autouse=True)
def built():
    cxx.build()


def test_philox_tokens_match_the_numpy_oracle():
    rng = np.random.default_rng(3)
    for _ in range(20):
        seed = int(rng.integers(0, 2 ** 63))
        block, step = int(rng.integers(0, 50)), int(rng.integers(0, 300))
        vocab = int(rng.choice([512, 1000, 32768, 262144]))
        pos = np.arange(256)
        assert np.array_equal(cxx.philox_tokens(seed, block, step, pos, vocab),
                              philox.draw_tokens(seed, block, step, pos, vocab))


def _tiny(seed=0):
    w = synth.WORKLOADS["tiny"]
    tw = synth.make_weights(w, seed=seed)
    return w, tw, helpers.oracle_config(w), helpers.oracle_weights(w, tw)


def test_tiny_generation_matches_the_numpy_oracle():
    """The tiny fp32 model's whole generation: identical tokens and step counts,
    and every step's entropies equal to float64 rounding."""
    w, tw, ocfg, ow = _tiny()
    m = cxx.Model(ocfg, tw, bf16_points=False)
    prompt = synth.make_prompt(w, seed=0)
    scfg = oracle.SamplerConfig(tau=w.tau, max_steps=w.max_steps)
    st_n = oracle.new_request(ocfg, 7, w.max_ctx)
    oracle.prefill(st_n, prompt, ocfg, ow, oracle.Precision())
    st_c = cxx.new_request(m, 7, w.max_ctx)
    cxx.prefill(m, st_c, prompt)
    for l in range(ocfg.n_layers):
        np.testing.assert_allclose(st_c.cache_k[l][:64], st_n.cache_k[l][:64], rtol=0, atol=1e-12)
        np.testing.assert_allclose(st_c.cache_v[l][:64], st_n.cache_v[l][:64], rtol=0, atol=1e-12)
    for s in range(w.max_steps):
        rn = oracle.denoise_step(st_n, ocfg, scfg, ow, oracle.Precision())
        rc = cxx.denoise_step(m, st_c, w.tau, w.max_steps)
        np.testing.assert_allclose(rc["entropy"], rn.entropy, rtol=1e-12, atol=0)
        np.testing.assert_allclose(rc["lse"], rn.lse, rtol=1e-12, atol=0)
        assert np.array_equal(rc["argmax"], rn.argmax)
        assert np.array_equal(rc["ids_after"], rn.ids_after) and np.array_equal(rc["accepted_after"],
                                                                              rn.accepted_after)
        for l in range(ocfg.n_layers):
            assert np.array_equal(np.sort(rc["layers"][l][3], axis=1), np.sort(rn.layers[l].ids, axis=1))
        if rn.done:
            break
    assert rc["done"] and rn.done
    out_n = oracle.commit_block(st_n, ocfg, ow, oracle.Precision())
    out_c = cxx.commit_block(m, st_c)
    assert np.array_equal(out_n, out_c)
    for l in range(ocfg.n_layers):
        np.testing.assert_allclose(st_c.cache_k[l][:st_c.P], st_n.cache_k[l][:st_n.P], rtol=0, atol=1e-12)


def test_mid_step_matches_the_numpy_oracle_with_bf16_points():
    """The mid-size bf16 model (8 layers, 32 experts top-4, vocab 32768) with the
    bf16 rounding points: a 96-token prefill and one denoising step through every
    layer agree with the numpy oracle to float64 rounding -- the same roundings
    are taken, so routing and the accepted position are identical."""
    w = synth.WORKLOADS["mid"]
    tw = synth.make_weights(w, seed=0)
    ocfg = helpers.oracle_config(w)
    ow = helpers.oracle_weights(w, tw)
    prec = oracle.Precision(bf16_points=True)
    m = cxx.Model(ocfg, tw, bf16_points=True)
    prompt = synth.make_prompt(w, seed=0, length=96)
    st_n = oracle.new_request(ocfg, 3, 96 + 256)
    oracle.prefill(st_n, prompt, ocfg, ow, prec)
    st_c = cxx.new_request(m, 3, 96 + 256)
    cxx.prefill(m, st_c, prompt)
    rn = oracle.denoise_step(st_n, ocfg, oracle.SamplerConfig(tau=w.tau, max_steps=w.max_steps), ow, prec)
    rc = cxx.denoise_step(m, st_c, w.tau, w.max_steps)
    for l in range(ocfg.n_layers):
        np.testing.assert_allclose(rc["layers"][l][0], rn.layers[l].k, rtol=0, atol=1e-9)
        np.testing.assert_allclose(rc["layers"][l][2], rn.layers[l].router_logits, rtol=0, atol=1e-9)
        assert np.array_equal(rc["layers"][l][3], rn.layers[l].ids)
        np.testing.assert_allclose(rc["layers"][l][4], rn.layers[l].gates, rtol=0, atol=1e-12)
    np.testing.assert_allclose(rc["hidden"], rn.hidden, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(rc["entropy"], rn.entropy, rtol=1e-11, atol=0)
    assert np.array_equal(rc["argmax"], rn.argmax)
    assert np.array_equal(rc["ids_after"], rn.ids_after)
