"""Whole denoising steps of the GPU library against the oracle, at any workload
shape: the harness shared by tests/test_gpu_step_parity.py.

Both sides start from the same seeded inputs and neither takes a value from
the other:
  * weights: synth.make_weights on the GPU; the oracle reads host float64
    copies of the same tensors, one layer at a time and each routed expert only
    when some row is routed to it (oracle.stream), so that the full-size model
    (50 GB of bf16 weights) never has to sit in host memory as float64;
  * the committed prefix: synth.make_prefix_kv keys and values, written into
    the library's cache and read, as float64, by the oracle (oracle.stream);
  * the canvas: Philox at step 0, drawn by each side itself.

Two comparisons per step:
  * teacher_forced(): layer by layer, the library's attention half and MoE half
    (dg_op_attention, dg_op_moe: the kernels and launch shapes of the step) run
    on the oracle's own input rows of that layer, so both sides take every
    routing decision from the same values: expert sets bit-exact except where
    the oracle's k-th - (k+1)-th router logit gap is below GAP (1e-3), gates
    within GATE_TOL, each half's update within RL2 relative L2 per row;
  * free_running(): the library's own dg_denoise_step against the oracle's
    step, with the per-layer rows read back through the debug taps.  Every bf16
    rounding point turns a sub-ulp difference upstream into whole-ulp flips in a
    few elements, so over many layers two correct bf16 implementations drift
    apart by about an ulp.  The bands are therefore SPREAD_MARGIN (2) times the
    oracle's own spread (oracle_spread: the bf16 model against exact
    arithmetic, on the same step), never a measure of the library's error:
    routing differences only at router gaps below twice the widest the two
    oracles decide differently in this or an earlier layer; hidden rows and
    logits within twice the oracles' median and largest spread; entropies
    within twice the entropy spread; argmax equal except at top-1 - top-2 gaps
    below twice the widest the rounding overturns or moves; the accepted
    position the oracle's except where its two lowest open entropies lie within
    twice the entropy band; accepted tokens and Philox re-draws exact.  Every
    band has the floor of the teacher-forced one (GAP, RL2, H_TOL).
"""
import numpy as np
import torch

import oracle
from oracle import philox, stream
from block_diffusion_decoding_dg_amd import synth
from tests import helpers
from tests.gpu_common import GAP, H_TOL, RL2, SPREAD_MARGIN, log, oracle_spread, rel_l2, topk_gap

GATE_TOL = 1e-3   # teacher-forced gates: with equal inputs the router logits differ only where the fp32
                  # norm rounds an element of the normalised row to the other bf16 neighbour


def _f64(t):
    return stream.f64(t)


def oracle_weights(tw_gpu):
    """The oracle's weights over the GPU tensors of synth.make_weights, copied to
    host float64 one layer (and one routed expert) at a time."""
    return stream.lazy_weights(tw_gpu)


def oracle_request(w, P, prefix_seed, seed):
    """An oracle request whose committed length is P with the synthetic prefix
    synth.make_prefix_kv(w, P, layer, prefix_seed), generated on the GPU."""
    return stream.request_with_prefix(w.n_layers, P, w.canvas_len,
                                      lambda l: synth.make_prefix_kv(w, P, l, prefix_seed, device="cuda"), seed)


def fill_prefix(dec, w, req, P, prefix_seed):
    """Write the synthetic prefix of request req into the library's cache and
    set its committed length."""
    for l in range(w.n_layers):
        k, vt = dec.kv_views(req, l)
        kk, vv = synth.make_prefix_kv(w, P, l, prefix_seed, device="cuda")
        k[:, :P, :] = kk
        vt[:, :, :P] = vv.transpose(1, 2)
    torch.cuda.synchronize()


def teacher_forced(dec, w, reqs, results, Ps, stats):
    """Run the library's attention and MoE halves of every layer on the oracle's
    inputs of that layer (results: the oracle's StepResults of the requests in
    reqs, whose committed lengths are Ps) and compare."""
    ocfg = helpers.oracle_config(w)
    C, k = w.canvas_len, w.top_k
    n_rows = C * len(reqs)
    flips_total = 0
    for l in range(w.n_layers):
        # attention half, one request at a time (its own prefix and canvas)
        x_attn_g = []
        for i, (req, r) in enumerate(zip(reqs, results)):
            tr = r.layers[l]
            x = torch.from_numpy(tr.x_in.astype(np.float32)).cuda()
            dec.dg_op_attention(req, l, x, Ps[i], False)
            xg = x.cpu().numpy().astype(np.float64)
            d_g, d_o = xg - tr.x_in.astype(np.float32), tr.x_attn - tr.x_in
            errs = [rel_l2(d_g[t], d_o[t]) for t in range(C)]
            stats.setdefault("attn_rl2", []).append(float(np.max(errs)))
            stats.setdefault("attn_rl2_med", []).append(float(np.median(errs)))
            assert max(errs) <= RL2, ("attention half", l, i, max(errs))
            x_attn_g.append(xg)
        # MoE half over all the step's rows at once (the step's launch shape)
        xa = np.concatenate([r.layers[l].x_attn for r in results]).astype(np.float32)
        x = torch.from_numpy(xa).cuda()
        ids = torch.empty((n_rows, k), dtype=torch.int32, device="cuda")
        gates = torch.empty((n_rows, k), dtype=torch.float32, device="cuda")
        dec.dg_op_moe(l, x, ids, gates)
        xg = x.cpu().numpy().astype(np.float64)
        ids, gates = ids.cpu().numpy(), gates.cpu().numpy()
        for i, r in enumerate(results):
            tr = r.layers[l]
            rows = slice(i * C, (i + 1) * C)
            x_next = r.layers[l + 1].x_in if l + 1 < w.n_layers else r.hidden
            gap = topk_gap(tr.router_logits.astype(np.float32), k)
            d_g, d_o = xg[rows] - xa[rows], x_next - tr.x_attn
            moe_errs = []
            for t in range(C):
                gi, gg = ids[rows][t], gates[rows][t]
                if set(gi.tolist()) != set(tr.ids[t].tolist()):
                    assert gap[t] < GAP, ("router set differs outside the band", l, i, t, gap[t])
                    flips_total += 1
                    continue
                og = dict(zip(tr.ids[t].tolist(), tr.gates[t].tolist()))
                for e, g in zip(gi.tolist(), gg.tolist()):
                    assert abs(g - og[e]) <= GATE_TOL, ("gate", l, i, t, e, g, og[e])
                e_ = rel_l2(d_g[t], d_o[t])
                moe_errs.append(e_)
                assert e_ <= RL2, ("MoE half", l, i, t, e_)
            stats.setdefault("moe_rl2", []).append(float(max(moe_errs)))
            stats.setdefault("moe_rl2_med", []).append(float(np.median(moe_errs)))
        log("  teacher-forced layer %2d: attention update rel L2 median %.2e max %.2e; MoE update median %.2e "
            "max %.2e" % (l, stats["attn_rl2_med"][-1], stats["attn_rl2"][-1], stats["moe_rl2_med"][-1],
                          stats["moe_rl2"][-1]))
    stats["tf_router_flips"] = flips_total
    # LM head on the oracle's final rows (the open ones): entropies and
    # log-sum-exp within H_TOL, argmax equal except at top-1 - top-2 gaps < GAP
    am_flips = 0
    for i, r in enumerate(results):
        open_ = np.nonzero(~r.accepted_before)[0]
        h = torch.from_numpy(r.hidden[open_].astype(np.float32)).cuda()
        ent, lse, am = (t.cpu().numpy() for t in dec.dg_op_lm_head(h))
        dH = np.abs(ent.astype(np.float64) - r.entropy[open_])
        dL = np.abs(lse.astype(np.float64) - r.lse[open_])
        stats.setdefault("tf_lm_dH", []).append(float(dH.max()))
        stats.setdefault("tf_lm_dlse", []).append(float(dL.max()))
        assert dH.max() <= H_TOL and dL.max() <= H_TOL, ("LM head", i, float(dH.max()), float(dL.max()))
        gap = topk_gap(r.logits[open_].astype(np.float32), 1)
        for j in np.nonzero(am != r.argmax[open_])[0]:
            assert gap[j] < GAP, ("argmax differs outside the band", i, int(open_[j]), float(gap[j]))
            am_flips += 1
    stats["tf_argmax_flips"] = am_flips
    log("  teacher-forced: %d layers x %d rows; routing differences (all inside the %.0e band): %d; "
        "max attention rel L2 %.2e, max MoE rel L2 %.2e; LM head on the oracle's final rows: |dH| max %.2e, "
        "|dLSE| max %.2e, argmax differences (all inside the band) %d"
        % (w.n_layers, n_rows, GAP, flips_total, max(stats["attn_rl2"]), max(stats["moe_rl2"]),
           max(stats["tf_lm_dH"]), max(stats["tf_lm_dlse"]), am_flips))


def free_running(dec, w, reqs, results, states_before, stats, spread, plain_results=None, n_logit_rows=8):
    """The library's own last dg_denoise_step (run with the tap buffer set)
    against the oracle's step from the same state, with the bands of `spread`
    (oracle_spread).  Every measure is logged before any is asserted."""
    C, k, L = w.canvas_len, w.top_k, w.n_layers
    rows = dec.dg_last_step_rows()
    n_rows = rows["rows"]
    assert n_rows == C * len(reqs)
    taps = [dec.dg_debug_tap(0, l, n_rows) for l in range(L + 1)]
    rlog = [dec.dg_debug_tap(2, l, n_rows) for l in range(L)]
    flipped = np.zeros(n_rows, dtype=bool)
    layer_err, flip_gaps, bad = [], [], []
    for l in range(L):
        n_flip, errs, dr = 0, [], 0.0
        band = max(GAP, SPREAD_MARGIN * spread["router_gap"][l])
        for i, r in enumerate(results):
            tr = r.layers[l]
            sl = slice(i * C, (i + 1) * C)
            gap = topk_gap(tr.router_logits.astype(np.float32), k)
            x_g = taps[l][sl].astype(np.float64)
            for t in range(C):
                row = i * C + t
                if flipped[row]:
                    continue
                errs.append(rel_l2(x_g[t], tr.x_in[t]))
                dr = max(dr, float(np.max(np.abs(rlog[l][row] - tr.router_logits[t]))))
                if set(rows["router_ids"][l][row].tolist()) != set(tr.ids[t].tolist()):
                    flip_gaps.append(float(gap[t]))
                    if gap[t] >= band:
                        bad.append(("router set differs outside the band", l, i, t, float(gap[t]), band))
                    flipped[row] = True
                    n_flip += 1
        if (np.median(errs) > max(RL2, SPREAD_MARGIN * spread["hidden_med"][l])
                or max(errs) > max(RL2, SPREAD_MARGIN * spread["hidden_max"][l])):
            bad.append(("hidden rows entering layer", l, float(np.median(errs)), max(errs),
                        spread["hidden_med"][l], spread["hidden_max"][l]))
        layer_err.append((float(np.median(errs)), float(max(errs)), spread["hidden_med"][l], spread["hidden_max"][l],
                          n_flip, int(spread["router_flips"][l]), dr, band))
    stats["layer_err"] = layer_err
    stats["flip_gaps"] = sorted(flip_gaps)
    for l in range(L):
        log("  free-running layer %2d: hidden rel L2 median %.2e max %.2e (oracle spread %.2e / %.2e); routing "
            "differences %d (oracle vs oracle %d); router logits max diff %.2e; routing band %.1e"
            % ((l,) + layer_err[l]))
    log("  free-running: rows with a routing difference in some layer: %d of %d; their oracle gaps %s"
        % (flipped.sum(), n_rows, ["%.1e" % g for g in stats["flip_gaps"]]))
    # final rows, entropies, argmax, sampler, canvas
    fin = taps[L]
    for i, r in enumerate(results):
        req = reqs[i]
        sl = slice(i * C, (i + 1) * C)
        open_b = ~r.accepted_before
        cmp = open_b & ~flipped[sl]
        e_fin = [rel_l2(fin[sl][t], r.hidden[t]) for t in np.nonzero(~flipped[sl])[0]]
        if max(e_fin) > max(RL2, SPREAD_MARGIN * spread["hidden_max"][L]):
            bad.append(("final rows", i, max(e_fin), spread["hidden_max"][L]))
        Hg = rows["entropy"][sl].astype(np.float64)
        dH = np.abs(Hg - r.entropy)[cmp]
        stats.setdefault("dH_max", []).append(float(dH.max()))
        stats.setdefault("dH_median", []).append(float(np.median(dH)))
        h_band = max(H_TOL, SPREAD_MARGIN * spread["entropy"])
        if dH.max() > h_band:
            bad.append(("entropy", i, float(dH.max()), h_band))
        am_g = rows["argmax"][sl]
        lgap = topk_gap(r.logits.astype(np.float32), 1)
        diff = np.nonzero(cmp & (am_g != r.argmax))[0]
        z_band = max(GAP, SPREAD_MARGIN * spread["argmax_gap"])
        for t in diff:
            if lgap[t] >= z_band:
                bad.append(("argmax differs outside the band", i, int(t), float(lgap[t]), z_band))
        stats.setdefault("argmax_diff_gaps", []).extend(float(lgap[t]) for t in diff)
        # the sampler: the GPU's choice is the rule on its own entropies; the
        # oracle's choice may differ only between near-equal lowest entropies
        ids_g, acc_g = dec.dg_get_canvas(req)
        idx = np.nonzero(open_b)[0]
        Hg32 = rows["entropy"][sl].astype(np.float32)
        take_g = np.zeros(C, bool)
        take_g[idx[np.argmin(Hg32[idx])]] = True
        take_g |= open_b & (Hg32 < np.float32(w.tau))
        assert np.array_equal(acc_g, r.accepted_before | take_g), "accept set is not the rule on the GPU's entropies"
        newly_o = r.accepted_after & ~r.accepted_before
        h_sorted = np.sort(r.entropy[open_b])
        stats.setdefault("lowest_two_gap", []).append(float(h_sorted[1] - h_sorted[0]))
        if not np.array_equal(newly_o, take_g):
            near = h_sorted[1] - h_sorted[0] < 2 * h_band
            involved = np.nonzero(newly_o != take_g)[0]
            if not (near or flipped[sl][involved].any()):
                bad.append(("accepted position differs", i, float(h_sorted[1] - h_sorted[0])))
            stats.setdefault("accept_diffs", []).append(i)
        else:
            for t in np.nonzero(newly_o)[0]:
                assert ids_g[t] == am_g[t]
                if ids_g[t] != r.ids_after[t] and not (lgap[t] < z_band or flipped[sl][t]):
                    bad.append(("accepted token differs", i, int(t)))
        still = ~acc_g
        st = states_before[i]
        assert np.array_equal(ids_g[still], philox.draw_tokens(st["seed"], st["block"], st["step"] + 1,
                                                               np.nonzero(still)[0], w.vocab)), "Philox re-draws"
        assert np.array_equal(ids_g[r.accepted_before], r.ids_before[r.accepted_before])
        if plain_results is not None:
            dHp = float(np.max(np.abs(Hg - plain_results[i].entropy)[cmp]))
            stats.setdefault("dH_plain_max", []).append(dHp)
            if dHp > max(H_TOL, SPREAD_MARGIN * spread["entropy"]):
                bad.append(("entropy against the plain-arithmetic oracle", i, dHp, spread["entropy"]))
        # logits of sampled rows, against the oracle and (if given) the plain-arithmetic
        # oracle, on rows all of them route alike: there the library may lie no
        # further from exact arithmetic than twice the bf16 model does
        cand = np.nonzero(cmp & spread["alike"][i])[0] if plain_results is not None else np.nonzero(cmp)[0]
        if len(cand) == 0:
            # every open row was routed differently in some layer by one of the
            # sides (usual over 30 layers): the LM head itself is held by the
            # teacher-forced check on the oracle's final rows
            log("  free-running: request %d: no open row routed alike by all sides; logits not sampled" % i)
            continue
        pick = np.sort(np.random.default_rng(i).choice(cand, size=min(n_logit_rows, len(cand)), replace=False))
        lg = dec.dg_last_step_logits(pick + i * C).cpu().numpy().astype(np.float64)
        el = [rel_l2(lg[n], r.logits[t]) for n, t in enumerate(pick)]
        stats.setdefault("logit_rl2", []).append(float(max(el)))
        if max(el) > max(RL2, SPREAD_MARGIN * spread["logit_max"]):
            bad.append(("logits", i, max(el), spread["logit_max"]))
        if plain_results is not None:
            pr = plain_results[i]
            ep = [rel_l2(lg[n], pr.logits[t]) for n, t in enumerate(pick)]
            stats.setdefault("logit_rl2_plain", []).append(float(max(ep)))
            if max(ep) > max(RL2, SPREAD_MARGIN * spread["logit_max"]):
                bad.append(("logits against the plain-arithmetic oracle", i, max(ep), spread["logit_max"]))
    log("  free-running: |dH| max %.2e median %.2e (oracle spread %.2e); argmax differences at oracle gaps %s "
        "(band %.1e, oracle-vs-oracle differences %d); accept differences %s (lowest-two entropy gaps %s); logits "
        "rel L2 %s (oracle spread median %.2e max %.2e)%s"
        % (max(stats["dH_max"]), max(stats["dH_median"]), spread["entropy"], stats["argmax_diff_gaps"],
           max(GAP, SPREAD_MARGIN * spread["argmax_gap"]), spread["argmax_flips"], stats.get("accept_diffs", []),
           ["%.1e" % g for g in stats["lowest_two_gap"]],
           "%.2e" % max(stats["logit_rl2"]) if stats.get("logit_rl2") else "not sampled", spread["logit_med"],
           spread["logit_max"],
           "" if plain_results is None else
           " (against the plain-arithmetic oracle: logits %s, |dH| max %.2e)"
           % ("%.2e" % max(stats["logit_rl2_plain"]) if stats.get("logit_rl2_plain") else "not sampled",
              max(stats["dH_plain_max"]))))
    assert not bad, bad[:10]
    return flipped
