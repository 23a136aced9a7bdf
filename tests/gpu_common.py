"""Shared helpers of the GPU parity tests: build a decoder from synthetic weights,
and compare one denoising step of the GPU library with the oracle's step from
the same state, applying the near-tie exemptions."""
import sys

import numpy as np
import torch

import oracle
from block_diffusion_decoding_dg_amd import dg, synth
from tests import helpers

# Bands.  Where both sides take a decision from the same input (the op-level
# and teacher-forced checks), a router set or an argmax may differ only where
# the oracle's gap between the last kept and the first dropped value is below
# GAP (1e-3), and a sampler decision only where the oracle's entropy is within
# TAU_BAND (1e-2 nats) of tau.  Whole bf16 steps carry the rounding drift of
# every layer before them; their bands come from the oracle's own spread
# (oracle_spread, SPREAD_MARGIN), computed on the same step.
TAU_BAND = 1e-2
# fp32 model: entropies are held to ENT_F32 * max(|H|, 1); the lowest-entropy
# choice may differ only between entropies within twice that.
ENT_F32 = 1e-4
GAP = 1e-3        # routing / argmax band where both sides see the same input
RL2 = 1e-2        # bf16: relative L2 per row (updates of a layer half, logits)
H_TOL = 1e-3      # nats: entropy floor of the free-running bands
# Free-running bands are SPREAD_MARGIN times the oracle spread: the library's
# step and the bf16 oracle differ by a rounding-flip process of the same kind as
# the one that separates the bf16 model from exact arithmetic, started by smaller
# differences (measured 0.6 - 0.9 times the spread at the mid shape), so twice
# the spread bounds it without following the library's own error.
SPREAD_MARGIN = 2.0


def oracle_spread(results, plain_results, k):
    """How far the bf16 model itself (the oracle with its bf16 rounding points)
    lies from exact arithmetic (the oracle without them) on the same step.
    Oracle values only.  A free-running bf16 step is held to these: it may not
    stray further from the bf16 model than the bf16 model strays from exact
    arithmetic.  Per layer, over the rows both oracles have routed alike so far:
      * router_gap: how wide a router gap the rounding can overturn -- the
        larger of the widest k-th - (k+1)-th gap the two decide differently and
        the most the rounding moves that gap on any row; an envelope over
        layers 0..l;
      * router_rl2, gate_max: the largest relative L2 of the router logits and
        the largest gate difference (rows whose sets agree);
      * hidden_med, hidden_max: median and largest relative L2 of the rows
        entering the layer (index n_layers: the final rows).
    At the end: the logits' median and largest relative L2 (open rows routed
    alike), the largest entropy difference (open rows), and argmax_gap, the
    larger of the widest top-1 - top-2 logit gap the two decide differently
    and the most the rounding moves that gap on any such row."""
    L = len(results[0].layers)
    sp = {"router_gap": np.zeros(L), "hidden_med": np.zeros(L + 1), "hidden_max": np.zeros(L + 1),
          "router_flips": np.zeros(L, dtype=int), "router_rl2": np.zeros(L), "gate_max": np.zeros(L)}
    fin = dict(logit_med=0.0, logit_max=0.0, entropy=0.0, argmax_gap=0.0, argmax_flips=0)
    hid = [[] for _ in range(L + 1)]
    logit_e = []
    sp["alike"] = []  # per request: rows the two oracles route alike in every layer
    for r, q in zip(results, plain_results):
        C = len(r.hidden)
        alike = np.ones(C, dtype=bool)
        for l in range(L):
            a, b = r.layers[l], q.layers[l]
            hid[l].extend(rel_l2(a.x_in[t], b.x_in[t]) for t in np.nonzero(alike)[0])
            gap = topk_gap(a.router_logits.astype(np.float32), k)
            order = np.argsort(-a.router_logits, axis=1, kind="stable")
            for t in range(C):
                if not alike[t]:
                    continue
                sp["router_rl2"][l] = max(sp["router_rl2"][l], rel_l2(a.router_logits[t], b.router_logits[t]))
                if k < a.router_logits.shape[1]:
                    # how far the rounding moves the k-th - (k+1)-th gap of this row
                    ek, ek1 = order[t, k - 1], order[t, k]
                    move = abs((a.router_logits[t, ek] - a.router_logits[t, ek1]) -
                               (b.router_logits[t, ek] - b.router_logits[t, ek1]))
                    sp["router_gap"][l] = max(sp["router_gap"][l], float(move))
                if set(a.ids[t].tolist()) != set(b.ids[t].tolist()):
                    sp["router_gap"][l] = max(sp["router_gap"][l], float(gap[t]))
                    sp["router_flips"][l] += 1
                    alike[t] = False
                else:
                    gb = dict(zip(b.ids[t].tolist(), b.gates[t].tolist()))
                    sp["gate_max"][l] = max(sp["gate_max"][l], max(abs(g - gb[e]) for e, g in
                                                                   zip(a.ids[t].tolist(), a.gates[t].tolist())))
        hid[L].extend(rel_l2(r.hidden[t], q.hidden[t]) for t in np.nonzero(alike)[0])
        sp["alike"].append(alike)
        open_ = ~r.accepted_before
        logit_e.extend(rel_l2(r.logits[t], q.logits[t]) for t in np.nonzero(open_ & alike)[0])
        fin["entropy"] = max(fin["entropy"], float(np.max(np.abs(r.entropy - q.entropy)[open_])))
        lgap = topk_gap(r.logits.astype(np.float32), 1)
        for t in np.nonzero(open_ & alike & (r.argmax != q.argmax))[0]:
            fin["argmax_gap"] = max(fin["argmax_gap"], float(lgap[t]))
            fin["argmax_flips"] += 1
        # how far the rounding moves the top-1 - top-2 gap itself: a gap that
        # narrow can be overturned even where no row happens to flip
        for t in np.nonzero(open_ & alike)[0]:
            i1 = int(r.argmax[t])
            z = r.logits[t].copy()
            z[i1] = -np.inf
            i2 = int(np.argmax(z))
            move = abs((r.logits[t][i1] - r.logits[t][i2]) - (q.logits[t][i1] - q.logits[t][i2]))
            fin["argmax_gap"] = max(fin["argmax_gap"], float(move))
    for l in range(L + 1):
        if hid[l]:
            sp["hidden_med"][l], sp["hidden_max"][l] = float(np.median(hid[l])), float(np.max(hid[l]))
    # the gaps the bf16 rounding overturns within the first l + 1 layers
    sp["router_gap"] = np.maximum.accumulate(sp["router_gap"])
    if logit_e:
        fin["logit_med"], fin["logit_max"] = float(np.median(logit_e)), float(np.max(logit_e))
    sp.update(fin)
    return sp


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_gpu(tw):
    out = {"embed": tw["embed"].cuda(), "final_norm": tw["final_norm"].cuda(),
           "layers": [{k: v.cuda() for k, v in lt.items()} for lt in tw["layers"]]}
    for n in ("sc_w1", "sc_w3", "sc_w2"):
        if n in tw:
            out[n] = tw[n].cuda()
    return out


def make_decoder(w, tw_gpu, max_requests=None, max_ctx=None, prefill_chunk=0, tau=None, max_steps=None,
                 sampler="threshold", budget=0.1, stop_entropy=0.005):
    cfg = dg.model_config(w, max_requests=max_requests, max_ctx=max_ctx, prefill_chunk=prefill_chunk)
    return dg.Decoder(cfg, w.tau if tau is None else tau, w.max_steps if max_steps is None else max_steps, tw_gpu,
                      sampler=sampler, budget=budget, stop_entropy=stop_entropy)


def normwise(a, b):
    """max |a - b| / max |b| (row-wise normwise relative error, worst row)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    num = np.max(np.abs(a - b), axis=-1)
    den = np.maximum(np.max(np.abs(b), axis=-1), 1e-30)
    return float(np.max(num / den))


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def topk_gap(vals, k):
    """Gap between the k-th and (k+1)-th largest entries of each row (inf if k == n)."""
    s = -np.sort(-np.asarray(vals, dtype=np.float64), axis=-1)
    if s.shape[-1] <= k:
        return np.full(s.shape[:-1], np.inf)
    return s[..., k - 1] - s[..., k]


def compare_router(gpu_ids, gpu_gates, tr, k, gate_tol, band=GAP, skip=None, gpu_logits=None, logit_rtol=None):
    """Router decisions of one layer.  Returns the rows whose expert set differs.

    A set may differ only where the oracle's k-th - (k+1)-th router logit gap is
    below `band`; on rows whose sets agree the gates are held to gate_tol, and
    with gpu_logits (the GPU's fp32 router logits of this layer) each compared
    row's logits to logit_rtol relative L2.  Rows in `skip` (whose routing
    already differed in an earlier layer, so that their hidden state
    legitimately differs here) are not compared."""
    o_ids = tr.ids
    gap = topk_gap(tr.router_logits.astype(np.float32), k)
    flips = []
    for t in range(o_ids.shape[0]):
        if skip is not None and skip[t]:
            continue
        if gpu_logits is not None:
            e = rel_l2(gpu_logits[t], tr.router_logits[t])
            assert e <= logit_rtol, ("router logits", t, e, logit_rtol)
        if set(gpu_ids[t]) != set(o_ids[t]):
            assert gap[t] < band, ("router set differs outside the band", t, gpu_ids[t], o_ids[t], gap[t], band)
            flips.append(t)
            continue
        og = dict(zip(o_ids[t].tolist(), tr.gates[t].tolist()))
        for e, g in zip(gpu_ids[t].tolist(), gpu_gates[t].tolist()):
            assert abs(g - og[e]) <= gate_tol, ("gate", t, e, g, og[e], gate_tol)
    return flips


def rule_on(H, accepted, tau, step, cap):
    """Positions the sampler rule takes at 1-based step `step`, given entropies H
    (fp32) and the accepted mask before the step: open positions with H < tau, the
    open position of lowest H (lowest index on ties), and at the cap every open
    position.  Used as a property check of the GPU's decision on its own H."""
    H = np.asarray(H, dtype=np.float32)
    open_ = ~np.asarray(accepted, dtype=bool)
    take = open_ & (H < np.float32(tau))
    if open_.any():
        idx = np.nonzero(open_)[0]
        take[idx[np.argmin(H[idx])]] = True
    if step >= cap:
        take |= open_
    return take


def _budget_diff_explained(i, Ho, open_b, acc_o, budget, flipped, h_band):
    """Whether position i may legitimately be decided differently by the budget
    rule on the GPU's entropies than on the oracle's, each entropy being held to
    h_band: a routing difference, an order swap with an open position of the
    other decision whose oracle entropy lies within 2 h_band, or a running sum
    through i (in the oracle's order) within (terms + 1) h_band of the budget."""
    if flipped[i]:
        return True
    idx = np.nonzero(open_b)[0]
    other = idx[acc_o[idx] != acc_o[i]]
    if other.size and np.min(np.abs(Ho[other] - Ho[i])) < 2 * h_band:
        return True
    order = sorted(idx, key=lambda j: (np.float32(Ho[j]), j))
    k = order.index(i)
    run = float(np.sum(Ho[order[:k + 1]]))
    return abs(run - float(np.float32(budget))) <= (k + 2) * h_band


def step_bands(w, r, q):
    """The bands of one step.  fp32 model (q None): the fixed ones -- GAP for the
    router and the argmax, entropies to ENT_F32 * max(|H|, 1), gates to 1e-4,
    router logits to 1e-4 relative L2.  bf16 model: SPREAD_MARGIN times the
    spread between the oracle's step r (bf16 rounding points) and q (exact
    arithmetic) from the same state (oracle_spread), with the same-input bands
    as floors: router gaps per layer, router logits, gates, entropy, argmax gap,
    logits."""
    L = w.n_layers
    if q is None:
        return {"router": np.full(L, GAP), "router_rl2": np.full(L, 1e-4), "gate": np.full(L, 1e-4),
                "entropy": None, "argmax": GAP, "logits": None, "spread": None}
    sp = oracle_spread([r], [q], w.top_k)
    m = SPREAD_MARGIN
    return {"router": np.maximum(GAP, m * sp["router_gap"]), "router_rl2": np.maximum(RL2, m * sp["router_rl2"]),
            "gate": np.maximum(2e-3, m * sp["gate_max"]), "entropy": max(H_TOL, m * sp["entropy"]),
            "argmax": max(GAP, m * sp["argmax_gap"]), "logits": max(RL2, m * sp["logit_max"]), "spread": sp}


class PlainTwin:
    """The exact-arithmetic oracle's copy of a bf16 oracle request: its own
    prefill and block commits, so that its cache carries none of the bf16
    rounding, and before each step it runs, the canvas of the bf16 oracle's
    request.  The spread of a step between the two then covers the drift of
    the committed cache as well as the step's own."""

    FIELDS = ("P", "block", "step", "active", "ids", "accepted", "prev_argmax", "sc_state")

    def __init__(self, st, prompt, ocfg, ow):
        self.st = oracle.new_request(ocfg, st.seed, st.max_ctx)
        self.ocfg, self.ow = ocfg, ow
        oracle.prefill(self.st, prompt, ocfg, ow, oracle.Precision(bf16_points=False))

    def sync(self, st):
        for f in self.FIELDS:
            v = getattr(st, f)
            setattr(self.st, f, v.copy() if isinstance(v, np.ndarray) else v)

    def commit(self, st):
        """Commit the canvas of st (the bf16 oracle's request, not yet committed)."""
        self.sync(st)
        oracle.commit_block(self.st, self.ocfg, self.ow, oracle.Precision(bf16_points=False))


def check_step(w, dec, st, ocfg, scfg, ow, prec, sample_rows=8, check_router=True, req=0, rng=None, stats=None,
               gstate=None, bands=None, plain=None):
    """Run one GPU step and the oracle step from the same state; compare.

    The bands are step_bands(): fixed for the fp32 model; for the bf16 model
    twice the spread between the bf16 oracle and the exact-arithmetic oracle on
    this same step (unless `bands` is given; the exact-arithmetic step runs on
    `plain`, a PlainTwin, when the two sides' caches come from their own
    prefills, else on a copy of st), never a measure of the library's own
    error.
    Continuous values (entropy, log-sum-exp, sampled logits) are compared on the
    open rows whose routing agreed with the oracle's in every layer; a row whose
    expert set differs in some layer (allowed only inside the router band) is
    left out of them.  Integer decisions:
      * argmax: equal unless the oracle's top-1 - top-2 gap is inside the argmax
        band, and then the GPU's choice is the maximum of its own logits;
      * sampler: the GPU's accept set must be the rule applied to the GPU's own
        entropies (exact); where it differs from the oracle's, the difference must
        lie in the tau band (TAU_BAND), or be the choice of the lowest-entropy
        position among oracle entropies within twice the entropy band;
      * Philox re-draws: bit-exact.
    After a permitted difference the GPU is re-synchronised to the oracle's state.
    With the budget sampler (scfg.mode == "budget") the GPU's decision is checked
    against the rule on its own entropies, argmax canvas and previous argmax
    canvas (kept in `gstate`, a dict the caller passes from step to step);
    differences from the oracle must be explained by _budget_diff_explained or,
    for the early stop, by a mean entropy within the entropy band of the
    threshold or an argmax near-tie.  Decisions excused at gaps of GAP or more
    are counted in stats ("excused_router", "excused_argmax").
    Returns (oracle StepResult, resynced, GPU step info, bands)."""
    import copy
    ids_g0, acc_g0 = dec.dg_get_canvas(req) if dec.dg_get_request(req)["active"] else (None, None)
    if ids_g0 is not None and st.active:
        assert np.array_equal(ids_g0, st.ids) and np.array_equal(acc_g0, st.accepted), "states diverged before step"
    need_spread = prec.bf16_points and bands is None
    if need_spread and plain is not None:
        plain.sync(st)
    st_plain = (plain.st if plain is not None else copy.deepcopy(st)) if need_spread else None
    info = dec.dg_denoise_step()[req]
    rows = dec.dg_last_step_rows()
    r = oracle.denoise_step(st, ocfg, scfg, ow, prec, keep_logits=True)
    if bands is None:
        q = None
        if st_plain is not None:
            q = oracle.denoise_step(st_plain, ocfg, scfg, ow, oracle.Precision(bf16_points=False), keep_logits=True)
        bands = step_bands(w, r, q)
    C = ocfg.canvas_len
    row0 = 0
    open_b = ~r.accepted_before
    # router decisions of every layer
    flipped = np.zeros(C, dtype=bool)
    n_excused_router = 0
    if check_router:
        glog = dec.dg_last_step_router_logits(rows["rows"])
        for l, tr in enumerate(r.layers):
            fl = compare_router(rows["router_ids"][l][row0:row0 + C], rows["router_gates"][l][row0:row0 + C], tr,
                                ocfg.top_k, gate_tol=bands["gate"][l], band=bands["router"][l], skip=flipped,
                                gpu_logits=glog[l][row0:row0 + C], logit_rtol=bands["router_rl2"][l])
            gap_l = topk_gap(tr.router_logits.astype(np.float32), ocfg.top_k)
            n_excused_router += int(np.sum(gap_l[fl] >= GAP))
            flipped[fl] = True
    cmp = open_b & ~flipped
    He = r.entropy[cmp]
    Hg = rows["entropy"][row0:row0 + C][cmp].astype(np.float64)
    err_h = np.abs(Hg - He)
    if bands["entropy"] is None:   # fp32
        h_tol = ENT_F32 * np.maximum(np.abs(He), 1.0)
        h_band = float(ENT_F32 * max(1.0, float(np.max(np.abs(r.entropy[open_b])))))
    else:
        h_tol = np.full_like(He, bands["entropy"])
        h_band = bands["entropy"]
    assert np.all(err_h <= h_tol), ("entropy", float(err_h.max()), h_band)
    lse_err = np.abs(rows["lse"][row0:row0 + C][cmp] - r.lse[cmp])
    lse_tol = ENT_F32 * np.maximum(np.abs(r.lse[cmp]), 1.0) if bands["entropy"] is None else bands["entropy"]
    assert np.all(lse_err <= lse_tol), ("lse", float(lse_err.max()))
    gap = topk_gap(r.logits.astype(np.float32), 1)
    am_g = rows["argmax"][row0:row0 + C]
    am_diff = np.nonzero(cmp & (am_g != r.argmax))[0]
    if am_diff.size:
        lgd = dec.dg_last_step_logits(am_diff + row0).cpu().numpy().astype(np.float64)
        for n, i in enumerate(am_diff):
            a_o, a_g = int(r.argmax[i]), int(am_g[i])
            # (the read-back logits come from another kernel: fp32 rounding apart)
            assert lgd[n, a_g] >= lgd[n, a_o] - 1e-4 * max(1.0, abs(lgd[n, a_o])), (
                "GPU argmax is not the maximum of its own logits", int(i))
            assert gap[i] < bands["argmax"], ("argmax differs outside the band", int(i), a_g, a_o, gap[i],
                                              bands["argmax"])
    n_excused_argmax = int(np.sum(gap[am_diff] >= GAP))
    # logits of a sample of compared rows
    cand = np.nonzero(cmp)[0]
    rng = rng or np.random.default_rng(0)
    pick = np.sort(rng.choice(cand, size=min(sample_rows, len(cand)), replace=False))
    lg = dec.dg_last_step_logits(pick + row0).cpu().numpy()
    if bands["logits"] is None:   # fp32: normwise relative error
        assert normwise(lg, r.logits[pick]) <= ENT_F32, normwise(lg, r.logits[pick])
    else:
        for n, t in enumerate(pick):
            e = rel_l2(lg[n], r.logits[t])
            assert e <= bands["logits"], ("logits rel L2", int(t), e, bands["logits"])
    if stats is not None:
        stats.setdefault("ent_err", []).append(float(err_h.max()) if err_h.size else 0.0)
        stats.setdefault("router_flip_rows", []).append(int(flipped.sum()))
        stats.setdefault("argmax_flips", []).append(int(len(am_diff)))
        stats.setdefault("excused_router", []).append(n_excused_router)
        stats.setdefault("excused_argmax", []).append(n_excused_argmax)
        stats["flipped"] = flipped  # rows whose routing differed in some layer (this step)
    # sampler: the GPU's accept set is the rule applied to its own (H, argmax)
    ids_g, acc_g = dec.dg_get_canvas(req)
    Hg_all = rows["entropy"][row0:row0 + C]
    budget = getattr(scfg, "mode", "threshold") == "budget"
    if budget:
        canvas_g = np.where(r.accepted_before, r.ids_before, am_g)
        te, tf, stop_g = oracle.budget_decide(Hg_all, am_g, r.accepted_before, canvas_g, gstate.get("prev"),
                                              scfg.budget, scfg.stop_entropy, st.step, scfg.max_steps)
        take_g = te | tf
        gstate["prev"] = canvas_g
    else:
        take_g = rule_on(Hg_all, r.accepted_before, scfg.tau, st.step, scfg.max_steps)
    assert np.array_equal(acc_g, r.accepted_before | take_g), "GPU accept set is not the rule on its own entropies"
    exp_ids = r.ids_before.copy()
    exp_ids[take_g] = am_g[take_g]
    still = ~(r.accepted_before | take_g)
    from oracle import philox
    exp_ids[still] = philox.draw_tokens(st.seed, st.block, st.step, np.nonzero(still)[0], ocfg.vocab)
    assert np.array_equal(ids_g, exp_ids), "GPU canvas is not accepted argmax + Philox re-draws"
    resync = False
    if not (np.array_equal(ids_g, r.ids_after) and np.array_equal(acc_g, r.accepted_after)):
        newly_o = r.accepted_after & ~r.accepted_before
        newly_g = acc_g & ~r.accepted_before
        h_o_min = float(np.min(r.entropy[open_b]))
        if budget:
            stop_o = r.stopped
            if stop_o != bool(stop_g):
                mean_o = float(np.mean(r.entropy[open_b]))
                near_mean = abs(mean_o - scfg.stop_entropy) <= h_band
                near_tie = bool(np.any(open_b & (am_g != r.argmax) & (gap < bands["argmax"])))
                assert near_mean or near_tie or flipped[open_b].any(), ("early stop differs", mean_o, h_band)
            else:
                acc_o = r.accept_entropy | r.accepted_before
                for i in np.nonzero(r.accept_entropy != te)[0]:
                    assert _budget_diff_explained(i, r.entropy, open_b, acc_o, scfg.budget, flipped, h_band), (
                        "budget decision differs outside the bands", int(i), h_band)
        for i in np.nonzero(newly_o != newly_g)[0] if not budget else []:
            near_tau = abs(r.entropy[i] - scfg.tau) < TAU_BAND
            lowest_choice = r.entropy[i] - h_o_min < 2 * h_band
            assert near_tau or lowest_choice or flipped[i], ("accept decision differs outside the bands", int(i),
                                                             r.entropy[i] - h_o_min, h_band)
        for i in np.nonzero(newly_o & newly_g & (ids_g != r.ids_after))[0]:
            assert gap[i] < bands["argmax"] or flipped[i], ("accepted token differs outside the argmax band", int(i))
        dec.dg_set_canvas(req, st.ids, st.accepted, st.step, st.block)
        if budget:   # the library forgets the previous argmax canvas on a set; so does the oracle here
            st.prev_argmax = None
            gstate["prev"] = None
        resync = True
        log("  resync at block %d step %d" % (st.block, st.step))
    assert info["step"] == st.step
    return r, resync, info, bands
