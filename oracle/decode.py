"""Prefill, denoising step, entropy-bound sampler and block commit (oracle side).

Test infrastructure: only the tests, the package's smoke check and the bench's
CPU-baseline leg use this package; the GPU library never imports or links it.

The decoding loop follows "DiffusionGemma hits ~1,500 TPS on one H100",
sections "What DiffusionGemma is" and "How the sampler actually works", and
"DiffusionGemma Hits 1,000 Tokens per Second", section "How diffusion text
generation changes the bottleneck":

1. a 256-token canvas starts filled with random tokens;
2. each step runs the decoder bidirectionally over the whole canvas, with the
   committed prefix in the KV cache visible to every canvas position;
3. a candidate is chosen at every position, confident positions are accepted
   and the rest are re-randomized for the next step;
4. the loop ends when the block has converged or at the step cap;
5. a finished block is committed to the KV cache and the next canvas is
   conditioned on it; nothing of the canvas enters the cache before that.

Two accept rules, both with the argmax token as the candidate, accepted
positions never changing and every open position forced to its argmax at the
step cap:

* "threshold" (a stated reading where the pages leave the rule open): among
  open positions accept those whose softmax entropy is strictly below tau, and
  always the single open position of lowest entropy (ties to the lower
  position).
* "budget", the default sampler of "DiffusionGemma hits ~1,500 TPS on one
  H100", section "How the sampler actually works" (budget 0.1, stop threshold
  0.005), which the pages describe in words only.  Readings taken: open
  positions are taken in order of rising entropy (ties to the lower position)
  while the running sum of their entropies, this one included, stays within
  the budget, and the first of them always (so that every step makes
  progress); the block stops early when the argmax canvas (accepted positions
  at their token, open ones at this step's argmax) equals the previous step's
  and the mean entropy of the open positions is below the stop threshold: then
  every open position is forced to its argmax, as at the cap.  The sums and
  the mean are taken exactly on entropies in 64-bit fixed point (2^-40 nat
  units, see `entropy_fixed`), so that their decisions do not depend on the
  order of summation.  The
committed K/V of a block are those of one more forward over the final canvas.
Prompt positions attend causally (the parent model is autoregressive).
"""
import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from .model import (ModelConfig, Weights, Precision, layer_forward, lm_head_stats, self_cond_input,
                    self_cond_embedding)
from .philox import draw_tokens


@dataclass
class SamplerConfig:
    tau: float
    max_steps: int  # step cap per block
    mode: str = "threshold"      # or "budget"
    budget: float = 0.1          # entropy budget per step ("budget" mode)
    stop_entropy: float = 0.005  # early-stop mean entropy ("budget" mode)


@dataclass
class RequestState:
    seed: int
    max_ctx: int
    cache_k: List[np.ndarray] = field(default_factory=list)  # per layer [max_ctx, Hkv, hd]
    cache_v: List[np.ndarray] = field(default_factory=list)
    P: int = 0              # committed length (prompt + committed blocks)
    block: int = 0          # index of the current / next canvas
    step: int = 0           # denoising steps taken on the current canvas
    active: bool = False
    ids: Optional[np.ndarray] = None       # [C] int64 canvas token ids
    accepted: Optional[np.ndarray] = None  # [C] bool
    prev_argmax: Optional[np.ndarray] = None  # [C] argmax canvas of the previous step of this block
    sc_state: Optional[np.ndarray] = None     # [C, d] self-conditioning state (cfg.self_cond_hidden > 0)


@dataclass
class StepResult:
    entropy: np.ndarray      # [C] float64 (every row, open or not)
    argmax: np.ndarray       # [C] int64
    lse: np.ndarray          # [C]
    accept_entropy: np.ndarray  # [C] bool: accepted this step by the entropy rule
    accept_forced: np.ndarray   # [C] bool: forced at the step cap
    redrawn: np.ndarray      # [C] bool: re-randomized this step
    ids_before: np.ndarray
    accepted_before: np.ndarray
    ids_after: np.ndarray
    accepted_after: np.ndarray
    n_open: int
    done: bool
    layers: list             # per-layer LayerTrace (router decisions etc.)
    logits: Optional[np.ndarray] = None
    hidden: Optional[np.ndarray] = None
    stopped: bool = False    # "budget" mode: the early stop fired this step


def new_request(cfg: ModelConfig, seed: int, max_ctx: int) -> RequestState:
    st = RequestState(seed=seed, max_ctx=max_ctx)
    for _ in range(cfg.n_layers):
        st.cache_k.append(np.zeros((max_ctx, cfg.n_kv_heads, cfg.head_dim)))
        st.cache_v.append(np.zeros((max_ctx, cfg.n_kv_heads, cfg.head_dim)))
    return st


def prefill(st: RequestState, prompt, cfg: ModelConfig, w: Weights, prec: Precision, keep_traces=False):
    """Causal forward over the prompt; stores post-RoPE K/V at [0, n).
    Returns the final rows, and with keep_traces also the per-layer traces."""
    prompt = np.asarray(prompt, dtype=np.int64)
    n = prompt.shape[0]
    if n > st.max_ctx:
        raise ValueError("prompt longer than max_ctx")
    st.P = n
    st.block = 0
    st.active = False
    if n == 0:
        x = np.zeros((0, cfg.d_model))
        return (x, []) if keep_traces else x
    x = w.embed[prompt]
    pos = np.arange(n)
    mask = np.tril(np.ones((n, n), dtype=bool))
    empty = np.zeros((0, cfg.n_kv_heads, cfg.head_dim))
    traces = []
    for l, lw in enumerate(w.layers):
        x, tr = layer_forward(x, pos, lw, cfg, prec, empty, empty, mask=mask,
                              skip_ffn=(l == cfg.n_layers - 1))
        st.cache_k[l][:n] = tr.k
        st.cache_v[l][:n] = tr.v
        traces.append(tr)
    return (x, traces) if keep_traces else x


def start_canvas(st: RequestState, cfg: ModelConfig):
    """Canvas initialisation: step index 0 of the current block."""
    c = cfg.canvas_len
    st.ids = draw_tokens(st.seed, st.block, 0, np.arange(c), cfg.vocab)
    st.accepted = np.zeros(c, dtype=bool)
    st.prev_argmax = None
    st.sc_state = np.zeros((c, cfg.d_model)) if cfg.self_cond_hidden > 0 else None
    st.step = 0
    st.active = True


def canvas_forward(st: RequestState, cfg: ModelConfig, w: Weights, prec: Precision,
                   for_commit=False):
    """Bidirectional forward of the canvas over [committed prefix ; canvas]."""
    c = cfg.canvas_len
    P = st.P
    if P + c > st.max_ctx:
        raise ValueError("canvas does not fit in max_ctx")
    x = w.embed[st.ids]
    if cfg.self_cond_hidden > 0:
        x = x + self_cond_embedding(st.sc_state, w, prec)
    pos = P + np.arange(c)
    traces = []
    for l, lw in enumerate(w.layers):
        last = l == cfg.n_layers - 1
        x, tr = layer_forward(x, pos, lw, cfg, prec, st.cache_k[l][:P], st.cache_v[l][:P],
                              mask=None, skip_ffn=(for_commit and last))
        traces.append(tr)
    return x, traces


def canvas_forward_batch(states, cfg: ModelConfig, w: Weights, prec: Precision):
    """canvas_forward for several requests in one pass, layer after layer: every
    request's rows go through layer l before any goes through layer l + 1, so
    each layer's weights are touched once per step.  Requests never mix: each
    canvas attends only to its own prefix and its own rows, and the other parts
    of a layer act row by row, so the result is that of canvas_forward on each
    request alone."""
    c = cfg.canvas_len
    xs, pos, traces = [], [], []
    for st in states:
        if st.P + c > st.max_ctx:
            raise ValueError("canvas does not fit in max_ctx")
        x = w.embed[st.ids]
        if cfg.self_cond_hidden > 0:
            x = x + self_cond_embedding(st.sc_state, w, prec)
        xs.append(x)
        pos.append(st.P + np.arange(c))
        traces.append([])
    for l, lw in enumerate(w.layers):
        for i, st in enumerate(states):
            xs[i], tr = layer_forward(xs[i], pos[i], lw, cfg, prec, st.cache_k[l][:st.P], st.cache_v[l][:st.P],
                                      mask=None)
            traces[i].append(tr)
    return xs, traces


def sampler_decide(entropy, argmax, accepted, tau, step, max_steps):
    """Entropy-bound accept rule on one canvas (pure function).

    entropy, argmax: per position; accepted: bool mask before the step; step:
    the 1-based index of this denoising step.  Decisions are taken on float32
    entropies.  Returns (accept_entropy, accept_forced) bool masks."""
    open_ = ~np.asarray(accepted, dtype=bool)
    h32 = np.asarray(entropy, dtype=np.float32)
    acc = open_ & (h32 < np.float32(tau))
    if open_.any():
        cand = np.where(open_, h32, np.float32(np.inf))
        lowest = int(np.argmin(cand))  # first minimum = lowest position
        acc[lowest] = True
    forced = np.zeros_like(acc)
    if step >= max_steps:
        forced = open_ & ~acc
    return acc, forced


FIX_FRAC_BITS = 40   # fixed-point entropies: units of 2^-40 nat
FIX_MAX_NATS = 64.0  # clamp; NaN counts as this (least confident)


def entropy_fixed(h) -> int:
    """Entropy (taken as float32) in fixed point: floor(clamp(h, 0, 64) * 2^40).

    Every float32 in [0, 64] times 2^40 is exact in float64, so the floor is
    exact and so are sums of up to 2^16 such values in 64 bits."""
    h = float(np.float32(h))
    if not h >= 0.0:
        h = 0.0 if h < 0.0 else FIX_MAX_NATS
    h = min(h, FIX_MAX_NATS)
    return int(math.floor(h * 2.0 ** FIX_FRAC_BITS))


def budget_decide(entropy, argmax, accepted, argmax_canvas, prev_argmax, budget, stop_entropy, step,
                  max_steps):
    """Entropy-budget accept rule on one canvas (pure function).

    entropy, argmax: per position (entries of accepted positions unused);
    accepted: mask before the step; argmax_canvas: this step's argmax canvas;
    prev_argmax: the previous step's, or None at the first step of a block;
    step: 1-based.  Returns (accept_budget, accept_forced, stopped)."""
    accepted = np.asarray(accepted, dtype=bool)
    n = len(accepted)
    open_pos = [i for i in range(n) if not accepted[i]]
    q = {i: entropy_fixed(entropy[i]) for i in open_pos}
    limit = entropy_fixed(budget)
    acc = np.zeros(n, dtype=bool)
    spent = 0
    for rank, i in enumerate(sorted(open_pos, key=lambda i: (q[i], i))):
        spent += q[i]
        if rank > 0 and spent > limit:
            break
        acc[i] = True
    stable = prev_argmax is not None and np.array_equal(np.asarray(argmax_canvas), np.asarray(prev_argmax))
    low = bool(open_pos) and sum(q.values()) < len(open_pos) * entropy_fixed(stop_entropy)
    stopped = stable and low
    forced = np.zeros(n, dtype=bool)
    if stopped or step >= max_steps:
        forced[open_pos] = True
        forced &= ~acc
    return acc, forced, stopped


def denoise_step(st: RequestState, cfg: ModelConfig, scfg: SamplerConfig, w: Weights,
                 prec: Precision, keep_logits=False) -> StepResult:
    if not st.active:
        start_canvas(st, cfg)
    x, traces = canvas_forward(st, cfg, w, prec)
    return _finish_step(st, x, traces, cfg, scfg, w, prec, keep_logits)


def denoise_step_batch(states, cfg: ModelConfig, scfg: SamplerConfig, w: Weights, prec: Precision,
                       keep_logits=False):
    """One denoising step of several requests together (canvases started as in
    denoise_step), their forwards taken layer by layer (canvas_forward_batch);
    returns one StepResult per request, each what denoise_step gives alone."""
    for st in states:
        if not st.active:
            start_canvas(st, cfg)
    xs, traces = canvas_forward_batch(states, cfg, w, prec)
    return [_finish_step(st, x, tr, cfg, scfg, w, prec, keep_logits) for st, x, tr in zip(states, xs, traces)]


def _finish_step(st: RequestState, x, traces, cfg: ModelConfig, scfg: SamplerConfig, w: Weights,
                 prec: Precision, keep_logits):
    """LM head, self-conditioning update and sampler of one canvas whose forward
    gave final rows x."""
    sc = cfg.self_cond_hidden > 0
    stats = lm_head_stats(x, w.embed, w.final_norm, cfg, prec, keep_logits=keep_logits or sc)
    if sc:
        # positions open at the start of the step take this step's softmax
        open_ = ~st.accepted
        st.sc_state = st.sc_state.copy()
        st.sc_state[open_] = self_cond_input(stats["logits"][open_], stats["lse"][open_], w.embed, prec)
    s = st.step + 1
    ids_before = st.ids.copy()
    acc_before = st.accepted.copy()
    argmax_canvas = np.where(st.accepted, st.ids, stats["argmax"])
    if scfg.mode == "budget":
        acc_e, acc_f, stopped = budget_decide(stats["entropy"], stats["argmax"], st.accepted, argmax_canvas,
                                        st.prev_argmax, scfg.budget, scfg.stop_entropy, s, scfg.max_steps)
    elif scfg.mode == "threshold":
        stopped = False
        acc_e, acc_f = sampler_decide(stats["entropy"], stats["argmax"], st.accepted, scfg.tau, s,
                                      scfg.max_steps)
    else:
        raise ValueError("unknown sampler mode %r" % scfg.mode)
    st.prev_argmax = argmax_canvas
    take = acc_e | acc_f
    ids = st.ids.copy()
    ids[take] = stats["argmax"][take]
    accepted = st.accepted | take
    redraw = ~accepted
    if redraw.any():
        pos = np.nonzero(redraw)[0]
        ids[pos] = draw_tokens(st.seed, st.block, s, pos, cfg.vocab)
    st.ids, st.accepted, st.step = ids, accepted, s
    n_open = int((~accepted).sum())
    return StepResult(entropy=stats["entropy"], argmax=stats["argmax"], lse=stats["lse"],
                      accept_entropy=acc_e, accept_forced=acc_f, redrawn=redraw,
                      ids_before=ids_before, accepted_before=acc_before,
                      ids_after=ids.copy(), accepted_after=accepted.copy(),
                      n_open=n_open, done=(n_open == 0), layers=traces,
                      logits=stats.get("logits") if keep_logits else None, hidden=x, stopped=stopped)


def commit_block(st: RequestState, cfg: ModelConfig, w: Weights, prec: Precision, keep_traces=False):
    """Write the K/V of a forward over the final canvas to [P, P + C); P += C.
    Returns the block's ids, and with keep_traces also the per-layer traces."""
    if not st.active or not st.accepted.all():
        raise ValueError("commit before the canvas is done")
    _, traces = canvas_forward(st, cfg, w, prec, for_commit=True)
    c = cfg.canvas_len
    for l, tr in enumerate(traces):
        st.cache_k[l][st.P:st.P + c] = tr.k
        st.cache_v[l][st.P:st.P + c] = tr.v
    out = st.ids.copy()
    st.P += c
    st.block += 1
    st.active = False
    st.ids = None
    st.accepted = None
    st.prev_argmax = None
    st.sc_state = None
    return (out, traces) if keep_traces else out


def generate(prompt, n_out, seed, cfg: ModelConfig, scfg: SamplerConfig, w: Weights,
             prec: Precision, max_ctx=None, on_step=None):
    """Whole generation for one request: prefill, then block after block.

    Output length n_out is rounded up to whole canvases and truncated."""
    c = cfg.canvas_len
    n_blocks = -(-n_out // c)
    if max_ctx is None:
        max_ctx = len(prompt) + n_blocks * c
    st = new_request(cfg, seed, max_ctx)
    prefill(st, prompt, cfg, w, prec)
    out = []
    steps = []
    for b in range(n_blocks):
        n = 0
        while True:
            r = denoise_step(st, cfg, scfg, w, prec)
            n += 1
            if on_step is not None:
                on_step(b, n, r, st)
            if r.done:
                break
        steps.append(n)
        out.append(commit_block(st, cfg, w, prec))
    return np.concatenate(out)[:n_out], steps, st
