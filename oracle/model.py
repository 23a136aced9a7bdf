"""Plain fp64 forward pass of the block-diffusion decoder (oracle side).

Test infrastructure: only the tests, the package's smoke check and the bench's
CPU-baseline leg use this package; the GPU library never imports or links it.

What the pages fix about the network ("Google open-sources DiffusionGemma",
section "26B MoE Architecture, but Only 3.8B Activated"; "DiffusionGemma Hits
1,000 Tokens per Second", section "The speed numbers and the hardware they
require"; "DiffusionGemma: Google open-sources a diffusion-based 26B MoE text
model", section "What's new"): a mixture-of-experts decoder with 8 routed
experts of 128 active per token plus one shared expert, and bidirectional
attention in which every canvas token sees its whole context.  Everything else
below is the plainest reading, listed with the rest in the design notes:

* pre-norm blocks; RMSNorm y = x / sqrt(mean(x^2) + eps) * g;
* grouped-query attention, q-head h reads kv-head h // (Hq / Hkv); RoPE in the
  rotate-half form on pairs (j, j + hd/2) with angle pos * theta^(-2j/hd) at
  absolute positions; scores scaled by 1/sqrt(hd); no softcap, no qk-norm;
* router logits r = b Wg^T; the k largest (ties to the lower expert id) are
  kept and their gates are the softmax over those k logits; the shared expert
  is added with weight 1; each expert is the SwiGLU FFN W2 (silu(W1 b) * W3 b);
* embedding without scaling; the LM head is the embedding matrix (tied);
* self-conditioning (optional; "DiffusionGemma hits ~1,500 TPS on one H100",
  section "How the sampler actually works", says only that the previous
  step's softmax goes back in through a small gated MLP): every canvas
  position keeps the expectation u = sum_v p_v E_v of the embedding under its
  softmax from the last step at which it was open (zero when the canvas
  starts), and each forward over the canvas adds W2 (silu(W1 u) * W3 u) to the
  token's embedding.

Arithmetic: float64 everywhere.  `Precision.bf16_points` optionally rounds
the operands that the bf16 GPU path feeds to its matrix cores (normalised
activations, q/k/v after RoPE, attention output, SwiGLU hidden) to bf16 with
round-to-nearest-even, so that both sides take integer decisions (top-k,
argmax, entropy argmin) from values of the same precision.  With it off the
forward is the exact-arithmetic definition.
"""
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np


@dataclass
class ModelConfig:
    vocab: int
    d_model: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_experts: int
    top_k: int
    expert_hidden: int
    shared_hidden: int
    canvas_len: int = 256
    rope_theta: float = 10000.0
    rms_eps: float = 1e-6
    self_cond_hidden: int = 0   # width of the self-conditioning MLP; 0 = no self-conditioning


@dataclass
class LayerWeights:
    attn_norm: np.ndarray   # [d]
    wq: np.ndarray          # [Hq*hd, d]
    wk: np.ndarray          # [Hkv*hd, d]
    wv: np.ndarray          # [Hkv*hd, d]
    wo: np.ndarray          # [d, Hq*hd]
    ffn_norm: np.ndarray    # [d]
    router: np.ndarray      # [E, d]
    w1: np.ndarray          # [E, eh, d]
    w3: np.ndarray          # [E, eh, d]
    w2: np.ndarray          # [E, d, eh]
    sw1: np.ndarray         # [sh, d]
    sw3: np.ndarray         # [sh, d]
    sw2: np.ndarray         # [d, sh]


@dataclass
class Weights:
    embed: np.ndarray       # [V, d]; also the LM head
    final_norm: np.ndarray  # [d]
    layers: List[LayerWeights]
    sc_w1: Optional[np.ndarray] = None   # [m, d] self-conditioning MLP (gate)
    sc_w3: Optional[np.ndarray] = None   # [m, d] (up)
    sc_w2: Optional[np.ndarray] = None   # [d, m] (down)


@dataclass
class Precision:
    bf16_points: bool = False


def round_bf16(x):
    """Round float64 values to the nearest bf16 (ties to even), returned as float64.

    Goes through float32 first; the float32 step is itself round-to-nearest,
    and no float64 value lands on a bf16 tie after it unless it already was one
    in float32 (bf16 keeps 8 of float32's 24 significand bits)."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16) << np.uint64(16)
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _maybe_bf16(x, prec):
    return round_bf16(x) if prec.bf16_points else x


def rmsnorm(x, g, eps):
    """y = x / sqrt(mean(x^2) + eps) * g over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def rope(x, positions, theta):
    """Rotate-half RoPE.  x: [T, H, hd]; positions: [T] absolute positions."""
    hd = x.shape[-1]
    half = hd // 2
    j = np.arange(half, dtype=np.float64)
    inv_freq = theta ** (-2.0 * j / hd)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]  # [T, half]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def attention(q, k, v, mask=None):
    """softmax(q k^T / sqrt(hd)) v per query head, grouped-query.

    q: [Tq, Hq, hd]; k, v: [Tk, Hkv, hd]; mask: optional bool [Tq, Tk], True
    where the query may see the key.  Returns [Tq, Hq, hd]."""
    tq, hq, hd = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    out = np.empty_like(q)
    scale = 1.0 / np.sqrt(hd)
    for h in range(hq):
        g = h // group
        s = (q[:, h, :] @ k[:, g, :].T) * scale  # [Tq, Tk]
        if mask is not None:
            s = np.where(mask, s, -np.inf)
        m = np.max(s, axis=1, keepdims=True)
        p = np.exp(s - m)
        p = p / np.sum(p, axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, g, :]
    return out


def silu(x):
    return x / (1.0 + np.exp(-x))


def topk_select(logits, k):
    """Indices of the k largest entries per row, largest first, ties to the
    lower index.  Plain repeated selection of the maximum.  logits: [T, E]."""
    t, e = logits.shape
    work = np.array(logits, dtype=np.float64, copy=True)
    ids = np.empty((t, k), dtype=np.int64)
    for j in range(k):
        best = np.argmax(work, axis=1)  # np.argmax returns the first maximum
        ids[:, j] = best
        work[np.arange(t), best] = -np.inf
    return ids


def route(b, router_w, k):
    """Router: logits r = b Wg^T, top-k ids, gates = softmax of the k kept logits.

    The integer decision (top-k) is taken on the logits rounded to float32,
    the precision in which the GPU path takes it."""
    r = b @ router_w.T
    r32 = r.astype(np.float32).astype(np.float64)
    ids = topk_select(r32, k)
    sel = np.take_along_axis(r, ids, axis=1)
    sel = sel - np.max(sel, axis=1, keepdims=True)
    gates = np.exp(sel)
    gates = gates / np.sum(gates, axis=1, keepdims=True)
    return r, ids, gates


def swiglu_ffn(b, w1, w3, w2, prec):
    h = silu(b @ w1.T) * (b @ w3.T)
    h = _maybe_bf16(h, prec)
    return h @ w2.T


def moe(b, lw: LayerWeights, cfg: ModelConfig, prec: Precision):
    """Routed top-k experts (gate-weighted) plus the shared expert.
    Returns (ffn_out [T, d], router_logits [T, E], ids [T, k], gates [T, k])."""
    r, ids, gates = route(b, lw.router, cfg.top_k)
    out = np.zeros_like(b)
    for e in range(cfg.n_experts):
        rows, slots = np.nonzero(ids == e)
        if rows.size == 0:
            continue
        y = swiglu_ffn(b[rows], lw.w1[e], lw.w3[e], lw.w2[e], prec)
        out[rows] += gates[rows, slots][:, None] * y
    out += swiglu_ffn(b, lw.sw1, lw.sw3, lw.sw2, prec)
    return out, r, ids, gates


@dataclass
class LayerTrace:
    x_in: np.ndarray = None         # [T, d] rows entering the layer
    x_attn: np.ndarray = None       # [T, d] rows after the attention half (residual added)
    k: np.ndarray = None            # [T, Hkv, hd] post-RoPE keys of the processed rows
    v: np.ndarray = None            # [T, Hkv, hd]
    ffn_in: np.ndarray = None       # [T, d] normalised FFN input
    router_logits: np.ndarray = None
    ids: np.ndarray = None
    gates: np.ndarray = None


def layer_forward(x, positions, lw: LayerWeights, cfg: ModelConfig, prec: Precision,
                  k_prefix, v_prefix, mask=None, skip_ffn=False):
    """One pre-norm decoder block over rows x [T, d] at absolute `positions`.

    Keys/values seen by the rows are [k_prefix ; own keys] (prefix: [P, Hkv, hd],
    already post-RoPE).  mask: bool [T, P + T] or None for full visibility.
    Returns (x_out, trace)."""
    t = x.shape[0]
    hq, hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    x_in = x
    a = _maybe_bf16(rmsnorm(x, lw.attn_norm, cfg.rms_eps), prec)
    q = (a @ lw.wq.T).reshape(t, hq, hd)
    k = (a @ lw.wk.T).reshape(t, hkv, hd)
    v = (a @ lw.wv.T).reshape(t, hkv, hd)
    q = _maybe_bf16(rope(q, positions, cfg.rope_theta), prec)
    k = _maybe_bf16(rope(k, positions, cfg.rope_theta), prec)
    v = _maybe_bf16(v, prec)
    keys = np.concatenate([k_prefix, k], axis=0)
    vals = np.concatenate([v_prefix, v], axis=0)
    o = attention(q, keys, vals, mask)
    o = _maybe_bf16(o.reshape(t, hq * hd), prec)
    x = x + o @ lw.wo.T
    tr = LayerTrace(x_in=x_in, x_attn=x, k=k, v=v)
    if skip_ffn:
        return x, tr
    b = _maybe_bf16(rmsnorm(x, lw.ffn_norm, cfg.rms_eps), prec)
    f, r, ids, gates = moe(b, lw, cfg, prec)
    tr.ffn_in, tr.router_logits, tr.ids, tr.gates = b, r, ids, gates
    return x + f, tr


def self_cond_input(z, lse, embed, prec: Precision):
    """Self-conditioning input of rows with logits z [R, V] and log-sum-exp lse
    [R]: the expectation of the embedding under the row's softmax, sum_v p_v E_v.
    The GPU rounds p to bf16 before the product (bf16 models)."""
    p = np.exp(z - np.asarray(lse)[:, None])
    return _maybe_bf16(p, prec) @ embed


def self_cond_embedding(u, w: Weights, prec: Precision):
    """Term added to the token embedding of canvas rows with self-conditioning
    state u [R, d]: the gated MLP W2 (silu(W1 u) * (W3 u)), u in bf16 on bf16
    models.  Zero for u = 0."""
    return swiglu_ffn(_maybe_bf16(u, prec), w.sc_w1, w.sc_w3, w.sc_w2, prec)


def lm_head_stats(h, embed, final_norm, cfg: ModelConfig, prec: Precision, keep_logits=False):
    """Final RMSNorm, tied LM head and per-row softmax statistics.

    Returns dict with entropy H = -sum p log p (nats), argmax (ties to the
    lower token id, decided on float32 logits), lse = log sum exp z, and the
    logits if asked.  h: [R, d]."""
    y = _maybe_bf16(rmsnorm(h, final_norm, cfg.rms_eps), prec)
    z = y @ embed.T  # [R, V]
    m = np.max(z, axis=1, keepdims=True)
    s = np.sum(np.exp(z - m), axis=1, keepdims=True)
    lse = m + np.log(s)
    logp = z - lse
    p = np.exp(logp)
    ent = -np.sum(p * logp, axis=1)
    z32 = z.astype(np.float32)
    out = {"entropy": ent, "argmax": np.argmax(z32, axis=1).astype(np.int64), "lse": lse[:, 0]}
    if keep_logits:
        out["logits"] = z
    return out
