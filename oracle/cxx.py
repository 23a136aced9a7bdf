"""Driver of the C++ oracle (oracle/cxx/dg_oracle.cpp).

TEST INFRASTRUCTURE ONLY: only `tests/`, `__graft_entry__` and the bench's
CPU-baseline leg use it; the GPU library never imports or links it.  Every
arithmetic step (norms, projections, RoPE, attention, routing, experts, LM
head, sampler, Philox) runs in the C++ library; this module only gathers
embedding rows, keeps the per-request cache arrays and calls the steps in the
order the numpy oracle's decode.py gives (prefill, canvas start, denoising
step, commit), so the two oracles can be compared step for step.
"""
import ctypes
import os
import subprocess

import numpy as np

from .decode import RequestState

_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "cxx")
SRC = os.path.join(_DIR, "dg_oracle.cpp")
LIB = os.path.join(_DIR, "libdg_oracle.so")


def build(verbose=False):
    """Compile the C++ oracle with g++ (plain -O2, OpenMP; no fast-math)."""
    cmd = ["g++", "-O2", "-std=c++17", "-fopenmp", "-fPIC", "-shared", SRC, "-o", LIB + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("g++ failed:\n%s\n%s" % (" ".join(cmd), r.stderr[-4000:]))
    os.replace(LIB + ".tmp", LIB)
    if verbose:
        print("built", LIB)
    return LIB


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("vocab", "d", "L", "hq", "hkv", "hd", "E", "k", "eh", "sh", "C")] + [
        ("theta", ctypes.c_double), ("eps", ctypes.c_double), ("bf16_points", ctypes.c_int32),
        ("wdtype", ctypes.c_int32)]


_LAYER = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "router", "w1", "w3", "w2", "sw1", "sw3", "sw2")


class Layer(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _LAYER]


_lib = None


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB):
        build()
    lib = ctypes.CDLL(LIB)
    P, I32, U64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64
    lib.dgo_philox_tokens.argtypes = [U64, I32, I32, P, I32, I32, P]
    lib.dgo_philox_tokens.restype = None
    lib.dgo_layer.argtypes = [P, P, P, I32, P, P, P, I32, I32, I32, P, P, P, P, P]
    lib.dgo_layer.restype = None
    lib.dgo_lm_head.argtypes = [P, P, P, P, I32, P, P, P, P]
    lib.dgo_lm_head.restype = None
    lib.dgo_sample.argtypes = [P, P, P, P, I32, ctypes.c_float, I32, I32, U64, I32, I32, P]
    lib.dgo_sample.restype = I32
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _weights_array(t):
    """Host array of a weight tensor: float32 as is, bf16 as its raw 16-bit words."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.to(torch.float32).numpy()


class Model:
    """The model's weights (torch tensors of synth.make_weights, native expert
    format) as host arrays the C++ oracle reads, and its configuration."""

    def __init__(self, cfg, tw, bf16_points):
        import torch
        self.lib = load()
        self.cfg = cfg
        wd = 1 if tw["embed"].dtype == torch.bfloat16 else 0
        self.c = Config(vocab=cfg.vocab, d=cfg.d_model, L=cfg.n_layers, hq=cfg.n_q_heads, hkv=cfg.n_kv_heads,
                        hd=cfg.head_dim, E=cfg.n_experts, k=cfg.top_k, eh=cfg.expert_hidden, sh=cfg.shared_hidden,
                        C=cfg.canvas_len, theta=cfg.rope_theta, eps=cfg.rms_eps, bf16_points=int(bf16_points),
                        wdtype=wd)
        self.embed = _weights_array(tw["embed"])
        self.final_norm = _weights_array(tw["final_norm"])
        self.arrays = [{n: _weights_array(lt[n]) for n in _LAYER} for lt in tw["layers"]]
        self.layers = [Layer(**{n: a[n].ctypes.data for n in _LAYER}) for a in self.arrays]

    def embed_rows(self, ids):
        e = self.embed[np.asarray(ids)]
        if e.dtype == np.uint16:
            return (e.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return e.astype(np.float64)

    def forward(self, x, pos, st, causal, kv_only=False, P=None):
        """Rows x through every layer against st's cache prefix [0, P); returns
        (x, per-layer (k, v, router logits, ids, gates))."""
        c, L = self.cfg, self.cfg.n_layers
        T = x.shape[0]
        P = st.P if P is None else P
        x = np.ascontiguousarray(x, dtype=np.float64)
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        out = []
        for l in range(L):
            skip = kv_only and l == L - 1
            kp = np.ascontiguousarray(st.cache_k[l][:P])
            vp = np.ascontiguousarray(st.cache_v[l][:P])
            k = np.zeros((T, c.n_kv_heads, c.head_dim))
            v = np.zeros_like(k)
            rl = np.zeros((T, c.n_experts))
            ids = np.zeros((T, c.top_k), dtype=np.int32)
            g = np.zeros((T, c.top_k))
            self.lib.dgo_layer(ctypes.byref(self.c), ctypes.byref(self.layers[l]), _p(x), T, _p(pos), _p(kp), _p(vp),
                               P, int(causal), int(skip), _p(k), _p(v), _p(rl), _p(ids), _p(g))
            out.append((k, v, rl, ids, g))
        return x, out

    def lm_head(self, h, keep_logits=False):
        n = h.shape[0]
        h = np.ascontiguousarray(h, dtype=np.float64)
        ent, lse = np.zeros(n), np.zeros(n)
        am = np.zeros(n, dtype=np.int32)
        z = np.zeros((n, self.cfg.vocab)) if keep_logits else None
        self.lib.dgo_lm_head(ctypes.byref(self.c), _p(self.embed), _p(self.final_norm), _p(h), n, _p(ent), _p(lse),
                             _p(am), _p(z))
        return ent, lse, am, z


def philox_tokens(seed, block, step, positions, vocab):
    pos = np.ascontiguousarray(positions, dtype=np.int32)
    out = np.zeros(len(pos), dtype=np.int32)
    load().dgo_philox_tokens(seed, block, step, _p(pos), len(pos), vocab, _p(out))
    return out


def new_request(m: Model, seed, max_ctx):
    c = m.cfg
    st = RequestState(seed=seed, max_ctx=max_ctx)
    for _ in range(c.n_layers):
        st.cache_k.append(np.zeros((max_ctx, c.n_kv_heads, c.head_dim)))
        st.cache_v.append(np.zeros((max_ctx, c.n_kv_heads, c.head_dim)))
    return st


def prefill(m: Model, st, prompt):
    """Causal forward over the prompt; its post-RoPE K/V at [0, n)."""
    prompt = np.asarray(prompt)
    n = len(prompt)
    st.P, st.block, st.active = n, 0, False
    if n == 0:
        return
    _, layers = m.forward(m.embed_rows(prompt), np.arange(n), st, causal=True, kv_only=True, P=0)
    for l, (k, v, *_rest) in enumerate(layers):
        st.cache_k[l][:n] = k
        st.cache_v[l][:n] = v


def start_canvas(m: Model, st):
    C = m.cfg.canvas_len
    st.ids = philox_tokens(st.seed, st.block, 0, np.arange(C), m.cfg.vocab).astype(np.int64)
    st.accepted = np.zeros(C, dtype=bool)
    st.step, st.active = 0, True


def denoise_step(m: Model, st, tau, max_steps, keep_logits=False):
    """One step of the threshold sampler; returns a dict of the step's values."""
    if not st.active:
        start_canvas(m, st)
    C = m.cfg.canvas_len
    x, layers = m.forward(m.embed_rows(st.ids), st.P + np.arange(C), st, causal=False)
    ent, lse, am, z = m.lm_head(x, keep_logits)
    s = st.step + 1
    ids = np.ascontiguousarray(st.ids, dtype=np.int32).copy()
    acc = st.accepted.astype(np.uint8).copy()
    before_ids, before_acc = st.ids.copy(), st.accepted.copy()
    take = np.zeros(C, dtype=np.uint8)
    n_open = load().dgo_sample(_p(ent.astype(np.float32)), _p(am), _p(ids), _p(acc), C, tau, s, max_steps, st.seed,
                               st.block, m.cfg.vocab, _p(take))
    st.ids, st.accepted, st.step = ids.astype(np.int64), acc.astype(bool), s
    return {"entropy": ent, "lse": lse, "argmax": am, "logits": z, "hidden": x, "layers": layers,
            "ids_before": before_ids, "accepted_before": before_acc, "ids_after": st.ids.copy(),
            "accepted_after": st.accepted.copy(), "take": take.astype(bool), "n_open": int(n_open),
            "done": n_open == 0}


def commit_block(m: Model, st):
    """The final canvas's K/V at [P, P + C); P grows by C."""
    C = m.cfg.canvas_len
    _, layers = m.forward(m.embed_rows(st.ids), st.P + np.arange(C), st, causal=False, kv_only=True)
    for l, (k, v, *_rest) in enumerate(layers):
        st.cache_k[l][st.P:st.P + C] = k
        st.cache_v[l][st.P:st.P + C] = v
    out = st.ids.copy()
    st.P += C
    st.block += 1
    st.active = False
    return out


def generate(m: Model, prompt, n_out, seed, tau, max_steps):
    C = m.cfg.canvas_len
    n_blocks = -(-n_out // C)
    st = new_request(m, seed, len(prompt) + n_blocks * C)
    prefill(m, st, prompt)
    out, steps = [], []
    for _ in range(n_blocks):
        n = 0
        while True:
            r = denoise_step(m, st, tau, max_steps)
            n += 1
            if r["done"]:
                break
        steps.append(n)
        out.append(commit_block(m, st))
    return np.concatenate(out)[:n_out], steps
