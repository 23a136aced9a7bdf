"""Weights and committed prefixes read by the oracle one layer at a time.

TEST INFRASTRUCTURE ONLY (with the rest of this package): the tests and the
bench's CPU-baseline leg use it to run the float64 oracle on models whose
float64 copy would not fit in host memory (the full-size model holds 25
billion parameters).  No arithmetic of the method lives here: the adaptors
only copy torch tensors to host float64 arrays when the oracle first indexes
them -- a layer's dense matrices when it enters the layer, a routed expert
when some row is routed to it, a layer's committed keys and values when its
attention reads them -- and keep the last layer's copies.
"""
import numpy as np

from .model import LayerWeights, Weights
from .decode import RequestState


def f64(t):
    """A torch tensor (any device, any float dtype) as a host float64 array."""
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


class LazyExperts:
    """Stacked expert matrices [E, out, in] of one layer; expert e is copied to
    the host as float64 on first use."""

    def __init__(self, t):
        self.t = t
        self.cache = {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            self.cache[e] = f64(self.t[e])
        return self.cache[e]


class LazyLayers:
    """The oracle's per-layer weights, built from the torch tensors of one
    {name: tensor} dict per layer as each layer is entered (the last layer used
    is kept).  Bf16 weights only: quantized experts have their own decoders."""

    def __init__(self, layers):
        self.layers = layers
        self.cur, self.lw = -1, None

    def __len__(self):
        return len(self.layers)

    def __getitem__(self, l):
        if l != self.cur:
            self.lw = None
            d = {}
            for k, v in self.layers[l].items():
                if k in ("w1", "w3", "w2"):
                    d[k] = LazyExperts(v)
                elif not k.endswith("scale"):
                    d[k] = f64(v)
            self.lw = LayerWeights(**d)
            self.cur = l
        return self.lw

    def __iter__(self):
        for l in range(len(self)):
            yield self[l]


def lazy_weights(tw):
    """oracle.Weights over the torch weights {"embed", "final_norm", "layers"}."""
    return Weights(embed=f64(tw["embed"]), final_norm=f64(tw["final_norm"]), layers=LazyLayers(tw["layers"]))


class LazyPrefix:
    """cache_k or cache_v of a request whose committed prefix [0, P) comes from
    gen(l) -> (k, v), torch tensors [n_kv_heads, P, head_dim]: layer l's rows are
    produced on first use, as float64 [rows, n_kv_heads, head_dim] with rows
    [P, rows) zero (room for a commit); the K/V pair of the last layer is kept
    in `shared`."""

    def __init__(self, n_layers, gen, which, shared, rows):
        self.n_layers, self.gen, self.which, self.shared, self.rows = n_layers, gen, which, shared, rows

    def __len__(self):
        return self.n_layers

    def __getitem__(self, l):
        sh = self.shared
        if sh.get("layer") != l:
            sh.clear()
            k, v = self.gen(l)
            sh["layer"] = l
            for name, t in (("k", k), ("v", v)):
                a = f64(t.transpose(0, 1))
                full = np.zeros((self.rows,) + a.shape[1:])
                full[:a.shape[0]] = a
                sh[name] = full
        return sh[self.which]


def request_with_prefix(n_layers, P, canvas_len, gen, seed):
    """A request whose committed length is P, its prefix read through gen."""
    shared = {}
    rows = P + canvas_len
    st = RequestState(seed=seed, max_ctx=rows, cache_k=LazyPrefix(n_layers, gen, "k", shared, rows),
                      cache_v=LazyPrefix(n_layers, gen, "v", shared, rows))
    st.P = P
    return st
