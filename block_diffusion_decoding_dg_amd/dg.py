"""Thin ctypes binding of libdg (include/dg.h).  Argument marshalling only:
every step of the decoding path runs in the library's HIP kernels.  PyTorch is
used for device memory and the stream.  There is no fallback: if the library
is not built, loading it raises."""
import ctypes
import os

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# DG_LIBRARY selects another build of the same library (e.g. one compiled with
# different tile parameters); the default is the in-tree build.
LIB_PATH = os.environ.get("DG_LIBRARY") or os.path.join(_PKG, "libdg.so")

DG_OK, DG_ERR_INVALID_ARG, DG_ERR_WORKSPACE, DG_ERR_STATE, DG_ERR_CAPACITY, DG_ERR_HIP, DG_ERR_UNSUPPORTED = \
    0, -1, -2, -3, -4, -5, -6
DG_F32, DG_BF16 = 0, 1

EXPORTS = ("dg_workspace_size", "dg_create", "dg_prefill", "dg_denoise_step", "dg_commit_block", "dg_generate",
           "dg_destroy", "dg_last_error", "dg_get_request", "dg_get_canvas", "dg_set_canvas", "dg_set_committed",
           "dg_last_step_rows", "dg_last_step_router_logits", "dg_last_step_logits", "dg_op_attention", "dg_op_moe", "dg_op_lm_head",
           "dg_op_sample", "dg_philox_tokens", "dg_kernel_timer", "dg_kernel_timer_read", "dg_kernel_timer_every",
           "dg_get_self_cond", "dg_set_self_cond", "dg_op_self_cond", "dg_debug_tap_size", "dg_debug_set_tap_buffer",
           "dg_debug_tap", "dg_debug_refusal_count", "dg_debug_refusal_case", "dg_op_lm_head_noalloc")

DG_TAP_LAYER_INPUT, DG_TAP_AFTER_ATTENTION, DG_TAP_ROUTER_LOGITS = 0, 1, 2

KERNEL_FAMILIES = {"embed": 1, "rmsnorm": 2, "qkv": 3, "attention": 4, "out_proj": 5, "router": 6, "permute": 7,
                   "expert_up": 8, "expert_down": 9, "shared_up": 10, "shared_down": 11, "combine": 12,
                   "lm_head": 13, "sample": 14, "self_cond": 15}


class DgError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("dg status %d: %s" % (status, msg))
        self.status = status


class ModelConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "vocab", "d_model", "n_layers", "n_q_heads", "n_kv_heads", "head_dim", "n_experts", "top_k",
        "expert_hidden", "shared_hidden", "canvas_len", "max_ctx", "max_requests", "prefill_chunk")] + [
        ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float), ("dtype", ctypes.c_int32),
        ("expert_format", ctypes.c_int32), ("self_cond_hidden", ctypes.c_int32)]


SAMPLER_MODES = {"threshold": 0, "budget": 1}


class SamplerConfig(ctypes.Structure):
    _fields_ = [("tau", ctypes.c_float), ("max_steps", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("budget", ctypes.c_float), ("stop_entropy", ctypes.c_float)]


_LAYER_FIELDS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "router", "w1", "w3", "w2", "sw1", "sw3", "sw2",
                 "w1_scale", "w3_scale", "w2_scale", "w1_mx_scale", "w3_mx_scale", "w2_mx_scale")
_SCALE_FIELDS = ("w1_scale", "w3_scale", "w2_scale", "w1_mx_scale", "w3_mx_scale", "w2_mx_scale")
DG_EXPERTS_NATIVE, DG_EXPERTS_FP8, DG_EXPERTS_MXFP4 = 0, 1, 2
EXPERT_FORMATS = {"native": DG_EXPERTS_NATIVE, "fp8": DG_EXPERTS_FP8, "mxfp4": DG_EXPERTS_MXFP4}


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _LAYER_FIELDS]


class Weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("layers", ctypes.POINTER(LayerWeights)), ("sc_w1", ctypes.c_void_p), ("sc_w3", ctypes.c_void_p),
                ("sc_w2", ctypes.c_void_p)]


class StepInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("active", "block", "step", "n_accepted", "n_forced", "n_open", "done")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class Stats(ctypes.Structure):
    _fields_ = [("prefill_ms", ctypes.c_double), ("decode_ms", ctypes.c_double), ("commit_ms", ctypes.c_double),
                ("steps", ctypes.c_int64), ("tokens", ctypes.c_int64)]


class RequestState(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("prefilled", "committed", "block", "step", "active", "done")] + [
        ("seed", ctypes.c_uint64)]


_lib = None


def load():
    """Load libdg.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libdg.so is not built (%s); run python -m block_diffusion_decoding_dg_amd.build"
                           % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, U64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t
    sig = {
        "dg_workspace_size": [ctypes.POINTER(ModelConfig), ctypes.POINTER(SZ), ctypes.POINTER(SZ)],
        "dg_create": [ctypes.POINTER(ModelConfig), ctypes.POINTER(SamplerConfig), ctypes.POINTER(Weights), P, SZ, P,
                      SZ, P, ctypes.POINTER(P)],
        "dg_prefill": [P, I32, P, I32, U64],
        "dg_denoise_step": [P, ctypes.POINTER(StepInfo)],
        "dg_commit_block": [P, I32, P],
        "dg_generate": [P, I32, P, P, I32, P, P, ctypes.POINTER(Stats)],
        "dg_get_request": [P, I32, ctypes.POINTER(RequestState)],
        "dg_get_canvas": [P, I32, P, P],
        "dg_set_canvas": [P, I32, P, P, I32, I32],
        "dg_set_committed": [P, I32, I32, U64],
        "dg_last_step_rows": [P, P, P, P, P, P, P],
        "dg_last_step_router_logits": [P, P],
        "dg_last_step_logits": [P, P, I32, P],
        "dg_get_self_cond": [P, I32, P],
        "dg_set_self_cond": [P, I32, P],
        "dg_op_self_cond": [P, P, I32, P],
        "dg_op_attention": [P, I32, I32, P, I32, I32, I32],
        "dg_op_moe": [P, I32, P, I32, P, P],
        "dg_op_lm_head": [P, P, I32, P, P, P],
        "dg_op_lm_head_noalloc": [P, P, I32, P, P, P],
        "dg_op_sample": [P, I32, P, P, I32, ctypes.POINTER(StepInfo)],
        "dg_philox_tokens": [U64, I32, I32, I32, I32, P, P],
        "dg_kernel_timer": [P, I32],
        "dg_kernel_timer_read": [P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)],
        "dg_kernel_timer_every": [P, ctypes.c_int32],
        "dg_debug_tap_size": [ctypes.POINTER(ModelConfig), ctypes.POINTER(SZ)],
        "dg_debug_set_tap_buffer": [P, P, SZ],
        "dg_debug_tap": [P, I32, I32, P, SZ],
        "dg_debug_refusal_count": [],
        "dg_debug_refusal_case": [I32, ctypes.c_char_p, SZ],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.dg_destroy.argtypes = [P]
    lib.dg_destroy.restype = None
    lib.dg_last_error.argtypes = [P]
    lib.dg_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _np_ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _stream_handle():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def model_config(w, max_requests=None, max_ctx=None, prefill_chunk=0):
    """dg_model_config for a synth.Workload."""
    dtype = DG_BF16 if w.dtype == "bf16" else DG_F32
    return ModelConfig(vocab=w.vocab, d_model=w.d_model, n_layers=w.n_layers, n_q_heads=w.n_q_heads,
                       n_kv_heads=w.n_kv_heads, head_dim=w.head_dim, n_experts=w.n_experts, top_k=w.top_k,
                       expert_hidden=w.expert_hidden, shared_hidden=w.shared_hidden, canvas_len=w.canvas_len,
                       max_ctx=w.max_ctx if max_ctx is None else max_ctx,
                       max_requests=w.n_requests if max_requests is None else max_requests,
                       prefill_chunk=prefill_chunk, rope_theta=w.rope_theta, rms_eps=w.rms_eps, dtype=dtype,
                       expert_format=EXPERT_FORMATS[w.expert_format],
                       self_cond_hidden=getattr(w, "self_cond_hidden", 0))


def dg_workspace_size(cfg):
    lib = load()
    kv, sc = ctypes.c_size_t(), ctypes.c_size_t()
    st = lib.dg_workspace_size(ctypes.byref(cfg), ctypes.byref(kv), ctypes.byref(sc))
    if st != DG_OK:
        raise DgError(st, lib.dg_last_error(None).decode())
    return kv.value, sc.value


def dg_debug_refusal_cases():
    """(status, message) of every launcher refusal case (host only, no GPU)."""
    lib = load()
    out = []
    for i in range(lib.dg_debug_refusal_count()):
        buf = ctypes.create_string_buffer(512)
        st = lib.dg_debug_refusal_case(i, buf, len(buf))
        out.append((st, buf.value.decode()))
    return out


def dg_philox_tokens(seed, block, step, n, vocab, out):
    lib = load()
    st = lib.dg_philox_tokens(seed, block, step, n, vocab, _ptr(out), _stream_handle())
    if st != DG_OK:
        raise DgError(st, lib.dg_last_error(None).decode())


class Decoder:
    """A dg context with caller-owned (torch) device buffers.

    weights: {"embed", "final_norm", "layers": [ {name: tensor} ]} on the GPU in
    the model dtype (see synth.make_weights)."""

    def __init__(self, cfg: ModelConfig, tau, max_steps, weights, device="cuda", sampler="threshold",
                 budget=0.1, stop_entropy=0.005):
        self.lib = load()
        self.cfg = cfg
        kv_bytes, sc_bytes = dg_workspace_size(cfg)
        self.kv = torch.empty(kv_bytes, dtype=torch.uint8, device=device)
        self.scratch = torch.empty(sc_bytes, dtype=torch.uint8, device=device)
        self.weights = weights  # keep the tensors alive
        L = cfg.n_layers
        self._layers = (LayerWeights * L)()
        for l, lt in enumerate(weights["layers"]):
            for n in _LAYER_FIELDS:
                if n in _SCALE_FIELDS and n not in lt:
                    continue  # scales of another expert format
                setattr(self._layers[l], n, lt[n].data_ptr())
        sc = {n: (weights[n].data_ptr() if n in weights else None) for n in ("sc_w1", "sc_w3", "sc_w2")}
        self._w = Weights(embed=weights["embed"].data_ptr(), final_norm=weights["final_norm"].data_ptr(),
                          layers=self._layers, **sc)
        if sampler not in SAMPLER_MODES:
            raise ValueError("unknown sampler %r" % (sampler,))
        self.scfg = SamplerConfig(tau=tau, max_steps=max_steps, mode=SAMPLER_MODES[sampler], budget=budget,
                                  stop_entropy=stop_entropy)
        self.ctx = ctypes.c_void_p()
        st = self.lib.dg_create(ctypes.byref(cfg), ctypes.byref(self.scfg), ctypes.byref(self._w),
                                _ptr(self.kv), kv_bytes, _ptr(self.scratch), sc_bytes, _stream_handle(),
                                ctypes.byref(self.ctx))
        if st != DG_OK:
            raise DgError(st, self.lib.dg_last_error(None).decode())
        self.C = cfg.canvas_len
        self.R = cfg.max_requests

    def close(self):
        if self.ctx:
            self.lib.dg_destroy(self.ctx)
            self.ctx = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, st):
        if st != DG_OK:
            raise DgError(st, self.lib.dg_last_error(self.ctx).decode())

    # --- the five calls ---------------------------------------------------
    def dg_prefill(self, req, prompt, seed):
        p = np.ascontiguousarray(prompt, dtype=np.int32)
        self._check(self.lib.dg_prefill(self.ctx, req, _np_ptr(p), len(p), seed))

    def dg_denoise_step(self):
        info = (StepInfo * self.R)()
        self._check(self.lib.dg_denoise_step(self.ctx, info))
        return [i.as_dict() for i in info]

    def dg_commit_block(self, req):
        out = np.zeros(self.C, dtype=np.int32)
        self._check(self.lib.dg_commit_block(self.ctx, req, _np_ptr(out)))
        return out

    def dg_generate(self, prompts, n_out, seeds):
        n = len(prompts)
        ps = [np.ascontiguousarray(p, dtype=np.int32) for p in prompts]
        pp = (ctypes.c_void_p * n)(*[p.ctypes.data for p in ps])
        npr = np.array([len(p) for p in ps], dtype=np.int32)
        sd = np.array(seeds, dtype=np.uint64)
        outs = [np.zeros(n_out, dtype=np.int32) for _ in range(n)]
        op = (ctypes.c_void_p * n)(*[o.ctypes.data for o in outs])
        stats = Stats()
        self._check(self.lib.dg_generate(self.ctx, n, pp, _np_ptr(npr), n_out, _np_ptr(sd), op,
                                         ctypes.byref(stats)))
        return outs, {n_: getattr(stats, n_) for n_, _ in Stats._fields_}

    # --- inspection / injection ------------------------------------------
    def dg_get_request(self, req):
        st = RequestState()
        self._check(self.lib.dg_get_request(self.ctx, req, ctypes.byref(st)))
        return {n: getattr(st, n) for n, _ in RequestState._fields_}

    def dg_get_canvas(self, req):
        ids = np.zeros(self.C, dtype=np.int32)
        acc = np.zeros(self.C, dtype=np.uint8)
        self._check(self.lib.dg_get_canvas(self.ctx, req, _np_ptr(ids), _np_ptr(acc)))
        return ids, acc.astype(bool)

    def dg_set_canvas(self, req, ids, accepted, step, block):
        i = np.ascontiguousarray(ids, dtype=np.int32)
        a = np.ascontiguousarray(accepted, dtype=np.uint8)
        self._check(self.lib.dg_set_canvas(self.ctx, req, _np_ptr(i), _np_ptr(a), step, block))

    def dg_set_committed(self, req, committed, seed):
        self._check(self.lib.dg_set_committed(self.ctx, req, committed, seed))

    def dg_last_step_rows(self):
        rows = self.R * self.C
        L, k = self.cfg.n_layers, self.cfg.top_k
        n = ctypes.c_int32()
        ent = np.full(rows, np.nan, dtype=np.float32)
        lse = np.full(rows, np.nan, dtype=np.float32)
        am = np.full(rows, -1, dtype=np.int32)
        rid = np.zeros(L * rows * k, dtype=np.int32)
        rg = np.zeros(L * rows * k, dtype=np.float32)
        self._check(self.lib.dg_last_step_rows(self.ctx, ctypes.byref(n), _np_ptr(ent), _np_ptr(lse), _np_ptr(am),
                                               _np_ptr(rid), _np_ptr(rg)))
        m = n.value
        return {"rows": m, "entropy": ent[:m], "lse": lse[:m], "argmax": am[:m],
                "router_ids": rid[:L * m * k].reshape(L, m, k), "router_gates": rg[:L * m * k].reshape(L, m, k)}

    def dg_last_step_router_logits(self, rows):
        """[n_layers][rows][n_experts] fp32 router logits of the last step."""
        out = np.zeros((self.cfg.n_layers, rows, self.cfg.n_experts), dtype=np.float32)
        self._check(self.lib.dg_last_step_router_logits(self.ctx, _np_ptr(out)))
        return out

    # --- debug taps ------------------------------------------------------------
    def enable_taps(self, on=True):
        """Register (or drop) a device tap buffer: later steps copy their hidden
        rows at every layer into it (dg_debug_set_tap_buffer)."""
        if not on:
            self._check(self.lib.dg_debug_set_tap_buffer(self.ctx, None, 0))
            self.tap_buf = None
            return
        n = ctypes.c_size_t()
        self._check(self.lib.dg_debug_tap_size(ctypes.byref(self.cfg), ctypes.byref(n)))
        self.tap_buf = torch.empty(n.value, dtype=torch.uint8, device="cuda")
        self._check(self.lib.dg_debug_set_tap_buffer(self.ctx, _ptr(self.tap_buf), n.value))

    def dg_debug_tap(self, which, layer, rows):
        """fp32 [rows][d_model] (router logits: [rows][n_experts]) of the last step."""
        width = self.cfg.n_experts if which == DG_TAP_ROUTER_LOGITS else self.cfg.d_model
        out = np.zeros((rows, width), dtype=np.float32)
        self._check(self.lib.dg_debug_tap(self.ctx, which, layer, _np_ptr(out), out.nbytes))
        return out

    def dg_last_step_logits(self, rows):
        r = np.ascontiguousarray(rows, dtype=np.int32)
        out = torch.empty((len(r), self.cfg.vocab), dtype=torch.float32, device="cuda")
        self._check(self.lib.dg_last_step_logits(self.ctx, _np_ptr(r), len(r), _ptr(out)))
        return out

    def dg_get_self_cond(self, req):
        """Self-conditioning state of request req's canvas, fp32 [canvas_len][d_model]."""
        out = np.zeros((self.C, self.cfg.d_model), dtype=np.float32)
        self._check(self.lib.dg_get_self_cond(self.ctx, req, _np_ptr(out)))
        return out

    def dg_set_self_cond(self, req, state):
        st = np.ascontiguousarray(state, dtype=np.float32)
        assert st.shape == (self.C, self.cfg.d_model)
        self._check(self.lib.dg_set_self_cond(self.ctx, req, _np_ptr(st)))

    # --- single operations -------------------------------------------------
    def dg_op_attention(self, req, layer, x, pos0, causal):
        assert x.dtype == torch.float32 and x.is_contiguous()
        self._check(self.lib.dg_op_attention(self.ctx, req, layer, _ptr(x), x.shape[0], pos0, int(causal)))

    def dg_op_moe(self, layer, x, ids=None, gates=None):
        assert x.dtype == torch.float32 and x.is_contiguous()
        self._check(self.lib.dg_op_moe(self.ctx, layer, _ptr(x), x.shape[0], _ptr(ids), _ptr(gates)))

    def dg_op_lm_head(self, h):
        n = h.shape[0]
        ent = torch.empty(n, dtype=torch.float32, device=h.device)
        lse = torch.empty(n, dtype=torch.float32, device=h.device)
        am = torch.empty(n, dtype=torch.int32, device=h.device)
        self._check(self.lib.dg_op_lm_head(self.ctx, _ptr(h), n, _ptr(ent), _ptr(lse), _ptr(am)))
        return ent, lse, am

    def dg_op_lm_head_noalloc(self, h, ent, lse, am):
        """dg_op_lm_head into caller-given outputs, with the library's static
        scratch; asynchronous on the library's stream."""
        self._check(self.lib.dg_op_lm_head_noalloc(self.ctx, _ptr(h), h.shape[0], _ptr(ent), _ptr(lse), _ptr(am)))

    def dg_op_self_cond(self, u):
        """Self-conditioning MLP term of the rows of u (fp32 [n][d_model], device)."""
        assert u.dtype == torch.float32 and u.is_contiguous()
        out = torch.empty_like(u)
        self._check(self.lib.dg_op_self_cond(self.ctx, _ptr(u), u.shape[0], _ptr(out)))
        return out

    def dg_op_sample(self, req, entropy, argmax, step):
        info = StepInfo()
        self._check(self.lib.dg_op_sample(self.ctx, req, _ptr(entropy), _ptr(argmax), step, ctypes.byref(info)))
        return info.as_dict()

    # --- kernel timer ----------------------------------------------------------
    def dg_kernel_timer(self, family):
        f = KERNEL_FAMILIES[family] if isinstance(family, str) else int(family)
        self._check(self.lib.dg_kernel_timer(self.ctx, f))

    def dg_kernel_timer_every(self, every):
        self._check(self.lib.dg_kernel_timer_every(self.ctx, every))

    def dg_kernel_timer_read(self):
        ms, n = ctypes.c_double(), ctypes.c_int64()
        self._check(self.lib.dg_kernel_timer_read(self.ctx, ctypes.byref(ms), ctypes.byref(n)))
        return ms.value, n.value

    def kv_views(self, req, layer):
        """(K [Hkv][max_ctx][hd], Vt [Hkv][hd][max_ctx]) views of the caller-owned cache."""
        c = self.cfg
        dt = torch.bfloat16 if c.dtype == DG_BF16 else torch.float32
        es = 2 if c.dtype == DG_BF16 else 4
        per = c.n_kv_heads * c.max_ctx * c.head_dim
        base = ((req * c.n_layers + layer) * 2) * per * es
        k = self.kv[base:base + per * es].view(dt).view(c.n_kv_heads, c.max_ctx, c.head_dim)
        v = self.kv[base + per * es:base + 2 * per * es].view(dt).view(c.n_kv_heads, c.head_dim, c.max_ctx)
        return k, v
