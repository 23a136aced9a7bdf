"""Seeded synthetic inputs: workload shapes, random-init weights and prompts.

This module is shared by the GPU tests, the CPU oracle's callers and the
bench.  It holds none of the decoder's arithmetic: it only draws numbers.

Workloads (the pages give one real configuration, DiffusionGemma 26B A4B: a
mixture of experts with 128 experts, 8 routed plus 1 shared active, 25.2B
total / 3.8B active parameters, 256-token canvases, batch 1, 4096 input /
1024 output tokens -- "DiffusionGemma hits ~1,500 TPS on one H100", section
"The specs that matter for serving"; "DiffusionGemma Hits 1,000 Tokens per
Second", section "The speed numbers and the hardware they require").  The
pages' own runs use real prompts and trained weights; here every matrix is
N(0, 0.02), norm gains are 1 and prompts are uniform random token ids.

Generators: torch's seeded normal generator (CPU or GPU device) per tensor,
seed = hash of (workload seed, tensor index); fp32 then round-to-nearest-even
bf16 for the bf16 workloads.  Prompts: numpy PCG64 uniform integers.
"""
from dataclasses import dataclass, asdict, replace
from typing import List, Optional

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16"
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
    prompt_len: int
    n_out: int            # output tokens per request
    n_requests: int
    tau: float
    max_steps: int
    canvas_len: int = 256
    rope_theta: float = 10000.0
    rms_eps: float = 1e-6
    init_std: float = 0.02
    expert_format: str = "native"   # or "fp8": routed experts as E4M3 codes + row scales
    self_cond_hidden: int = 0       # width of the self-conditioning MLP (0: none)

    @property
    def n_blocks(self):
        return -(-self.n_out // self.canvas_len)

    @property
    def max_ctx(self):
        return self.prompt_len + self.n_blocks * self.canvas_len

    def model_dict(self):
        keys = ("vocab", "d_model", "n_layers", "n_q_heads", "n_kv_heads", "head_dim", "n_experts",
                "top_k", "expert_hidden", "shared_hidden", "canvas_len", "rope_theta", "rms_eps",
                "self_cond_hidden")
        return {k: getattr(self, k) for k in keys}

    def param_count(self):
        d, hd = self.d_model, self.head_dim
        per_layer = ((self.n_q_heads + 2 * self.n_kv_heads) * hd * d + self.n_q_heads * hd * d
                     + self.n_experts * d + self.n_experts * 3 * d * self.expert_hidden
                     + 3 * d * self.shared_hidden + 2 * d)
        return self.n_layers * per_layer + self.vocab * d + d

    def active_param_count(self):
        """Parameters one token touches in a forward pass: attention, router, its
        top_k routed experts, the shared expert, norms, and the tied embedding /
        LM head counted once."""
        d, hd = self.d_model, self.head_dim
        per_layer = ((self.n_q_heads + 2 * self.n_kv_heads) * hd * d + self.n_q_heads * hd * d
                     + self.n_experts * d + self.top_k * 3 * d * self.expert_hidden
                     + 3 * d * self.shared_hidden + 2 * d)
        return self.n_layers * per_layer + self.vocab * d + d


# The five workloads.  The tiny one leaves the shared-expert width unstated;
# it is taken equal to the routed experts' width.
WORKLOADS = {
    "tiny": Workload("tiny", "f32", vocab=512, d_model=64, n_layers=2, n_q_heads=4, n_kv_heads=2,
                     head_dim=16, n_experts=8, top_k=2, expert_hidden=128, shared_hidden=128,
                     prompt_len=64, n_out=256, n_requests=1, tau=0.5, max_steps=64),
    "mid": Workload("mid", "bf16", vocab=32768, d_model=1024, n_layers=8, n_q_heads=16,
                    n_kv_heads=4, head_dim=64, n_experts=32, top_k=4, expert_hidden=512,
                    shared_hidden=1536, prompt_len=1024, n_out=512, n_requests=1, tau=1.0,
                    max_steps=256),
    "full": Workload("full", "bf16", vocab=262144, d_model=2816, n_layers=30, n_q_heads=16,
                     n_kv_heads=8, head_dim=256, n_experts=128, top_k=8, expert_hidden=704,
                     shared_hidden=2112, prompt_len=4096, n_out=1024, n_requests=1, tau=1.0,
                     max_steps=256),
    "full_x8": Workload("full_x8", "bf16", vocab=262144, d_model=2816, n_layers=30, n_q_heads=16,
                        n_kv_heads=8, head_dim=256, n_experts=128, top_k=8, expert_hidden=704,
                        shared_hidden=2112, prompt_len=4096, n_out=1024, n_requests=8, tau=1.0,
                        max_steps=256),
    "full_long": Workload("full_long", "bf16", vocab=262144, d_model=2816, n_layers=30,
                          n_q_heads=16, n_kv_heads=8, head_dim=256, n_experts=128, top_k=8,
                          expert_hidden=704, shared_hidden=2112, prompt_len=131072, n_out=512,
                          n_requests=1, tau=1.0, max_steps=256),
}

# The mid-size and full-size shapes with FP8 (E4M3) routed experts.
WORKLOADS["mid_fp8"] = replace(WORKLOADS["mid"], name="mid_fp8", expert_format="fp8")
WORKLOADS["full_fp8"] = replace(WORKLOADS["full"], name="full_fp8", expert_format="fp8")
# ... and with MXFP4 (E2M1 + E8M0 block scales) routed experts.
WORKLOADS["mid_mxfp4"] = replace(WORKLOADS["mid"], name="mid_mxfp4", expert_format="mxfp4")
WORKLOADS["full_mxfp4"] = replace(WORKLOADS["full"], name="full_mxfp4", expert_format="mxfp4")
# ... and with self-conditioning through a gated MLP of width 256.
WORKLOADS["mid_sc"] = replace(WORKLOADS["mid"], name="mid_sc", self_cond_hidden=256)
WORKLOADS["full_sc"] = replace(WORKLOADS["full"], name="full_sc", self_cond_hidden=256)

LAYER_TENSORS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "router",
                 "w1", "w3", "w2", "sw1", "sw3", "sw2")


def layer_shapes(w: Workload):
    d, hd, E = w.d_model, w.head_dim, w.n_experts
    return {
        "attn_norm": (d,), "wq": (w.n_q_heads * hd, d), "wk": (w.n_kv_heads * hd, d),
        "wv": (w.n_kv_heads * hd, d), "wo": (d, w.n_q_heads * hd), "ffn_norm": (d,),
        "router": (E, d), "w1": (E, w.expert_hidden, d), "w3": (E, w.expert_hidden, d),
        "w2": (E, d, w.expert_hidden), "sw1": (w.shared_hidden, d), "sw3": (w.shared_hidden, d),
        "sw2": (d, w.shared_hidden),
    }


def torch_dtype(w: Workload):
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def _tensor_seed(seed: int, index: int) -> int:
    return (seed * 1_000_003 + index * 7_919 + 12_345) % (2 ** 63)


def _normal(shape, std, seed, index, device, dtype):
    g = torch.Generator(device=device)
    g.manual_seed(_tensor_seed(seed, index))
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    t.mul_(std)
    return t.to(dtype)


def make_weights(w: Workload, seed: int = 0, device="cpu", layers: Optional[List[int]] = None):
    """Random-init weights as torch tensors on `device`, in the workload dtype.

    Returns {"embed": [V, d], "final_norm": [d], "layers": [ {name: tensor} ]}.
    `layers` restricts generation to the listed layer indices (others None);
    the values of a layer do not depend on which others are generated."""
    dt = torch_dtype(w)
    out = {"embed": _normal((w.vocab, w.d_model), w.init_std, seed, 0, device, dt),
           "final_norm": torch.ones(w.d_model, device=device, dtype=dt), "layers": []}
    shapes = layer_shapes(w)
    for l in range(w.n_layers):
        if layers is not None and l not in layers:
            out["layers"].append(None)
            continue
        lt = {}
        for i, name in enumerate(LAYER_TENSORS):
            if name.endswith("norm"):
                lt[name] = torch.ones(shapes[name], device=device, dtype=dt)
            else:
                lt[name] = _normal(shapes[name], w.init_std, seed, 1 + l * 64 + i, device, dt)
        if w.expert_format == "fp8":
            for name in ("w1", "w3", "w2"):
                lt[name], lt[name + "_scale"] = quantize_rows_e4m3(lt[name])
        elif w.expert_format == "mxfp4":
            for name in ("w1", "w3", "w2"):
                lt[name], lt[name + "_mx_scale"] = quantize_blocks_mxfp4(lt[name])
        out["layers"].append(lt)
    out.update(make_self_cond_weights(w, seed, device))
    return out


def make_self_cond_weights(w: Workload, seed: int = 0, device="cpu"):
    """The self-conditioning MLP's weights of make_weights alone ({} without
    self-conditioning): sc_w1, sc_w3 [m, d] and sc_w2 [d, m] in the workload dtype."""
    out = {}
    if w.self_cond_hidden > 0:
        dt = torch_dtype(w)
        m, d = w.self_cond_hidden, w.d_model
        for i, (name, shape) in enumerate((("sc_w1", (m, d)), ("sc_w3", (m, d)), ("sc_w2", (d, m)))):
            out[name] = _normal(shape, w.init_std, seed, 1 + w.n_layers * 64 + i, device, dt)
    return out


def quantize_rows_e4m3(w: torch.Tensor):
    """Stand-in for an FP8 checkpoint of a weight tensor [..., out, in]: per output
    row a float32 scale max|w| / 448 (1 for a zero row) and the E4M3 codes of
    w / scale (torch's round-to-nearest-even cast), as uint8.  The random bf16
    weights are drawn first, so the FP8 model is the bf16 one quantized."""
    wf = w.float()
    amax = wf.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    codes = (wf / scale[..., None]).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale.contiguous()


# E2M1 magnitudes by code (index = code & 7) and the midpoints between neighbours.
_E2M1_MIDS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def quantize_blocks_mxfp4(w: torch.Tensor):
    """Stand-in for an MXFP4 checkpoint of a weight tensor [..., out, in] (in a
    multiple of 32), following the OCP MX conversion: per block of 32 weights of
    a row the shared exponent X = floor(log2 max|w|) - 2 (2 = E2M1's largest
    exponent; X = 0 for an all-zero block, clamped to [-126, 127]), scale byte
    X + 127, and the E2M1 codes of w / 2^X rounded to nearest, ties to the even
    code, saturating at 6.  Returns (packed codes uint8 [..., out, in / 2], lower
    index in the low nibble; scale bytes uint8 [..., out, in / 32])."""
    wf = w.float()
    shape = wf.shape
    blocks = wf.reshape(*shape[:-1], shape[-1] // 32, 32)
    amax = blocks.abs().amax(dim=-1)
    _, e = torch.frexp(amax)  # amax = f * 2^e with f in [0.5, 1): floor(log2 amax) = e - 1
    x = torch.where(amax > 0, e - 3, torch.zeros_like(e)).clamp_(-126, 127)
    y = blocks / torch.ldexp(torch.ones_like(amax), x)[..., None]  # exact: a power of two
    a = y.abs()
    idx = torch.zeros(a.shape, dtype=torch.uint8, device=a.device)
    for j, m in enumerate(_E2M1_MIDS):
        # at a midpoint the tie goes to the even neighbour: up when the lower one is odd
        idx += ((a > m) | ((a == m) & (j % 2 == 1))).to(torch.uint8)
    del a
    code = (idx | ((y < 0).to(torch.uint8) << 3)).reshape(shape)
    del idx, y
    packed = code[..., 0::2] | (code[..., 1::2] << 4)
    return packed.contiguous(), (x + 127).to(torch.uint8).contiguous()


def make_prompt(w: Workload, seed: int = 0, length: Optional[int] = None):
    n = w.prompt_len if length is None else length
    rng = np.random.Generator(np.random.PCG64(seed + 0x5EED))
    return rng.integers(0, w.vocab, size=n, dtype=np.int64).astype(np.int32)


def make_prefix_kv(w: Workload, P: int, layer: int, seed: int = 0, device="cpu"):
    """A synthetic committed prefix for one layer of one request: post-RoPE keys
    and values of positions [0, P), both [n_kv_heads, P, head_dim] in the
    workload dtype, drawn N(0, s^2) with s = init_std * sqrt(d_model) -- the
    spread of a unit-RMS row projected by N(0, init_std^2) weights, i.e. the
    spread of the keys and values a prefill of the random-init model writes.
    It stands in for the K/V of a long random prompt wherever running the
    prompt's prefill on the CPU would be out of reach."""
    std = w.init_std * float(np.sqrt(w.d_model))
    shape = (w.n_kv_heads, P, w.head_dim)
    dt = torch_dtype(w)
    k = _normal(shape, std, seed, 0x100000 + 2 * layer, device, dt)
    v = _normal(shape, std, seed, 0x100000 + 2 * layer + 1, device, dt)
    return k, v


def make_normal(shape, seed, std=1.0, device="cpu", dtype=torch.float32):
    """Seeded N(0, std) tensor for op-level test inputs (activations, caches)."""
    return _normal(shape, std, seed, 0x7FFF, device, dtype)


def make_uniform_ints(n, high, seed):
    rng = np.random.Generator(np.random.PCG64(seed + 0xA11))
    return rng.integers(0, high, size=n, dtype=np.int64).astype(np.int32)
