"""Test-side glue: turns the synthetic torch weights into the oracle's float64 form."""
import numpy as np
import torch

import oracle
from block_diffusion_decoding_dg_amd import synth


def to_f64(t):
    if t is None:
        return None
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def oracle_config(w: synth.Workload) -> oracle.ModelConfig:
    return oracle.ModelConfig(**w.model_dict())


def oracle_weights(w: synth.Workload, tw) -> oracle.Weights:
    layers = []
    for lt in tw["layers"]:
        if lt is None:
            layers.append(None)
            continue
        d = {k: to_f64(v) for k, v in lt.items() if not k.endswith("_scale")}
        if "w1_scale" in lt:   # FP8 experts: the oracle's own decoding of the codes
            for n in ("w1", "w3", "w2"):
                d[n] = oracle.dequantize_rows(lt[n].cpu().numpy(), lt[n + "_scale"].cpu().numpy())
        if "w1_mx_scale" in lt:   # MXFP4 experts: likewise
            for n in ("w1", "w3", "w2"):
                d[n] = oracle.dequantize_mxfp4(lt[n].cpu().numpy(), lt[n + "_mx_scale"].cpu().numpy())
        layers.append(oracle.LayerWeights(**d))
    return oracle.Weights(embed=to_f64(tw["embed"]), final_norm=to_f64(tw["final_norm"]),
                          layers=layers, sc_w1=to_f64(tw.get("sc_w1")), sc_w3=to_f64(tw.get("sc_w3")),
                          sc_w2=to_f64(tw.get("sc_w2")))


def oracle_precision(w: synth.Workload, bf16_points=True) -> oracle.Precision:
    return oracle.Precision(bf16_points=(w.dtype == "bf16" and bf16_points))


def small_workload(**kw):
    """A tiny fp32 workload with overrides (for oracle pins)."""
    base = synth.WORKLOADS["tiny"]
    d = {**base.__dict__, **kw}
    return synth.Workload(**d)
