#!/usr/bin/env python3
"""Denoising-step benchmark: output tok/s at batch 1 and ms per 256-token step.

Workload (default "full"): a 30-layer, 25.2B-parameter (3.8B active) bf16 MoE
decoder with the shape the pages give for DiffusionGemma 26B A4B (128 experts,
8 routed + 1 shared, bidirectional attention over 256-token canvases; "DiffusionGemma
hits ~1,500 TPS on one H100", section "The specs that matter for serving").
Weights are random N(0, 0.02), and the prompt is 4096 uniform random ids.
1024 output tokens are produced as 4 canvases of 256.  The timed region is
`--steps` denoising steps (1024 by default = the whole 4096-in / 1024-out
generation) together with every block commit that falls inside it.  Weights
and the prompt's KV cache are resident in HBM before timing starts.

The JSON line carries:
  value        output tokens / timed seconds (tokens accepted by the sampler);
  ms_per_step  timed ms / steps;
  roofline     the dominant kernel (routed-expert W1/W3 projection) measured
               with HIP events on the library's stream: algorithmic bytes per
               launch / mean launch time against 8 TB/s; "traffic" is the HBM
               bytes per launch that rocprofv3's counters measured for this
               kernel source (profiles/ws_hbm_traffic.md), null once it changed;
  step_roofline  the whole step: algorithmic bytes and FLOPs per step against
               max(bytes / 8 TB/s, FLOPs / 2.5 PFLOP/s);
  cpu_baseline the float64 oracle timed on the first step(s) of block 0 at full
               size (all layers, LM head, sampler; optionally the commit),
               with its BLAS thread count and the host's nproc / lscpu.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
MFMA_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s
MFMA_F32_TFLOPS = 157.3

# Routed-expert W1/W3 kernel: the largest single kernel of the step (2/3 of the
# routed expert bytes, which are ~89% of the step's bytes at the full shape).
DOMINANT = "expert_up"
TIMER_EVERY = 8  # the dominant kernel is timed on one timed step in this many


def esize(w):
    return 2 if w.dtype == "bf16" else 4


def expert_matrix_bytes(w, rows, cols):
    """Bytes of one routed expert matrix [rows, cols]: the model dtype, one byte
    per E4M3 code plus a float32 scale per row, or half a byte per E2M1 code plus
    one E8M0 byte per 32 weights."""
    if w.expert_format == "fp8":
        return rows * cols + 4 * rows
    if w.expert_format == "mxfp4":
        return rows * cols // 2 + rows * cols // 32
    return rows * cols * esize(w)


def expert_up_bytes(w, touched, rows):
    """Algorithmic HBM bytes of one routed W1/W3 launch: the touched experts' W1 and
    W3 once, the normalised rows once, the SwiGLU output once."""
    es = esize(w)
    return (touched * 2 * expert_matrix_bytes(w, w.expert_hidden, w.d_model) + rows * w.d_model * es
            + rows * w.top_k * w.expert_hidden * es)


def step_bytes(w, P, rows, touched_per_layer, weights=True):
    """Algorithmic HBM bytes of one denoising step over `rows` canvas rows whose
    request has committed length P: every weight the step needs once (routed
    experts: only those touched), the KV prefix once, the canvas K/V written once.
    weights=False: the request's own bytes only (its KV), for the second and later
    requests of a step that denoises several canvases against the same weights."""
    es = esize(w)
    d, hd = w.d_model, w.head_dim
    dense = ((w.n_q_heads + 2 * w.n_kv_heads) * hd * d + w.n_q_heads * hd * d + w.n_experts * d
             + 3 * d * w.shared_hidden)
    total = 0
    per_expert = 2 * expert_matrix_bytes(w, w.expert_hidden, d) + expert_matrix_bytes(w, d, w.expert_hidden)
    kv = w.n_layers * 2 * w.n_kv_heads * hd * es
    total += P * kv + rows * kv          # prefix read + canvas K/V write
    if not weights:
        return total
    for t in touched_per_layer:
        total += dense * es + t * per_expert
    total += w.vocab * d * es            # LM head
    m = getattr(w, "self_cond_hidden", 0)
    if m:
        # self-conditioning: the transposed embedding once, the open rows' logits
        # (fp32) and softmax (bf16) written and read once, the MLP weights once
        total += w.vocab * d * es + rows * w.vocab * 2 * (4 + 2) + 3 * d * m * es
    return total


def step_flops(w, P, rows, n_open):
    d, hd = w.d_model, w.head_dim
    per_tok = ((w.n_q_heads + 2 * w.n_kv_heads) * hd * d + w.n_q_heads * hd * d + w.n_experts * d
               + 3 * d * w.shared_hidden + w.top_k * 3 * d * w.expert_hidden)
    f = 2 * rows * w.n_layers * per_tok
    f += 4 * w.n_layers * w.n_q_heads * hd * rows * (P + rows)
    f += 2 * n_open * d * w.vocab
    m = getattr(w, "self_cond_hidden", 0)
    if m:
        f += 2 * n_open * d * w.vocab + 2 * rows * 3 * d * m  # softmax x embedding; the MLP
    return f


def measured_traffic(w):
    """HBM bytes per launch of the dominant kernel (bf16, FP8 or MXFP4 experts, per the
    workload) from the committed rocprofv3 counter summary (FETCH_SIZE +
    WRITE_SIZE, copy-calibrated), or None when the kernel's source has changed
    since the counters were taken or the summary has no figure for it.  The bf16,
    FP8 and MXFP4 experts run on k_wsd."""
    import hashlib
    prof = os.path.join(ROOT, "profiles", "ws_hbm_traffic.md")
    src_name, sha_key = "k_wsd.hip", "k_wsd_source_sha256"
    src = os.path.join(ROOT, "block_diffusion_decoding_dg_amd", "csrc", src_name)
    try:
        key = {"fp8": "expert_up_fp8_traffic_bytes_per_launch",
               "mxfp4": "expert_up_mxfp4_traffic_bytes_per_launch"}.get(w.expert_format,
                                                                         "expert_up_traffic_bytes_per_launch")
        fields = dict(l.split(": ", 1) for l in open(prof).read().splitlines() if ": " in l and l.split(": ", 1)[0]
                      in (key, sha_key))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    if fields.get(sha_key, "").strip() != sha or key not in fields:
        return None
    if w.n_requests != 1 or w.prompt_len != 4096:  # the counters were taken on the one-request workload
        return None
    return int(fields[key])


def host_cpu():
    """nproc and lscpu's model, sockets, cores and threads of this host."""
    import subprocess
    info = {"nproc": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        keys = {"Model name": "model", "Socket(s)": "sockets", "Core(s) per socket": "cores_per_socket",
                "Thread(s) per core": "threads_per_core", "CPU(s)": "cpus"}
        for line in out.splitlines():
            k, _, v = line.partition(":")
            if k.strip() in keys:
                info[keys[k.strip()]] = v.strip()
    except (OSError, subprocess.SubprocessError):
        pass
    return info


def cpu_baseline(w, tw, n_steps=1, commit=False):
    """Time the float64 oracle (numpy) on real denoising steps of the same
    workload: the first n_steps steps of block 0 of one request -- each through
    every layer, the LM head over the open rows and the sampler -- and, with
    commit, the block commit's forward after them.  The request's committed prefix is
    prompt_len rows of synthetic keys and values (synth.make_prefix_kv; the
    oracle's own prefill of the prompt would take many times longer than the
    steps).  The oracle reads the model's weights from the GPU one layer at a
    time as float64 (oracle.stream): those copies are inside the timed region,
    the embedding's is not."""
    import numpy as np
    import threadpoolctl
    import oracle
    from oracle import stream
    from block_diffusion_decoding_dg_amd import synth

    cfg = oracle.ModelConfig(**w.model_dict())
    scfg = oracle.SamplerConfig(tau=w.tau, max_steps=w.max_steps)
    prec = oracle.Precision(bf16_points=(w.dtype == "bf16"))
    P = w.prompt_len
    ow = stream.lazy_weights(tw)
    st = stream.request_with_prefix(w.n_layers, P, w.canvas_len,
                                    lambda l: synth.make_prefix_kv(w, P, l, seed=1, device=tw["embed"].device),
                                    seed=0)
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] + [1])
    tokens, per_step, commit_s = 0, [], None
    t0 = time.perf_counter()
    for _ in range(n_steps):
        ts = time.perf_counter()
        r = oracle.denoise_step(st, cfg, scfg, ow, prec)
        per_step.append(time.perf_counter() - ts)
        tokens += int(np.sum(r.accepted_after & ~r.accepted_before))
        if r.done:
            break
    if commit:
        # the commit's forward (every layer's K/V over the canvas, kv only); the
        # canvas is not finished after a few steps, so it runs over the canvas
        # as it stands, which costs the same
        from oracle.decode import canvas_forward
        tc = time.perf_counter()
        canvas_forward(st, cfg, ow, prec, for_commit=True)
        commit_s = time.perf_counter() - tc
    elapsed = time.perf_counter() - t0
    host = host_cpu()
    return {"value": tokens / elapsed, "unit": "tok/s", "cores": int(threads), "kind": "oracle",
            "sample": ("float64 numpy oracle, the first %d step(s) of block 0%s of one request over a %d-row "
                       "synthetic KV prefix, every layer at full size (weights copied from the GPU layer by layer "
                       "inside the timed region): %.1f s per step%s, %d tokens accepted in %.1f s; %d BLAS threads "
                       "on a host with nproc %s (%s, %s socket(s) x %s cores x %s threads)"
                       % (len(per_step), " and the block commit" if commit else "", P,
                          float(np.mean(per_step)), "" if commit_s is None else ", commit %.1f s" % commit_s,
                          tokens, elapsed, threads, host.get("nproc"), host.get("model", "?"),
                          host.get("sockets", "?"), host.get("cores_per_socket", "?"),
                          host.get("threads_per_core", "?"))),
            "ms_per_step": float(np.mean(per_step)) * 1e3, "host": host}


def describe(w, K):
    C = w.canvas_len
    return ("%s: vocab %d, d_model %d, %d layers, %d/%d heads x %d, %d experts top-%d + 1 shared, expert hidden "
            "%d, shared hidden %d%s; %d requests x %d-token prompt, %d timed steps (%d canvases of %d)" % (
                w.name, w.vocab, w.d_model, w.n_layers, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_experts,
                w.top_k, w.expert_hidden, w.shared_hidden,
                {"fp8": ", routed experts in FP8 E4M3 with row scales",
                 "mxfp4": ", routed experts in MXFP4 (E2M1, E8M0 scale per 32 weights)"}.get(w.expert_format, "")
                + (", self-conditioning MLP of width %d" % w.self_cond_hidden if w.self_cond_hidden else ""),
                w.n_requests, w.prompt_len, K, max(1, -(-K // C)), C))


def timed_run(w, tw, K, W, kernel, seed, log):
    """Prefill, W untimed warm-up steps, prefill again, then K timed steps with
    the block commits that fall inside them.  Returns the measured figures."""
    import numpy as np
    import torch
    from block_diffusion_decoding_dg_amd import dg
    from block_diffusion_decoding_dg_amd import synth
    C = w.canvas_len
    R = w.n_requests
    n_blocks = max(1, -(-K // C))
    max_ctx = w.prompt_len + n_blocks * C
    cfg = dg.model_config(w, max_ctx=max_ctx)
    dec = dg.Decoder(cfg, w.tau, w.max_steps, tw)
    prompts = [synth.make_prompt(w, seed=seed + r) for r in range(R)]
    seeds = [seed + r for r in range(R)]

    def prefill_all():
        t0 = time.perf_counter()
        for r in range(R):
            dec.dg_prefill(r, prompts[r], seeds[r])
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3

    log("bench: %s: prefill %d x %d tokens" % (w.name, R, w.prompt_len))
    prefill_ms = prefill_all()
    log("bench: prefill %.1f ms; warmup %d steps" % (prefill_ms, W))
    # Experts touched per layer, sampled on the untimed warmup steps (the routing
    # of a canvas changes little from step to step) and on the last timed step.
    touched_samples = []

    def sample_touched():
        rids = dec.dg_last_step_rows()["router_ids"]
        touched_samples.append([int(np.unique(rids[l]).size) for l in range(w.n_layers)])

    for _ in range(W):
        dec.dg_denoise_step()
        sample_touched()
    prefill_ms = prefill_all()  # reset to block 0, step 0

    dec.dg_kernel_timer(kernel)
    # HIP events on every 8th step only: each event pair holds the stream for a
    # few microseconds, which timing every launch would add to the step time
    dec.dg_kernel_timer_every(TIMER_EVERY)
    torch.cuda.synchronize()
    log("bench: timing %d steps" % K)
    trace = []  # (block, step, first active request of its step) per request per step
    tokens = 0
    commits = 0
    t0 = time.perf_counter()
    for i in range(K):
        infos = dec.dg_denoise_step()
        first = True  # the step's first active request carries the weight bytes
        for r in range(R):
            inf = infos[r]
            if not inf["active"]:
                continue
            tokens += inf["n_accepted"] + inf["n_forced"]
            trace.append((inf["block"], inf["step"], first))
            first = False
        if all(infos[r]["done"] or not infos[r]["active"] for r in range(R)):
            for r in range(R):
                if infos[r]["active"] and infos[r]["done"]:
                    dec.dg_commit_block(r)
                    commits += 1
        if (i + 1) % 128 == 0:
            log("bench: %d steps, %.1f s" % (i + 1, time.perf_counter() - t0))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kt_ms, kt_n = dec.dg_kernel_timer_read()
    elapsed = t1 - t0

    sample_touched()
    touched = [float(np.mean([t[l] for t in touched_samples])) for l in range(w.n_layers)]
    dec.close()

    # Algorithmic bytes and FLOPs of every timed step, from its block and its open rows.
    tot_bytes = 0
    tot_flops = 0
    # With R concurrent requests a step reads the weights once (touched experts
    # as sampled for the whole batch) and each request's KV.
    for blk, step, first in trace:
        P = w.prompt_len + blk * C
        n_open = C - (step - 1)  # one acceptance per step before this one (random weights)
        tot_bytes += step_bytes(w, P, C, touched, weights=first)
        tot_flops += step_flops(w, P, C, n_open)
    mean_bytes = tot_bytes / max(1, len(trace)) * R
    mean_flops = tot_flops / max(1, len(trace)) * R
    ms_per_step = elapsed * 1e3 / K
    roof_ms = max(mean_bytes / (HBM_PEAK_GBS * 1e9), mean_flops / (MFMA_BF16_TFLOPS * 1e12)) * 1e3

    launch_ms = kt_ms / max(1, kt_n)
    bpl = expert_up_bytes(w, sum(touched) / len(touched), R * C)
    achieved = bpl / (launch_ms * 1e-3) / 1e9 if (kt_n and kernel == DOMINANT) else None
    return {
        "value": tokens / elapsed, "ms_per_step": ms_per_step, "tokens_per_step": tokens / K,
        "commits": commits, "prefill_ms": prefill_ms,
        "roofline": {"scope": "one kernel: the step's dominant launch (routed-expert W1/W3 projection, one per "
                              "layer); the whole step's fraction is step_roofline.frac",
                     "bound": "hbm", "kernel": kernel, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": (achieved / HBM_PEAK_GBS) if achieved else None, "traffic": None,
                     "launch_ms": launch_ms, "launches": kt_n, "bytes_per_launch": bpl},
        "step_roofline": {"scope": "the whole denoising step against max(bytes / 8 TB/s, FLOPs / 2.5 PFLOP/s)",
                          "bytes_per_step": mean_bytes, "flops_per_step": mean_flops,
                          "roofline_ms": roof_ms, "frac": roof_ms / ms_per_step,
                          "touched_experts_per_layer": sum(touched) / len(touched),
                          "touched_sampled_steps": len(touched_samples)},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="full")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel", default=DOMINANT, help="kernel family timed with HIP events")
    ap.add_argument("--cpu-steps", type=int, default=1,
                    help="denoising steps of block 0 the CPU oracle baseline times (about 20 s each at full size)")
    ap.add_argument("--cpu-commit", action="store_true", help="the CPU oracle baseline also times the block commit")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--fp8-steps", type=int, default=256,
                    help="steps timed again with the routed experts in FP8 (full workload only; 0 = skip)")
    ap.add_argument("--mxfp4-steps", type=int, default=256,
                    help="steps timed again with the routed experts in MXFP4 (full workload only; 0 = skip)")
    ap.add_argument("--sc-steps", type=int, default=256,
                    help="steps timed again with a self-conditioning MLP of width 256 (full workload only; 0 = skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-sized device buffer 8 times (calibrates rocprofv3 FETCH_SIZE/WRITE_SIZE "
                         "against a kernel of known traffic) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 8}))
        return

    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only (no sharding, no collectives); --gpus %d is not "
              "supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from block_diffusion_decoding_dg_amd import dg, synth

    if not torch.cuda.is_available():
        print("bench.py: needs a GPU", file=sys.stderr)
        sys.exit(2)
    w = synth.WORKLOADS[args.workload]
    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    log("bench: generating %s weights on the GPU" % w.name)
    tw = synth.make_weights(w, seed=args.seed, device="cuda")
    torch.cuda.synchronize()
    res = timed_run(w, tw, args.steps, args.warmup, args.kernel, args.seed, log)
    K, W, R, C = args.steps, args.warmup, w.n_requests, w.canvas_len
    out = {
        "metric": "output tok/s at bs=1, 4096-in/1024-out; ms per 256-token denoise step",
        "value": res["value"],
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic: random N(0,0.02) weights, uniform random prompt ids",
        "config": {"workload": describe(w, K),
                   "global_batch": R, "seq_len": w.prompt_len, "parallelism": "none"},
        "tokens_per_step": res["tokens_per_step"],
        "commits": res["commits"],
        "prefill_ms": res["prefill_ms"],
        "roofline": res["roofline"],
        "step_roofline": res["step_roofline"],
    }
    if w.expert_format == "fp8":
        out["dtype"] = "bf16, fp8 (e4m3) routed-expert weights"
    elif w.expert_format == "mxfp4":
        out["dtype"] = "bf16, mxfp4 (e2m1 + e8m0 block scales) routed-expert weights"
    if args.kernel == DOMINANT:
        out["roofline"]["traffic"] = measured_traffic(w)
    # The same model with its routed experts quantized to E4M3 + row scales (the
    # pages' FP8 checkpoint, as read here) and to MXFP4, each timed on its own.
    legs = (("fp8", args.fp8_steps, synth.quantize_rows_e4m3, "_scale"),
            ("mxfp4", args.mxfp4_steps, synth.quantize_blocks_mxfp4, "_mx_scale"))
    for fmt, steps, quant, suffix in legs:
        if steps <= 0 or w.name != "full":
            continue
        wq = synth.WORKLOADS["full_" + fmt]
        log("bench: quantizing the routed experts to %s" % fmt)
        layers = []
        for lt in tw["layers"]:
            lq = dict(lt)
            for n in ("w1", "w3", "w2"):
                lq[n], lq[n + suffix] = quant(lt[n])
            layers.append(lq)
        tq = dict(tw, layers=layers)
        torch.cuda.synchronize()
        rq = timed_run(wq, tq, steps, args.warmup, args.kernel, args.seed, log)
        if args.kernel == DOMINANT:
            rq["roofline"]["traffic"] = measured_traffic(wq)
        out[fmt + "_experts"] = {"workload": describe(wq, steps), "steps": steps,
                                 "value": rq["value"], "unit": "tok/s", "ms_per_step": rq["ms_per_step"],
                                 "roofline": rq["roofline"], "step_roofline": rq["step_roofline"]}
        del tq, layers
        torch.cuda.empty_cache()
    # The same model with self-conditioning (an MLP of width 256 on the previous
    # step's softmax expectation of the embedding), its kernels timed as a family.
    if args.sc_steps > 0 and w.name == "full":
        ws = synth.WORKLOADS["full_sc"]
        log("bench: self-conditioning leg")
        tsc = dict(tw, **synth.make_self_cond_weights(ws, seed=args.seed, device="cuda"))
        torch.cuda.synchronize()
        rs = timed_run(ws, tsc, args.sc_steps, args.warmup, "self_cond", args.seed, log)
        out["self_cond"] = {"workload": describe(ws, args.sc_steps), "steps": args.sc_steps, "value": rs["value"],
                            "unit": "tok/s", "ms_per_step": rs["ms_per_step"],
                            "self_cond_kernels_ms_per_launch": rs["roofline"]["launch_ms"],
                            "self_cond_launches_timed": rs["roofline"]["launches"],
                            "note": "two timed units per step: the MLP term added to the embedding, and the state "
                                    "update after the LM head (logits to bf16 softmax, split-vocabulary product with "
                                    "the transposed embedding, fold)",
                            "step_roofline": rs["step_roofline"]}
        del tsc
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("bench: CPU oracle baseline (%d step(s)%s)" % (args.cpu_steps, " and a commit" if args.cpu_commit else ""))
        out["cpu_baseline"] = cpu_baseline(w, tw, args.cpu_steps, args.cpu_commit)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
