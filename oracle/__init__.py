"""CPU oracle for one denoising step of a block-autoregressive text-diffusion decoder.

TEST INFRASTRUCTURE ONLY.  A plain, slow float64 implementation (numpy; its
matrix product is the only library primitive used) of what the GPU library
computes.  Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg
of `bench.py` may import it.  It shares no code with the GPU library and
imports nothing from it.

Parity pins (see tests/test_oracle_*.py): Philox against numpy's own
Philox4x64-10; attention and RoPE against closed forms; the MoE against a
dense all-experts evaluation with a gate mask; entropy against scipy and
closed forms; the sampler against its invariants and brute-force
enumeration; the commit against a one-shot forward under the block mask; the
E4M3 decoding against torch's float8_e4m3fn and the format's closed forms.
Logit values of a whole random-weight model have no printed worked example in
the pages: beyond those pins they are "parity unpinned".
"""
from .model import (ModelConfig, LayerWeights, Weights, Precision, round_bf16, rmsnorm, rope,
                    attention, silu, topk_select, route, moe, layer_forward, lm_head_stats,
                    self_cond_input, self_cond_embedding)
from .philox import philox4x64_10, draw_tokens
from .quant import (decode_e4m3, dequantize_rows, E4M3_MAX, decode_e2m1, decode_e8m0, unpack_fp4,
                    dequantize_mxfp4, MX_BLOCK, E2M1_MAX)
from .decode import (SamplerConfig, RequestState, StepResult, new_request, prefill, start_canvas,
                     canvas_forward, canvas_forward_batch, sampler_decide, entropy_fixed, budget_decide, denoise_step, denoise_step_batch, commit_block, generate)
