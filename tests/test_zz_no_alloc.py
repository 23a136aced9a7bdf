"""dg_op_lm_head_noalloc (the LM head on the library's static device scratch)
against dg_op_lm_head (the same kernels on the context's workspace): two calls
in a row, the second with fewer rows, on the fp32 and the bf16 path; and a row
count whose buffers exceed the static scratch is rejected before any launch."""
import numpy as np
import pytest
import torch

from block_diffusion_decoding_dg_amd import dg, synth
from tests.gpu_common import log, make_decoder

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wname", ["tiny", "mid"])
def test_lm_head_noalloc_matches_lm_head(wname):
    w = synth.WORKLOADS[wname]
    tw = synth.make_weights(w, seed=0, device="cuda")
    dec = make_decoder(w, tw)
    for n, seed in ((200, 1), (37, 2)):
        h = synth.make_normal((n, w.d_model), seed=seed, std=1.0, device="cuda")
        ent, lse, am = dec.dg_op_lm_head(h)
        ent2 = torch.full((n,), float("nan"), device="cuda")
        lse2 = torch.full((n,), float("nan"), device="cuda")
        am2 = torch.full((n,), -1, dtype=torch.int32, device="cuda")
        dec.dg_op_lm_head_noalloc(h, ent2, lse2, am2)
        torch.cuda.synchronize()
        log("%s no-alloc LM head, %d rows: entropy equal %s, lse equal %s, argmax equal %s"
            % (wname, n, torch.equal(ent, ent2), torch.equal(lse, lse2), torch.equal(am, am2)))
        assert torch.equal(ent, ent2) and torch.equal(lse, lse2) and torch.equal(am, am2)
    # more rows than the static scratch holds: refused on the host, nothing launched
    n_big = 65536  # past 16 MiB of buffers at both shapes
    h = torch.zeros((n_big, w.d_model), device="cuda")
    out_f = torch.zeros(n_big, device="cuda")
    out_i = torch.zeros(n_big, dtype=torch.int32, device="cuda")
    with pytest.raises(dg.DgError) as e:
        dec.dg_op_lm_head_noalloc(h, out_f, out_f, out_i)
    assert e.value.status == dg.DG_ERR_INVALID_ARG and "static scratch" in str(e.value)
    dec.close()
