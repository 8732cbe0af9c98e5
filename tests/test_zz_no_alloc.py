"""The entry point that allocates nothing (moe_layer_forward_noalloc) against moe_layer_forward with a
caller workspace, through the C ABI: two calls in a row, the second on a smaller input, each bit for
bit equal to the workspace entry point's result (same kernels, same order), and the routing too."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_gemm_amd as moe
from _gpu_helpers import dev_tensor, say, upload_layer
from synth import WORKLOADS, gen_layer_inputs

pytestmark = pytest.mark.gpu


def _pair(spec, seed):
    """(noalloc y, workspace y, noalloc routing, workspace routing) for one layer call."""
    say(f"noalloc {spec.name}: S={spec.S} seed={seed}")
    inp = gen_layer_inputs(spec, seed=seed)
    x = dev_tensor(inp.x, inp.bits.get("x"), spec.dtype)
    wt = upload_layer(inp)              # the tensors must outlive the calls: the struct holds raw addresses
    w = moe.weights_struct(wt)
    desc = moe.desc_from_spec(spec)
    assert moe.moe_workspace_bytes(desc) <= moe.MOE_NOALLOC_SCRATCH_BYTES
    outs = []
    for noalloc in (True, False):
        rb = moe.alloc_routing(desc)
        y = torch.empty_like(x)
        logits = torch.empty((spec.S, spec.E_routed), dtype=torch.float32, device="cuda")
        if noalloc:
            moe.moe_layer_forward_noalloc(desc, x, w, None, logits, rb.struct, None, x, y)
        else:
            ws = moe.workspace(desc)
            moe.moe_layer_forward(desc, x, w, None, logits, rb.struct, None, x, y, ws)
        torch.cuda.synchronize()
        outs.append((y, logits, rb))
    del wt
    return outs


@pytest.mark.parametrize("first,second", [
    (("dit_moe_xl", 1200), ("dit_moe_xl", 333)),          # tiled GEMMs, then a smaller call
    (("des_vote_b025", 32), ("des_vote_b025", 8)),         # a decode block, then a smaller block
])
def test_noalloc_matches_workspace_entry_point(first, second):
    for name, S in (first, second):
        spec = WORKLOADS[name].replace(S=S)
        (y0, l0, r0), (y1, l1, r1) = _pair(spec, seed=S)
        assert torch.equal(l0, l1)
        assert torch.equal(y0, y1)
        for key in ("topk_idx", "topk_w", "counts", "offsets", "row_token", "n_rows"):
            assert torch.equal(r0[key], r1[key]), key
        say(f"  bit-identical: y {tuple(y0.shape)}, rows {int(r0['n_rows'][0])}")
