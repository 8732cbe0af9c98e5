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


def _sweep_cases():
    """The random-shape sweep's configurations without a cache (the entry point's calls here pass
    none) whose workspace fits the static scratch."""
    from test_gpu_random_layers import CONFIGS
    return [spec for spec, _ in CONFIGS
            if spec.reuse_tau == 0 and moe.moe_workspace_bytes(moe.desc_from_spec(spec)) <= moe.MOE_NOALLOC_SCRATCH_BYTES]


SWEEP = _sweep_cases()


@pytest.mark.parametrize("spec", SWEEP, ids=[s.name for s in SWEEP])
def test_noalloc_matches_workspace_entry_point_on_the_sweep(spec):
    """Every routing mode, precision and expert mix of the random-shape sweep: the output, the logits
    and every routing array are bit-identical to the workspace entry point's."""
    (y0, l0, r0), (y1, l1, r1) = _pair(spec, seed=int(spec.name[4:]) + 11)
    assert torch.equal(l0, l1)
    assert torch.equal(y0, y1)
    for key, t in r0.tensors.items():
        assert torch.equal(t, r1[key]), key


def test_noalloc_under_graph_capture():
    """The callers it is for: a decode-block layer captured into a HIP graph through the entry point
    that allocates nothing, replayed four times with eager calls of the same entry point (other
    inputs, the same static scratch) between the replays; every replay equals the eager result."""
    spec = WORKLOADS["des_vote_b025"]
    desc = moe.desc_from_spec(spec)
    bufs = []
    for seed in (0, 1):
        inp = gen_layer_inputs(spec, seed=seed)
        x = dev_tensor(inp.x, inp.bits.get("x"), spec.dtype)
        wt = upload_layer(inp)
        bufs.append((x, wt, moe.weights_struct(wt), torch.empty_like(x), moe.alloc_routing(desc)))
    (x, _, w, y, rb), (x2, _, w2, y2, rb2) = bufs
    logits = torch.empty((spec.S, spec.E_routed), dtype=torch.float32, device="cuda")

    def call(stream):
        moe.moe_layer_forward_noalloc(desc, x, w, None, logits, rb.struct, None, x, y, stream=stream)

    call(torch.cuda.current_stream().cuda_stream)   # eager reference (also sets up the scratch address)
    torch.cuda.synchronize()
    y_ref, l_ref = y.clone(), logits.clone()

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            call(side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep in range(4):
        y.fill_(0)
        logits.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"replay {rep}: output differs from eager"
        assert torch.equal(logits, l_ref), f"replay {rep}: logits differ from eager"
        moe.moe_layer_forward_noalloc(desc, x2, w2, None, None, rb2.struct, None, x2, y2)
        torch.cuda.synchronize()
    say("  graph replays of the no-allocation entry point: bit-identical")
