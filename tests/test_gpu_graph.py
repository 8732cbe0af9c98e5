"""moe_layer_forward captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library only enqueues kernels on the caller's stream (no allocation, no memset, no host
synchronisation), so a layer call can be captured once and replayed. Every replay must give the
eager result bit for bit (the kernels are deterministic). The replays are separated by eager work
on other buffers and by synchronisations, and every replay is checked, not only the last.
"""
import pytest
import torch

import mixture_experts_layer_gemm_amd as moe
from _gpu_helpers import dev_tensor, say, torch_dtype, upload_layer
from synth import WORKLOADS, gen_layer_inputs

pytestmark = pytest.mark.gpu


def _buffers(spec, seed):
    inp = gen_layer_inputs(spec, seed=seed)
    x = dev_tensor(inp.x, inp.bits.get("x"), spec.dtype)
    return x, upload_layer(inp)


@pytest.mark.parametrize("name,S", [("dit_moe_xl", 700), ("des_vote_b025", 32), ("ec_dit", 1024),
                                    ("dit_moe_xl_reuse", 600)])
def test_graph_replay_matches_eager(name, S):
    spec = WORKLOADS[name].replace(S=S)
    say(f"graph {name}: S={S}")
    desc = moe.desc_from_spec(spec)
    x, wt = _buffers(spec, 0)
    w = moe.weights_struct(wt)
    ws = moe.workspace(desc)
    rb = moe.alloc_routing(desc)
    dt = torch_dtype(spec)
    y = torch.empty((spec.S, spec.d), dtype=dt, device="cuda")
    logits = torch.empty((spec.S, spec.E_routed), dtype=torch.float32, device="cuda")
    cache = torch.zeros((spec.S, spec.d), dtype=dt, device="cuda") if spec.reuse_tau > 0 else None
    cache0 = cache.clone() if cache is not None else None

    def call(stream):
        moe.moe_layer_forward(desc, x, w, None, logits, rb.struct, cache, None, y, ws, stream=stream)

    # eager reference (the cache, when used, starts from the same contents every time)
    call(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    y_ref, l_ref = y.clone(), logits.clone()
    c_ref = cache.clone() if cache is not None else None

    # other eager work on separate buffers, run between replays
    x2, wt2 = _buffers(spec, 1)
    w2 = moe.weights_struct(wt2)
    ws2 = moe.workspace(desc)
    y2 = torch.empty_like(y)
    cache2 = torch.zeros_like(cache) if cache is not None else None

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        if cache is not None:
            cache.copy_(cache0)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            call(side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep in range(4):
        y.fill_(0)
        logits.fill_(0)
        if cache is not None:
            cache.copy_(cache0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"replay {rep}: output differs from eager"
        assert torch.equal(logits, l_ref), f"replay {rep}: logits differ from eager"
        if cache is not None:
            assert torch.equal(cache, c_ref), f"replay {rep}: cache differs from eager"
        moe.moe_layer_forward(desc, x2, w2, None, None, None, cache2, None, y2, ws2)
        torch.cuda.synchronize()
