"""GPU parity of the DICE denoising-step loop ("DICE: Staleness-Centric Optimizations for Parallel
Diffusion MoE Inference", 关键设计): a 2-layer DiT-MoE-XL-shaped stack run for 4 steps with a
drifting input, where layer 0 lets low-score tokens reuse its cached routed output (条件通信) except
on stride-refresh steps, and layer 1 stays synchronous (选择性同步). Every step's output and every
layer's cache are compared with the oracle's step loop, which keeps its own caches."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_gemm_amd as moe
import oracle as orc
from _gpu_helpers import assert_close, dev_tensor, reconcile_tc, routing_np, say, to_np, upload_layer
from synth import WORKLOADS, gen_layer_inputs, gen_tensor

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(600)
def test_dice_step_loop_matches_oracle():
    spec = WORKLOADS["dit_moe_xl"].replace(S=640, n_layers=2)
    T, stride, tau, reuse_layers = 4, 3, 0.3, (0,)
    inp = gen_layer_inputs(spec, seed=0)
    rng = np.random.default_rng(5)
    xs, x = [], inp.x.astype(np.float64)
    for _ in range(T):                    # the step-to-step drift of the latent tokens, stored in bf16
        xs.append(orc.bf16_round(x))
        x = xs[-1] + gen_tensor(rng, (spec.S, spec.d), 0.05, "f32")[0]
    wts = [upload_layer(inp, layer) for layer in range(spec.n_layers)]
    d_fresh = moe.desc_from_spec(spec.replace(reuse_tau=0.0))
    d_reuse = moe.desc_from_spec(spec.replace(reuse_tau=tau))
    ws = moe.workspace(d_reuse)
    caches = [torch.zeros((spec.S, spec.d), dtype=torch.bfloat16, device="cuda") for _ in range(spec.n_layers)]
    got = {}

    def hook(t, layer, h, L, rt, sp):
        say(f"step {t} layer {layer} tau={sp.reuse_tau}")
        desc = d_fresh if sp.reuse_tau == 0 else d_reuse
        h_dev = dev_tensor(h.astype(np.float32), None, "bf16")
        rb = moe.alloc_routing(desc)
        y = torch.empty_like(h_dev)
        logits = torch.empty((spec.S, spec.E_routed), dtype=torch.float32, device="cuda")
        prev_cache = caches[layer].clone()
        moe.moe_layer_forward(desc, h_dev, moe.weights_struct(wts[layer]), None, logits, rb.struct, caches[layer],
                              h_dev, y, ws)
        torch.cuda.synchronize()
        assert np.allclose(to_np(logits), L, atol=2e-5 * max(1.0, np.abs(L).max()))
        g = routing_np(rb, sp)
        rt = reconcile_tc(sp, L, rt, g["topk_idx"], g["reuse"] if sp.reuse_tau > 0 else None)
        reuse = g["reuse"].astype(bool) if sp.reuse_tau > 0 else np.zeros(spec.S, bool)
        # reused tokens left the cache alone, bit for bit
        assert torch.equal(caches[layer][torch.from_numpy(reuse).cuda()], prev_cache[torch.from_numpy(reuse).cuda()])
        got[(t, layer)] = (to_np(y), to_np(caches[layer]), reuse)
        return rt

    steps = orc.dice_step_loop(spec, inp, xs, tau=tau, stride=stride, reuse_layers=reuse_layers, rt_hook=hook,
                               h_store="bf16")
    n_reused = 0
    for t in range(T):
        for layer in range(spec.n_layers):
            y_gpu, c_gpu, reuse = got[(t, layer)]
            r = steps[t][layer]
            assert np.array_equal(reuse, r["reuse"])
            n_reused += int(reuse.sum())
            assert_close(y_gpu, r["y_exact"], "bf16", f"step {t} layer {layer} y")
            # fresh tokens wrote their routed part (one rounding to bf16 on each side); reused tokens
            # kept the previous cache (checked bit for bit in the hook)
            fresh = ~reuse
            assert_close(c_gpu[fresh], r["routed"][fresh], "bf16", f"step {t} layer {layer} cache")
            if layer not in reuse_layers or t % stride == 0:
                assert not reuse.any()
    say(f"  (token, layer) pairs reused: {n_reused} of {T * spec.n_layers * spec.S}")
    assert n_reused > 0
