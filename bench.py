"""Benchmark of the MoE FFN layer forward on one MI355X.

Default workload: the largest configuration, the MMOE MoE++ stack (64 x 256 = 16384 tokens, d=1152,
16 heavy GELU experts 1152->4608->1152 + identity, zero and constant experts + 1 shared expert, top-2
over 19 with gate-residual routing, 4 stacked layers), bf16, seeded synthetic inputs. A step is one
pass of the stack: per layer one moe_layer_forward call (router GEMM + the previous layer's logits,
softmax + top-k, counting-sort dispatch, the grouped expert GEMMs with the gather fused, and the
combine with the residual add). Inputs are resident in HBM before timing starts.

Prints one JSON line: tokens/s, the roofline of the dominant kernel (its duration read live with
HIP events attached to its launches on its own stream), and the fp64 CPU oracle timed on a bounded
sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--graph]

Other modes (each prints its own JSON lines): --des-fit (the DES per-expert latency model fitted on
the streaming kernels), --dice-steps (DICE reuse over a denoising-step loop), --dense (the GEMM
kernels on dense single-expert problems, with torch.matmul on the same shapes), --attnres (the
attention-residual aggregation's HBM rate), --calibrate-copy (a plain copy for the HBM counters).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E

METRIC = "MoE-layer tokens/s + % bf16 MFMA peak (GEMM) / % HBM peak (routing, DES)"

DESCRIPTIONS = {
    "dit_moe_tiny_f32": "1 x 256 tokens, d=384, 8 GELU experts 384->1536->384, top-2 renormalised, fp32",
    "dit_moe_xl": "32 x 256 = 8192 tokens, d=1152, 8 SwiGLU experts 1152->4608->1152 + 2 shared, top-2 renormalised",
    "dit_moe_xl_reuse": "dit_moe_xl with cached routed outputs reused for tokens whose top softmax score < 0.3",
    "ec_dit": "64 x 128 = 8192 tokens, d=1536, 32 GELU experts 1536->6144->1536, expert choice C=512",
    "des_vote_b025": "DES-Vote decode block: 32 tokens, d=2048, 64 SwiGLU experts 2048->1024->2048, top-8, core 16",
    "des_vote_b050": "DES-Vote decode block: 32 tokens, d=2048, 64 SwiGLU experts 2048->1024->2048, top-8, core 32",
    "des_seq": "DES-Seq decode block: 32 tokens, d=2048, 64 SwiGLU experts 2048->1024->2048, core = union of each "
               "token's top-2, tokens re-route top-8 inside it",
    "vanilla_top8": "vanilla decode block: 32 tokens, d=2048, 64 SwiGLU experts 2048->1024->2048, each token its own "
                    "top-8 (experts loaded = their union)",
    "mmoe": "MMOE MoE++ stack: 64 x 256 = 16384 tokens, d=1152, 16 GELU experts + identity/zero/constant + 1 shared, "
            "top-2 with gate residual, 4 layers",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mmoe", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0, help="oracle sample size (0 = automatic)")
    ap.add_argument("--dice-steps", action="store_true",
                    help="DICE denoising-step loop: reuse fraction and time per step under three policies")
    ap.add_argument("--des-fit", action="store_true",
                    help="fit the DES per-expert latency model f(c) = a*c + b on the streaming kernels")
    ap.add_argument("--rho", type=float, default=0.0,
                    help="with --des-fit: tokens of a block correlate by rho (shared component); 0 = independent")
    ap.add_argument("--dense", action="store_true",
                    help="the grouped GEMM kernels on dense single-expert problems, with torch.matmul on the same "
                         "shapes for context")
    ap.add_argument("--attnres", action="store_true",
                    help="attention-residual aggregation over n block states (MMOE width, 16384 tokens): "
                         "HBM throughput per n")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured once into a HIP graph and replayed (adds a 'graph' field)")
    ap.add_argument("--zero-operands", action="store_true",
                    help="with --dense: zero tokens and weights (the clock then stays at its peak)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (3 times): the reference for scaling "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes")
    return ap.parse_args()


def calibrate_copy():
    """A plain copy of known size. Under rocprofv3 --pmc its FETCH_SIZE and WRITE_SIZE per dispatch,
    divided by 1 GiB read and 1 GiB written, give the factors that turn the counters into bytes."""
    import torch

    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "dispatches": 3}), flush=True)


def des_fit(args):
    """The DES latency model ("Dynamic Expert Sharing", 2.1): an expert that serves c rows costs
    f(c) = a*c + b, b being the fetch of its weights, so a block costs a*(rows) + b*(experts used).
    Decode blocks of N in {8, 16, 32, 64} tokens are routed by vanilla top-8, DES-Vote (core 16 and
    32) and DES-Seq (core = union of each token's top-k_seq, k_seq in {1, 2, 4}, then top-8 inside
    it; 2.3, 3.1, 4.3); the two streaming kernels' time per block (HIP events on their launches) is
    fitted by least squares to t = a*rows + b*experts + c0 (c0: the fixed cost of the two launches).
    At N = 32 each DES-Seq block is also set against DES-Vote with a core of the same size, and
    every block reports its routing fidelity against vanilla top-8 (4.4): the cosine similarity of
    the per-expert hit counts, and the share of the vanilla top-8 routing mass the chosen experts
    keep. With --rho the block's tokens share a component (x_i = sqrt(rho) z + sqrt(1 - rho) e_i), a
    stand-in for the coupled tokens of one decoding block that gives vanilla routing fewer distinct
    experts. Prints one JSON line per block and one with the fit."""
    import numpy as np
    import torch

    import mixture_experts_layer_gemm_amd as moe
    from synth import WORKLOADS, gen_coupled_tokens, gen_layer_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    base = WORKLOADS["des_vote_b025"].replace(S=64)
    inp = gen_layer_inputs(base, seed=0)

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    copies = []
    for _ in range(4):   # rotated so the 256 MB MALL cannot keep a block's experts between calls
        t = {"w_router": up(inp.bits["w_router.0"]), "w1": up(inp.bits["w1.0"]), "w2": up(inp.bits["w2.0"]),
             "w3": up(inp.bits["w3.0"])}
        copies.append((t, moe.weights_struct(t)))
    if args.rho > 0.0:
        _, xbits = gen_coupled_tokens(np.random.default_rng(7), base.S, base.d, args.rho)
        x_all = up(xbits)
    else:
        x_all = up(inp.bits["x"])
    stream = torch.cuda.current_stream()
    rows, experts, times = [], [], []
    vanilla_hits = {}

    def run_block(name, spec, n):
        desc = moe.desc_from_spec(spec)
        ws = moe.workspace(desc, device=dev)
        rb = moe.alloc_routing(desc, device=dev)
        x = x_all[:n].contiguous()
        y = torch.empty_like(x)

        def call(i):
            moe.moe_layer_forward(desc, x, copies[i % 4][1], None, None, rb.struct, None, None, y, ws,
                                  stream=stream.cuda_stream)

        for i in range(args.warmup):
            call(i)
        torch.cuda.synchronize()
        moe.moe_profile_begin()
        for i in range(args.steps):
            call(i)
        prof = moe.moe_profile_end()
        torch.cuda.synchronize()
        # per layer call (a kernel may be launched more than once per call)
        t_us = sum(prof[k][0] * 1e3 / args.steps for k in ("stream_up", "stream_down") if k in prof)
        layer_us = sum(v[0] * 1e3 / args.steps for v in prof.values())
        counts = rb["counts"].cpu().numpy()[: spec.E_heavy]
        kk = min(spec.k, spec.m_core) if spec.mode == "des" else spec.k
        idx = rb["topk_idx"].cpu().numpy().reshape(-1)[: n * kk].reshape(n, kk)
        probs = rb["probs"].cpu().numpy()
        r, e = int(counts.sum()), int(np.count_nonzero(counts))
        line = {"block": name, "tokens": n, "rows": r, "experts": e,
                "weight_bytes": e * 3 * spec.d * spec.f * 2, "stream_us": round(t_us, 2),
                "kernels_us": round(layer_us, 2)}
        # routing fidelity against vanilla top-8 on the same tokens
        hits = np.bincount(idx[idx >= 0], minlength=spec.E_heavy).astype(float)
        if name == "vanilla":
            vanilla_hits[n] = (hits, np.sort(probs, axis=1)[:, ::-1][:, :8].sum(1))
        vh, vmass = vanilla_hits[n]
        kept = np.take_along_axis(probs, np.where(idx >= 0, idx, 0), 1) * (idx >= 0)
        line["hit_cosine_vs_vanilla"] = round(float(hits @ vh / (np.linalg.norm(hits) * np.linalg.norm(vh))), 4)
        line["routing_mass_kept_vs_vanilla"] = round(float(np.mean(kept.sum(1) / vmass)), 4)
        print(json.dumps(line), flush=True)
        rows.append(r)
        experts.append(e)
        times.append(t_us)
        return e

    for n in (8, 16, 32, 64):
        run_block("vanilla", WORKLOADS["vanilla_top8"].replace(S=n), n)
        for name, spec0 in (("vote16", WORKLOADS["des_vote_b025"]), ("vote32", WORKLOADS["des_vote_b050"])):
            run_block(name, spec0.replace(S=n), n)
        for kq in (1, 2, 4):
            e = run_block(f"seq_k{kq}", WORKLOADS["des_seq"].replace(S=n, vote_k=kq), n)
            if n == 32:   # DES-Vote with a core of the same size
                run_block(f"vote_core{e}", WORKLOADS["des_vote_b025"].replace(S=n, m_core=e), n)
    A = np.stack([np.asarray(rows, float), np.asarray(experts, float), np.ones(len(rows))], axis=1)
    coef, *_ = np.linalg.lstsq(A, np.asarray(times), rcond=None)
    pred = A @ coef
    d, f = base.d, base.f
    bytes_per_expert = 3 * d * f * 2
    print(json.dumps({"fit": "stream_us = a*rows + b*experts + c0", "rho": args.rho,
                      "a_us_per_row": round(float(coef[0]), 4),
                      "b_us_per_expert": round(float(coef[1]), 4), "c0_us": round(float(coef[2]), 3),
                      "max_abs_residual_us": round(float(np.abs(pred - np.asarray(times)).max()), 3),
                      "blocks": len(rows), "bytes_per_expert": bytes_per_expert,
                      "b_as_bandwidth_GBps": round(bytes_per_expert / (float(coef[1]) * 1e-6) / 1e9, 1)}),
          flush=True)


def dense_gemm(args):
    """The grouped GEMM kernels on dense problems: one heavy expert that every token takes (top-1 of
    1), so through moe_layer_forward the up projection is a plain S x (m*f) x d GEMM over the tokens
    in order (m = 2 for SwiGLU) and the down projection S x d x f. Their rates come from the
    library's own event timing of the two launches. torch.matmul (the vendor GEMM: bf16 out, no
    activation, no gather) runs the same shapes on operands drawn the same way, for context. One
    JSON line per shape."""
    import numpy as np
    import torch

    import mixture_experts_layer_gemm_amd as moe
    from synth import WORKLOADS, gen_layer_inputs, gen_tensor

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    S = 16384

    def up(bits):
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)
        return t.zero_() if args.zero_operands else t

    def vendor_us(a, b):
        for _ in range(3):
            torch.matmul(a, b.t())
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            torch.matmul(a, b.t())
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / args.steps

    for d, f, act in ((1152, 4608, "swiglu"), (1536, 6144, "gelu"), (4608, 4608, "swiglu")):
        spec = WORKLOADS["dit_moe_xl"].replace(S=S, d=d, f=f, act=act, E_heavy=1, n_shared=0, k=1)
        inp = gen_layer_inputs(spec, seed=0)
        b = inp.bits
        t = {"w_router": up(b["w_router.0"]), "w1": up(b["w1.0"]), "w2": up(b["w2.0"])}
        if act == "swiglu":
            t["w3"] = up(b["w3.0"])
        x = up(b["x"])
        desc = moe.desc_from_spec(spec)
        ws = moe.workspace(desc, device=dev)
        rb = moe.alloc_routing(desc, device=dev)
        y = torch.empty_like(x)
        wts = moe.weights_struct(t)
        stream = torch.cuda.current_stream()
        for _ in range(args.warmup):
            moe.moe_layer_forward(desc, x, wts, None, None, rb.struct, None, None, y, ws, stream=stream.cuda_stream)
        torch.cuda.synchronize()
        moe.moe_profile_begin()
        for _ in range(args.steps):
            moe.moe_layer_forward(desc, x, wts, None, None, rb.struct, None, None, y, ws, stream=stream.cuda_stream)
        prof = moe.moe_profile_end()
        torch.cuda.synchronize()
        m = 2 if act == "swiglu" else 1
        # per layer call: a projection may run as two launches (a column remainder split off)
        up_us = prof["gemm_up"][0] * 1e3 / args.steps
        down_us = prof["gemm_down"][0] * 1e3 / args.steps
        flops_up, flops_down = 2.0 * S * d * f * m, 2.0 * S * d * f
        # vendor GEMMs on the same shapes: tokens x (gate and up rows side by side), hidden x W2
        w_up = t["w1"].reshape(-1, d)
        if act == "swiglu":
            w_up = torch.cat([w_up, t["w3"].reshape(-1, d)], 0)
        h = up(gen_tensor(np.random.default_rng(1), (S, f), 1.0, "bf16")[1])
        v_up, v_down = vendor_us(x, w_up.contiguous()), vendor_us(h, t["w2"].reshape(-1, f).contiguous())
        print(json.dumps({"problem": f"{act} d={d} f={f} S={S}", "operands": "zero" if args.zero_operands else "random",
                          "up": f"{S} x {m * f} x {d}", "up_us": round(up_us, 1),
                          "up_tflops": round(flops_up / up_us / 1e6, 1),
                          "down": f"{S} x {d} x {f}", "down_us": round(down_us, 1),
                          "down_tflops": round(flops_down / down_us / 1e6, 1),
                          "vendor_up_tflops": round(flops_up / v_up / 1e6, 1),
                          "vendor_down_tflops": round(flops_down / v_down / 1e6, 1)}), flush=True)
        del t, x, y, ws, rb, h, w_up
        torch.cuda.empty_cache()


def attnres_bench(args):
    """Attention-residual aggregation ("MMOE: Modernizing Diffusion Transformers with Efficient Expert
    Design", 方法论) on the MMOE shape: 64 x 256 = 16384 tokens, d = 1152, bf16, with n = 5, 9 and 17
    states (4, 8, 16 completed block states and the partial one). The kernel reads every state once
    and writes the output: (n + 1) * S * d * 2 bytes per call, its HBM roofline. Successive calls
    take their states from a pool of 17 distinct ones (641 MB), so the 256 MB MALL cannot hold a
    call's inputs. Times are the library's event timing of the launches. One JSON line per n."""
    import numpy as np
    import torch

    import mixture_experts_layer_gemm_amd as moe
    from synth import gen_tensor

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    S, d = 16384, 1152
    rng = np.random.default_rng(0)

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    pool = [up(gen_tensor(rng, (S, d), 1.0, "bf16")[1]) for _ in range(17)]
    q = up(gen_tensor(rng, (d,), 1.0 / np.sqrt(d), "bf16")[1])
    out = torch.empty((S, d), dtype=torch.bfloat16, device=dev)
    for n in (5, 9, 17):
        sets = [[pool[(i * n + j) % len(pool)] for j in range(n)] for i in range(max(args.steps, args.warmup))]
        for i in range(args.warmup):
            moe.moe_attnres_aggregate(moe.MOE_BF16, S, d, sets[i], q, 1e-6, out)
        torch.cuda.synchronize()
        moe.moe_profile_begin()
        for i in range(args.steps):
            moe.moe_attnres_aggregate(moe.MOE_BF16, S, d, sets[i], q, 1e-6, out)
        prof = moe.moe_profile_end()
        torch.cuda.synchronize()
        us = prof["attnres"][0] * 1e3 / prof["attnres"][1]
        nbytes = (n + 1) * S * d * 2 + d * 2
        gbs = nbytes / us / 1e3
        print(json.dumps({"kernel": "attnres", "states": n, "tokens": S, "d": d, "dtype": "bf16", "us": round(us, 2),
                          "bytes_per_call": nbytes,
                          "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                       "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}}), flush=True)


def dice_steps(args):
    """The DICE step loop on one GPU ("DICE: Staleness-Centric Optimizations for Parallel Diffusion MoE
    Inference", 关键设计). A stack of 4 DiT-MoE-XL-shaped MoE layers (residual stream) runs T = 10
    denoising steps whose input drifts a little each step. Per layer and step, tokens whose top
    routing score is below tau reuse the layer's cached routed output (conditional communication,
    here: skipped expert rows); every `stride`-th step refreshes all tokens; with selective sync the
    deeper half of the layers never reuses. Policies: no reuse; reuse in every layer; DICE (shallow
    half reuses, deep half synchronous). Prints one JSON line per policy: time per step (HIP events
    over the whole loop), the fraction of (token, layer) pairs reused, and the speed-up over no reuse."""
    import numpy as np
    import torch

    import mixture_experts_layer_gemm_amd as moe
    from synth import WORKLOADS, gen_layer_inputs, gen_tensor

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L, T, stride, tau = 4, 10, 4, 0.3
    spec = WORKLOADS["dit_moe_xl"].replace(n_layers=L)
    inp = gen_layer_inputs(spec, seed=0)

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    ws_l = []
    for layer in range(L):
        t = {"w_router": up(inp.bits[f"w_router.{layer}"])}
        for n in ("w1", "w3", "w2", "s_w1", "s_w3", "s_w2"):
            t[n] = up(inp.bits[f"{n}.{layer}"])
        ws_l.append((t, moe.weights_struct(t)))
    x0 = up(inp.bits["x"])
    rng = np.random.default_rng(3)
    drift = []
    for _ in range(T):   # the step-to-step change of the latent tokens
        v, b = gen_tensor(rng, (spec.S, spec.d), 0.02, "bf16")
        drift.append(up(b))
    d_fresh = moe.desc_from_spec(spec.replace(reuse_tau=0.0))
    d_reuse = moe.desc_from_spec(spec.replace(reuse_tau=tau))
    ws = moe.workspace(d_reuse, device=dev)
    rbs = [moe.alloc_routing(d_reuse, device=dev) for _ in range(L)]
    stream = torch.cuda.current_stream()
    caches = [torch.zeros((spec.S, spec.d), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    hs = [torch.empty_like(x0) for _ in range(L)]
    xt = torch.empty_like(x0)
    results = {}
    for policy in ("none", "all", "dice"):
        def run(count):
            reused = 0
            xt.copy_(x0)
            for t in range(T):
                xt.add_(drift[t])
                h = xt
                for layer in range(L):
                    use = policy == "all" or (policy == "dice" and layer < L // 2)
                    fresh = (not use) or t % stride == 0
                    desc = d_fresh if fresh else d_reuse
                    moe.moe_layer_forward(desc, h, ws_l[layer][1], None, None, rbs[layer].struct, caches[layer], h,
                                          hs[layer], ws, stream=stream.cuda_stream)
                    if count and not fresh:
                        reused += int(rbs[layer]["reuse"].sum().item())
                    h = hs[layer]
            return reused

        run(False)   # warm-up (also fills the caches)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        run(False)
        ev1.record(stream)
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / T
        reused = run(True)
        frac = reused / float(T * L * spec.S)
        results[policy] = ms
        line = {"dice_policy": policy, "layers": L, "steps": T, "stride": stride, "tau": tau, "tokens": spec.S,
                "ms_per_step": round(ms, 4), "reused_fraction": round(frac, 4),
                "speedup_vs_no_reuse": round(results["none"] / ms, 3)}
        print(json.dumps(line), flush=True)


def sha256_of(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def read_traffic(kernel, workload):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it was taken on the current
    kernel source; None otherwise."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_src = re.search(r"source_sha256:\s*([0-9a-f]{64})", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    m_file = re.search(r"source_file:\s*(\S+)", txt)
    if not (m_src and m_b and m_file):
        return None
    if sha256_of(os.path.join(ROOT, m_file.group(1))) != m_src.group(1):
        return None
    return float(m_b.group(1))


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.des_fit:
        des_fit(args)
        return
    if args.dice_steps:
        dice_steps(args)
        return
    if args.dense:
        dense_gemm(args)
        return
    if args.attnres:
        attnres_bench(args)
        return

    import numpy as np
    import torch

    import mixture_experts_layer_gemm_amd as moe
    from synth import WORKLOADS, gen_layer_inputs, gen_tensor

    spec = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32

    def up(vals, bits):
        if bits is None:
            return torch.from_numpy(np.ascontiguousarray(vals, np.float32)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    t0 = time.time()
    inp = gen_layer_inputs(spec, seed=0)
    x = up(inp.x, inp.bits.get("x"))
    # decode blocks stream their experts' weights: rotate 4 weight copies so the 256 MB MALL cannot hold them
    streamed = bool(spec.E_heavy) and spec.S * spec.k / spec.E_heavy <= 64 and spec.mode != "ec"
    copies = 4 if streamed else 1
    layers = []
    for layer in range(spec.n_layers):
        per_copy = []
        for c in range(copies):
            b = inp.bits
            t = {"w_router": up(inp.w_router[layer], b.get(f"w_router.{layer}"))}
            if spec.E_heavy:
                t["w1"] = up(inp.w1[layer], b.get(f"w1.{layer}"))
                t["w2"] = up(inp.w2[layer], b.get(f"w2.{layer}"))
                if inp.w3[layer] is not None:
                    t["w3"] = up(inp.w3[layer], b.get(f"w3.{layer}"))
            if spec.n_shared:
                t["s_w1"] = up(inp.s_w1[layer], b.get(f"s_w1.{layer}"))
                t["s_w2"] = up(inp.s_w2[layer], b.get(f"s_w2.{layer}"))
                if inp.s_w3[layer] is not None:
                    t["s_w3"] = up(inp.s_w3[layer], b.get(f"s_w3.{layer}"))
            if spec.n_const:
                t["const_vec"] = up(inp.const_vec[layer], b.get(f"const_vec.{layer}"))
            per_copy.append((t, moe.weights_struct(t)))
        layers.append(per_copy)
    desc = moe.desc_from_spec(spec)
    ws = moe.workspace(desc, device=dev)
    rb = moe.alloc_routing(desc, device=dev)
    stream = torch.cuda.current_stream()
    cache = None
    if spec.reuse_tau > 0:
        # the cache holds the routed part of a previous call on slightly different tokens
        xv, xb = gen_tensor(np.random.default_rng(1), (spec.S, spec.d), 0.05, spec.dtype)
        x_prev = up(np.asarray(inp.x, np.float32) + xv, None).to(dt)
        cache = torch.zeros((spec.S, spec.d), dtype=dt, device=dev)
        d0 = moe.desc_from_spec(spec.replace(reuse_tau=0.0))
        ws0 = moe.workspace(d0, device=dev)
        y0 = torch.empty_like(x)
        moe.moe_layer_forward(d0, x_prev, layers[0][0][1], None, None, None, cache, None, y0, ws0)
        torch.cuda.synchronize()
    hs = [torch.empty_like(x) for _ in range(spec.n_layers)]
    logits = [torch.empty((spec.S, spec.E_routed), dtype=torch.float32, device=dev) for _ in range(spec.n_layers)]
    setup_s = time.time() - t0

    def step(i, st=None):
        h = x
        prev = None
        for layer in range(spec.n_layers):
            w = layers[layer][i % copies][1]
            res = h if spec.n_layers > 1 else None
            moe.moe_layer_forward(desc, h, w, prev, logits[layer] if spec.n_layers > 1 else None,
                                  rb.struct if layer == spec.n_layers - 1 else None, cache, res, hs[layer], ws,
                                  stream=(st or stream).cuda_stream)
            h = hs[layer]
            prev = logits[layer]

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - wall0) * 1e3 / args.steps
    ms = ev0.elapsed_time(ev1) / args.steps

    # the same steps captured once into a HIP graph (one step per weight copy) and replayed: the
    # launch gaps between the layer's kernels go away
    graph = None
    if args.graph:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            for i in range(copies):
                step(i, side)
        torch.cuda.synchronize()
        reps = max(1, args.steps // copies)
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        gev0, gev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gev0.record()
        for _ in range(reps):
            g.replay()
        gev1.record()
        torch.cuda.synchronize()
        gms = gev0.elapsed_time(gev1) / (reps * copies)
        graph = {"ms_per_step": round(gms, 4), "value": round(spec.S / (gms / 1e3), 1), "steps": reps * copies}

    # per-kernel times: a second pass with event pairs attached to every launch
    moe.moe_profile_begin()
    for i in range(args.steps):
        step(i)
    prof = moe.moe_profile_end()
    torch.cuda.synchronize()
    # avg_us: per layer call (the sum of a kernel's launches in one call: a GEMM projection may be split
    # into two launches); launches: over the whole pass
    calls = args.steps * spec.n_layers
    kernels = {k: {"avg_us": round(v[0] * 1e3 / calls, 2), "launches": v[1]} for k, v in prof.items()}

    # algorithmic work per launch from the actual routing
    n_rows = int(rb["n_rows"][0].item())
    counts = rb["counts"].cpu().numpy()
    n_active = int(np.count_nonzero(counts[: spec.E_heavy])) if spec.E_heavy else 0
    d, f = spec.d, spec.f
    mats_up = 2 if spec.act == "swiglu" else 1
    rows_gemm = n_rows + spec.S * spec.n_shared
    work = {
        "gemm_up": ("mfma", rows_gemm * 2.0 * d * f * mats_up),
        "gemm_down": ("mfma", rows_gemm * 2.0 * d * f),
        "stream_up": ("hbm", n_active * mats_up * f * d * (2 if spec.dtype == "bf16" else 4)),
        "stream_down": ("hbm", n_active * d * f * (2 if spec.dtype == "bf16" else 4)),
    }
    if streamed:
        # streamed experts: the shared experts (if any) still run on the tiled GEMM
        work["gemm_up"] = ("mfma", spec.S * spec.n_shared * 2.0 * d * f * mats_up)
        work["gemm_down"] = ("mfma", spec.S * spec.n_shared * 2.0 * d * f)
    cand = [k for k in work if k in prof and work[k][1] > 0]
    dom = max(cand, key=lambda k: prof[k][0]) if cand else None
    roofline = None
    if dom:
        avg_s = prof[dom][0] / calls / 1e3   # per layer call, like work_per_launch
        bound, amount = work[dom]
        if bound == "mfma":
            peak = PEAK_BF16_TFLOPS if spec.dtype == "bf16" else PEAK_F32_TFLOPS
            achieved = amount / avg_s / 1e12
            unit = "TFLOP/s"
        else:
            peak = PEAK_HBM_GBS
            achieved = amount / avg_s / 1e9
            unit = "GB/s"
        roofline = {"kernel": dom, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                    "frac": round(achieved / peak, 4), "traffic": read_traffic(dom, args.workload),
                    "work_per_launch": amount, "avg_us": round(avg_s * 1e6, 2)}

    layer_flops = spec.n_layers * (2.0 * spec.S * d * spec.E_routed + rows_gemm * 2.0 * d * f * (mats_up + 1))
    tokens_per_s = spec.S / (ms / 1e3)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(spec, inp, args.cpu_tokens)

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded N(0,1) tokens, N(0,0.02) weights)",
        "config": {"workload": f"{args.workload}: {DESCRIPTIONS[args.workload]}", "tokens_per_step": spec.S,
                   "layers": spec.n_layers, "dispatched_rows": n_rows, "active_experts": n_active},
        "layer_tflops": round(layer_flops / (ms / 1e3) / 1e12, 2),
        "wall_ms_per_step": round(wall_ms, 4),
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
    if graph is not None:
        out["graph"] = graph
    print(json.dumps(out), flush=True)


def cpu_baseline(spec, inp, n_tokens):
    """The fp64 oracle, untuned, on the first n tokens of the same inputs (bounded so the run stays
    around 10-30 s). Token choice and DES routing of a token do not depend on other tokens of the
    sample; for expert choice the sample is routed on its own."""
    import numpy as np

    import oracle as orc

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        cores = os.cpu_count()

    def run(n):
        sub = spec.replace(S=n)
        x = inp.x[:n].astype(np.float64)
        t = time.perf_counter()
        h, prev = x, None
        for layer in range(spec.n_layers):
            r = orc.layer_forward(sub, inp, h, layer=layer, prev_logits=prev,
                                  cache=np.zeros_like(x) if spec.reuse_tau > 0 else None,
                                  residual=h if spec.n_layers > 1 else None)
            h, prev = r["y"], r["logits"]
        return time.perf_counter() - t

    target = 12.0   # seconds of oracle work
    if n_tokens <= 0:
        n0 = min(spec.S, 128)
        t0 = run(n0)
        n_tokens = int(min(spec.S, max(n0, n0 * target / max(t0, 1e-3))))
    n_tokens = min(n_tokens, spec.S)
    # the first n tokens, repeated until about `target` seconds have passed when one pass is short
    t, reps = 0.0, 0
    while reps == 0 or (t < target and t / reps < target / 2 and reps < 50):
        t += run(n_tokens)
        reps += 1
    rep_note = f", {reps} passes" if reps > 1 else ""
    return {"value": round(n_tokens * reps / t, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {n_tokens} of {spec.S} tokens{rep_note}, whole layer ({spec.n_layers} layer(s)), "
                      f"numpy fp64",
            "seconds": round(t, 2)}


if __name__ == "__main__":
    main()
