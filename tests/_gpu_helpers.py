"""Helpers for the GPU parity tests: uploads, layer runs through the C ABI, tolerance checks and
near-tie reconciliation (routing decisions that fp32 and fp64 may legitimately take differently)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import mixture_experts_layer_gemm_amd as moe
import oracle as orc

BF16_REL_L2 = 5e-3     # layer-output tolerances for bf16 workloads
BF16_MAX_ABS = 2e-2
F32_REL = 1e-5         # fp32 workloads: relative L2 and max-abs relative to max |y|


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_tensor(vals: np.ndarray, bits, dtype: str, device="cuda"):
    """Device copy of a stored tensor: bf16 from its exact encodings, fp32 from its values."""
    if dtype == "bf16":
        if bits is None:
            u = np.ascontiguousarray(vals, np.float32).view(np.uint32)
            assert np.all((u & 0xFFFF) == 0), "values are not bf16 numbers"
            bits = (u >> 16).astype(np.uint16)
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(vals, np.float32)).to(device)


def slots(spec) -> int:
    """Slots per token that the library fills densely: min(k, m_core) for DES-Vote, else k."""
    return min(spec.k, spec.m_core) if spec.mode == "des" else spec.k


def routing_np(rb, spec) -> dict:
    """Host copies of the routing buffers, with the per-slot arrays viewed as [S, slots]."""
    g = {k: v.cpu().numpy() for k, v in rb.tensors.items()}
    if spec.mode == "ec":
        return g
    ks = slots(spec)
    for name in ("topk_idx", "topk_w", "token_rows"):
        g[name] = g[name].reshape(-1)[: spec.S * ks].reshape(spec.S, ks)
    return g


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def upload_layer(inp, layer=0, device="cuda"):
    spec = inp.spec
    dt = spec.dtype
    b = inp.bits
    t = {"w_router": dev_tensor(inp.w_router[layer], b.get(f"w_router.{layer}"), dt, device)}
    if spec.E_heavy:
        t["w1"] = dev_tensor(inp.w1[layer], b.get(f"w1.{layer}"), dt, device)
        t["w2"] = dev_tensor(inp.w2[layer], b.get(f"w2.{layer}"), dt, device)
        if inp.w3[layer] is not None:
            t["w3"] = dev_tensor(inp.w3[layer], b.get(f"w3.{layer}"), dt, device)
    if spec.n_shared:
        t["s_w1"] = dev_tensor(inp.s_w1[layer], b.get(f"s_w1.{layer}"), dt, device)
        t["s_w2"] = dev_tensor(inp.s_w2[layer], b.get(f"s_w2.{layer}"), dt, device)
        if inp.s_w3[layer] is not None:
            t["s_w3"] = dev_tensor(inp.s_w3[layer], b.get(f"s_w3.{layer}"), dt, device)
    if spec.n_const:
        t["const_vec"] = dev_tensor(inp.const_vec[layer], b.get(f"const_vec.{layer}"), dt, device)
    return t


def torch_dtype(spec):
    return torch.bfloat16 if spec.dtype == "bf16" else torch.float32


def run_layer(spec, x_dev, wt, flags=0, prev=None, cache=None, residual=None, ws=None, routing=None):
    """One moe_layer_forward through the C ABI. Returns (y, logits, routing buffers)."""
    desc = moe.desc_from_spec(spec, flags)
    if routing is None:
        routing = moe.alloc_routing(desc)
    if ws is None:
        ws = moe.workspace(desc)
    y = torch.empty((spec.S, spec.d), dtype=torch_dtype(spec), device="cuda")
    logits = torch.empty((spec.S, spec.E_routed), dtype=torch.float32, device="cuda")
    w = moe.weights_struct(wt)
    moe.moe_layer_forward(desc, x_dev, w, prev, logits, routing.struct, cache, residual, y, ws)
    torch.cuda.synchronize()
    return y, logits, routing


def bf16_half_ulp(a: np.ndarray) -> np.ndarray:
    """Half the spacing of bfloat16 numbers at |a| (8 significant bits): 2^(e - 8) for
    2^e <= |a| < 2^(e+1); 0 at a = 0."""
    a = np.abs(np.asarray(a, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 8), 0.0)


def assert_close(y_gpu: np.ndarray, y_ref: np.ndarray, dtype: str, what=""):
    """Layer-output tolerance against the fp64 oracle.

    bf16: rel-L2 <= 5e-3 and max-abs <= 2e-2. The output is stored in bf16, so it carries up to
    half a bf16 ulp of rounding that no implementation can avoid; the max-abs bound applies to the
    value before that rounding, i.e. |y_gpu - y_ref| - half_ulp(max(|y_gpu|, |y_ref|)) <= 2e-2.
    fp32: rel-L2 <= 1e-5 and max-abs <= 1e-5 * max |y_ref|. Prints the measured values and the
    margin (bound / measured) of each bound."""
    y_gpu = np.asarray(y_gpu, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    assert y_gpu.shape == y_ref.shape, (y_gpu.shape, y_ref.shape)
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite output"
    diff = np.abs(y_gpu - y_ref)
    rel = np.linalg.norm(diff) / max(np.linalg.norm(y_ref), 1e-30)
    raw = float(diff.max()) if diff.size else 0.0
    if dtype == "bf16":
        excess = diff - bf16_half_ulp(np.maximum(np.abs(y_gpu), np.abs(y_ref)))
        mx = max(0.0, float(excess.max())) if diff.size else 0.0
        say(f"  {what}: rel-L2 {rel:.3e} (<= {BF16_REL_L2}, margin {BF16_REL_L2 / max(rel, 1e-30):.1f}x), "
            f"max-abs {raw:.3e}, beyond the output's half-ulp {mx:.3e} (<= {BF16_MAX_ABS}, "
            f"margin {BF16_MAX_ABS / max(mx, 1e-30):.1f}x), n={y_ref.size}")
        assert rel <= BF16_REL_L2, f"{what}: rel-L2 {rel}"
        assert mx <= BF16_MAX_ABS, f"{what}: max-abs beyond half-ulp {mx}"
    else:
        scale = max(float(np.abs(y_ref).max()) if y_ref.size else 0.0, 1e-30)
        say(f"  {what}: rel-L2 {rel:.3e} (<= {F32_REL}, margin {F32_REL / max(rel, 1e-30):.1f}x), "
            f"max-abs/max|y| {raw / scale:.3e} (<= {F32_REL}, margin {F32_REL * scale / max(raw, 1e-30):.1f}x)")
        assert rel <= F32_REL, f"{what}: rel-L2 {rel}"
        assert raw <= F32_REL * scale, f"{what}: max-abs {raw}"


def h_store(spec):
    """Storage precision of the hidden activation between the two projections: the layer dtype
    (bf16 layers keep H in bf16; fp32 layers keep it exact to fp32)."""
    return "bf16" if spec.dtype == "bf16" else None


def assert_rel_exact(y_gpu: np.ndarray, y_exact: np.ndarray, what=""):
    """The relative bound against the oracle with exact (fp64) hidden activations: the layer's bf16
    storage of H is the only intermediate rounding that comparison does not model, and it stays
    within rel-L2 5e-3."""
    y_gpu = np.asarray(y_gpu, np.float64)
    y_exact = np.asarray(y_exact, np.float64)
    rel = np.linalg.norm(y_gpu - y_exact) / max(np.linalg.norm(y_exact), 1e-30)
    say(f"  {what} vs exact-H oracle: rel-L2 {rel:.3e} (<= {BF16_REL_L2}, margin {BF16_REL_L2 / max(rel, 1e-30):.1f}x), "
        f"max-abs {np.abs(y_gpu - y_exact).max() if y_gpu.size else 0.0:.3e} (information)")
    assert rel <= BF16_REL_L2, f"{what}: rel-L2 vs exact-H oracle {rel}"


# ------------------------------------------------------------------------------------------------
# Near-tie reconciliation. The GPU decides on fp32 logits from an fp32-accumulated GEMM, the oracle
# on fp64 logits; they differ by ~1e-6. Where the oracle's own decision margin is below `eps`, both
# choices are correct. The GPU's choice is accepted there only after checking it is one of the
# valid choices; everywhere else the decisions must match exactly.

def reconcile_tc(spec, L64, rt, idx_gpu, reuse_gpu=None, eps=1e-4, max_frac=1e-3):
    """eps: the decision margin below which both choices are accepted, a scalar or one per token
    (a layer deep in a stack sees inputs that differ by rounding from the oracle's)."""
    idx_gpu = np.asarray(idx_gpu, np.int64)
    eps = np.broadcast_to(np.asarray(eps, np.float64), (L64.shape[0],))
    P = rt["P"]
    k = idx_gpu.shape[1]
    keys = L64
    if spec.mode in ("des", "des_seq"):
        core = rt["core"]
        mask = np.full(L64.shape, -np.inf)
        mask[:, core] = 0.0
        keys = L64 + mask
    srt = -np.sort(-keys, axis=1)
    kth = srt[:, k - 1]
    nxt = srt[:, k] if keys.shape[1] > k else np.full(len(kth), -np.inf)
    same = np.all(np.sort(idx_gpu, 1) == np.sort(rt["idx"], 1), axis=1)
    ordered = np.all(idx_gpu == rt["idx"], axis=1)
    bad = np.nonzero(~ordered)[0]
    n_fix = 0
    for s in bad:
        # every chosen GPU expert must be within eps of the k-th oracle key, and the order flip
        # must be between near-equal keys
        g = keys[s, idx_gpu[s]]
        assert np.all(g >= kth[s] - eps[s]), f"token {s}: GPU took {idx_gpu[s]}, oracle {rt['idx'][s]}"
        if not same[s]:
            assert kth[s] - nxt[s] < eps[s], f"token {s}: set differs without a near tie"
        assert np.all(np.diff(g) <= eps[s]), f"token {s}: GPU slot order not by key"
        n_fix += 1
    if len(bad):
        rt = dict(rt)
        idx = rt["idx"].copy()
        idx[bad] = idx_gpu[bad]
        rt["idx"] = idx
        rt["w"] = orc.tc_weights(P, idx, spec.renorm)
    if reuse_gpu is not None and spec.reuse_tau > 0:
        reuse_gpu = np.asarray(reuse_gpu, bool)
        diff = np.nonzero(reuse_gpu != rt["reuse"])[0]
        for s in diff:
            assert abs(rt["pmax"][s] - spec.reuse_tau) < 1e-5, f"token {s}: reuse flag differs"
        if len(diff):
            rt = dict(rt)
            r = rt["reuse"].copy()
            r[diff] = reuse_gpu[diff]
            rt["reuse"] = r
        n_fix += len(diff)
    frac = n_fix / max(1, L64.shape[0])
    say(f"  near-tie tokens reconciled: {n_fix} ({frac:.2e} of tokens)")
    assert frac <= max_frac
    return rt


def reconcile_ec(spec, rt, row_token_gpu, C, eps=1e-7):
    """Per expert, the GPU's C tokens must equal the oracle's except among tokens whose affinity
    is within eps of the C-th largest."""
    P = rt["P"]
    E = P.shape[1]
    tok_gpu = np.asarray(row_token_gpu, np.int64)[: E * C].reshape(E, C)
    n_fix = 0
    tokens = rt["tokens"].copy()
    for i in range(E):
        a, b = set(tokens[i].tolist()), set(tok_gpu[i].tolist())
        if a == b:
            continue
        thr = np.sort(P[:, i])[::-1][C - 1]
        for s in a ^ b:
            assert abs(P[s, i] - thr) < eps, f"expert {i}: token {s} differs without a near tie"
        tokens[i] = np.sort(tok_gpu[i])
        n_fix += len(a ^ b)
    if n_fix:
        rt = dict(rt)
        rt["tokens"] = tokens
        rt["gates"] = np.take_along_axis(P.T, tokens, axis=1)
    say(f"  near-tie expert-choice swaps reconciled: {n_fix}")
    return rt


def reconcile_des(spec, rt, core_gpu, L64, eps=1e-5):
    core_gpu = np.sort(np.asarray(core_gpu, np.int64))
    if np.array_equal(core_gpu, rt["core"]):
        return rt
    v = np.asarray(rt["votes"], np.float64)
    order = orc.rank_desc(v[None, :])[0]
    m = spec.m_core
    edge = v[order[m - 1]] - (v[order[m]] if len(order) > m else -np.inf)
    assert edge < eps, f"core differs without a near tie (gap {edge})"
    for e in set(core_gpu.tolist()) ^ set(rt["core"].tolist()):
        assert abs(v[e] - v[order[m - 1]]) < eps
    rt = dict(rt)
    rt["core"] = core_gpu
    P = rt["P"]
    idx, w = orc.core_reroute(L64, P, core_gpu, spec.k, spec.renorm)
    rt["idx"], rt["w"] = idx, w
    say("  near-tie DES core reconciled")
    return rt


def reconcile_des_seq(spec, rt, core_gpu, L64, eps=1e-4):
    """DES-Seq: the core is the union of each token's top-k_seq. An expert may be in one side's core
    and not the other's only through a near tie at some token's k_seq boundary; then the GPU's core
    is taken and the oracle re-routes inside it."""
    core_gpu = np.asarray(core_gpu, np.int64)
    core_gpu = np.sort(core_gpu[core_gpu >= 0])
    if np.array_equal(core_gpu, rt["core"]):
        return rt
    kq = spec.vote_k
    srt = -np.sort(-L64, axis=1)
    kth = srt[:, kq - 1]
    nxt = srt[:, kq] if L64.shape[1] > kq else np.full(L64.shape[0], -np.inf)
    for e in set(core_gpu.tolist()) ^ set(rt["core"].tolist()):
        near = (np.abs(L64[:, e] - kth) < eps) & (kth - nxt < eps)
        assert near.any(), f"DES-Seq core differs at expert {e} without a near tie"
    rt = dict(rt)
    rt["core"] = core_gpu
    idx, w = orc.core_reroute(L64, rt["P"], core_gpu, spec.k, spec.renorm)
    rt["idx"], rt["w"] = idx, w
    say("  near-tie DES-Seq core reconciled")
    return rt
