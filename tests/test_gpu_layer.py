"""GPU parity of the whole layer (moe_layer_forward and the four-call path) against the fp64 oracle,
on every workload shape: reduced token counts that span several tiles with ragged tails, and every
token of every workload at its full size, in the launch configuration the benchmark uses."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_gemm_amd as moe
import oracle as orc
from _gpu_helpers import (assert_close, assert_rel_exact, dev_tensor, h_store, reconcile_des, reconcile_des_seq,
                          reconcile_ec, reconcile_tc, routing_np, run_layer, say, to_np, upload_layer)
from synth import WORKLOADS, gen_layer_inputs, gen_tensor

pytestmark = pytest.mark.gpu


def _oracle_rt(spec, L64, got_rb, reuse=True, eps=1e-4, max_frac=1e-3):
    """The oracle's routing of L64, with near-tie decisions taken from the GPU where both are valid."""
    rt = orc.route(spec, L=L64)
    g = routing_np(got_rb, spec)
    if spec.mode == "ec":
        return reconcile_ec(spec, rt, g["row_token"], rt["C"])
    if spec.mode == "des":
        rt = reconcile_des(spec, rt, g["core"][: spec.m_core], L64)
    idx_gpu = g["topk_idx"]
    if spec.mode == "des_seq":
        rt = reconcile_des_seq(spec, rt, g["core"], L64)
        kp = rt["idx"].shape[1]                      # min(k, |core|); the rest are empty slots
        assert np.all(idx_gpu[:, kp:] == -1) and np.all(g["topk_w"][:, kp:] == 0)
        assert np.all(g["token_rows"][:, kp:] == -1)
        idx_gpu = idx_gpu[:, :kp]
    return reconcile_tc(spec, L64, rt, idx_gpu, g["reuse"] if (reuse and spec.reuse_tau > 0) else None,
                        eps=eps, max_frac=max_frac)


def _layer_case(spec, seed=0, flags=0, with_cache=False, residual=False):
    say(f"layer {spec.name}: S={spec.S} d={spec.d} f={spec.f} E_r={spec.E_routed} mode={spec.mode} flags={flags}")
    inp = gen_layer_inputs(spec, seed=seed)
    x = dev_tensor(inp.x, inp.bits.get("x"), spec.dtype)
    wt = upload_layer(inp)
    cache_np = cache = None
    if with_cache:
        rng = np.random.default_rng(seed + 100)
        cv, cb = gen_tensor(rng, (spec.S, spec.d), 0.5, spec.dtype)
        cache_np = cv.astype(np.float64)
        cache = dev_tensor(cv, cb, spec.dtype)
    res = x if residual else None
    y, logits, rb = run_layer(spec, x, wt, flags=flags, cache=cache, residual=res)
    L64 = orc.router_logits(inp.x, inp.w_router[0])
    assert np.allclose(to_np(logits), L64, atol=2e-5 * max(1.0, np.abs(L64).max()))
    rt = _oracle_rt(spec, L64, rb)
    res_np = inp.x if residual else None
    ref = orc.layer_forward(spec, inp, inp.x, cache=cache_np, rt=rt, residual=res_np, h_store=h_store(spec))
    assert_close(to_np(y), ref["y"], spec.dtype, spec.name)
    if h_store(spec):
        exact = orc.layer_forward(spec, inp, inp.x, cache=cache_np, rt=rt, residual=res_np)
        assert_rel_exact(to_np(y), exact["y"], spec.name)
    if with_cache:
        # fresh tokens wrote their routed part to the cache; reused tokens left it alone
        fresh = ~rt["reuse"]
        got_cache = to_np(cache)
        assert np.array_equal(got_cache[rt["reuse"]], cache_np[rt["reuse"]])
        assert_close(got_cache[fresh], ref["routed"][fresh], spec.dtype, spec.name + " cache")
    return inp, rt, y, rb


def test_tiny_f32_layer_full_size():
    spec = WORKLOADS["dit_moe_tiny_f32"]
    _layer_case(spec)
    _layer_case(spec, flags=moe.MOE_F_FORCE_TILED)
    _layer_case(spec, flags=moe.MOE_F_FORCE_STREAM)


F32_CASES = {
    # every routing mode and expert kind in fp32 end to end (fp32 MFMA, register weight streaming)
    "des_vote": (WORKLOADS["des_vote_b025"].replace(S=32, d=256, f=256, m_core=8, dtype="f32"), 0, False, False),
    "des_seq": (WORKLOADS["des_seq"].replace(S=24, d=256, f=256, dtype="f32"), 0, False, False),
    "ec": (WORKLOADS["ec_dit"].replace(S=300, d=128, f=256, E_heavy=8, dtype="f32"), 0, False, False),
    "mmoe_light_shared": (WORKLOADS["mmoe"].replace(S=200, d=128, f=256, n_layers=1, dtype="f32"), 0, False, True),
    "reuse_stream": (WORKLOADS["dit_moe_xl_reuse"].replace(S=96, d=128, f=256, reuse_tau=0.2, dtype="f32"),
                     moe.MOE_F_FORCE_STREAM, True, False),
}


@pytest.mark.parametrize("name", list(F32_CASES))
def test_f32_layer_modes(name):
    spec, flags, with_cache, residual = F32_CASES[name]
    _layer_case(spec, flags=flags, with_cache=with_cache, residual=residual)


def test_dit_moe_xl_layer_reduced():
    spec = WORKLOADS["dit_moe_xl"].replace(S=700)
    _layer_case(spec)
    _layer_case(spec, seed=1, flags=moe.MOE_F_FORCE_STREAM, residual=True)


def test_dit_moe_xl_reuse_layer_reduced():
    spec = WORKLOADS["dit_moe_xl_reuse"].replace(S=900)
    _, rt, _, _ = _layer_case(spec, with_cache=True)
    assert 0 < rt["reuse"].sum() < spec.S


def test_reuse_extremes():
    base = WORKLOADS["dit_moe_xl_reuse"].replace(S=300, d=256, f=512)
    _layer_case(base.replace(reuse_tau=1.5), with_cache=True)     # everything from the cache
    _layer_case(base.replace(reuse_tau=0.0))                      # reuse off


def test_ec_dit_layer_reduced():
    spec = WORKLOADS["ec_dit"].replace(S=1024)
    _, rt, _, _ = _layer_case(spec)
    assert rt["C"] == 64


@pytest.mark.parametrize("name", ["des_vote_b025", "des_vote_b050"])
def test_des_layer_full_size(name):
    spec = WORKLOADS[name]
    _layer_case(spec)
    _layer_case(spec, flags=moe.MOE_F_FORCE_TILED)


def test_vanilla_top8_block_full_size():
    """The vanilla decode block the DES variants are measured against: each token its own top-8; the
    experts streamed are the union of the tokens' choices."""
    spec = WORKLOADS["vanilla_top8"]
    inp, rt, _, rb = _layer_case(spec)
    counts = rb["counts"].cpu().numpy()[: spec.E_heavy]
    assert np.array_equal(np.flatnonzero(counts > 0), np.unique(rt["idx"]))
    assert counts.sum() == spec.S * spec.k


@pytest.mark.parametrize("k_seq", [1, 2, 4])
def test_des_seq_block_full_size(k_seq):
    """DES-Seq ("Dynamic Expert Sharing", 2.3, 3.1, 4.3): the core is the union of the tokens' top-k_seq
    and every token re-activates its top-8 inside it. The core and votes (selection counts) match the
    oracle, only core experts get rows, and the layer output matches; streamed and tiled paths."""
    spec = WORKLOADS["des_seq"].replace(vote_k=k_seq)
    for flags in (0, moe.MOE_F_FORCE_TILED):
        inp, rt, _, rb = _layer_case(spec, flags=flags)
        g = routing_np(rb, spec)
        core = g["core"]
        n = int(np.count_nonzero(core >= 0))
        assert np.array_equal(core[:n], rt["core"]) and np.all(core[n:] == -1)
        L64 = orc.router_logits(inp.x, inp.w_router[0])
        if np.array_equal(rt["core"], orc.route(spec, L=L64)["core"]):
            assert np.array_equal(g["votes"], orc.des_seq_counts(L64, k_seq, spec.E_routed).astype(np.float32))
        counts = g["counts"][: spec.E_heavy]
        assert set(np.flatnonzero(counts > 0)) <= set(rt["core"].tolist())
        assert counts.sum() == spec.S * min(spec.k, n)


def test_des_seq_core_smaller_than_k():
    """A 3-token block with k_seq = 1 and k = 8: the core holds at most 3 experts, so every token keeps
    all of them and its other slots are empty (expert -1, weight 0)."""
    spec = WORKLOADS["des_seq"].replace(S=3, vote_k=1, d=256, f=256)
    _, rt, _, rb = _layer_case(spec, flags=moe.MOE_F_FORCE_STREAM)
    g = routing_np(rb, spec)
    n = rt["core"].size
    assert n <= 3 and np.all(g["topk_idx"][:, n:] == -1) and np.all(g["topk_w"][:, n:] == 0)


@pytest.mark.parametrize("d,f,act,S,m_core", [
    (256, 256, "swiglu", 32, 16),     # up: 2 stages per wave (the ring's minimum); down: 2
    (384, 640, "swiglu", 40, 16),     # odd stage counts (3 and 5)
    (256, 128, "gelu", 32, 16),       # down K=128 is below the ring's minimum: register streaming
    (512, 256, "gelu_tanh", 24, 16),
    (256, 384, "gelu", 200, 16),      # many rows per expert: several 32-row passes
    (2048, 256, "gelu", 32, 16),      # wide down projection (32 x 16 workgroups)
    (1024, 2048, "gelu", 100, 32),    # 32 active experts, 64-row passes
])
def test_stream_shapes(d, f, act, S, m_core):
    spec = WORKLOADS["des_vote_b025"].replace(S=S, d=d, f=f, act=act, m_core=m_core)
    _layer_case(spec, flags=moe.MOE_F_FORCE_STREAM)


@pytest.mark.parametrize("E", [20, 48, 100, 200])
def test_router_expert_slices_many_tokens(E):
    """Above 1024 tokens a router workgroup covers 32 tokens and all experts (16-expert tiles x 2,
    4 or 8), or 16 tokens and 256 experts: logits and the layer against the oracle for each slice
    width, with a ragged last token tile (1500 = 46 x 32 + 28)."""
    spec = WORKLOADS["dit_moe_xl"].replace(S=1500, d=256, f=256, E_heavy=E, n_shared=0)
    _layer_case(spec)


@pytest.mark.parametrize("mode", ["tc", "ec"])
def test_single_expert_layer_is_a_dense_mlp(mode):
    """One heavy expert that every token takes (top-1 of 1, or expert choice with C clipped to S):
    the layer is a dense MLP over the tokens in order, the shape of bench.py --dense."""
    base = WORKLOADS["dit_moe_xl"] if mode == "tc" else WORKLOADS["ec_dit"]
    spec = base.replace(S=700, E_heavy=1, n_shared=0, k=1)
    _, rt, _, _ = _layer_case(spec)
    if mode == "ec":
        assert rt["C"] == spec.S


@pytest.mark.parametrize("d", [1088, 1216])
def test_down_projection_column_remainders(d):
    """Model widths whose last 256-wide output tile of the down projection is a quarter used (1088 =
    4 x 256 + 64: that tile runs the 128-wide body, half of it past N) or three quarters used (1216:
    the 256-wide body). 6000 tokens make the 256-wide tiles the planner's choice."""
    spec = WORKLOADS["dit_moe_xl"].replace(S=6000, d=d, f=512)
    _layer_case(spec)


def test_light_experts_only_layer():
    """No heavy experts: identity, zero and constant experts plus a shared expert."""
    spec = WORKLOADS["mmoe"].replace(S=500, d=256, f=512, E_heavy=0, n_layers=1)
    _layer_case(spec)


def test_identity_only_is_exact():
    spec = WORKLOADS["mmoe"].replace(S=333, d=256, f=512, E_heavy=0, n_identity=1, n_zero=0, n_const=0,
                                     n_shared=0, k=1, n_layers=1)
    inp = gen_layer_inputs(spec)
    x = dev_tensor(inp.x, inp.bits["x"], "bf16")
    y, _, _ = run_layer(spec, x, upload_layer(inp))
    assert torch.equal(y, x)


def _stack_case(spec, end_to_end=True):
    """Stacked MoE++ layers with gate residual on a residual stream, each layer in the benchmark's
    launch configuration (one moe_layer_forward with the residual fused into the combine).

    Per layer, both sides start from the same inputs: the oracle's bf16 stream h_l and its logits
    L_{l-1} rounded to fp32 go to the GPU layer, so each layer is checked on its own. Then the GPU
    runs the whole stack on its own outputs and the final stream is compared end to end."""
    say(f"stack {spec.name}: S={spec.S} layers={spec.n_layers}")
    inp = gen_layer_inputs(spec)
    h64 = inp.x.astype(np.float64)
    prev32 = None
    desc = moe.desc_from_spec(spec)
    ws = moe.workspace(desc)
    wts = [upload_layer(inp, layer) for layer in range(spec.n_layers)]
    for layer in range(spec.n_layers):
        h_dev = dev_tensor(h64.astype(np.float32), None, "bf16")
        prev_dev = None if prev32 is None else torch.from_numpy(prev32).cuda()
        rb = moe.alloc_routing(desc)
        y = torch.empty_like(h_dev)
        logits = torch.empty((spec.S, spec.E_routed), dtype=torch.float32, device="cuda")
        moe.moe_layer_forward(desc, h_dev, moe.weights_struct(wts[layer]), prev_dev, logits, rb.struct, None, h_dev,
                              y, ws)
        torch.cuda.synchronize()
        prev64 = None if prev32 is None else prev32.astype(np.float64)
        L64 = orc.router_logits(h64, inp.w_router[layer], prev64)
        assert np.allclose(to_np(logits), L64, atol=2e-5 * max(1.0, np.abs(L64).max()))
        rt = _oracle_rt(spec, L64, rb)
        ref = orc.layer_forward(spec, inp, h64, layer=layer, prev_logits=prev64, residual=h64, rt=rt, h_store="bf16")
        assert_close(to_np(y), ref["y"], "bf16", f"layer {layer}")
        exact = orc.layer_forward(spec, inp, h64, layer=layer, prev_logits=prev64, residual=h64, rt=rt)
        assert_rel_exact(to_np(y), exact["y"], f"layer {layer}")
        h64 = orc.bf16_round(ref["y"])
        prev32 = ref["logits"].astype(np.float32)
        del rb, y, logits, h_dev, prev_dev
    if not end_to_end:
        return
    h_dev = dev_tensor(inp.x, inp.bits["x"], "bf16")
    prev_dev = None
    for layer in range(spec.n_layers):
        y = torch.empty_like(h_dev)
        logits = torch.empty((spec.S, spec.E_routed), dtype=torch.float32, device="cuda")
        moe.moe_layer_forward(desc, h_dev, moe.weights_struct(wts[layer]), prev_dev, logits, None, None, h_dev, y, ws)
        h_dev, prev_dev = y, logits
    torch.cuda.synchronize()
    got = to_np(h_dev)
    rel = np.linalg.norm(got - h64) / np.linalg.norm(h64)
    say(f"  end-to-end stack rel-L2 {rel:.3e} (information; each layer is checked above)")
    # Chained on its own stream, the GPU meets near-tied routing decisions in deeper layers that go
    # the other way; each such token changes by O(|y|). Only a sanity bound is asserted here.
    assert rel <= 5e-2


def test_mmoe_stack_reduced():
    _stack_case(WORKLOADS["mmoe"].replace(S=600))


@pytest.mark.parametrize("name", ["dit_moe_xl", "ec_dit", "des_vote_b025", "des_seq", "mmoe"])
def test_empty_batch_resets_routing(name):
    """S = 0 routes nothing: moe_layer_forward and moe_route set the per-expert counts and offsets,
    n_rows and the capacity to 0, DES votes to 0 and the DES core slots to -1, with null token
    arrays and no workspace."""
    spec = WORKLOADS[name].replace(S=4, n_layers=1)
    say(f"empty batch {name}")
    wt = upload_layer(gen_layer_inputs(spec))
    rb = moe.alloc_routing(moe.desc_from_spec(spec))
    d0 = moe.desc_from_spec(spec.replace(S=0))

    def garbage():
        for t in rb.tensors.values():
            t.fill_(7)

    def check():
        torch.cuda.synchronize()
        g = {k: v.cpu() for k, v in rb.tensors.items()}
        assert int(g["counts"].abs().sum()) == 0 and int(g["offsets"].abs().sum()) == 0
        assert int(g["n_rows"][0]) == 0
        if "capacity" in g:
            assert int(g["capacity"][0]) == 0
        if spec.mode in ("des", "des_seq"):
            assert float(g["votes"].abs().sum()) == 0.0
            ncore = spec.m_core if spec.mode == "des" else spec.E_routed
            assert bool((g["core"][:ncore] == -1).all())
        # arrays of S rows are left alone
        assert bool((g["topk_idx"] == 7).all()) if "topk_idx" in g else True

    garbage()
    assert moe.moe_layer_forward(d0, None, moe.weights_struct(wt), None, None, rb.struct, None, None, None, None,
                                 0) == moe.MOE_OK
    check()
    garbage()
    assert moe.moe_route(d0, None, rb.struct, None, 0) == moe.MOE_OK
    check()


def test_des_with_full_cover_is_token_choice():
    """Degenerate DES cases ("Dynamic Expert Sharing", 2.2-2.4): a DES-Vote core of every expert
    (beta = 1), or a DES-Seq core built from each token's own top-k (k_seq = k), leaves every token its
    plain top-k, so the layer equals token choice bit for bit (same streaming kernels)."""
    base = WORKLOADS["des_vote_b025"]
    tc = base.replace(mode="tc")
    vote_all = base.replace(m_core=base.E_heavy)
    seq_k = WORKLOADS["des_seq"].replace(vote_k=base.k)
    inp = gen_layer_inputs(tc, seed=11)
    x = dev_tensor(inp.x, inp.bits["x"], "bf16")
    wt = upload_layer(inp)
    outs = {}
    for name, spec in (("tc", tc), ("vote_all", vote_all), ("seq_k", seq_k)):
        y, logits, rb = run_layer(spec, x, wt, flags=moe.MOE_F_FORCE_STREAM)
        outs[name] = (y, logits, routing_np(rb, spec))
    y0, l0, g0 = outs["tc"]
    for name in ("vote_all", "seq_k"):
        y1, l1, g1 = outs[name]
        say(f"  {name}: equal to token choice")
        assert torch.equal(l0, l1)
        assert np.array_equal(g0["topk_idx"], g1["topk_idx"]), name
        assert np.array_equal(g0["topk_w"], g1["topk_w"]), name
        assert torch.equal(y0, y1), name


SPLIT_ROUTER_CASES = {
    "des_vote_b025": WORKLOADS["des_vote_b025"],
    "des_seq": WORKLOADS["des_seq"],
    "vanilla_top8": WORKLOADS["vanilla_top8"],
    # gate residual on a small batch: 4 K splits of 9 steps at d = 1152
    "mmoe_s32": WORKLOADS["mmoe"].replace(S=32, n_layers=1),
    "f32_s20": WORKLOADS["dit_moe_tiny_f32"].replace(S=20),
    # one token, and a block of 5: one token tile, every split
    "vanilla_s1": WORKLOADS["vanilla_top8"].replace(S=1),
    "des_s5": WORKLOADS["des_vote_b025"].replace(S=5),
}


@pytest.mark.parametrize("name", list(SPLIT_ROUTER_CASES))
def test_split_router_paths_agree(name):
    """With few token tiles the router splits K over several workgroups per tile. The one-workgroup
    routing adds the partial sums itself; the multi-launch path adds them with a summing kernel.
    Both give the same logits (checked against the oracle, with the previous layer's logits added),
    routing and output, bit for bit."""
    spec = SPLIT_ROUTER_CASES[name]
    say(f"split router {name}: S={spec.S} d={spec.d} E_r={spec.E_routed}")
    inp = gen_layer_inputs(spec, seed=5)
    x = dev_tensor(inp.x, inp.bits.get("x"), spec.dtype)
    wt = upload_layer(inp)
    prev32 = np.random.default_rng(6).standard_normal((spec.S, spec.E_routed)).astype(np.float32)
    outs = {}
    for with_prev in (False, True):
        prev = torch.from_numpy(prev32).cuda() if with_prev else None
        for multi in (False, True):
            flags = moe.MOE_F_ROUTE_MULTI if multi else 0
            y, logits, rb = run_layer(spec, x, wt, flags=flags, prev=prev)
            outs[with_prev, multi] = (y, logits, routing_np(rb, spec))
        L64 = orc.router_logits(inp.x, inp.w_router[0], prev32.astype(np.float64) if with_prev else None)
        assert np.allclose(to_np(outs[with_prev, False][1]), L64, atol=2e-5 * max(1.0, np.abs(L64).max()))
        (y0, l0, r0), (y1, l1, r1) = outs[with_prev, False], outs[with_prev, True]
        assert torch.equal(l0, l1), "logits"
        for key in ("topk_idx", "topk_w", "counts", "offsets", "row_token", "row_w", "token_rows", "n_rows"):
            assert np.array_equal(r0[key], r1[key]), key
        assert torch.equal(y0, y1), "output"
    assert not torch.equal(outs[False, False][1], outs[True, False][1])


FOUR_CALL_CASES = {
    # grouped GEMMs, then the combine kernel
    "dit_moe_xl": (WORKLOADS["dit_moe_xl"].replace(S=513), 0, False, False),
    # weight streaming: moe_layer_forward combines inside the streaming down projection, the
    # four-call path with the combine kernel
    "des_vote_b025": (WORKLOADS["des_vote_b025"], 0, False, False),
    "des_seq_k1": (WORKLOADS["des_seq"].replace(vote_k=1), 0, False, False),
    # shared and zero-computation experts, residual: the shared GEMMs run before the streamed experts
    "mmoe_stream": (WORKLOADS["mmoe"].replace(S=64, d=256, f=512, n_layers=1), moe.MOE_F_FORCE_STREAM, False, True),
    # cached routed parts of low-score tokens (written by the fused combine for fresh tokens)
    "reuse_stream": (WORKLOADS["dit_moe_xl_reuse"].replace(S=96, d=384, f=256, reuse_tau=0.2), moe.MOE_F_FORCE_STREAM,
                     True, True),
}


@pytest.mark.parametrize("name", list(FOUR_CALL_CASES))
def test_four_call_path_matches_layer_forward(name):
    """moe_route + moe_dispatch + moe_expert_ffn + moe_combine == moe_layer_forward (bitwise), also
    where the layer forward fuses the combine into the streaming down projection."""
    spec, flags, with_cache, residual = FOUR_CALL_CASES[name]
    _four_call_case(name, spec, flags, with_cache, residual, seed=4)


def _four_call_case(name, spec, flags, with_cache, residual, seed):
    """Runs the bf16 layer both ways and checks the four-call path against moe_layer_forward."""
    say(f"four-call {name}: S={spec.S} d={spec.d} f={spec.f} flags={flags}")
    inp = gen_layer_inputs(spec, seed=seed)
    x = dev_tensor(inp.x, inp.bits["x"], "bf16")
    wt = upload_layer(inp)
    cache0 = None
    if with_cache:
        rng = np.random.default_rng(9)
        cv, cb = gen_tensor(rng, (spec.S, spec.d), 0.5, spec.dtype)
        cache0 = dev_tensor(cv, cb, spec.dtype)
    res = x if residual else None
    c_a = cache0.clone() if with_cache else None
    y_ref, logits, _ = run_layer(spec, x, wt, flags=flags, cache=c_a, residual=res)
    desc = moe.desc_from_spec(spec, flags)
    rb = moe.alloc_routing(desc)
    ws = moe.workspace(desc)
    moe.moe_route(desc, logits, rb.struct, ws)
    xp = torch.empty((rb.rows, spec.d), dtype=torch.bfloat16, device="cuda")
    moe.moe_dispatch(desc, x, rb.struct, xp)
    yp = torch.empty((rb.rows, spec.d), dtype=torch.float32, device="cuda")
    ys = torch.empty((spec.S, spec.d), dtype=torch.float32, device="cuda")
    w = moe.weights_struct(wt)
    moe.moe_expert_ffn(desc, x, xp, rb.struct, w, yp, ys, ws)
    y = torch.empty_like(x)
    c_b = cache0.clone() if with_cache else None
    moe.moe_combine(desc, x, rb.struct, yp, ys, wt.get("const_vec"), c_b, res, y)
    torch.cuda.synchronize()
    n = int(rb["n_rows"][0])
    tok = rb["row_token"][:n].long()
    assert torch.equal(xp[:n], x[tok])
    assert torch.equal(y, y_ref)
    if with_cache:
        reused = rb["reuse"].bool()
        assert 0 < int(reused.sum()) < spec.S
        assert torch.equal(c_a, c_b)
        assert torch.equal(c_a[reused], cache0[reused])


# ------------------------------------------------------------------------------------------------
# Full sizes, every token, in the launch configuration the benchmark uses.

@pytest.mark.timeout(600)
def test_dit_moe_xl_full_size():
    spec = WORKLOADS["dit_moe_xl"]
    _, rt, y1, rb = _layer_case(spec)
    g = routing_np(rb, spec)
    assert g["n_rows"][0] == g["counts"].sum() == g["offsets"][-1] == spec.S * spec.k
    # determinism: a second call is bit-identical
    inp = gen_layer_inputs(spec)
    y2, _, _ = run_layer(spec, dev_tensor(inp.x, inp.bits["x"], "bf16"), upload_layer(inp))
    assert torch.equal(y1, y2)


@pytest.mark.timeout(600)
def test_dit_moe_xl_reuse_full_size():
    spec = WORKLOADS["dit_moe_xl_reuse"]
    _, rt, _, rb = _layer_case(spec, with_cache=True)
    n_reuse = int(rt["reuse"].sum())
    say(f"  reused tokens: {n_reuse} of {spec.S}")
    assert 0 < n_reuse < spec.S
    assert int(rb["n_rows"][0]) == spec.k * (spec.S - n_reuse)


@pytest.mark.timeout(600)
def test_ec_dit_full_size():
    spec = WORKLOADS["ec_dit"]
    _, rt, _, rb = _layer_case(spec)
    assert rt["C"] == 512 and int(rb["n_rows"][0]) == 32 * 512 and int(rb["capacity"][0]) == 512
    assert np.array_equal(rb["counts"].cpu().numpy(), np.full(32, 512))


@pytest.mark.timeout(900)
def test_mmoe_stack_full_size():
    """All four MoE++ layers at 64 x 256 = 16384 tokens: routers above 1024 tokens take the 32-token
    workgroups with the previous layer's logits added, and the GEMMs the benchmark's tile widths."""
    _stack_case(WORKLOADS["mmoe"], end_to_end=False)
