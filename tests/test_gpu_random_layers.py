"""GPU parity of the layer on a seeded sweep of shapes no workload has: model and hidden widths that
leave ragged and half-used tiles, few or many experts, every routing mode and activation, light
and shared experts, cache reuse and the residual add, small and mid-sized token counts (the
one-workgroup and the multi-launch routing, the streaming and the tiled expert kernels)."""
import numpy as np
import pytest

import oracle as orc
from synth import LayerSpec, gen_layer_inputs
from test_gpu_layer import _four_call_case, _layer_case

pytestmark = pytest.mark.gpu


def _configs(n=64, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        mode = ["tc", "tc", "tc", "ec", "des", "des_seq"][rng.integers(6)]
        dtype = "f32" if rng.random() < 0.2 else "bf16"
        # widths that are multiples of 128 (bf16) or 64 (f32) also allow the weight-streaming kernel
        d = int(rng.choice([64, 128, 256, 320, 576, 1024, 1088] if dtype == "bf16" else [64, 192, 320]))
        f = int(rng.choice([64, 128, 192, 256, 448, 640, 960, 1024] if dtype == "bf16" else [128, 320]))
        act = ["gelu", "gelu_tanh", "swiglu"][rng.integers(3)]
        E = int(rng.integers(1, 41))
        light = mode == "tc" and rng.random() < 0.4
        n_id, n_zero, n_const = (int(rng.integers(0, 2)), int(rng.integers(0, 2)), int(rng.integers(0, 2))) if light \
            else (0, 0, 0)
        E_r = E + n_id + n_zero + n_const
        n_shared = int(rng.integers(0, 3))
        S = int(rng.choice([int(rng.integers(1, 70)), int(rng.integers(70, 2600))]))
        k = int(rng.integers(1, min(E_r, 8) + 1))
        kw = dict(name=f"rand{len(out)}", S=S, d=d, f=f, E_heavy=E, n_identity=n_id, n_zero=n_zero,
                  n_const=n_const, n_shared=n_shared, act=act, mode=mode, k=k, renorm=bool(rng.random() < 0.7),
                  dtype=dtype)
        if mode == "ec":
            fc = float(rng.choice([1.0, 2.0, 4.0]))
            if int(np.floor(np.float32(fc) * S / E_r)) < 1:
                continue
            kw.update(capacity_factor=fc, k=2)
        elif mode == "des":
            kw.update(vote_k=int(rng.integers(1, k + 1)), m_core=int(rng.integers(1, E_r + 1)))
        elif mode == "des_seq":
            kw.update(vote_k=int(rng.integers(1, min(3, E_r) + 1)))
        elif rng.random() < 0.3:
            kw.update(reuse_tau=0.3)
        out.append((LayerSpec(**kw), bool(rng.random() < 0.5)))
    return out


CONFIGS = _configs()


def _median_tau(spec, seed):
    """With cache reuse: a threshold between two middle values of the tokens' top probability, so
    that about half of the tokens reuse the cache (with near-uniform routing a fixed 0.3 would take
    them all)."""
    if spec.reuse_tau <= 0:
        return spec
    inp = gen_layer_inputs(spec, seed=seed)
    pmax = np.sort(orc.softmax(orc.router_logits(inp.x, inp.w_router[0])).max(axis=1))
    m = len(pmax) // 2
    tau = 0.5 * (pmax[m] + pmax[min(m + 1, len(pmax) - 1)]) if len(pmax) > 1 else pmax[0] * 1.5
    return spec.replace(reuse_tau=float(tau))


@pytest.mark.parametrize("spec,residual", CONFIGS, ids=[c[0].name for c in CONFIGS])
def test_random_layer(spec, residual):
    seed = int(spec.name[4:]) + 11
    spec = _median_tau(spec, seed)
    _layer_case(spec, seed=seed, with_cache=spec.reuse_tau > 0, residual=residual)


def _flag_cases():
    """The first configurations again, each with one flag that picks the other kernel path: the
    tiled grouped GEMM or the weight-streaming kernel for the heavy experts, or the multi-launch
    routing instead of the one-workgroup kernel. Combinations the library rejects are left out."""
    import mixture_experts_layer_gemm_amd as moe
    out = []
    for i, (spec, residual) in enumerate(CONFIGS[:36]):
        flag = [moe.MOE_F_FORCE_TILED, moe.MOE_F_FORCE_STREAM, moe.MOE_F_ROUTE_MULTI][i % 3]
        if flag == moe.MOE_F_ROUTE_MULTI and spec.mode == "ec":
            continue
        if flag != moe.MOE_F_ROUTE_MULTI and spec.E_heavy == 0:
            continue
        if moe.lib().moe_workspace_bytes(moe.desc_from_spec(spec, flag)) == 0:
            continue
        out.append((spec, residual, flag))
    return out


FLAG_CASES = _flag_cases()


@pytest.mark.parametrize("spec,residual,flag", FLAG_CASES, ids=[f"{c[0].name}-f{c[2]:#x}" for c in FLAG_CASES])
def test_random_layer_forced_path(spec, residual, flag):
    seed = int(spec.name[4:]) + 11
    spec = _median_tau(spec, seed)
    _layer_case(spec, seed=seed, flags=flag, with_cache=spec.reuse_tau > 0, residual=residual)


FOUR_CALL_RANDOM = [c for c in CONFIGS if c[0].dtype == "bf16"][:24]


@pytest.mark.parametrize("spec,residual", FOUR_CALL_RANDOM, ids=[c[0].name for c in FOUR_CALL_RANDOM])
def test_random_four_call_path(spec, residual):
    """moe_route + moe_dispatch + moe_expert_ffn + moe_combine equal moe_layer_forward bit for bit on
    the sweep's bf16 shapes."""
    seed = int(spec.name[4:]) + 11
    spec = _median_tau(spec, seed)
    _four_call_case(spec.name, spec, 0, spec.reuse_tau > 0, residual, seed=seed)
