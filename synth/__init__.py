"""Seeded synthetic inputs for the sparse MoE FFN layer (shared by tests, bench and smoke).

This module only draws random numbers and rounds them to the storage precision. It holds
none of the layer's arithmetic: no logits, softmax, routing, capacity, expert MLP or combine.
Both the fp64 oracle and the GPU library consume what it returns.

Recipe (the pages' datasets and trained weights are not available, so seeded tensors of the
pages' shapes stand in for them):
  * x ~ N(0, 1); every weight (router, experts, shared experts, constant-expert vectors) ~ N(0, 0.02).
  * One ``numpy.random.default_rng(seed)`` (PCG64) stream, drawn in a fixed order:
    x, then per layer: router weight, per heavy expert (W_up, W_gate [SwiGLU only], W_down),
    per shared expert (same), constant-expert vectors.
  * fp32 draws, rounded to bf16 round-to-nearest-even for bf16 workloads.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

__all__ = ["LayerSpec", "WORKLOADS", "bf16_rne", "LayerInputs", "gen_layer_inputs", "gen_tensor"]


@dataclass(frozen=True)
class LayerSpec:
    """Shape and hyper-parameters of one MoE FFN layer call (no arithmetic here)."""

    name: str
    S: int                      # tokens in the call (batch x sequence)
    d: int                      # model dim
    f: int                      # expert hidden dim
    E_heavy: int                # heavy (MLP) routed experts
    n_identity: int = 0         # zero-computation experts: identity ...
    n_zero: int = 0             # ... zero ...
    n_const: int = 0            # ... and learned-constant
    n_shared: int = 0           # always-on experts, weight 1
    act: str = "gelu"           # "gelu" (erf) | "gelu_tanh" | "swiglu"
    mode: str = "tc"            # "tc" token choice | "ec" expert choice | "des" DES-Vote | "des_seq" DES-Seq
    k: int = 2                  # token-choice / DES re-route top-k
    renorm: bool = True         # renormalise the selected weights
    capacity_factor: float = 2.0
    vote_k: int = 0             # DES-Vote filter K; DES-Seq local selection count k_seq
    m_core: int = 0             # DES core-set size
    reuse_tau: float = 0.0      # DICE-style low-score reuse threshold (0 = off)
    dtype: str = "bf16"         # "bf16" | "f32"
    n_layers: int = 1           # stacked layers (gate residual + residual stream)

    @property
    def E_routed(self) -> int:
        return self.E_heavy + self.n_identity + self.n_zero + self.n_const

    def replace(self, **kw) -> "LayerSpec":
        return dataclasses.replace(self, **kw)


# The five workloads, at full size.
WORKLOADS: dict[str, LayerSpec] = {
    # 1 image x 256 tokens, d=384, 8 GELU experts 384->1536->384, top-2 renormalised, fp32.
    "dit_moe_tiny_f32": LayerSpec("dit_moe_tiny_f32", S=256, d=384, f=1536, E_heavy=8, act="gelu",
                                  mode="tc", k=2, renorm=True, dtype="f32"),
    # 32 x 256 tokens, d=1152, 8 SwiGLU experts 1152->4608->1152 + 2 shared, top-2.
    "dit_moe_xl": LayerSpec("dit_moe_xl", S=8192, d=1152, f=4608, E_heavy=8, n_shared=2, act="swiglu",
                            mode="tc", k=2, renorm=True),
    # Same layer, tokens whose top softmax score < 0.3 reuse the cached routed output.
    "dit_moe_xl_reuse": LayerSpec("dit_moe_xl_reuse", S=8192, d=1152, f=4608, E_heavy=8, n_shared=2,
                                  act="swiglu", mode="tc", k=2, renorm=True, reuse_tau=0.3),
    # 64 x 128 tokens, d=1536, 32 GELU experts 1536->6144->1536, expert choice with f_c = 2.
    "ec_dit": LayerSpec("ec_dit", S=8192, d=1536, f=6144, E_heavy=32, act="gelu", mode="ec",
                        capacity_factor=2.0),
    # DES-Vote decode block: N=32 tokens, d=2048, 64 SwiGLU experts 2048->1024->2048, top-8,
    # vote filter K=8, core = beta*64 experts.
    "des_vote_b025": LayerSpec("des_vote_b025", S=32, d=2048, f=1024, E_heavy=64, act="swiglu",
                               mode="des", k=8, renorm=True, vote_k=8, m_core=16),
    "des_vote_b050": LayerSpec("des_vote_b050", S=32, d=2048, f=1024, E_heavy=64, act="swiglu",
                               mode="des", k=8, renorm=True, vote_k=8, m_core=32),
    # DES-Seq on the same block: the core is the union of every token's top-2 (local selection
    # count k_seq = 2); tokens then re-route top-8 inside it.
    "des_seq": LayerSpec("des_seq", S=32, d=2048, f=1024, E_heavy=64, act="swiglu", mode="des_seq", k=8,
                         renorm=True, vote_k=2),
    # The vanilla block the DES variants are measured against: every token its own top-8; the
    # experts loaded are their union.
    "vanilla_top8": LayerSpec("vanilla_top8", S=32, d=2048, f=1024, E_heavy=64, act="swiglu", mode="tc", k=8,
                              renorm=True),
    # MMOE MoE++: 64 x 256 tokens, d=1152, 16 heavy GELU experts + identity/zero/constant + 1 shared,
    # top-2 over 19 with gate residual, 4 stacked layers.
    "mmoe": LayerSpec("mmoe", S=16384, d=1152, f=4608, E_heavy=16, n_identity=1, n_zero=1, n_const=1,
                      n_shared=1, act="gelu", mode="tc", k=2, renorm=True, n_layers=4),
}


def bf16_rne(a: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns (bits as uint16, the rounded values as float32). Inputs here are finite.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    bits = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    vals = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return bits, vals


def gen_tensor(rng: np.random.Generator, shape, std: float, dtype: str):
    """One N(0, std^2) tensor in the storage precision: (values float32, bf16 bits or None)."""
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if dtype == "bf16":
        bits, vals = bf16_rne(a)
        return vals, bits
    return a, None


def gen_coupled_tokens(rng: np.random.Generator, n: int, d: int, rho: float):
    """A decode block of n bf16 tokens that share part of their content: x_i = sqrt(rho) * z +
    sqrt(1 - rho) * e_i, with z and every e_i drawn N(0, I_d), so each token is N(0, I_d) and any two
    correlate by rho (a stand-in for the semantically coupled tokens of one parallel-decoding
    block). rho = 0 gives independent tokens. Returns (values float32, bf16 bits)."""
    z = rng.standard_normal(size=(1, d), dtype=np.float32)
    e = rng.standard_normal(size=(n, d), dtype=np.float32)
    a = np.float32(np.sqrt(rho)) * z + np.float32(np.sqrt(1.0 - rho)) * e
    bits, vals = bf16_rne(a)
    return vals, bits


@dataclass
class LayerInputs:
    """Values are float32 arrays holding exactly the stored (bf16 or fp32) numbers.

    ``bits[name]`` holds the bf16 encodings for bf16 workloads (None for fp32).
    Per-layer weights are lists indexed by layer.
    """

    spec: LayerSpec
    x: np.ndarray
    w_router: list
    w1: list        # [E_h, f, d]  up projection (SwiGLU: the linear "up" branch)
    w3: list        # [E_h, f, d]  SwiGLU gate branch, or None
    w2: list        # [E_h, d, f]  down projection
    s_w1: list
    s_w3: list
    s_w2: list
    const_vec: list  # [n_const, d] or None
    bits: dict


def gen_layer_inputs(spec: LayerSpec, seed: int = 0, std: float = 0.02) -> LayerInputs:
    rng = np.random.default_rng(seed)
    dt = spec.dtype
    bits: dict = {}

    def draw(name, shape, s):
        v, b = gen_tensor(rng, shape, s, dt)
        bits[name] = b
        return v

    x = draw("x", (spec.S, spec.d), 1.0)
    wr, w1, w3, w2, sw1, sw3, sw2, cv = [], [], [], [], [], [], [], []
    swiglu = spec.act == "swiglu"
    for layer in range(spec.n_layers):
        wr.append(draw(f"w_router.{layer}", (spec.E_routed, spec.d), std))
        up, gate, down = [], [], []
        for _ in range(spec.E_heavy):
            up.append(draw(None, (spec.f, spec.d), std))
            if swiglu:
                gate.append(draw(None, (spec.f, spec.d), std))
            down.append(draw(None, (spec.d, spec.f), std))
        bits.pop(None, None)
        w1.append(_stack(up, (0, spec.f, spec.d)))
        w3.append(_stack(gate, (0, spec.f, spec.d)) if swiglu else None)
        w2.append(_stack(down, (0, spec.d, spec.f)))
        sup, sgate, sdown = [], [], []
        for _ in range(spec.n_shared):
            sup.append(draw(None, (spec.f, spec.d), std))
            if swiglu:
                sgate.append(draw(None, (spec.f, spec.d), std))
            sdown.append(draw(None, (spec.d, spec.f), std))
        bits.pop(None, None)
        sw1.append(_stack(sup, (0, spec.f, spec.d)) if spec.n_shared else None)
        sw3.append(_stack(sgate, (0, spec.f, spec.d)) if (spec.n_shared and swiglu) else None)
        sw2.append(_stack(sdown, (0, spec.d, spec.f)) if spec.n_shared else None)
        cv.append(draw(f"const_vec.{layer}", (spec.n_const, spec.d), std) if spec.n_const else None)
    inp = LayerInputs(spec, x, wr, w1, w3, w2, sw1, sw3, sw2, cv, bits)
    if dt == "bf16":
        # Encodings of the stacked expert tensors (exact: values are already bf16 numbers).
        for name in ("w1", "w3", "w2", "s_w1", "s_w3", "s_w2"):
            for layer, v in enumerate(getattr(inp, name)):
                bits[f"{name}.{layer}"] = None if v is None else _exact_bits(v)
    return inp


def _stack(lst, empty_shape):
    if not lst:
        return np.zeros(empty_shape, dtype=np.float32)
    return np.stack(lst)


def _exact_bits(v: np.ndarray) -> np.ndarray:
    """bf16 encodings of float32 values that are already bf16 numbers (low half is zero)."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)
