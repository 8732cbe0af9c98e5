"""GPU parity of the attention-residual aggregation (moe_attnres_aggregate) against the fp64 oracle.

Tolerance, per element: the kernel rounds its fp32 result once to the output dtype (at most half a
unit in the last place, 2^-9 relative for bf16, 2^-24 for fp32). Its fp32 scores z carry a
relative error of a few 1e-7 (two length-d sums and a square root), and an error dz in the scores
moves the weights by at most 2 |dz| alpha_j, so the output by at most 2 max|dz| times the token's
largest input magnitude: about 4e-6 of it for scores up to 6. The test allows one full unit in the
last place plus 2e-5 (bf16) / 1e-5 (fp32) of that magnitude, and, for saturated softmaxes with
scores in the hundreds, 5e-3 of it.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_gemm_amd as moe
import oracle as orc
from _gpu_helpers import say
from synth import gen_tensor

pytestmark = pytest.mark.gpu


def _make(seed, n, S, d, dtype):
    """n states of [S, d] with per-state scales (so the RMS normalisation matters) and a query whose
    scores spread over a few units."""
    rng = np.random.default_rng(seed)
    vals, bits = [], []
    for j in range(n):
        v, b = gen_tensor(rng, (S, d), float(0.25 + 2.0 * rng.random()), dtype)
        vals.append(np.asarray(v, np.float64))
        bits.append(b)
    qv, qb = gen_tensor(rng, (d,), 1.5 / np.sqrt(d), dtype)
    return vals, bits, np.asarray(qv, np.float64), qb


def _dev(vals, bits, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(vals, np.float32)).cuda()


def _run(vals, bits, qv, qb, dtype, eps=1e-6):
    S, d = vals[0].shape
    states = [_dev(v, b, dtype) for v, b in zip(vals, bits)]
    q = _dev(qv, qb, dtype)
    out = torch.empty((S, d), dtype=states[0].dtype, device="cuda")
    moe.moe_attnres_aggregate(moe.MOE_BF16 if dtype == "bf16" else moe.MOE_F32, S, d, states, q, eps, out)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def _check(got, ref, vals, dtype, rel_amax=None):
    ulp = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -23
    amax = np.max(np.abs(np.stack(vals)), axis=(0, 2))[:, None]   # per token
    if rel_amax is None:
        rel_amax = 2e-5 if dtype == "bf16" else 1e-5
    tol = ulp * np.abs(ref) + rel_amax * amax
    err = np.abs(got - ref)
    assert np.all(err <= tol), f"max err {err.max():.3e}, worst ratio {(err / tol).max():.3f}"


@pytest.mark.parametrize("S,d,n,dtype", [
    (1000, 1152, 5, "bf16"),     # MMOE width: 2.25 chunks per lane (3 in registers, ragged)
    (777, 2048, 3, "bf16"),      # 4 chunks per lane
    (513, 4096, 12, "bf16"),     # widest bf16 row, 8 chunks per lane
    (333, 64, 1, "bf16"),        # one state: the output is that state
    (5, 8, 64, "bf16"),          # the most states, one 16-byte chunk per row
    (129, 384, 7, "f32"),
    (64, 4096, 2, "f32"),        # widest fp32 row, 16 chunks per lane
    (3, 1536, 17, "f32"),
])
def test_attnres_matches_oracle(S, d, n, dtype):
    say(f"attnres S={S} d={d} n={n} {dtype}")
    vals, bits, qv, qb = _make(S * 7 + d + n, n, S, d, dtype)
    ref, _ = orc.attnres_aggregate(np.stack(vals), qv)
    got = _run(vals, bits, qv, qb, dtype)
    _check(got, ref, vals, dtype)
    if n == 1:
        assert np.array_equal(got, vals[0])


def test_attnres_zero_query_is_the_mean_and_s0_is_a_noop():
    vals, bits, qv, qb = _make(11, 4, 200, 1152, "bf16")
    zq = np.zeros_like(qv)
    got = _run(vals, bits, zq, np.zeros_like(qb), "bf16")
    _check(got, np.mean(np.stack(vals), axis=0), vals, "bf16")
    out = torch.full((4, 64), 3.0, dtype=torch.bfloat16, device="cuda")
    st = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    moe.moe_attnres_aggregate(moe.MOE_BF16, 0, 64, [st], q, 1e-6, out)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)


def test_attnres_large_scores_stay_finite():
    """Scores of a few hundred (a large query) must not overflow the running softmax."""
    vals, bits, qv, qb = _make(5, 6, 64, 512, "f32")
    q_big = qv * 400.0
    ref, alpha = orc.attnres_aggregate(np.stack(vals), q_big)
    assert alpha.max() > 0.99   # the softmax is saturated
    got = _run(vals, bits, q_big, None, "f32")
    assert np.all(np.isfinite(got))
    _check(got, ref, vals, "f32", rel_amax=5e-3)


def test_attnres_bench_shape_sampled():
    """The shape bench.py --attnres times (16384 tokens, d = 1152, 17 states, bf16), checked on 512
    sampled tokens: each token's output depends only on that token's rows."""
    S, d, n = 16384, 1152, 17
    say(f"attnres full size S={S} d={d} n={n}")
    vals, bits, qv, qb = _make(123, n, S, d, "bf16")
    got = _run(vals, bits, qv, qb, "bf16")
    rows = np.sort(np.random.default_rng(7).choice(S, 512, replace=False))
    sub = [v[rows] for v in vals]
    ref, _ = orc.attnres_aggregate(np.stack(sub), qv)
    _check(got[rows], ref, sub, "bf16")
