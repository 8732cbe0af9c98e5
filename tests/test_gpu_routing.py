"""GPU parity of the routing entry point (moe_route) against the oracle: bit-exact indices, core sets,
permutations and counts when both sides decide on the same fp32 keys."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_gemm_amd as moe
import oracle as orc
from _gpu_helpers import reconcile_des, reconcile_des_seq, reconcile_ec, routing_np, say
from synth import LayerSpec

pytestmark = pytest.mark.gpu


def _spec(**kw):
    base = dict(name="route", S=64, d=256, f=256, E_heavy=8, act="gelu", mode="tc", k=2, renorm=True, dtype="bf16")
    base.update(kw)
    return LayerSpec(**base)


def _route(spec, keys32, input_probs=False, multi=False):
    flags = (moe.MOE_F_INPUT_PROBS if input_probs else 0) | (moe.MOE_F_ROUTE_MULTI if multi else 0)
    desc = moe.desc_from_spec(spec, flags)
    rb = moe.alloc_routing(desc)
    ws = moe.workspace(desc)
    keys = torch.from_numpy(np.ascontiguousarray(keys32, np.float32)).cuda()
    moe.moe_route(desc, keys, rb.struct, ws)
    torch.cuda.synchronize()
    return routing_np(rb, spec), rb


def _logits(rng, S, E, scale=0.7, tie_rows=0.2):
    L = (rng.standard_normal((S, E)) * scale).astype(np.float32)
    ties = rng.random(S) < tie_rows
    L[ties] = rng.integers(-1, 2, size=(int(ties.sum()), E)).astype(np.float32)   # exact ties
    # half of those zeros negative: -0 and +0 are equal keys, the lower expert first
    L[(L == 0) & (rng.random((S, E)) < 0.5)] = np.float32(-0.0)
    return L


def _check_permutation(spec, got, idx, reuse=None):
    E_r = spec.E_routed
    valid = (idx >= 0) & (idx < spec.E_heavy)       # -1: an empty DES-Seq slot
    if reuse is not None:
        valid &= ~reuse[:, None]
    counts, offsets, row_token, row_slot, token_rows = orc.counting_sort(idx, E_r, valid)
    R = int(offsets[-1])
    assert got["n_rows"][0] == R
    assert np.array_equal(got["counts"], counts)
    assert np.array_equal(got["offsets"], offsets)
    assert np.array_equal(got["row_token"][:R], row_token)
    assert np.array_equal(got["token_rows"], token_rows)
    # row weights are the slot weights, moved
    assert np.array_equal(got["row_w"][:R], got["topk_w"][row_token, row_slot])


TC_CASES = [
    # S, E_heavy, n_id, n_zero, n_const, k
    (1000, 8, 0, 0, 0, 2),
    # the library's limits: 256 routed experts, k = 16 (one-workgroup kernel at S * E_r = 8192)
    (32, 256, 0, 0, 0, 16),
    (300, 256, 0, 0, 0, 16),
    (777, 16, 1, 1, 1, 2),
    (333, 64, 0, 0, 0, 8),
    (129, 200, 0, 0, 0, 16),
    (1, 8, 0, 0, 0, 2),
    (64, 5, 0, 0, 0, 5),
    (300, 1, 0, 0, 0, 1),
    (5000, 0, 1, 1, 1, 2),
    # one-workgroup kernel with a wave per token: 1, 2 and 4 experts per lane
    (100, 64, 0, 0, 0, 8),
    (60, 100, 0, 0, 0, 6),
    (40, 200, 0, 0, 0, 16),
]


# multi=False lets small calls take the one-workgroup kernel; multi=True forces the multi-launch path
@pytest.mark.parametrize("multi", [False, True])
@pytest.mark.parametrize("case", TC_CASES)
def test_tc_route_bitexact_on_logits(case, multi):
    S, Eh, ni, nz, nc, k = case
    spec = _spec(S=S, E_heavy=Eh, n_identity=ni, n_zero=nz, n_const=nc, k=k)
    say(f"tc route logits S={S} E_r={spec.E_routed} k={k} multi={multi}")
    rng = np.random.default_rng(S + Eh)
    L = _logits(rng, S, spec.E_routed)
    got, _ = _route(spec, L, multi=multi)
    L64 = L.astype(np.float64)
    idx = orc.tc_select(L64, k)
    assert np.array_equal(got["topk_idx"], idx)
    P = orc.softmax(L64)
    assert np.allclose(got["probs"], P, rtol=0, atol=2e-7)
    assert np.allclose(got["topk_w"], orc.tc_weights(P, idx, True), rtol=2e-6, atol=1e-7)
    _check_permutation(spec, got, idx)


@pytest.mark.parametrize("renorm,S", [(True, 3000), (False, 3000), (True, 1500)])
def test_tc_route_bitexact_on_probs_with_reuse(renorm, S):
    E = 8
    spec = _spec(S=S, E_heavy=E, k=2, renorm=renorm, reuse_tau=0.3)
    rng = np.random.default_rng(7)
    L = _logits(rng, S, E, scale=1.2, tie_rows=0.1).astype(np.float64)
    P32 = orc.softmax(L).astype(np.float32)
    say(f"tc route probs renorm={renorm} S={S}")
    got, _ = _route(spec, P32, input_probs=True)
    P = P32.astype(np.float64)
    idx = orc.tc_select(P, 2)
    assert np.array_equal(got["topk_idx"], idx)
    w = orc.tc_weights(P, idx, renorm)
    assert np.allclose(got["topk_w"], w, rtol=2e-7, atol=0)
    reuse = P32.max(axis=1) < np.float32(0.3)
    assert 0 < reuse.sum() < S
    assert np.array_equal(got["reuse"].astype(bool), reuse)
    _check_permutation(spec, got, idx, reuse)


EC_CASES = [
    # S, E, f_c
    (8192, 32, 2.0),
    (1024, 256, 2.0),   # 256 experts (the limit), C = 8
    (1000, 7, 1.3),
    (50, 4, 8.0),
    (2049, 64, 1.0),
]


@pytest.mark.parametrize("case", EC_CASES)
def test_ec_route_bitexact_on_probs(case):
    S, E, fc = case
    spec = _spec(S=S, E_heavy=E, mode="ec", capacity_factor=fc)
    rng = np.random.default_rng(S + E)
    L = _logits(rng, S, E, scale=0.8, tie_rows=0.3).astype(np.float64)
    P32 = orc.softmax(L).astype(np.float32)
    say(f"ec route S={S} E={E} f_c={fc}")
    got, _ = _route(spec, P32, input_probs=True)
    C = orc.ec_capacity(S, E, np.float32(fc).item())
    tokens, gates = orc.ec_select(P32.astype(np.float64), C)
    assert got["capacity"][0] == C and got["n_rows"][0] == E * C
    assert np.array_equal(got["counts"], np.full(E, C))
    assert np.array_equal(got["offsets"], np.arange(E + 1) * C)
    assert np.array_equal(got["row_token"][: E * C].reshape(E, C), tokens)
    assert np.array_equal(got["row_w"][: E * C].reshape(E, C), gates.astype(np.float32))
    off, lst = orc.ec_token_csr(tokens, S)
    assert np.array_equal(got["token_off"], off)
    assert np.array_equal(got["token_list"][: E * C], lst)


def _structured_ec_keys(rng, S):
    """Columns of fp32 probabilities whose bit patterns differ in few or many bits: every key equal;
    differing in the lowest 4 bits; in the lowest 12; softmax-like; two values with many ties; and
    keys spread over 20 binades."""
    base = np.float32(0.125).view(np.uint32)
    cols = [
        np.full(S, base, np.uint32),
        base + rng.integers(0, 16, S).astype(np.uint32),
        base + rng.integers(0, 4096, S).astype(np.uint32),
        np.abs(rng.standard_normal(S) * 0.02 + 0.1).astype(np.float32).view(np.uint32),
        np.where(rng.random(S) < 0.5, np.float32(0.25), np.float32(0.5)).astype(np.float32).view(np.uint32),
        (np.float32(2.0) ** rng.uniform(-20, 0, S)).astype(np.float32).view(np.uint32),
    ]
    return np.stack(cols, axis=1).view(np.float32)


@pytest.mark.parametrize("S", [3000, 20000])
def test_ec_route_bitexact_structured_keys(S):
    """Expert choice on keys whose common leading bits differ from column to column, so the radix
    select starts at different digits (every key equal: no digit at all; a single digit that
    overlaps no fixed bit, or several); 20000 tokens take the path that reads the keys from memory
    on every pass."""
    E = 6
    spec = _spec(S=S, E_heavy=E, mode="ec", capacity_factor=1.0)
    P32 = _structured_ec_keys(np.random.default_rng(S), S)
    say(f"ec route structured keys S={S} E={E}")
    got, _ = _route(spec, P32, input_probs=True)
    C = orc.ec_capacity(S, E, 1.0)
    tokens, gates = orc.ec_select(P32.astype(np.float64), C)
    assert np.array_equal(got["row_token"][: E * C].reshape(E, C), tokens)
    assert np.array_equal(got["row_w"][: E * C].reshape(E, C), gates.astype(np.float32))
    assert np.array_equal(tokens[0], np.arange(C))   # all keys equal: the lowest tokens
    off, lst = orc.ec_token_csr(tokens, S)
    assert np.array_equal(got["token_off"], off)
    assert np.array_equal(got["token_list"][: E * C], lst)


def test_ec_route_on_logits_full_size():
    S, E = 8192, 32
    spec = _spec(S=S, E_heavy=E, mode="ec", capacity_factor=2.0)
    rng = np.random.default_rng(3)
    L = (rng.standard_normal((S, E)) * 0.78).astype(np.float32)
    got, _ = _route(spec, L)
    rt = orc.route(spec, L=L.astype(np.float64))
    assert np.allclose(got["probs"], rt["P"], atol=2e-7)
    rt2 = reconcile_ec(spec, rt, got["row_token"], rt["C"])
    assert np.array_equal(got["row_token"][: E * rt["C"]].reshape(E, -1), rt2["tokens"])


DES_CASES = [
    # N, E, K, M, k
    (32, 64, 8, 16, 8),
    (32, 256, 16, 64, 16),   # the limits: 256 experts, k = 16
    (32, 64, 8, 32, 8),
    (6, 10, 3, 4, 2),
    (100, 19, 4, 3, 8),
    (257, 128, 16, 40, 16),
    # one-workgroup kernel with 2 and 4 experts per lane
    (60, 100, 6, 20, 6),
    (50, 150, 8, 40, 8),
]


@pytest.mark.parametrize("multi", [False, True])
@pytest.mark.parametrize("case", DES_CASES)
def test_des_route_bitexact_on_probs(case, multi):
    N, E, K, M, k = case
    spec = _spec(S=N, E_heavy=E, mode="des", k=k, vote_k=K, m_core=M)
    rng = np.random.default_rng(N * E)
    L = _logits(rng, N, E, scale=0.9, tie_rows=0.2).astype(np.float64)
    P32 = orc.softmax(L).astype(np.float32)
    say(f"des route N={N} E={E} K={K} M={M} k={k} multi={multi}")
    got, _ = _route(spec, P32, input_probs=True, multi=multi)
    P = P32.astype(np.float64)
    votes, core = orc.des_vote(P, P, K, M, vote_dtype=np.float32)
    assert np.array_equal(got["votes"], votes)
    assert np.array_equal(got["core"][:M], core)
    idx, w = orc.core_reroute(P, P, core, k, True)
    assert np.array_equal(got["topk_idx"], idx)
    # fp32 sum of k weights: relative error below k * 2^-23
    assert np.allclose(got["topk_w"], w, rtol=k * 1.2e-7, atol=0)
    _check_permutation(spec, got, idx)
    assert np.unique(got["row_token"][: got["n_rows"][0]]).size <= N
    assert np.count_nonzero(got["counts"]) <= M


def test_des_route_dyadic_matches_bruteforce_core():
    N, E, K, M = 5, 9, 3, 4
    spec = _spec(S=N, E_heavy=E, mode="des", k=2, vote_k=K, m_core=M)
    rng = np.random.default_rng(11)
    raw = rng.integers(1, 40, size=(N, E)).astype(np.float64)
    P32 = (raw / 1024.0).astype(np.float32)          # dyadic: fp32 sums exact
    got, _ = _route(spec, P32, input_probs=True)
    votes, core = orc.des_vote(P32, P32, K, M)
    assert np.array_equal(got["votes"].astype(np.float64), votes)
    assert np.array_equal(got["core"][:M], core)


def test_des_route_on_logits_full_size():
    spec = _spec(S=32, E_heavy=64, mode="des", k=8, vote_k=8, m_core=16)
    rng = np.random.default_rng(5)
    L = (rng.standard_normal((32, 64)) * 0.91).astype(np.float32)
    got, _ = _route(spec, L)
    L64 = L.astype(np.float64)
    rt = orc.route(spec, L=L64)
    rt = reconcile_des(spec, rt, got["core"][: spec.m_core], L64)
    assert np.allclose(got["votes"], rt["votes"], atol=1e-6)
    assert np.array_equal(got["topk_idx"], rt["idx"])


DES_SEQ_CASES = [
    # N, E, k_seq, k
    (32, 64, 1, 8),
    (32, 256, 4, 16),   # the limits: 256 experts, k = 16
    (32, 64, 2, 8),
    (32, 64, 4, 8),
    (6, 10, 1, 4),      # small union: |core| may fall below k (empty slots)
    (3, 40, 1, 8),      # |core| <= 3 < k
    (100, 19, 3, 8),
    (257, 128, 2, 16),
    (60, 100, 2, 6),    # one-workgroup kernel with 2 experts per lane
    (50, 150, 3, 8),    # and 4 per lane
]


@pytest.mark.parametrize("multi", [False, True])
@pytest.mark.parametrize("case", DES_SEQ_CASES)
def test_des_seq_route_bitexact_on_probs(case, multi):
    """DES-Seq ("Dynamic Expert Sharing", 2.3, 4.3): core = union of the tokens' top-k_seq (listed
    ascending, then -1), votes = selection counts, each token's top-min(k, |core|) inside the core,
    the remaining slots empty; bit-exact on given fp32 probabilities with exact ties."""
    N, E, kq, k = case
    spec = _spec(S=N, E_heavy=E, mode="des_seq", k=k, vote_k=kq)
    rng = np.random.default_rng(N * E + kq)
    L = _logits(rng, N, E, scale=0.9, tie_rows=0.2).astype(np.float64)
    P32 = orc.softmax(L).astype(np.float32)
    say(f"des-seq route N={N} E={E} k_seq={kq} k={k} multi={multi}")
    got, _ = _route(spec, P32, input_probs=True, multi=multi)
    P = P32.astype(np.float64)
    rt = orc.route(spec, P=P, input_probs=True)
    n = rt["core"].size
    assert np.array_equal(got["core"][:n], rt["core"]) and np.all(got["core"][n:] == -1)
    assert np.array_equal(got["votes"], rt["votes"].astype(np.float32))
    kp = rt["idx"].shape[1]
    assert kp == min(k, n)
    assert np.array_equal(got["topk_idx"][:, :kp], rt["idx"])
    assert np.all(got["topk_idx"][:, kp:] == -1) and np.all(got["topk_w"][:, kp:] == 0)
    assert np.allclose(got["topk_w"][:, :kp], rt["w"], rtol=k * 1.2e-7, atol=0)
    idx = np.concatenate([rt["idx"], np.full((N, k - kp), -1)], axis=1)
    _check_permutation(spec, got, idx)
    assert set(np.flatnonzero(got["counts"])) <= set(rt["core"].tolist())


def test_des_seq_route_on_logits_full_size():
    spec = _spec(S=32, E_heavy=64, mode="des_seq", k=8, vote_k=2)
    rng = np.random.default_rng(6)
    L = (rng.standard_normal((32, 64)) * 0.91).astype(np.float32)
    got, _ = _route(spec, L)
    L64 = L.astype(np.float64)
    rt = reconcile_des_seq(spec, orc.route(spec, L=L64), got["core"], L64)
    kp = rt["idx"].shape[1]
    assert np.array_equal(got["topk_idx"][:, :kp], rt["idx"])


def test_route_is_deterministic():
    spec = _spec(S=4096, E_heavy=16, n_identity=1, n_zero=1, n_const=1, k=2)
    L = _logits(np.random.default_rng(2), 4096, 19)
    a, _ = _route(spec, L)
    b, _ = _route(spec, L)
    for key in ("topk_idx", "topk_w", "row_token", "row_w", "token_rows", "counts"):
        assert np.array_equal(a[key], b[key]), key
