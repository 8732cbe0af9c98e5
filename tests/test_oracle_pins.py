"""Pins of the fp64 oracle against what the pages and the mathematics fix (CPU only).

Each test checks the oracle against something other than itself: closed forms, tabulated values,
brute force over all subsets on tiny inputs, invariants the pages state, or hand-derived numbers.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle as orc
from synth import LayerSpec, gen_layer_inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _brute_topk(keys_row, k):
    """Brute force: the k-subset with the largest key sum; ties to the lexicographically smallest
    sorted index tuple. Keys here are exact in fp64 (small integers or dyadic)."""
    best, best_sum = None, -math.inf
    for sub in itertools.combinations(range(len(keys_row)), k):   # lexicographic order
        s = sum(keys_row[i] for i in sub)
        if s > best_sum:
            best, best_sum = sub, s
    return best


# ------------------------------------------------------------------------------ softmax


def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(1)
    L = rng.standard_normal((300, 19)) * 3
    P = orc.softmax(L)
    assert np.all(P > 0)
    assert np.max(np.abs(P.sum(axis=1) - 1.0)) <= 1e-12


def test_softmax_two_experts_is_logistic():
    g = _gold("logistic.json")
    for z, sig in g["values"]:
        # p_0 of a two-expert row [l0, l1] = sigma(l0 - l1); check at several offsets.
        for base in (-3.0, 0.0, 7.5):
            P = orc.softmax(np.array([[base + z, base]]))
            assert abs(P[0, 0] - sig) <= g["tolerance"]
            assert abs(P[0, 1] - (1 - sig)) <= g["tolerance"]


# ------------------------------------------------------------------------------ token choice


@pytest.mark.parametrize("seed", range(6))
def test_tc_matches_bruteforce_with_ties(seed):
    rng = np.random.default_rng(seed)
    S, E = 8, int(rng.integers(2, 9))
    L = rng.integers(-2, 3, size=(S, E)).astype(float)    # many exact ties
    for k in range(1, E + 1):
        idx = orc.tc_select(L, k)
        for s in range(S):
            assert tuple(sorted(idx[s])) == _brute_topk(L[s], k)
            # slots in key order: keys non-increasing, equal keys by ascending index
            for a, b in zip(idx[s][:-1], idx[s][1:]):
                assert L[s, a] > L[s, b] or (L[s, a] == L[s, b] and a < b)


def test_tc_k_equals_E_selects_all():
    rng = np.random.default_rng(3)
    L = rng.standard_normal((50, 7))
    idx = orc.tc_select(L, 7)
    assert np.all(np.sort(idx, axis=1) == np.arange(7))


def test_tc_weights_renorm_is_softmax_over_chosen():
    rng = np.random.default_rng(4)
    L = rng.standard_normal((40, 8))
    idx = orc.tc_select(L, 2)
    w = orc.tc_weights(orc.softmax(L), idx, renorm=True)
    # Closed form for two chosen logits a >= b: weights sigma(a-b), sigma(b-a).
    a = np.take_along_axis(L, idx[:, :1], 1)[:, 0]
    b = np.take_along_axis(L, idx[:, 1:2], 1)[:, 0]
    sig = 1.0 / (1.0 + np.exp(-(a - b)))
    assert np.allclose(w[:, 0], sig, rtol=0, atol=1e-14)
    assert np.allclose(w[:, 1], 1 - sig, rtol=0, atol=1e-14)
    wr = orc.tc_weights(orc.softmax(L), idx, renorm=False)
    ex = np.exp(L)
    assert np.allclose(wr, np.take_along_axis(ex, idx, 1) / ex.sum(1, keepdims=True), atol=1e-15)


# ------------------------------------------------------------------------------ expert choice


def test_capacity_page_values_and_rounding():
    for c in _gold("page_values.json")["capacity"]["cases"]:
        assert orc.ec_capacity(c["S"], c["E"], c["f_c"]) == c["C"]
    assert orc.ec_capacity(10, 3, 2.0) == 6           # 6.67 rounds down
    assert orc.ec_capacity(10, 1, 2.0) == 10          # clipped to S
    assert orc.ec_capacity(7, 4, 0.5) == 0            # rounds to 0 (the library rejects this)


@pytest.mark.parametrize("seed", range(5))
def test_ec_matches_bruteforce(seed):
    rng = np.random.default_rng(10 + seed)
    S, E = 8, 4
    A = rng.integers(0, 6, size=(S, E)) / 8.0          # dyadic, exact sums, ties
    C = orc.ec_capacity(S, E, 2.0)
    tokens, gates = orc.ec_select(A, C)
    for i in range(E):
        assert tuple(tokens[i]) == _brute_topk(A[:, i], C)
        assert np.array_equal(gates[i], A[tokens[i], i])


def test_ec_natural_balance_and_variable_experts_per_token():
    rng = np.random.default_rng(5)
    S, E = 512, 16
    A = orc.softmax(rng.standard_normal((S, E)))
    C = orc.ec_capacity(S, E, 2.0)
    tokens, _ = orc.ec_select(A, C)
    counts = np.bincount(tokens.ravel(), minlength=S)
    assert tokens.shape == (E, C) and C == 64
    assert all(len(set(t)) == C for t in tokens)       # every expert takes exactly C distinct tokens
    assert counts.sum() == E * C
    assert counts.min() >= 0 and counts.max() <= E
    assert counts.min() != counts.max()                # tokens get a variable number of experts
    off, lst = orc.ec_token_csr(tokens, S)
    assert np.array_equal(np.diff(off), counts)
    for s in range(0, S, 37):
        rows = lst[off[s]:off[s + 1]]
        experts = rows // C
        assert np.all(np.diff(experts) > 0)
        assert np.all(tokens[experts, rows % C] == s)


def _dense_spec(**kw):
    base = dict(name="t", S=24, d=8, f=12, E_heavy=1, act="gelu", mode="tc", k=1, dtype="f32")
    base.update(kw)
    return LayerSpec(**base)


def _textbook_ffn(x, w1, w3, w2, act):
    """Dense FFN written from scratch for the E=1 checks (matrix-vector loops)."""
    y = np.zeros((x.shape[0], w2.shape[0]))
    for s in range(x.shape[0]):
        u = np.array([sum(w1[o, i] * x[s, i] for i in range(x.shape[1])) for o in range(w1.shape[0])])
        if act == "swiglu":
            g = np.array([sum(w3[o, i] * x[s, i] for i in range(x.shape[1])) for o in range(w3.shape[0])])
            h = g / (1 + np.exp(-g)) * u
        else:
            h = np.array([v * 0.5 * (1 + math.erf(v / math.sqrt(2))) for v in u])
        y[s] = [sum(w2[o, i] * h[i] for i in range(h.size)) for o in range(w2.shape[0])]
    return y


@pytest.mark.parametrize("mode,act", [("tc", "gelu"), ("tc", "swiglu"), ("ec", "gelu")])
def test_single_expert_is_dense_mlp(mode, act):
    spec = _dense_spec(mode=mode, act=act)
    W = gen_layer_inputs(spec, seed=2, std=0.3)
    r = orc.layer_forward(spec, W, W.x)
    if mode == "ec":
        assert r["rt"]["C"] == spec.S
        assert np.all(r["rt"]["gates"] == 1.0)
    ref = _textbook_ffn(W.x.astype(float), W.w1[0][0].astype(float),
                        None if W.w3[0] is None else W.w3[0][0].astype(float),
                        W.w2[0][0].astype(float), act)
    assert np.allclose(r["y"], ref, rtol=1e-12, atol=1e-12)


def test_router_logits_hand_worked():
    """L = x . W_r^T with W_r stored [E, d]: x = (1, 2), expert rows (1, 0), (0, 1), (1, 1), (-2, 0.5)
    give L = (1, 2, 3, -1); the gate residual adds the previous logits elementwise."""
    x = np.array([[1.0, 2.0]])
    w = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [-2.0, 0.5]])
    assert orc.router_logits(x, w).tolist() == [[1.0, 2.0, 3.0, -1.0]]
    assert orc.router_logits(x, w, np.array([[0.5, -2.0, 0.0, 1.0]])).tolist() == [[1.5, 0.0, 3.0, 0.0]]


def test_expert_choice_two_experts_hand_affinities():
    """Two experts, f_c = 1.5, S = 4: C = 3. Logits ln 3 / ln 1, ln 1 / ln 3, 0 / 0, ln 7 / ln 1 give
    affinities (3/4, 1/4), (1/4, 3/4), (1/2, 1/2), (7/8, 1/8). Expert 0 takes tokens 3, 0, 2 and
    expert 1 tokens 1, 2, 0, so token 0 gets 3/4 F_0 + 1/4 F_1, token 1 gets 3/4 F_1, token 2 gets
    1/2 F_0 + 1/2 F_1 and token 3 gets 7/8 F_0 (EC-DiT 核心公式: the output sums A_{s,i} FFN_i over
    the experts that chose s)."""
    spec = LayerSpec(name="ec2", S=4, d=8, f=12, E_heavy=2, act="gelu", mode="ec", capacity_factor=1.5,
                     dtype="f32")
    W = gen_layer_inputs(spec, seed=14, std=0.4)
    x = W.x.astype(np.float64)
    L = np.log(np.array([[3.0, 1.0], [1.0, 3.0], [1.0, 1.0], [7.0, 1.0]]))
    rt = orc.route(spec, L=L)
    assert rt["C"] == 3
    assert rt["tokens"].tolist() == [[0, 2, 3], [0, 1, 2]]
    y = orc.layer_forward(spec, W, x, rt=rt)["y"]
    F = [_textbook_ffn(x, W.w1[0][i].astype(np.float64), None, W.w2[0][i].astype(np.float64), "gelu")
         for i in range(2)]
    want = np.stack([0.75 * F[0][0] + 0.25 * F[1][0], 0.75 * F[1][1], 0.5 * F[0][2] + 0.5 * F[1][2],
                     0.875 * F[0][3]])
    assert np.allclose(y, want, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------------------ DES


def _des_bruteforce(P, K, M):
    """Core set by brute force: per token the K-subset of largest probability sum; total vote of a
    candidate core = sum over tokens of the probabilities of its members inside that token's
    filtered set; the best M-subset, ties to the lexicographically smallest tuple."""
    N, E = P.shape
    T = [set(_brute_topk(P[n], K)) for n in range(N)]
    best, best_v = None, -math.inf
    for core in itertools.combinations(range(E), M):
        v = sum(P[n, e] for n in range(N) for e in core if e in T[n])
        if v > best_v:
            best, best_v = core, v
    return best


@pytest.mark.parametrize("seed", range(6))
def test_des_vote_core_matches_bruteforce(seed):
    rng = np.random.default_rng(20 + seed)
    N, E = int(rng.integers(2, 7)), int(rng.integers(4, 11))
    raw = rng.integers(0, 9, size=(N, E)).astype(float)
    raw[:, 0] += 1
    P = raw / 1024.0                                   # dyadic "routing weights" (exact sums)
    K = int(rng.integers(1, E + 1))
    M = int(rng.integers(1, E + 1))
    for vdt in (np.float64, np.float32):
        votes, core = orc.des_vote(P, P, K, M, vote_dtype=vdt)
        assert core.size == M and np.all(np.diff(core) > 0)
        assert tuple(core) == _des_bruteforce(P, K, M)


def test_des_core_size_page_values():
    for c in _gold("page_values.json")["core_size"]["cases"]:
        assert int(c["beta"] * c["M"]) == c["M_core"]
        rng = np.random.default_rng(0)
        L = rng.standard_normal((32, c["M"]))
        _, core = orc.des_vote(L, orc.softmax(L), 8, c["M_core"])
        assert core.size == c["M_core"]


def test_des_beta_one_and_full_cover_equal_token_choice():
    rng = np.random.default_rng(7)
    N, E, k = 32, 64, 8
    L = rng.standard_normal((N, E))
    P = orc.softmax(L)
    idx_tc = orc.tc_select(L, k)
    w_tc = orc.tc_weights(P, idx_tc, True)
    # beta = 1: the core is every expert
    _, core = orc.des_vote(L, P, k, E)
    idx, w = orc.core_reroute(L, P, core, k, True)
    assert np.array_equal(idx, idx_tc) and np.allclose(w, w_tc, atol=1e-15)
    # M_core >= number of experts with a vote, K >= k: the same as token choice
    n_voted = np.unique(orc.tc_select(L, k)).size
    _, core = orc.des_vote(L, P, k, n_voted)
    idx, w = orc.core_reroute(L, P, core, k, True)
    assert np.array_equal(idx, idx_tc)
    # a smaller core changes the routing and keeps every slot inside the core
    _, core = orc.des_vote(L, P, k, 16)
    idx, _ = orc.core_reroute(L, P, core, k, True)
    assert np.isin(idx, core).all() and np.unique(idx).size <= 16


def test_des_core_smaller_than_k():
    rng = np.random.default_rng(8)
    L = rng.standard_normal((5, 12))
    _, core = orc.des_vote(L, orc.softmax(L), 8, 3)
    idx, w = orc.core_reroute(L, orc.softmax(L), core, 8, True)
    assert idx.shape == (5, 3) and np.allclose(w.sum(1), 1.0)


def test_des_seq_is_union_of_topk():
    rng = np.random.default_rng(9)
    L = rng.standard_normal((6, 20))
    core = orc.des_seq_core(L, 2)
    want = sorted({e for s in range(6) for e in _brute_topk(L[s], 2)})
    assert list(core) == want


def _padded_route_bruteforce(L, core, k):
    """Per token, the top-min(k, |core|) experts inside the core by brute force (key sum, then the
    lexicographically smallest tuple), in key order."""
    out = []
    for s in range(L.shape[0]):
        kk = min(k, len(core))
        sub = _brute_topk(L[s, core], kk)
        chosen = [int(core[i]) for i in sub]
        chosen.sort(key=lambda e: (-L[s, e], e))
        out.append(chosen)
    return np.array(out, dtype=np.int64)


@pytest.mark.parametrize("seed", range(5))
def test_des_seq_route_matches_bruteforce(seed):
    """DES-Seq (Dynamic Expert Sharing, 2.3; 3.1 local count k_seq; 4.3 re-activate top-k in the core):
    the core is the union of each token's top-k_seq, every routed slot lies in it, and each token's
    slots are its brute-force top-k inside the core. Integer logits give exact ties."""
    rng = np.random.default_rng(40 + seed)
    N, E = int(rng.integers(2, 7)), int(rng.integers(5, 11))
    L = rng.integers(-3, 4, size=(N, E)).astype(float)
    for k_seq in range(1, E + 1):
        for k in (2, 4):
            if k > E:
                continue
            spec = LayerSpec(name="dseq", S=N, d=8, f=8, E_heavy=E, act="gelu", mode="des_seq", k=k,
                             vote_k=k_seq, dtype="f32")
            rt = orc.route(spec, L=L)
            want_core = sorted({e for s in range(N) for e in _brute_topk(L[s], k_seq)})
            assert list(rt["core"]) == want_core
            assert np.array_equal(np.flatnonzero(rt["votes"]), want_core)
            assert rt["votes"].sum() == N * k_seq
            assert np.array_equal(rt["idx"], _padded_route_bruteforce(L, np.array(want_core), k))
            assert np.allclose(rt["w"].sum(1), 1.0)


def test_des_seq_reduces_to_token_choice_when_k_seq_covers_k():
    """With k_seq >= k every token's own top-k lies in the core, so DES-Seq is vanilla top-k."""
    rng = np.random.default_rng(9)
    L = rng.standard_normal((32, 64))
    base = LayerSpec(name="dseq", S=32, d=8, f=8, E_heavy=64, act="gelu", mode="tc", k=8, dtype="f32")
    tc = orc.route(base, L=L)
    for k_seq in (8, 12, 64):
        rt = orc.route(base.replace(mode="des_seq", vote_k=k_seq), L=L)
        assert np.array_equal(rt["idx"], tc["idx"]) and np.allclose(rt["w"], tc["w"], atol=1e-15)


def test_des_seq_core_smaller_than_k():
    """One token with k_seq = 2 < k = 4: the core has 2 experts and the token keeps both."""
    L = np.array([[0.1, 2.0, -1.0, 1.5, 0.0]])
    spec = LayerSpec(name="dseq", S=1, d=8, f=8, E_heavy=5, act="gelu", mode="des_seq", k=4, vote_k=2, dtype="f32")
    rt = orc.route(spec, L=L)
    assert list(rt["core"]) == [1, 3]
    assert rt["idx"].tolist() == [[1, 3]]
    e = np.exp(np.array([2.0, 1.5]))
    assert np.allclose(rt["w"][0], e / e.sum(), atol=1e-15)


def test_des_latency_model():
    # f(c) = a c + b for c > 0: two experts with 3 and 5 tokens, one idle.
    assert orc.des_block_latency([3, 0, 5], a=2.0, b=10.0) == (2 * 3 + 10) + (2 * 5 + 10)


# ------------------------------------------------------------------------------ permutation


@pytest.mark.parametrize("seed", range(4))
def test_counting_sort_properties(seed):
    rng = np.random.default_rng(30 + seed)
    S, E, k = 97, 11, 3
    idx = np.stack([rng.permutation(E)[:k] for _ in range(S)])
    valid = rng.random((S, k)) > 0.2
    counts, offsets, row_token, row_slot, token_rows = orc.counting_sort(idx, E, valid)
    assert np.array_equal(offsets[1:] - offsets[:-1], counts)
    assert offsets[0] == 0 and offsets[-1] == valid.sum()
    # brute force grouping
    want = [(e, s, j) for e in range(E) for s in range(S) for j in range(k) if valid[s, j] and idx[s, j] == e]
    assert [(int(idx[s, j]), int(s), int(j)) for s, j in zip(row_token, row_slot)] == want
    for s in range(S):
        for j in range(k):
            r = token_rows[s, j]
            if valid[s, j]:
                assert row_token[r] == s and row_slot[r] == j
            else:
                assert r == -1


# ------------------------------------------------------------------------------ experts


def test_gelu_matches_normal_cdf_table():
    g = _gold("normal_cdf.json")
    for z, phi in g["values"]:
        assert abs(orc.gelu(z) - z * phi) <= abs(z) * g["tolerance"] + 1e-15


def test_silu_matches_logistic():
    g = _gold("logistic.json")
    for z, sig in g["values"]:
        assert abs(orc.silu(z) - z * sig) <= g["tolerance"]


def test_gelu_tanh_close_to_erf_form():
    z = np.linspace(-4, 4, 81)
    assert np.max(np.abs(orc.gelu_tanh(z) - orc.gelu(z))) < 1e-3


def test_gelu_tanh_matches_decimal_table():
    """The tanh form against 40-digit values of the published formula (a wrong constant, such as
    0.0447 for 0.044715 or 2/pi for sqrt(2/pi), fails by far more than the tolerance)."""
    g = _gold("gelu_tanh.json")
    for z, want in g["values"]:
        assert abs(orc.gelu_tanh(z) - want) <= g["tolerance"] * max(1.0, abs(want)), (z, orc.gelu_tanh(z), want)


def test_mlp_hand_worked():
    """d=2, f=3, GELU. x=(1,2). W1 rows (1,0), (-1,0), (2,-1) give pre-activations (1,-1,0);
    gelu = (Phi(1), -Phi(-1), 0). W2 = [[1,2,3],[0,-1,4]] then gives
    y = (Phi(1) - 2 Phi(-1), Phi(-1))."""
    phi = dict((z, p) for z, p in _gold("normal_cdf.json")["values"])
    x = np.array([[1.0, 2.0]])
    w1 = np.array([[1.0, 0.0], [-1.0, 0.0], [2.0, -1.0]])
    w2 = np.array([[1.0, 2.0, 3.0], [0.0, -1.0, 4.0]])
    y = orc.mlp(x, w1, None, w2, "gelu")
    assert np.allclose(y, [[phi[1.0] - 2 * phi[-1.0], phi[-1.0]]], atol=1e-10)
    # SwiGLU: gate rows (1,0),(0,1) -> (1,2); up rows (0,1),(1,1) -> (2,3);
    # h = (silu(1)*2, silu(2)*3) = (2 sigma(1), 6 sigma(2)); W2 = [[1,-1]] -> y = 2 sigma(1) - 6 sigma(2)
    sig = dict((z, p) for z, p in _gold("logistic.json")["values"])
    w3 = np.array([[1.0, 0.0], [0.0, 1.0]])
    w1 = np.array([[0.0, 1.0], [1.0, 1.0]])
    y = orc.mlp(x, w1, w3, np.array([[1.0, -1.0]]), "swiglu")
    assert abs(y[0, 0] - (2 * sig[1.0] - 6 * sig[2.0])) < 1e-12


def test_mlp_hidden_stored_in_bf16_hand_worked():
    """The hidden activation at its bf16 storage precision, rounded after the activation and before
    the down projection (ties to even). x = (1, 2), W1 rows (1, 0), (-1, 0), (3, 0): z = (1, -1, 3),
    gelu = (Phi(1), -Phi(-1), 3 Phi(3)) = (0.84134.., -0.15866.., 2.99595..), whose nearest bf16
    numbers are 215/256, -162/1024 and 3 (the last rounds up; truncation would give 2.984375).
    W2 = [[1, 2, 3], [0, -1, 4]] then gives exactly (9.5234375, 12.158203125)."""
    x = np.array([[1.0, 2.0]])
    w1 = np.array([[1.0, 0.0], [-1.0, 0.0], [3.0, 0.0]])
    w2 = np.array([[1.0, 2.0, 3.0], [0.0, -1.0, 4.0]])
    assert orc.mlp(x, w1, None, w2, "gelu", h_store="bf16").tolist() == [[9.5234375, 12.158203125]]
    phi = dict((z, p) for z, p in _gold("normal_cdf.json")["values"])
    exact = orc.mlp(x, w1, None, w2, "gelu")
    want = [phi[1.0] - 2 * phi[-1.0] + 9 * phi[3.0], phi[-1.0] + 12 * phi[3.0]]
    assert np.allclose(exact, [want], atol=1e-9)


def _light_spec(**kw):
    base = dict(name="light", S=40, d=16, f=8, E_heavy=2, n_identity=1, n_zero=1, n_const=1,
                act="gelu", mode="tc", k=1, renorm=True, dtype="f32")
    base.update(kw)
    return LayerSpec(**base)


def test_zero_and_identity_and_const_experts():
    spec = _light_spec()
    W = gen_layer_inputs(spec, seed=3)
    S, E = spec.S, spec.E_routed
    L = np.zeros((S, E))
    for target, kind in ((3, "zero"), (2, "identity"), (4, "const")):
        Lt = L.copy()
        Lt[:, target] = 5.0
        rt = orc.route(spec, L=Lt)
        assert np.all(rt["idx"][:, 0] == target) and np.all(rt["w"] == 1.0)
        r = orc.layer_forward(spec, W, W.x, rt=rt)
        if kind == "zero":
            assert np.all(r["y"] == 0.0)
        elif kind == "identity":
            assert np.array_equal(r["y"], W.x.astype(float))
        else:
            assert np.array_equal(r["y"], np.broadcast_to(W.const_vec[0][0].astype(float), (S, spec.d)))
    # top-2 without renorm: constant expert with weight g gives g * v_c
    spec2 = _light_spec(k=2, renorm=False)
    Lt = np.zeros((S, E))
    Lt[:, 4] = 3.0
    Lt[:, 3] = 2.0                                  # the zero expert takes the second slot
    rt = orc.route(spec2, L=Lt)
    r = orc.layer_forward(spec2, W, W.x, rt=rt)
    g = orc.softmax(Lt)[:, 4]
    assert np.allclose(r["y"], g[:, None] * W.const_vec[0][0][None, :].astype(float), atol=1e-15)


def test_combine_sensitivity_identity():
    """DICE, conditional communication: for y = sum_e s^e h^e, d||y|| / d h^e = s^e * y / ||y||.
    Checked through the oracle's layer: three constant experts (their outputs h^e are the vectors
    v_e, so they can be perturbed directly), top-3 of 3 without renormalisation and hand-chosen
    logits ln 5, ln 3, ln 2 per token, so the scores are exactly 1/2, 3/10, 1/5."""
    spec = LayerSpec(name="sens", S=2, d=10, f=8, E_heavy=0, n_const=3, act="gelu", mode="tc", k=3,
                     renorm=False, dtype="f32")
    W = gen_layer_inputs(spec, seed=11, std=1.0)
    L = np.log(np.array([[5.0, 3.0, 2.0], [2.0, 5.0, 3.0]]))
    rt = orc.route(spec, L=L)
    s_want = {0: [0.5, 0.3, 0.2], 1: [0.2, 0.5, 0.3]}            # score of expert e for token t
    for t in range(2):
        for j in range(3):
            assert abs(rt["w"][t, j] - s_want[t][rt["idx"][t, j]]) < 1e-15

    def ynorm(cv, t):
        W2 = gen_layer_inputs(spec, seed=11, std=1.0)
        W2.const_vec[0] = cv
        return np.linalg.norm(orc.layer_forward(spec, W2, W2.x, rt=rt)["y"][t])

    cv0 = W.const_vec[0].astype(np.float64)
    for t in range(2):
        y = orc.layer_forward(spec, W, W.x, rt=rt)["y"][t]
        ny = np.linalg.norm(y)
        assert np.allclose(y, sum(s_want[t][e] * cv0[e] for e in range(3)), atol=1e-15)
        eps = 1e-6
        for e in range(3):
            for i in range(spec.d):
                cp, cm = cv0.copy(), cv0.copy()
                cp[e, i] += eps
                cm[e, i] -= eps
                fd = (ynorm(cp, t) - ynorm(cm, t)) / (2 * eps)
                assert abs(fd - s_want[t][e] * y[i] / ny) < 1e-8


def test_shared_experts_sum_with_weight_one():
    """Two always-on shared experts (MMOE 共享专家; the DiT-MoE-XL workload has two): the oracle's
    shared part is the plain sum of the two dense MLPs, each written out as loops (SwiGLU and GELU),
    and a layer with only a zero expert routed returns exactly that sum."""
    for act in ("swiglu", "gelu"):
        spec = LayerSpec(name="shared2", S=5, d=8, f=12, E_heavy=0, n_zero=1, n_shared=2, act=act, mode="tc",
                         k=1, dtype="f32")
        W = gen_layer_inputs(spec, seed=12, std=0.4)
        x = W.x.astype(np.float64)
        want = np.zeros((spec.S, spec.d))
        for i in range(2):
            w3 = None if W.s_w3[0] is None else W.s_w3[0][i].astype(np.float64)
            want += _textbook_ffn(x, W.s_w1[0][i].astype(np.float64), w3, W.s_w2[0][i].astype(np.float64), act)
        assert np.allclose(orc.shared_out(spec, W, 0, x), want, rtol=1e-12, atol=1e-12)
        # each expert contributes: dropping either one changes the sum
        one = _textbook_ffn(x, W.s_w1[0][0].astype(np.float64),
                            None if W.s_w3[0] is None else W.s_w3[0][0].astype(np.float64),
                            W.s_w2[0][0].astype(np.float64), act)
        assert np.abs(want - one).max() > 1e-3
        r = orc.layer_forward(spec, W, x)
        assert np.all(r["rt"]["idx"] == 0) and np.all(r["routed"] == 0.0)
        assert np.allclose(r["y"], want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("renorm", [False, True])
def test_top2_two_heavy_experts_hand_logits(renorm):
    """Top-2 of three heavy experts with hand-chosen logits ln 5, ln 3, ln 2 (permuted per token):
    probabilities 1/2, 3/10, 1/5, so the two chosen weights are 1/2 and 3/10 (raw) or 5/8 and 3/8
    (renormalised). The layer must equal that weighted sum of the two chosen experts' dense MLPs,
    written out as loops."""
    spec = LayerSpec(name="top2", S=3, d=8, f=12, E_heavy=3, act="gelu", mode="tc", k=2, renorm=renorm,
                     dtype="f32")
    W = gen_layer_inputs(spec, seed=13, std=0.4)
    x = W.x.astype(np.float64)
    L = np.log(np.array([[5.0, 3.0, 2.0], [2.0, 3.0, 5.0], [3.0, 2.0, 5.0]]))
    pick = [(0, 1), (2, 1), (2, 0)]
    wts = (5 / 8, 3 / 8) if renorm else (0.5, 0.3)
    rt = orc.route(spec, L=L)
    for t in range(3):
        assert tuple(rt["idx"][t]) == pick[t]
        assert np.allclose(rt["w"][t], wts, rtol=0, atol=1e-15)
    y = orc.layer_forward(spec, W, x, rt=rt)["y"]
    for t in range(3):
        want = sum(wj * _textbook_ffn(x[t:t + 1], W.w1[0][e].astype(np.float64), None,
                                      W.w2[0][e].astype(np.float64), "gelu")[0] for wj, e in zip(wts, pick[t]))
        assert np.allclose(y[t], want, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------------------ layer-level


def test_dice_reuse_extremes():
    spec = _light_spec(E_heavy=4, n_identity=0, n_zero=0, n_const=0, n_shared=1, k=2, reuse_tau=0.0)
    W = gen_layer_inputs(spec, seed=4, std=0.2)
    cache = np.random.default_rng(5).standard_normal((spec.S, spec.d))
    base = orc.layer_forward(spec, W, W.x, cache=cache)
    assert not base["rt"]["reuse"].any()
    # tau > 1: every token reuses, routed part == cache exactly, nothing dispatched
    spec_all = spec.replace(reuse_tau=1.5)
    r = orc.layer_forward(spec_all, W, W.x, cache=cache)
    assert r["rt"]["reuse"].all()
    assert np.array_equal(r["routed"], cache)
    assert np.allclose(r["y"] - orc.shared_out(spec, W, 0, W.x), cache, atol=1e-14)
    valid = ~np.broadcast_to(r["rt"]["reuse"][:, None], r["rt"]["idx"].shape)
    assert orc.counting_sort(r["rt"]["idx"], spec.E_routed, valid)[0].sum() == 0


def test_gate_residual_with_zero_router_keeps_routing():
    spec = _light_spec(n_identity=0, n_zero=0, n_const=0, E_heavy=6, k=2, n_layers=3)
    W = gen_layer_inputs(spec, seed=6, std=0.3)
    for layer in range(1, spec.n_layers):
        W.w_router[layer][:] = 0.0
    outs = orc.stack_forward(spec, W, W.x, act_bf16=False)
    for r in outs[1:]:
        assert np.array_equal(r["rt"]["idx"], outs[0]["rt"]["idx"])
        assert np.allclose(r["logits"], outs[0]["logits"], atol=0)
    # and the residual stream adds each layer's output
    assert np.allclose(outs[1]["h_in"], outs[0]["y"])


def test_bf16_round_reference_values():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: ties to even -> 1.0; just above rounds up.
    assert orc.bf16_round(1.0 + 2 ** -8) == 1.0
    assert orc.bf16_round(1.0 + 2 ** -8 + 2 ** -12) == 1.0 + 2 ** -7
    assert orc.bf16_round(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6     # tie -> even mantissa
    assert orc.bf16_round(-3.0) == -3.0


# ------------------------------------------------------------------------------ attention-residual aggregation


def _states(rng, n, S, d, scale=1.0):
    return rng.standard_normal((n, S, d)) * scale


def test_attnres_single_state_is_identity():
    rng = np.random.default_rng(0)
    V = _states(rng, 1, 5, 16)
    out, alpha = orc.attnres_aggregate(V, rng.standard_normal(16))
    assert np.array_equal(alpha, np.ones((5, 1)))
    assert np.array_equal(out, V[0])


def test_attnres_zero_query_is_mean_and_identical_states_pass_through():
    rng = np.random.default_rng(1)
    V = _states(rng, 4, 6, 8)
    out, alpha = orc.attnres_aggregate(V, np.zeros(8))
    assert np.allclose(alpha, 0.25, atol=1e-15, rtol=0)
    assert np.allclose(out, V.mean(axis=0), atol=1e-14, rtol=0)
    same = np.repeat(V[:1], 3, axis=0)
    out2, _ = orc.attnres_aggregate(same, rng.standard_normal(8) * 5)
    assert np.allclose(out2, V[0], atol=1e-14, rtol=0)


def test_attnres_two_orthogonal_states_give_the_logistic():
    """v0 = a e_0, v1 = b e_1 in d = 4, q = t e_0, eps = 0: v0's RMS is |a| / 2, so z_0 = 2 t
    sign(a) and z_1 = 0, and the two-state softmax gives alpha_0 = sigma(2 t sign(a)), tabulated."""
    table = {z: p for z, p in _gold("logistic.json")["values"]}
    d = 4
    for a, b, t, zz in ((3.0, -7.0, 0.5, 1.0), (0.25, 2.0, 1.0, 2.0), (-5.0, 1.0, 0.5, -1.0), (2.0, 9.0, 0.0, 0.0)):
        V = np.zeros((2, 1, d))
        V[0, 0, 0] = a
        V[1, 0, 1] = b
        q = np.zeros(d)
        q[0] = t
        out, alpha = orc.attnres_aggregate(V, q, eps=0.0)
        p0 = table[zz]
        assert abs(alpha[0, 0] - p0) <= 1e-12 and abs(alpha[0, 1] - (1 - p0)) <= 1e-12
        assert abs(out[0, 0] - p0 * a) <= 1e-12 * abs(a)
        assert abs(out[0, 1] - (1 - p0) * b) <= 1e-12 * abs(b)
        assert out[0, 2] == 0 and out[0, 3] == 0


def test_attnres_scores_ignore_state_scale_and_order():
    """The keys are RMS-normalised, so scaling a state by c > 0 leaves every weight unchanged
    (eps = 0) while the output takes the scaled state; permuting the states permutes the weights
    and leaves the output unchanged."""
    rng = np.random.default_rng(2)
    V = _states(rng, 5, 7, 12)
    q = rng.standard_normal(12)
    out, alpha = orc.attnres_aggregate(V, q, eps=0.0)
    W = V.copy()
    W[2] *= 37.0
    out2, alpha2 = orc.attnres_aggregate(W, q, eps=0.0)
    assert np.allclose(alpha2, alpha, atol=1e-14, rtol=0)
    assert np.allclose(out2 - out, alpha[:, 2:3] * 36.0 * V[2], atol=1e-12, rtol=0)
    perm = [3, 0, 4, 2, 1]
    out3, alpha3 = orc.attnres_aggregate(V[perm], q, eps=0.0)
    assert np.allclose(alpha3, alpha[:, perm], atol=1e-15, rtol=0)
    assert np.allclose(out3, out, atol=1e-13, rtol=0)


def test_attnres_is_a_convex_combination():
    rng = np.random.default_rng(3)
    V = _states(rng, 6, 9, 10, scale=3.0)
    out, alpha = orc.attnres_aggregate(V, rng.standard_normal(10) * 2)
    assert np.all(alpha > 0)
    assert np.allclose(alpha.sum(axis=1), 1.0, atol=1e-15, rtol=0)
    assert np.all(out <= V.max(axis=0) + 1e-12) and np.all(out >= V.min(axis=0) - 1e-12)


# ------------------------------------------------------------------------------ DICE step loop


def _dice_spec(**kw):
    base = dict(name="dice", S=48, d=16, f=24, E_heavy=4, n_shared=1, act="swiglu", mode="tc", k=2, renorm=True,
                dtype="f32", n_layers=3)
    base.update(kw)
    return LayerSpec(**base)


def _steps(W, T, drift, seed=21):
    rng = np.random.default_rng(seed)
    x = W.x.astype(np.float64)
    xs = []
    for _ in range(T):
        xs.append(x.copy())
        x = x + drift * rng.standard_normal(x.shape)
    return xs


def test_dice_loop_without_reuse_is_a_fresh_stack_per_step():
    spec = _dice_spec()
    W = gen_layer_inputs(spec, seed=22, std=0.3)
    xs = _steps(W, 4, 0.1)
    for tau, layers in ((0.3, ()), (0.0, (0, 1, 2))):
        steps = orc.dice_step_loop(spec, W, xs, tau=tau, stride=3, reuse_layers=layers, act_bf16=False)
        for t, per in enumerate(steps):
            fresh = orc.stack_forward(spec, W, xs[t], act_bf16=False, gate_residual=False)
            for layer in range(spec.n_layers):
                assert not per[layer]["reuse"].any()
                assert np.array_equal(per[layer]["y"], fresh[layer]["y"])


def test_dice_loop_stationary_input_full_reuse_repeats_step_zero():
    """tau > 1 reuses every token on non-refresh steps: the routed part is the cache of step 0
    exactly, so with an unchanged input every step reproduces step 0 bit for bit (fp32 storage)."""
    spec = _dice_spec()
    W = gen_layer_inputs(spec, seed=23, std=0.3)
    xs = [W.x.astype(np.float64)] * 5
    steps = orc.dice_step_loop(spec, W, xs, tau=1.5, stride=4, reuse_layers=(0, 1, 2), act_bf16=False)
    for t in range(1, 5):
        for layer in range(spec.n_layers):
            if t % 4 != 0:
                assert steps[t][layer]["reuse"].all()
                assert np.array_equal(steps[t][layer]["routed"], steps[0][layer]["routed"])
            assert np.array_equal(steps[t][layer]["y"], steps[0][layer]["y"])


def test_dice_loop_reuse_refresh_and_selective_sync():
    """With a drifting input: on a reuse step, tokens below tau take the previous cache exactly and
    the others match a fresh computation; refresh steps and the synchronous (deep) layer always
    match a fresh layer call on their input; caches hold the fresh routed parts."""
    spec = _dice_spec(E_heavy=8)
    W = gen_layer_inputs(spec, seed=24, std=0.15)
    xs = _steps(W, 5, 0.05)
    tau, stride, layers = 0.3, 3, (0, 1)
    steps = orc.dice_step_loop(spec, W, xs, tau=tau, stride=stride, reuse_layers=layers, act_bf16=False)
    n_reused = 0
    for t, per in enumerate(steps):
        for layer, r in enumerate(per):
            h = r["h_in"]
            fresh = orc.layer_forward(spec, W, h, layer=layer, residual=h)
            P = fresh["rt"]["P"]
            reuse = r["reuse"]
            if layer in layers and t % stride != 0:
                assert np.array_equal(reuse, P.max(1) < tau)
                prev = steps[t - 1][layer]["cache"]
                assert np.array_equal(r["routed"][reuse], prev[reuse])
                assert np.array_equal(r["cache"][reuse], prev[reuse])
                n_reused += int(reuse.sum())
            else:
                assert not reuse.any()
            assert np.allclose(r["routed"][~reuse], fresh["routed"][~reuse], rtol=0, atol=1e-14)
            assert np.array_equal(r["cache"][~reuse], r["routed"][~reuse])
            assert np.allclose(r["y"], fresh["y"] - fresh["routed"] + r["routed"], rtol=0, atol=1e-13)
    assert 0 < n_reused < 5 * spec.S * len(layers)
