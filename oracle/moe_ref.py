"""Plain, slow, fp64 CPU oracle of the sparse Mixture-of-Experts FFN layer forward.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run this module. It shares no code with the HIP library (it imports
nothing from ``mixture_experts_layer_gemm_amd``) and the library never calls it.

Everything is NumPy float64 unless a function says otherwise. Dense products use ``numpy.matmul``;
selections use ``numpy.lexsort`` with the sort keys written out. There is no blocking, fusion or
reordering beyond the definitions below.

Pages followed (cited by title and section):
  [EC-DiT] "EC-DiT: Scaling Diffusion Transformers with Adaptive Expert-Choice Routing",
           part 三 (技术架构), 核心公式: token-choice vs expert-choice routing, the affinity softmax
           A = softmax(x'W_r) over experts, and 容量因子 (Capacity = f_c * S / E, f_c = 2.0).
  [DES]    "Dynamic Expert Sharing: Decoupling Memory from Parallelism in Mixture-of-Experts
           Diffusion LLMs": 2.1 latency model f(c) = a*c + b; 2.2 core-set function Phi; 2.3 DES-Seq;
           2.4 DES-Vote (filter to top-K, vote with routing weights, elect top M_core);
           3.1 M_core = beta * M; 4.3 re-activating top-8 inside the core set.
  [MMOE]   "MMOE: Modernizing Diffusion Transformers with Efficient Expert Design", 方法论:
           MoE++ expert layer (heavy MLP experts; identity, zero and constant zero-computation
           experts), gate-residual routing, shared always-on expert.
  [DICE]   "DICE: Staleness-Centric Optimizations for Parallel Diffusion MoE Inference", 关键设计:
           条件通信 (high-score tokens fresh, low-score tokens reuse cached results; the sensitivity
           of ||y|| to an expert output scales with its routing score) and 交织并行 (only combine
           results are cached).

Readings where the pages are silent or garbled are marked [R#]; each is listed in the design
notes of the repository with its justification.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py`` against closed forms,
brute force on tiny inputs, invariants the pages state, or hand-derived values. None is
"parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf

F64 = np.float64

# --------------------------------------------------------------------------------------------
# a1: router logits (+ gate residual)
# --------------------------------------------------------------------------------------------


def router_logits(x, w_router, prev_logits=None):
    """Router logits L = x . W_r^T, plus the previous MoE layer's logits when given.

    [EC-DiT] 核心公式: the router scores are x' W_r with W_r of shape d x E; the weight is stored
    here as [E, d] (linear-layer layout), so the product is x W_r^T.
    [MMOE] 方法论, gate-residual routing: the router adds the previous layer's gating logits
    (plain addition of its final logits [R17]).
    """
    L = np.asarray(x, F64) @ np.asarray(w_router, F64).T
    if prev_logits is not None:
        L = L + np.asarray(prev_logits, F64)
    return L


def softmax(L):
    """Row softmax over experts: p_{s,i} = exp(L_{s,i}) / sum_i exp(L_{s,i}).

    [EC-DiT] 核心公式 (the affinity A_{s,i}). The row max is subtracted first; that leaves the
    quotient unchanged. All routed experts (heavy and zero-computation) share one softmax [R16].
    """
    L = np.asarray(L, F64)
    z = np.exp(L - L.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


# --------------------------------------------------------------------------------------------
# a2: token choice
# --------------------------------------------------------------------------------------------


def rank_desc(keys):
    """Per row, the column indices ordered by (key descending, index ascending) [R2].

    This order decides every selection below: ties always go to the lower index.
    """
    keys = np.asarray(keys, F64)
    cols = np.broadcast_to(np.arange(keys.shape[-1]), keys.shape)
    # lexsort: last key is primary.
    return np.lexsort((cols, -keys), axis=-1)


def tc_select(keys, k):
    """Token choice: each token takes its top-k experts [EC-DiT] (Token-Choice 路由).

    ``keys`` are the router logits (equivalently the probabilities: softmax is strictly increasing
    within a row), or given probabilities. Slots are in key order [R3].
    """
    return rank_desc(keys)[:, :k].astype(np.int64)


def tc_weights(P, idx, renorm):
    """Gate weight of each chosen slot: the softmax probability, or with ``renorm`` the
    probability divided by the sum over the token's chosen experts [R1]."""
    P = np.asarray(P, F64)
    w = np.take_along_axis(P, idx, axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return w


# --------------------------------------------------------------------------------------------
# a2': expert choice
# --------------------------------------------------------------------------------------------


def ec_capacity(S, E, capacity_factor):
    """Tokens per expert: Capacity = f_c * S / E [EC-DiT] (容量因子), rounded down and clipped
    to S [R5]."""
    return int(min(S, math.floor(capacity_factor * S / E)))


def ec_select(A, C):
    """Expert choice: expert i takes the C tokens with the largest affinity A[:, i]
    (ties to the lower token index) [EC-DiT] (Expert-Choice 路由).

    Returns ``tokens`` [E, C] (each row ascending by token id) and ``gates`` [E, C] = A[token, i]
    (the raw affinity [R6]).
    """
    A = np.asarray(A, F64)
    order = rank_desc(A.T)[:, :C]          # [E, C] best-first
    tokens = np.sort(order, axis=1)
    gates = np.take_along_axis(A.T, tokens, axis=1)
    return tokens.astype(np.int64), gates


# --------------------------------------------------------------------------------------------
# a2'': DES-Vote (and DES-Seq)
# --------------------------------------------------------------------------------------------


def des_vote(filter_keys, P, vote_k, m_core, vote_dtype=F64, vote_renorm=False):
    """DES-Vote core set [DES] 2.4.

    1. Filter: token n keeps its top-K experts T_n (by ``filter_keys``: logits or probabilities).
    2. Vote: v_e = sum over tokens n (ascending) of [e in T_n] * p_{n,e}, with p the routing weight
       (raw softmax probability [R8]; ``vote_renorm`` renormalises p within T_n instead).
       ``vote_dtype`` fixes the accumulation precision; the sum runs over n in ascending order.
    3. Elect: the M_core experts with the largest vote, ties to the lower index; experts with no
       vote fill by index, so the core always has exactly M_core members [R10].

    Returns (votes [E] as vote_dtype, core [M_core] ascending).
    """
    P = np.asarray(P, F64)
    N, E = P.shape
    T = rank_desc(filter_keys)[:, :vote_k]
    wsel = np.take_along_axis(P, T, axis=1)
    if vote_renorm:
        wsel = wsel / wsel.sum(axis=1, keepdims=True)
    votes = np.zeros(E, dtype=vote_dtype)
    for n in range(N):                      # fixed accumulation order
        for j in range(vote_k):
            e = T[n, j]
            votes[e] = vote_dtype(votes[e] + vote_dtype(wsel[n, j]))
    core = np.sort(rank_desc(votes.astype(F64)[None, :])[0, :m_core])
    return votes, core.astype(np.int64)


def des_seq_core(filter_keys, k_seq):
    """DES-Seq core set [DES] 2.3: the union over tokens of each token's top-k experts [R14].
    Returns the members ascending (size varies)."""
    T = rank_desc(filter_keys)[:, :k_seq]
    return np.unique(T).astype(np.int64)


def des_seq_counts(filter_keys, k_seq, E):
    """For each expert, the number of tokens whose local top-k_seq holds it ([DES] 2.3: the local
    selections whose union is the core). The core is the set of experts with a nonzero count."""
    T = rank_desc(filter_keys)[:, :k_seq]
    return np.bincount(T.ravel(), minlength=E).astype(np.int64)


def core_reroute(keys, P, core, k, renorm):
    """Each token re-activates its top-k' experts inside the core set, k' = min(k, |core|)
    [DES] 4.3 [R12]. Keys restricted to the core decide (ties to lower index); weights are the
    probabilities, renormalised over the chosen experts when ``renorm`` [R11]."""
    keys = np.asarray(keys, F64)
    core = np.asarray(core, np.int64)
    kk = min(k, core.size)
    local = rank_desc(keys[:, core])[:, :kk]   # positions inside the ascending core list
    idx = core[local]                            # key order preserved (core ascending => ties ok)
    w = tc_weights(P, idx, renorm)
    return idx, w


# --------------------------------------------------------------------------------------------
# a3: counting sort (dispatch order)
# --------------------------------------------------------------------------------------------


def counting_sort(idx, E, valid=None):
    """Group the (token, slot) pairs by expert: experts ascending, then token ascending, then slot.

    ``valid[s, j]`` False drops a pair (a zero-computation expert, or a token reusing its cache).
    Returns counts [E], offsets [E+1] (exclusive prefix sum), row_token [R], row_slot [R], and
    token_rows [S, k] (the row of each valid pair, -1 otherwise).
    """
    idx = np.asarray(idx, np.int64)
    S, k = idx.shape
    if valid is None:
        valid = np.ones_like(idx, dtype=bool)
    tok = np.broadcast_to(np.arange(S)[:, None], (S, k))
    slot = np.broadcast_to(np.arange(k)[None, :], (S, k))
    e_v, t_v, j_v = idx[valid], tok[valid], slot[valid]
    order = np.lexsort((j_v, t_v, e_v))
    counts = np.bincount(e_v, minlength=E).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    row_token = t_v[order]
    row_slot = j_v[order]
    token_rows = np.full((S, k), -1, dtype=np.int64)
    token_rows[row_token, row_slot] = np.arange(order.size)
    return counts, offsets, row_token, row_slot, token_rows


def ec_token_csr(tokens, S):
    """For expert choice: rows are expert-major (row = i*C + position). For every token, the
    rows that hold it, by ascending expert. Returns (token_off [S+1], token_list)."""
    E, C = tokens.shape
    pairs = [(int(tokens[i, p]), i, i * C + p) for i in range(E) for p in range(C)]
    pairs.sort()
    cnt = np.bincount(np.asarray([p[0] for p in pairs], np.int64), minlength=S) if pairs else \
        np.zeros(S, np.int64)
    token_off = np.concatenate([[0], np.cumsum(cnt)]).astype(np.int64)
    token_list = np.asarray([p[2] for p in pairs], dtype=np.int64)
    return token_off, token_list


# --------------------------------------------------------------------------------------------
# a5-a8: experts
# --------------------------------------------------------------------------------------------


def gelu(z):
    """GELU, erf form: z * Phi(z) [R20]."""
    z = np.asarray(z, F64)
    return 0.5 * z * (1.0 + _erf(z / math.sqrt(2.0)))


def gelu_tanh(z):
    """GELU, tanh approximation (flag-selected variant) [R20]."""
    z = np.asarray(z, F64)
    return 0.5 * z * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))


def silu(z):
    z = np.asarray(z, F64)
    return z / (1.0 + np.exp(-z))


def mlp(xr, w1, w3, w2, act, h_store=None):
    """A heavy expert, the standard MLP of [MMOE] MoE++ (no biases [R20]).

    GELU:   W2 . gelu(W1 . x)
    SwiGLU: W2 . (silu(W_gate . x) * (W_up . x)), with w1 = W_up and w3 = W_gate [R21].
    Weights are [out, in]; rows of ``xr`` are tokens.

    ``h_store="bf16"`` keeps the hidden activation at the storage precision of a bf16 layer
    between the two projections [R23]: it is rounded to the nearest bf16 (ties to even) after the
    activation and before the down projection. Default: exact (fp64) throughout.
    """
    xr = np.asarray(xr, F64)
    up = xr @ np.asarray(w1, F64).T
    if act == "swiglu":
        h = silu(xr @ np.asarray(w3, F64).T) * up
    elif act == "gelu":
        h = gelu(up)
    elif act == "gelu_tanh":
        h = gelu_tanh(up)
    else:
        raise ValueError(act)
    if h_store == "bf16":
        h = bf16_round(h)
    elif h_store is not None:
        raise ValueError(h_store)
    return h @ np.asarray(w2, F64).T


def expert_kind(spec, e):
    """Routed expert ids: [0, E_h) heavy, then identity, zero, constant [MMOE] MoE++."""
    if e < spec.E_heavy:
        return "heavy", e
    e -= spec.E_heavy
    if e < spec.n_identity:
        return "identity", e
    e -= spec.n_identity
    if e < spec.n_zero:
        return "zero", e
    e -= spec.n_zero
    return "const", e


def expert_out(spec, W, layer, e, xr, h_store=None):
    """Output of routed expert e on token rows ``xr`` [MMOE] MoE++: heavy = MLP, identity = x,
    zero = 0, constant = its learned vector v_c (independent of x [R15])."""
    kind, j = expert_kind(spec, e)
    xr = np.asarray(xr, F64)
    if kind == "heavy":
        w3 = None if W.w3[layer] is None else W.w3[layer][j]
        return mlp(xr, W.w1[layer][j], w3, W.w2[layer][j], spec.act, h_store)
    if kind == "identity":
        return xr.copy()
    if kind == "zero":
        return np.zeros_like(xr)
    return np.broadcast_to(np.asarray(W.const_vec[layer][j], F64), xr.shape).copy()


def shared_out(spec, W, layer, x, h_store=None):
    """Sum of the always-on shared experts, weight 1 each [MMOE] (共享专家) [R19]."""
    x = np.asarray(x, F64)
    out = np.zeros_like(x)
    for i in range(spec.n_shared):
        w3 = None if W.s_w3[layer] is None else W.s_w3[layer][i]
        out += mlp(x, W.s_w1[layer][i], w3, W.s_w2[layer][i], spec.act, h_store)
    return out


# --------------------------------------------------------------------------------------------
# Routing decisions for a layer
# --------------------------------------------------------------------------------------------


def route(spec, L=None, P=None, input_probs=False, vote_dtype=F64):
    """All routing decisions of one layer call from logits L (or from given probabilities P
    when ``input_probs``). Returns a dict; see the keys below."""
    if input_probs:
        P = np.asarray(P, F64)
        keys = P
    else:
        L = np.asarray(L, F64)
        P = softmax(L)
        keys = L
    S, E = P.shape
    out = {"P": P, "pmax": P.max(axis=1)}
    if spec.mode == "tc":
        idx = tc_select(keys, spec.k)
        out.update(idx=idx, w=tc_weights(P, idx, spec.renorm))
    elif spec.mode == "des":
        votes, core = des_vote(keys, P, spec.vote_k, spec.m_core, vote_dtype=vote_dtype)
        idx, w = core_reroute(keys, P, core, spec.k, spec.renorm)
        out.update(idx=idx, w=w, votes=votes, core=core)
    elif spec.mode == "des_seq":
        # [DES] 2.3 core = union of each token's top-k_seq (k_seq = spec.vote_k, the local selection
        # count of 3.1); then, as in 4.3, every token re-activates its top-k inside that core
        core = des_seq_core(keys, spec.vote_k)
        idx, w = core_reroute(keys, P, core, spec.k, spec.renorm)
        out.update(idx=idx, w=w, votes=des_seq_counts(keys, spec.vote_k, E), core=core)
    elif spec.mode == "ec":
        C = ec_capacity(S, E, spec.capacity_factor)
        tokens, gates = ec_select(P, C)
        out.update(C=C, tokens=tokens, gates=gates)
    else:
        raise ValueError(spec.mode)
    if spec.mode in ("tc", "des", "des_seq"):
        out["reuse"] = (out["pmax"] < spec.reuse_tau) if spec.reuse_tau > 0 else np.zeros(S, bool)
    return out


# --------------------------------------------------------------------------------------------
# a9-a10: combine, and the whole layer
# --------------------------------------------------------------------------------------------


def routed_part(spec, W, layer, x, rt, h_store=None):
    """sum over a token's slots of gate weight * expert output (token / DES choice), or
    sum over the experts that picked the token of A_{s,i} * FFN_i(x_s) (expert choice;
    a token no expert picked gets 0 [R7]). [EC-DiT] 核心公式; [MMOE] MoE++."""
    x = np.asarray(x, F64)
    S = x.shape[0]
    out = np.zeros_like(x)
    if spec.mode == "ec":
        for i in range(rt["tokens"].shape[0]):
            t = rt["tokens"][i]
            out[t] += rt["gates"][i][:, None] * expert_out(spec, W, layer, i, x[t], h_store)
        return out
    idx, w = rt["idx"], rt["w"]
    live = ~rt["reuse"]
    for e in range(spec.E_routed):
        sel = (idx == e) & live[:, None]
        if not sel.any():
            continue
        s_ids, j_ids = np.nonzero(sel)
        out[s_ids] += w[s_ids, j_ids][:, None] * expert_out(spec, W, layer, e, x[s_ids], h_store)
    return out


def layer_forward(spec, W, x, layer=0, prev_logits=None, cache=None, residual=None, rt=None, h_store=None):
    """One MoE FFN layer call.

    y_s = residual_s + shared(x_s) + routed_s, with routed_s from ``routed_part`` for fresh tokens
    and routed_s = cache_s for tokens reusing their cached result ([DICE] 条件通信: a token whose
    top softmax score is below tau reuses the cached combine result [R22]). Fresh tokens' routed
    part is returned as the new cache.

    ``rt`` overrides the routing decisions (default: ``route`` on this call's logits).
    ``h_store`` is the storage precision of the experts' hidden activations (see ``mlp``).
    Returns dict(y, logits, rt, routed, new_cache).
    """
    x = np.asarray(x, F64)
    L = router_logits(x, W.w_router[layer], prev_logits)
    if rt is None:
        rt = route(spec, L=L)
    routed = routed_part(spec, W, layer, x, rt, h_store)
    if spec.mode != "ec" and rt["reuse"].any():
        if cache is None:
            raise ValueError("reuse needs a cache")
        routed = np.where(rt["reuse"][:, None], np.asarray(cache, F64), routed)
    y = routed + shared_out(spec, W, layer, x, h_store)
    if residual is not None:
        y = y + np.asarray(residual, F64)
    return {"y": y, "logits": L, "rt": rt, "routed": routed}


def bf16_round(a):
    """Round to the nearest bfloat16 (ties to even): the storage precision of a bf16 activation."""
    a32 = np.asarray(a, np.float64).astype(np.float32)
    u = a32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(F64)


def stack_forward(spec, W, x, act_bf16=True, gate_residual=True):
    """``spec.n_layers`` MoE layers on a residual stream h_{l+1} = h_l + y_l, each router adding
    the previous layer's logits ([MMOE] gate-residual routing) [R17, R18] unless ``gate_residual``
    is False (a DiT-MoE stack). The stream is stored in the layer precision (bf16 for a bf16
    workload) between layers. Returns per-layer results."""
    h = np.asarray(x, F64)
    prev = None
    outs = []
    for layer in range(spec.n_layers):
        r = layer_forward(spec, W, h, layer=layer, prev_logits=prev, residual=h)
        h_next = bf16_round(r["y"]) if act_bf16 else r["y"]
        r["h_in"] = h
        r["h_out"] = h_next
        outs.append(r)
        prev = r["logits"] if gate_residual else None
        h = h_next
    return outs


def dice_step_loop(spec, W, xs, tau, stride, reuse_layers, act_bf16=True, rt_hook=None, h_store=None):
    """DICE denoising-step loop on one device ([DICE] 关键设计).

    ``xs`` are the latent tokens of the successive steps t = 0, 1, ...; each step runs the
    ``spec.n_layers`` MoE layers on a residual stream (no gate residual: a DiT-MoE stack). Every
    layer keeps a cache of its routed output (交织并行: only the combine result is kept) across
    steps. At step t, layer l lets tokens whose top routing score is below ``tau`` reuse that
    cache (条件通信: low-score tokens take the stale result, high-score ones are recomputed)
    when l is in ``reuse_layers`` and t is not a multiple of ``stride``; otherwise every token is
    recomputed (the stride refresh, and 选择性同步: layers outside ``reuse_layers`` stay
    synchronous). Fresh tokens write their routed part into the cache, rounded to the storage
    precision (bf16 for a bf16 workload); reused tokens leave it alone. The stream between layers
    is stored in the same precision (``y``; ``y_exact`` is the layer output before that rounding).

    ``rt_hook(t, layer, h, L, rt, spec_l)`` may replace the routing decisions of a layer call (a
    test that accepts the other side's choice on near-ties). Returns, per step, a list of per-layer
    dicts: h_in, y, routed, cache (after the call), reuse (the mask used).
    """
    rnd = bf16_round if act_bf16 else (lambda a: np.asarray(a, F64))
    caches = [None] * spec.n_layers
    steps = []
    for t, x in enumerate(xs):
        h = np.asarray(x, F64)
        per = []
        for layer in range(spec.n_layers):
            fresh = (layer not in reuse_layers) or (t % stride == 0)
            sp = spec.replace(reuse_tau=0.0 if fresh else float(tau))
            L = router_logits(h, W.w_router[layer])
            rt = route(sp, L=L)
            if rt_hook is not None:
                rt = rt_hook(t, layer, h, L, rt, sp)
            r = layer_forward(sp, W, h, layer=layer, cache=caches[layer], residual=h, rt=rt, h_store=h_store)
            caches[layer] = np.where(rt["reuse"][:, None], caches[layer], rnd(r["routed"])) \
                if caches[layer] is not None else rnd(r["routed"])
            y = rnd(r["y"])
            per.append({"h_in": h, "y": y, "y_exact": r["y"], "routed": r["routed"], "cache": caches[layer],
                        "reuse": rt["reuse"]})
            h = y
        steps.append(per)
    return steps


# --------------------------------------------------------------------------------------------
# Attention-residual aggregation over block states (the block-level step next to the MoE layer)
# --------------------------------------------------------------------------------------------


def attnres_aggregate(states, query, eps=1e-6):
    """Depth aggregation of block states by a learned pseudo-query.

    [MMOE] 方法论, attention-residual aggregation: before a sub-layer, a learned pseudo-query
    aggregates the list of completed block states; the forward keeps those states and the current
    partial state as recurrent state. The page gives no formula. Reading [R33]: for every token s,
    each state v_j (the completed block states, then the current partial state) gets the score
    z_j = q . v_j / sqrt(mean(v_j^2) + eps) (the query against the state's RMS-normalised copy);
    the weights are the softmax of z over j, and the result is sum_j alpha_j v_j over the raw
    states.

    states: [n, S, d]; query: [d]. Returns (out [S, d], alpha [S, n]).
    """
    V = np.asarray(states, F64)
    q = np.asarray(query, F64)
    rms = np.sqrt(np.mean(V * V, axis=2) + eps)          # [n, S]
    z = (V @ q) / rms                                    # [n, S]
    alpha = softmax(z.T)                                 # [S, n], softmax over the states
    out = np.einsum("sj,jsd->sd", alpha, V)
    return out, alpha


# --------------------------------------------------------------------------------------------
# DES latency model (measurement model, not a kernel)
# --------------------------------------------------------------------------------------------


def des_block_latency(counts, a, b):
    """Block latency sum over active experts of f(c) = a*c + b (c > 0) [DES] 2.1 [R13]:
    a * (total routed pairs) + b * (number of distinct experts used)."""
    counts = np.asarray(counts)
    return float(a * counts.sum() + b * np.count_nonzero(counts))
