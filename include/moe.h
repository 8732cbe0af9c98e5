/*
 * moe.h - C ABI of the MI355X (gfx950) sparse Mixture-of-Experts FFN layer forward.
 *
 * The layer (one call, S tokens of width d):
 *   logits L = x . W_r^T (+ L_prev)                     router, gate residual
 *   p      = softmax(L) over the E_r routed experts      affinity
 *   routing: token choice (each token takes its top-k experts), expert choice (each expert takes
 *            its top-C tokens, C = floor(f_c * S / E_r)), DES-Vote (a core set of M_core experts
 *            elected by summed routing weights; tokens re-route top-k inside it) or DES-Seq (the core
 *            is the union of every token's top-k_seq; tokens re-route top-k inside it)
 *   dispatch: tokens grouped by expert (stable counting sort)
 *   experts:  heavy = GELU or SwiGLU MLP (grouped bf16/fp32 MFMA GEMMs); identity, zero and
 *             constant experts computed inline; shared experts on every token with weight 1
 *   combine:  y_s = residual_s + shared_s + sum_j w_{s,j} * out_{e_{s,j}}(x_s)
 *             (tokens whose top probability is below tau reuse their cached routed part).
 *
 * Sources (web pages; cited by title and section):
 *   "EC-DiT: Scaling Diffusion Transformers with Adaptive Expert-Choice Routing", part 三 技术架构,
 *     核心公式: token choice vs expert choice; affinity A = softmax(x' W_r); 容量因子 (capacity
 *     f_c * S / E with f_c = 2.0).
 *   "Dynamic Expert Sharing: Decoupling Memory from Parallelism in Mixture-of-Experts Diffusion
 *     LLMs": 2.1 latency model f(c) = a*c + b; 2.3 DES-Seq; 2.4 DES-Vote; 3.1 M_core = beta * M and
 *     the local selection count of DES-Seq; 4.3 top-8 re-activated inside the core set.
 *   "MMOE: Modernizing Diffusion Transformers with Efficient Expert Design", 方法论: MoE++ layer
 *     (heavy MLP experts, identity / zero / constant zero-computation experts), gate-residual
 *     routing, shared expert.
 *   "DICE: Staleness-Centric Optimizations for Parallel Diffusion MoE Inference", 关键设计,
 *     条件通信: low-score tokens reuse cached combine results.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked [host]. Arrays are dense row-major.
 *   - Weights use the linear-layer layout [out, in]: y = x . W^T.
 *   - Element type of x, weights, x_perm, residual, cache and y is desc->dtype (bf16 or fp32).
 *     Logits, probabilities, routing weights, y_perm and y_shared are fp32; indices are int32.
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL = the null stream). No call
 *     allocates or frees device memory, frees caller memory, or synchronises the host (unless
 *     MOE_F_SYNC_DEBUG is set). The caller owns every buffer; scratch memory comes from `ws`
 *     (at least moe_workspace_bytes(desc) bytes, 256-byte aligned).
 *   - Arguments are validated on the host before any launch. A call returns MOE_OK (0) or a
 *     negative moe_status and launches nothing on an argument error. No C++ exception crosses
 *     the ABI. Calls that overlap on one stream are ordered; calls on different streams that
 *     share a workspace race.
 *   - Token rows (x, x_perm, residual, cache, y), expert outputs (y_perm, y_shared), weights and
 *     constant vectors are read and written 16 bytes at a time: each must start on a 16-byte
 *     boundary, or the call returns MOE_EINVAL.
 *   - An empty batch (desc->S == 0) is valid. It reads no token array, which may then be NULL, and
 *     needs no workspace. moe_route and moe_layer_forward then only set the routing's
 *     per-expert counts and offsets, n_rows and capacity to 0, DES votes to 0 and DES core slots
 *     to -1 (moe_route needs `routing` for that; moe_layer_forward takes NULL). The other calls
 *     do nothing.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,        /* null pointer, inconsistent sizes, k/vote_k/m_core out of range, C rounds to 0 */
  MOE_EUNSUPPORTED = -2,  /* dtype / activation / shape alignment this library does not implement;
                             e.g. the tiled expert GEMMs (used when experts get many rows) need
                             d and d_ff to be multiples of 64 */
  MOE_EWORKSPACE = -3,    /* ws_bytes < moe_workspace_bytes(desc) or ws not 256-byte aligned */
  MOE_EHIP = -4,          /* a HIP launch or runtime error (the call's work may be partly enqueued) */
  MOE_ESCRATCH = -5       /* moe_layer_forward_noalloc: the call needs more scratch than its static
                             buffer holds (moe_workspace_bytes(desc) > MOE_NOALLOC_SCRATCH_BYTES) */
} moe_status;

typedef enum { MOE_BF16 = 0, MOE_F32 = 1 } moe_dtype;
typedef enum { MOE_ACT_GELU = 0 /* erf form */, MOE_ACT_GELU_TANH = 1, MOE_ACT_SWIGLU = 2 } moe_act;
typedef enum { MOE_TOKEN_CHOICE = 0, MOE_EXPERT_CHOICE = 1, MOE_DES_VOTE = 2, MOE_DES_SEQ = 3 } moe_mode;

/* desc->flags */
#define MOE_F_INPUT_PROBS   0x1u  /* moe_route: `logits` holds probabilities p (rows sum to 1);
                                     selection, votes and weights use them as given */
#define MOE_F_SYNC_DEBUG    0x4u  /* synchronise the stream after every launch and report errors */
#define MOE_F_FORCE_TILED   0x8u  /* heavy experts on the tiled grouped GEMM (default: chosen from the
                                     expected rows per expert) */
#define MOE_F_FORCE_STREAM  0x10u /* heavy experts on the weight-streaming kernel (few rows per expert) */
#define MOE_F_ROUTE_MULTI   0x20u /* token choice / DES: always route and dispatch with the multi-launch
                                     kernels (default: a small call, S * E_r <= 16384 and S * k <= 4096,
                                     runs both in one workgroup; the results are identical) */

/* Layer description [host]. Routed expert ids: [0, E_heavy) heavy, then n_identity identity,
 * n_zero zero and n_const constant experts; E_r = E_heavy + n_identity + n_zero + n_const. */
typedef struct {
  int32_t S, d, d_ff;           /* tokens (0: an empty batch), model dim, expert hidden dim      */
  int32_t E_heavy, n_identity, n_zero, n_const;
  int32_t n_shared;             /* always-on experts, weight 1                                     */
  int32_t dtype;                /* moe_dtype                                                       */
  int32_t act;                  /* moe_act                                                         */
  int32_t mode;                 /* moe_mode                                                        */
  int32_t k;                    /* token choice / DES re-route top-k (1 <= k <= E_r)               */
  int32_t renorm;               /* 1: chosen weights divided by their sum                          */
  float capacity_factor;        /* expert choice: C = min(S, floor(f_c * S / E_r)), C >= 1         */
  int32_t vote_k, m_core;       /* DES-Vote: filter top-K per token, core-set size;
                                   DES-Seq: vote_k = local selection count k_seq, m_core unused     */
  float reuse_tau;              /* token choice / DES: reuse cache where max_e p < tau; 0 = off
                                   (DICE, 关键设计 / 条件通信)                                        */
  uint32_t flags;               /* MOE_F_*                                                         */
} moe_desc;

/* Routing results, caller-allocated device arrays. k_eff = k (token choice, DES-Seq) or min(k, m_core)
 * (DES-Vote); R_max = S*k_eff (token choice, DES) or E_r*C (expert choice; S*E_r always suffices).
 * Pointers a mode does not use may be NULL. Limits: E_r <= 256, k_eff <= 16.
 * DES-Seq: the core's size |core| is only known on the device; a token re-routes to
 * k' = min(k, |core|) experts and its slots k'..k-1 hold expert -1 with weight 0 and row -1. */
typedef struct {
  int32_t *topk_idx;            /* [S,k_eff] chosen expert per slot, slots in descending key order  */
  float *topk_w;                /* [S,k_eff] gate weight per slot                                    */
  float *probs;                 /* [S,E_r] softmax probabilities (output; input with INPUT_PROBS); nullable */
  int32_t *counts;              /* [E_r] dispatched rows per expert (0 for zero-computation experts) */
  int32_t *offsets;             /* [E_r+1] exclusive prefix sum of counts                            */
  int32_t *row_token;           /* [R_max] token of each dispatched row; rows grouped by expert
                                   ascending, then token ascending, then slot                        */
  float *row_w;                 /* [R_max] gate weight of each dispatched row                        */
  int32_t *token_rows;          /* [S,k_eff] row of each slot; -1 for zero-computation experts and reused tokens */
  int32_t *token_off;           /* expert choice: [S+1] CSR offsets of each token's rows              */
  int32_t *token_list;          /* expert choice: [E_r*C] rows of each token, ascending expert        */
  int32_t *core;                /* DES-Vote: [m_core] core experts, ascending; DES-Seq: [E_r], the
                                   union ascending, then -1 up to E_r                                 */
  float *votes;                 /* DES-Vote: [E_r] summed routing weights (fp32, tokens in ascending
                                   order); DES-Seq: [E_r] tokens whose top-k_seq holds the expert      */
  uint8_t *reuse;               /* [S] 1 = token reuses its cache (nullable when reuse_tau == 0)      */
  int32_t *n_rows;              /* [1] total dispatched heavy rows R (<= R_max)                       */
  int32_t *capacity;            /* expert choice: [1] the C used                                      */
} moe_routing;

/* Weights (device, dtype of the layer). */
typedef struct {
  const void *w_router;         /* [E_r, d]                                                          */
  const void *w1;               /* [E_heavy, d_ff, d]  up projection (SwiGLU: linear "up" branch)    */
  const void *w3;               /* [E_heavy, d_ff, d]  SwiGLU gate branch (NULL for GELU)            */
  const void *w2;               /* [E_heavy, d, d_ff]  down projection                               */
  const void *s_w1, *s_w3, *s_w2; /* shared experts, same shapes with n_shared in place of E_heavy  */
  const void *const_vec;        /* [n_const, d] constant-expert vectors                              */
} moe_weights;

/* Bytes of scratch every entry point below may use for `desc` (>= 256, a multiple of 256). Returns 0
 * if `desc` is invalid. */
size_t moe_workspace_bytes(const moe_desc *desc /* [host] */);

/* Routing from logits [S,E_r] (or probabilities with MOE_F_INPUT_PROBS): softmax, then
 *   token choice: top-k per token by (logit desc, expert asc); weights p or p / sum p (renorm)
 *             (EC-DiT, 三 技术架构 / 核心公式, token choice);
 *   expert choice: each expert takes C tokens by (p desc, token asc); gate = p
 *             (EC-DiT, 核心公式, expert choice; 容量因子: C = floor(f_c * S / E_r), clipped to S);
 *   DES-Vote: top-vote_k filter per token, votes v_e = sum_n [e in T_n] p_{n,e}, core = top m_core
 *             by (v desc, e asc), re-route top-min(k, m_core) inside the core
 *             (Dynamic Expert Sharing, 2.4; 3.1 M_core = beta * M; 4.3 re-activation inside the core);
 *   DES-Seq:  core = union over tokens of each token's top-vote_k, re-route top-min(k, |core|) inside it
 *             (Dynamic Expert Sharing, 2.3; 3.1 local selection count; 4.3);
 * then the dispatch order (counts, offsets, row_token, row_w, token_rows, token CSR), and the
 * reuse mask when reuse_tau > 0 (DICE, 关键设计 / 条件通信: tokens whose top score is below tau). */
moe_status moe_route(const moe_desc *desc, const float *logits, moe_routing *routing /* [host] struct */,
                     void *ws, size_t ws_bytes, void *stream);

/* Dispatch: x_perm[r, :] = x[row_token[r], :] for r < n_rows. x [S,d], x_perm [R_max,d]; rows >= n_rows
 * untouched. The tokens grouped by expert for the experts' batched MLPs: EC-DiT, 核心公式 (each expert
 * processes the tokens routed to it); on one device DICE's all-to-all dispatch (关键设计) is this
 * local permute. MOE_EINVAL for null pointers. */
moe_status moe_dispatch(const moe_desc *desc, const void *x, const moe_routing *routing, void *x_perm,
                        void *stream);

/* Heavy and shared experts (MMOE MoE++ heavy experts and 共享专家).
 * y_perm[r] (fp32 [R_max,d]) = MLP_{e(r)}(row r) for r < n_rows, where row r is x_perm[r] when
 * x_perm is non-NULL, else x[row_token[r]] gathered inside the GEMM (no x_perm traffic).
 * y_shared (fp32 [S,d]; required iff n_shared > 0) = sum over shared experts of MLP_i(x).
 * GELU: W2 . gelu(W1 . x); SwiGLU: W2 . (silu(W3 . x) * (W1 . x)). The hidden activation is stored
 * in dtype between the two GEMMs; accumulation is fp32. */
moe_status moe_expert_ffn(const moe_desc *desc, const void *x, const void *x_perm, const moe_routing *routing,
                          const moe_weights *weights, float *y_perm, float *y_shared, void *ws, size_t ws_bytes,
                          void *stream);

/* Combine: y [S,d] = residual + y_shared + routed, routed_s = sum_j topk_w[s,j] * out_j in slot order,
 * where out_j = y_perm[token_rows[s,j]] (heavy), x_s (identity), 0 (zero), const_vec[c] (constant),
 * nothing for an empty DES-Seq slot (expert -1) (MMOE, 方法论: MoE++ zero-computation experts and the
 * shared expert); expert choice: sum over token_list rows (ascending expert) of row_w * y_perm (EC-DiT,
 * 核心公式: a token's output sums A_{s,i} FFN_i over the experts that chose it, 0 if none). fp32
 * accumulation, one rounding to dtype. With reuse: reused tokens take routed_s = cache_s, fresh
 * tokens write cache_s = routed_s rounded to dtype (DICE, 关键设计: 条件通信 reuses stale results for
 * low-score tokens; 交织并行 keeps only the combine results). residual, y_shared, cache are nullable.
 * MOE_EINVAL for a missing pointer the description needs (y_perm with heavy experts, y_shared with
 * shared experts, const_vec with constant experts, cache and reuse with reuse_tau > 0). */
moe_status moe_combine(const moe_desc *desc, const void *x, const moe_routing *routing, const float *y_perm,
                       const float *y_shared, const void *const_vec, void *cache, const void *residual, void *y,
                       void *stream);

/* The whole layer: router GEMM L = x . W_r^T (EC-DiT, 核心公式: scores x' W_r) plus prev_logits when
 * given (MMOE, 方法论: gate-residual routing adds the previous layer's logits), moe_route, the expert
 * GEMMs (gather fused), moe_combine. logits_out [S,E_r] fp32 (nullable) receives the final logits, the
 * next layer's prev_logits. routing may be NULL (then the workspace holds it). cache is required when
 * reuse_tau > 0 (DICE 条件通信). No device-to-host synchronisation. MOE_EINVAL with MOE_F_INPUT_PROBS
 * (probabilities are an input of moe_route only). */
moe_status moe_layer_forward(const moe_desc *desc, const void *x, const moe_weights *weights,
                             const float *prev_logits, float *logits_out, moe_routing *routing, void *cache,
                             const void *residual, void *y, void *ws, size_t ws_bytes, void *stream);

/* moe_layer_forward for callers that cannot allocate device memory (code under stream capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same layer, the same kernels and results, with
 * no workspace argument. Its scratch memory is a static device array of MOE_NOALLOC_SCRATCH_BYTES
 * (64 MiB) inside the library, one per GPU, held until the process ends; the call allocates nothing.
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU (different streams, or
 * threads) race and must be serialised by the caller. Runs on the current device, whose array
 * address is looked up on the first call there. MOE_ESCRATCH when moe_workspace_bytes(desc) exceeds
 * MOE_NOALLOC_SCRATCH_BYTES (e.g. beyond about 1300 tokens of the DiT-MoE-XL-shaped layer; decode
 * blocks need about 2.5 MiB); otherwise the statuses of moe_layer_forward. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_layer_forward_noalloc(const moe_desc *desc, const void *x, const moe_weights *weights,
                                     const float *prev_logits, float *logits_out, moe_routing *routing, void *cache,
                                     const void *residual, void *y, void *stream);

/* Attention-residual aggregation ("MMOE: Modernizing Diffusion Transformers with Efficient Expert
 * Design", 方法论: before a sub-layer a learned pseudo-query aggregates the completed block states,
 * which the forward keeps with the current partial state). The page gives no formula; per token s
 * this computes, over the n states v_j (states[j], each [S,d] of dtype, row-major; the completed
 * states, then the partial one):
 *   z_j = query . v_j[s] / sqrt(mean(v_j[s]^2) + eps),  out[s] = sum_j softmax_j(z)_j * v_j[s].
 * states: [host] array of n device pointers (1 <= n <= 64); query [d] and out [S,d] are device
 * buffers of dtype (MOE_BF16 or MOE_F32); every buffer is 16-byte aligned; out may not alias a
 * state. fp32 arithmetic, one rounding to dtype. S = 0 does nothing. MOE_EINVAL for null or
 * misaligned pointers, n < 1, d <= 0, S < 0 or a negative or non-finite eps; MOE_EUNSUPPORTED for n > 64, d not a multiple of 8 (bf16) / 4 (fp32), or d > 4096. */
moe_status moe_attnres_aggregate(int32_t dtype, int32_t S, int32_t d, int32_t n, const void *const *states,
                                 const void *query, float eps, void *out, void *stream);

/* Static description of a status code. Thread-safe. */
const char *moe_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
