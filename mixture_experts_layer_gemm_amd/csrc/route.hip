// Router GEMM, softmax + token-choice top-k, DES-Vote core set, and the counting-sort dispatch.
//
// Router and affinity: "EC-DiT: Scaling Diffusion Transformers with Adaptive Expert-Choice
// Routing", 三 技术架构 / 核心公式 (scores x' W_r, A = softmax over experts; token choice takes each
// token's top-k experts). Gate residual: "MMOE: Modernizing Diffusion Transformers with Efficient
// Expert Design", 方法论 (the router adds the previous MoE layer's logits). DES-Vote: "Dynamic
// Expert Sharing: Decoupling Memory from Parallelism in Mixture-of-Experts Diffusion LLMs", 2.4
// (filter to top-K, vote with routing weights, elect M_core) and 4.3 (re-activate top-k inside the
// core). Low-score reuse mask: "DICE: Staleness-Centric Optimizations for Parallel Diffusion MoE
// Inference", 关键设计 / 条件通信.
//
// Selection order everywhere: key descending, expert index ascending on ties. Keys are the fp32
// logits (or given probabilities), compared exactly.
#include <float.h>
#include <limits.h>

#include <algorithm>

#include "common.hpp"
#include "internal.hpp"

// Wave-wide reductions of the device library (DPP based; every lane of the wave must be active).
extern "C" __device__ __attribute__((const)) float __ockl_wfred_max_f32(float);
extern "C" __device__ __attribute__((const)) float __ockl_wfred_add_f32(float);

namespace moe {

// =============================================================================================
// Router GEMM. A workgroup computes 16 * TT tokens x (16 * ET) experts (grid.y covers the rest).
// Its W waves split the K axis (wave w takes K steps w, w + W, ...), so each wave has only a few
// dependent load rounds; the partial sums are then added in LDS in wave order (a fixed order:
// results do not depend on timing). 16x16 MFMA tiles with operand P = W_r rows (16 experts) and
// operand Q = x rows (16 tokens): each lane ends with 4 consecutive experts of one token. x is read
// once from HBM per expert slice; W_r stays in cache, and each of its fragments serves the TT
// token tiles (with many experts its cache reads would otherwise outnumber those of x).
template <typename T, int ET, int TT>
__global__ __launch_bounds__(1024) void k_router(const T* __restrict__ x, const T* __restrict__ w,
                                                 const float* __restrict__ prev, float* __restrict__ logits,
                                                 int S, int d, int E) {
  constexpr int EPC = Elem<T>::kPer16B;
  constexpr int STEP = 4 * EPC;   // K elements per MFMA step
  constexpr int EW = ET * 16;     // experts per workgroup
  constexpr int TW = TT * 16;     // tokens per workgroup
  extern __shared__ float s_part[];   // [W][TW][EW]
  const int W = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int s0 = blockIdx.x * TW;
  const int e0 = blockIdx.y * EW;
  const T* xrow[TT];
#pragma unroll
  for (int p = 0; p < TT; ++p) xrow[p] = x + (size_t)min(s0 + p * 16 + r, S - 1) * d + g * EPC;
  const T* wrow[ET];
  bool wok[ET];
  floatx4_t acc[TT][ET];
#pragma unroll
  for (int q = 0; q < ET; ++q) {
    const int e = e0 + q * 16 + r;
    wok[q] = e < E;
    wrow[q] = w + (size_t)min(e, E - 1) * d + g * EPC;
#pragma unroll
    for (int p = 0; p < TT; ++p) acc[p][q] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  }
  const int nsteps = d / STEP;
  // a wave takes about four K steps: unrolled, all of their loads are in flight together
#pragma unroll 4
  for (int t = wave; t < nsteps; t += W) {
    const size_t kk = (size_t)t * STEP;
    uint4 xv[TT];
#pragma unroll
    for (int p = 0; p < TT; ++p) xv[p] = *reinterpret_cast<const uint4*>(xrow[p] + kk);
#pragma unroll
    for (int q = 0; q < ET; ++q) {
      uint4 wv = *reinterpret_cast<const uint4*>(wrow[q] + kk);
      if (!wok[q]) wv = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int p = 0; p < TT; ++p) acc[p][q] = mfma16(wv, xv[p], acc[p][q], T());
    }
  }
  float* mine = s_part + (size_t)wave * TW * EW;
#pragma unroll
  for (int p = 0; p < TT; ++p)
#pragma unroll
    for (int q = 0; q < ET; ++q)
#pragma unroll
      for (int t = 0; t < 4; ++t) mine[(p * 16 + r) * EW + q * 16 + 4 * g + t] = acc[p][q][t];
  __syncthreads();
  const int ne = min(EW, E - e0);
  for (int o = threadIdx.x; o < TW * ne; o += blockDim.x) {
    const int tr = o / ne, el = o - tr * ne;
    const int st = s0 + tr, e = e0 + el;
    if (st >= S) continue;
    float v = 0.f;
    for (int q = 0; q < W; ++q) v += s_part[((size_t)q * TW + tr) * EW + el];
    if (prev) v += prev[(size_t)st * E + e];
    logits[(size_t)st * E + e] = v;
  }
}

template <typename T, int ET, int TT>
static void router_t(const void* x, const void* w_router, const float* prev, float* logits, int S, int d, int E,
                     hipStream_t st) {
  constexpr int STEP = 4 * Elem<T>::kPer16B;
  const int nsteps = d / STEP;
  // about 4 K steps per wave; the partial sums of all waves fit in 64 KB of LDS
  const int W = std::max(1, std::min({16, nsteps / 4, 64 / (ET * TT)}));
  const size_t lds = (size_t)W * 16 * TT * ET * 16 * sizeof(float);
  const dim3 grid((S + 16 * TT - 1) / (16 * TT), (E + ET * 16 - 1) / (ET * 16));
  auto kfn = k_router<T, ET, TT>;
  MOE_LAUNCH("router", kfn, grid, 64 * W, lds, st, (const T*)x, (const T*)w_router, prev, logits, S, d, E);
}

template <typename T>
static void router_dt(const void* x, const void* w_router, const float* prev, float* logits, int S, int d, int E,
                      hipStream_t st) {
  // few tokens: one 16-expert tile per workgroup, for more workgroups; many tokens: all experts in
  // one workgroup, so x is read once, and 32 tokens per workgroup, so each W_r fragment read from
  // the cache serves two token tiles
  if (E <= 16 || S <= 1024) router_t<T, 1, 1>(x, w_router, prev, logits, S, d, E, st);
  else if (E <= 32) router_t<T, 2, 2>(x, w_router, prev, logits, S, d, E, st);
  else if (E <= 64) router_t<T, 4, 2>(x, w_router, prev, logits, S, d, E, st);
  else if (E <= 128) router_t<T, 8, 2>(x, w_router, prev, logits, S, d, E, st);
  else router_t<T, 16, 1>(x, w_router, prev, logits, S, d, E, st);   // two tiles would spill
}

hipError_t launch_router(int dtype, const void* x, const void* w_router, const float* prev, float* logits, int S,
                         int d, int E, hipStream_t st) {
  if (S <= 0) return hipSuccess;
  if (E < 1 || E > 256) return hipErrorInvalidValue;
  if (dtype == 0) router_dt<bf16_t>(x, w_router, prev, logits, S, d, E, st);
  else router_dt<float>(x, w_router, prev, logits, S, d, E, st);
  return hipGetLastError();
}

// =============================================================================================
// Group primitives: a token's experts are spread over LPT lanes (LPT a power of two <= 64), each
// lane holding V = ceil(E/LPT) of them (expert e lives in lane e % LPT, slot e / LPT).
template <int LPT>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (LPT == 64) return __ockl_wfred_max_f32(v);   // whole wave: DPP reduction
#pragma unroll
  for (int o = LPT / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
template <int LPT>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (LPT == 64) return __ockl_wfred_add_f32(v);   // whole wave: DPP reduction
#pragma unroll
  for (int o = LPT / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Arg-best over the group under (key desc, index asc).
template <int LPT>
__device__ __forceinline__ void group_argbest(float& key, int& idx) {
#pragma unroll
  for (int o = LPT / 2; o > 0; o >>= 1) {
    const float ok = __shfl_xor(key, o, 64);
    const int oi = __shfl_xor(idx, o, 64);
    if (ok > key || (ok == key && oi < idx)) { key = ok; idx = oi; }
  }
}

constexpr int kMaxV = 4;   // E_r <= 256

// Per-token probabilities from logits (softmax with the row max subtracted) or as given.
template <int LPT, int V>
__device__ __forceinline__ void token_probs(const float* keys_row, bool live, int E, int sub, int input_probs,
                                            float (&key)[V], float (&p)[V]) {
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int e = sub + v * LPT;
    key[v] = (live && e < E) ? keys_row[e] : -FLT_MAX;
  }
  if (input_probs) {
#pragma unroll
    for (int v = 0; v < V; ++v) p[v] = (sub + v * LPT < E) ? key[v] : 0.f;
    return;
  }
  float m = -FLT_MAX;
#pragma unroll
  for (int v = 0; v < V; ++v) m = fmaxf(m, key[v]);
  m = group_max<LPT>(m);
  float z[V], zs = 0.f;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    z[v] = (sub + v * LPT < E) ? expf(key[v] - m) : 0.f;
    zs += z[v];
  }
  zs = group_sum<LPT>(zs);
  const float inv = 1.0f / zs;
#pragma unroll
  for (int v = 0; v < V; ++v) p[v] = z[v] * inv;
}

constexpr int kMaxK = 16;

// Top-k of the token's keys among experts allowed by `allow` (bit v of the lane's mask).
// Returns the lane's chosen-set bits; when sel_e is given (k <= kMaxK) also writes the k chosen
// experts and their probabilities in key order.
template <int LPT, int V>
__device__ __forceinline__ unsigned token_topk(const float (&key)[V], const float (&p)[V], unsigned allow, int E,
                                               int sub, int lane, int k, int* sel_e, float* sel_p) {
  unsigned taken = 0;
  for (int j = 0; j < k; ++j) {
    float bk = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e = sub + v * LPT;
      const bool ok = e < E && ((allow >> v) & 1u) && !((taken >> v) & 1u);
      if (ok && (key[v] > bk || (key[v] == bk && e < bi))) { bk = key[v]; bi = e; }
    }
    group_argbest<LPT>(bk, bi);
    // owner lane of expert bi supplies its probability
    float mine = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (sub + v * LPT == bi) { mine = p[v]; taken |= 1u << v; }
    const int owner = (lane & ~(LPT - 1)) + (bi & (LPT - 1));
    const float pw = __shfl(mine, owner, 64);
    if (sel_e) {
      sel_p[j] = pw;
      sel_e[j] = bi;
    }
  }
  return taken;
}

template <int LPT, int V>
__global__ __launch_bounds__(256) void k_route_topk(RouteArgs a) {
  const int lane = threadIdx.x & 63;
  const int sub = lane & (LPT - 1);
  const int s = blockIdx.x * (256 / LPT) + threadIdx.x / LPT;
  const bool live = s < a.S;
  const int E = a.E_r;
  float key[V], p[V];
  token_probs<LPT, V>(a.keys + (size_t)min(s, a.S - 1) * E, live, E, sub, a.input_probs, key, p);
  if (live && a.probs) {
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (sub + v * LPT < E) a.probs[(size_t)s * E + sub + v * LPT] = p[v];
  }
  float pm = 0.f;
#pragma unroll
  for (int v = 0; v < V; ++v) pm = fmaxf(pm, p[v]);
  pm = group_max<LPT>(pm);
  int sel_e[kMaxK];
  float sel_p[kMaxK];
  token_topk<LPT, V>(key, p, ~0u, E, sub, lane, a.k, sel_e, sel_p);
  if (live && sub == 0) {
    float denom = 1.f;
    if (a.renorm) {
      float t = 0.f;
      for (int j = 0; j < a.k; ++j) t += sel_p[j];
      denom = t;
    }
    for (int j = 0; j < a.k; ++j) {
      a.topk_idx[(size_t)s * a.k + j] = sel_e[j];
      a.topk_w[(size_t)s * a.k + j] = a.renorm ? sel_p[j] / denom : sel_p[j];
    }
    if (a.reuse) a.reuse[s] = (a.tau > 0.f && pm < a.tau) ? 1 : 0;
  }
}

template <int LPT, int V>
static void route_topk_t(const RouteArgs& a, hipStream_t st) {
  auto kfn = k_route_topk<LPT, V>;
  MOE_LAUNCH("route_topk", kfn, (a.S + 256 / LPT - 1) / (256 / LPT), 256, 0, st, a);
}

// Lanes per token (LPT) and experts per lane (V) for E_r routed experts, the same in every routing
// kernel (the softmax sums a token's experts per lane, then over its lanes, so the mapping fixes the
// rounding): up to 32 experts, 8 lanes of up to 4 experts, so a wave routes 8 tokens at once with
// 3-level shuffle reductions (mmoe, 19 experts: 6.9 -> 4.2 us); beyond, a whole wave per token,
// whose top-k is a radix select over ballots (cross-lane shuffles go through the LDS crossbar, and
// k rounds of 4- or 5-level shuffle reductions cost more than the ballots at 64 experts).
hipError_t launch_route_topk(const RouteArgs& a, hipStream_t st) {
  const int E = a.E_r;
  if (E <= 8) route_topk_t<8, 1>(a, st);
  else if (E <= 32) route_topk_t<8, 4>(a, st);
  else if (E <= 64) route_topk_t<64, 1>(a, st);
  else if (E <= 128) route_topk_t<64, 2>(a, st);
  else route_topk_t<64, 4>(a, st);
  return hipGetLastError();
}

// =============================================================================================
// DES, one workgroup for the whole block of N tokens (N = a.S).
//  1. per token: probabilities, top-K filter T_n; filt[n][e] = p_{n,e} (DES-Vote) or 1 (DES-Seq)
//     for e in T_n, else 0;
//  2. per expert: v_e = sum over n ascending of filt[n][e] (fp32, sequential: adding the zeros
//     of unfiltered entries leaves the sum unchanged); for DES-Seq the number of tokens whose
//     top-K holds e (exact integers);
//  3. DES-Vote: core = the m_core experts first under (v desc, e asc); DES-Seq: core = the experts
//     with v_e > 0 (the union of the T_n); listed ascending (DES-Seq: then -1 up to E_r);
//  4. per token: top-min(k, |core|) by key among core experts; weights p or renormalised p; slots
//     from min(k, |core|) up to the stride (DES-Seq only) hold expert -1 and weight 0.
template <int LPT, int V>
__global__ __launch_bounds__(256) void k_route_des(RouteArgs a, float* __restrict__ filt) {
  __shared__ float s_votes[256];
  __shared__ int s_incore[256];
  __shared__ int s_ncore;
  const int lane = threadIdx.x & 63;
  const int sub = lane & (LPT - 1);
  const int tpb = 256 / LPT;
  const int E = a.E_r;
  // 1. filter
  for (int base = 0; base < a.S; base += tpb) {
    const int s = base + threadIdx.x / LPT;
    const bool live = s < a.S;
    float key[V], p[V];
    token_probs<LPT, V>(a.keys + (size_t)min(s, a.S - 1) * E, live, E, sub, a.input_probs, key, p);
    const unsigned taken = token_topk<LPT, V>(key, p, ~0u, E, sub, lane, a.vote_k, nullptr, nullptr);
    float pm = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) pm = fmaxf(pm, p[v]);
    pm = group_max<LPT>(pm);
    if (live) {
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int e = sub + v * LPT;
        if (e < E) {
          filt[(size_t)s * E + e] = ((taken >> v) & 1u) ? (a.seq ? 1.f : p[v]) : 0.f;
          if (a.probs) a.probs[(size_t)s * E + e] = p[v];
        }
      }
      if (sub == 0 && a.reuse) a.reuse[s] = (a.tau > 0.f && pm < a.tau) ? 1 : 0;
    }
  }
  __syncthreads();
  // 2. votes
  for (int e = threadIdx.x; e < E; e += 256) {
    float v = 0.f;
    for (int n = 0; n < a.S; ++n) v += filt[(size_t)n * E + e];
    s_votes[e] = v;
    a.votes[e] = v;
  }
  __syncthreads();
  // 3. elect
  for (int e = threadIdx.x; e < E; e += 256) {
    const float ve = s_votes[e];
    if (a.seq) {
      s_incore[e] = ve > 0.f ? 1 : 0;
      continue;
    }
    int rank = 0;
    for (int q = 0; q < E; ++q) {
      const float vq = s_votes[q];
      rank += (vq > ve || (vq == ve && q < e)) ? 1 : 0;
    }
    s_incore[e] = rank < a.m_core ? 1 : 0;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0;
    for (int e = 0; e < E; ++e) n += s_incore[e];
    s_ncore = n;
  }
  for (int e = threadIdx.x; e < E; e += 256) {
    if (s_incore[e]) {
      int pos = 0;
      for (int q = 0; q < e; ++q) pos += s_incore[q];
      a.core[pos] = e;
    }
  }
  __syncthreads();
  const int ncore = s_ncore;
  if (a.seq)
    for (int j = ncore + threadIdx.x; j < E; j += 256) a.core[j] = -1;
  // 4. re-route inside the core; DES-Seq keeps the stride a.k and pads the slots past min(k, |core|)
  const int kk = min(a.k, ncore);
  const int ks = a.seq ? a.k : kk;
  for (int base = 0; base < a.S; base += tpb) {
    const int s = base + threadIdx.x / LPT;
    const bool live = s < a.S;
    float key[V], p[V];
    token_probs<LPT, V>(a.keys + (size_t)min(s, a.S - 1) * E, live, E, sub, a.input_probs, key, p);
    unsigned allow = 0;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e = sub + v * LPT;
      if (e < E && s_incore[e]) allow |= 1u << v;
    }
    int sel_e[kMaxK];
    float sel_p[kMaxK];
    token_topk<LPT, V>(key, p, allow, E, sub, lane, kk, sel_e, sel_p);
    if (live && sub == 0) {
      float denom = 1.f;
      if (a.renorm) {
        float t = 0.f;
        for (int j = 0; j < kk; ++j) t += sel_p[j];
        denom = t;
      }
      for (int j = 0; j < kk; ++j) {
        a.topk_idx[(size_t)s * ks + j] = sel_e[j];
        a.topk_w[(size_t)s * ks + j] = a.renorm ? sel_p[j] / denom : sel_p[j];
      }
      for (int j = kk; j < ks; ++j) {
        a.topk_idx[(size_t)s * ks + j] = -1;
        a.topk_w[(size_t)s * ks + j] = 0.f;
      }
    }
  }
}

template <int LPT, int V>
static void route_des_t(const RouteArgs& a, float* ws_filt, hipStream_t st) {
  auto kfn = k_route_des<LPT, V>;
  MOE_LAUNCH("route_des", kfn, 1, 256, 0, st, a, ws_filt);
}

hipError_t launch_route_des(const RouteArgs& a, float* ws_filt, hipStream_t st) {
  const int E = a.E_r;   // the lane mapping of launch_route_topk
  if (E <= 8) route_des_t<8, 1>(a, ws_filt, st);
  else if (E <= 32) route_des_t<8, 4>(a, ws_filt, st);
  else if (E <= 64) route_des_t<64, 1>(a, ws_filt, st);
  else if (E <= 128) route_des_t<64, 2>(a, ws_filt, st);
  else route_des_t<64, 4>(a, ws_filt, st);
  return hipGetLastError();
}

// =============================================================================================
// Counting sort of the (token, slot) pairs onto heavy experts. Pair p = s*k + j. A pair is
// dispatched when its expert is heavy and its token does not reuse its cache. Rows are grouped by
// expert ascending; inside an expert, by p ascending (token, then slot). Three passes, no atomics
// on the output order: per-chunk histograms, a scan, and a ranked scatter.
constexpr int kPermThreads = 256;
constexpr int kPermRounds = 4;
constexpr int kPermChunk = kPermThreads * kPermRounds;
constexpr int kPermMaxE = 1024;

int permute_num_blocks(int S, int k) { return (int)(((int64_t)S * k + kPermChunk - 1) / kPermChunk); }

__device__ __forceinline__ bool pair_live(const PermuteArgs& a, int64_t p, int& e) {
  if (p >= (int64_t)a.S * a.k) { e = -1; return false; }
  e = a.topk_idx[p];
  const int s = (int)(p / a.k);
  return e >= 0 && e < a.E_heavy && !(a.reuse && a.reuse[s]);
}

__global__ __launch_bounds__(kPermThreads) void k_perm_count(PermuteArgs a) {
  __shared__ int cnt[kPermMaxE];
  for (int i = threadIdx.x; i < a.E_heavy; i += kPermThreads) cnt[i] = 0;
  __syncthreads();
  for (int r = 0; r < kPermRounds; ++r) {
    const int64_t p = (int64_t)blockIdx.x * kPermChunk + r * kPermThreads + threadIdx.x;
    int e;
    if (pair_live(a, p, e)) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < a.E_heavy; i += kPermThreads) a.blk_cnt[(size_t)blockIdx.x * a.E_heavy + i] = cnt[i];
}

// One workgroup: per-expert exclusive bases over chunks (in place), counts, offsets.
__global__ __launch_bounds__(kPermThreads) void k_perm_scan(PermuteArgs a, int nblk) {
  __shared__ int tot[kPermMaxE];
  for (int e = threadIdx.x; e < a.E_heavy; e += kPermThreads) {
    int run = 0;
    for (int b0 = 0; b0 < nblk; b0 += 8) {   // eight loads in flight, then the eight bases in order
      int c[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = b0 + j < nblk ? a.blk_cnt[(size_t)(b0 + j) * a.E_heavy + e] : 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (b0 + j < nblk) a.blk_cnt[(size_t)(b0 + j) * a.E_heavy + e] = run;
        run += c[j];
      }
    }
    tot[e] = run;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int e = 0; e < a.E_r; ++e) {
      const int c = e < a.E_heavy ? tot[e] : 0;
      a.offsets[e] = run;
      a.counts[e] = c;
      run += c;
    }
    a.offsets[a.E_r] = run;
    *a.n_rows = run;
  }
}

__global__ __launch_bounds__(kPermThreads) void k_perm_scatter(PermuteArgs a, int nbits) {
  __shared__ int wcnt[kPermThreads / 64][kPermMaxE];
  __shared__ int run[kPermMaxE];
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < a.E_heavy; i += kPermThreads) {
    run[i] = 0;
    for (int w = 0; w < kPermThreads / 64; ++w) wcnt[w][i] = 0;
  }
  __syncthreads();
  const int* bbase = a.blk_cnt + (size_t)blockIdx.x * a.E_heavy;
  for (int r = 0; r < kPermRounds; ++r) {
    const int64_t p = (int64_t)blockIdx.x * kPermChunk + r * kPermThreads + threadIdx.x;
    int e;
    const bool ok = pair_live(a, p, e);
    const int key = ok ? e : a.E_heavy;       // one extra class for pairs not dispatched
    uint64_t peers = ~0ull;
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (key >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const uint64_t lower = peers & lanemask_lt();
    const int rank = __popcll(lower);
    if (ok && lower == 0) wcnt[wave][e] = __popcll(peers);
    __syncthreads();
    if (ok) {
      int base = run[e];
      for (int w = 0; w < wave; ++w) base += wcnt[w][e];
      const int row = a.offsets[e] + bbase[e] + base + rank;
      a.row_token[row] = (int)(p / a.k);
      a.row_w[row] = a.topk_w[p];
      a.token_rows[p] = row;
    } else if (p < (int64_t)a.S * a.k) {
      a.token_rows[p] = -1;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < a.E_heavy; i += kPermThreads) {
      int add = 0;
      for (int w = 0; w < kPermThreads / 64; ++w) { add += wcnt[w][i]; wcnt[w][i] = 0; }
      run[i] += add;
    }
    __syncthreads();
  }
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t st) {
  const int nblk = permute_num_blocks(a.S, a.k);
  int nbits = 1;
  while ((1 << nbits) <= a.E_heavy) ++nbits;   // classes 0..E_heavy
  if (nblk > 0) {
    auto kfn = k_perm_count;
    MOE_LAUNCH("perm_count", kfn, nblk, kPermThreads, 0, st, a);
  }
  {
    auto kfn = k_perm_scan;
    MOE_LAUNCH("perm_scan", kfn, 1, kPermThreads, 0, st, a, nblk);
  }
  if (nblk > 0) {
    auto kfn = k_perm_scatter;
    MOE_LAUNCH("perm_scatter", kfn, nblk, kPermThreads, 0, st, a, nbits);
  }
  return hipGetLastError();
}

// =============================================================================================
// Small calls (a DES decode block, a tiny batch): the whole routing of token choice or DES-Vote and
// the counting-sort dispatch in one workgroup: one launch instead of four. The selections are the
// same as in k_route_topk / k_route_des (the same keys, order and tie rule; for a token spread over
// a whole wave, wave_topk finds them by a radix select over ballots instead of shuffles; the core
// and the re-route inside it rank experts by comparison counts); votes are summed in the same
// order, and rows come out in the same (expert, token, slot) order as the three permute kernels.
// Barriers here wait for LDS only (lds_barrier).
constexpr int kSmallThreads = 1024;
constexpr int kSmallWaves = kSmallThreads / 64;
constexpr int kSmallMaxSE = 8192;     // S * E_r: keys and probabilities kept in LDS
constexpr int kSmallMaxPairs = 4096;  // S * k
constexpr int kSmallMaxS = 2048;
static_assert(kSmallMaxPairs % kSmallThreads == 0, "whole rounds of pairs");

bool route_small_supported(int S, int E_r, int k) {
  return S >= 1 && S <= kSmallMaxS && (int64_t)S * E_r <= kSmallMaxSE && (int64_t)S * k <= kSmallMaxPairs &&
         E_r <= 256 && k <= kMaxK;
}

// Barrier for LDS data only: waits for this wave's LDS operations but not for its global stores,
// which a full __syncthreads would also wait for (their results are not read back here).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Integer with the order of the float (finite values).
__device__ __forceinline__ int float_order(float f) {
  const int b = __float_as_int(f);
  return b >= 0 ? b : b ^ 0x7fffffff;
}

// Top-k of one token whose experts span the whole wave (expert e in lane e % 64, slot e / 64),
// among experts allowed by `allow` (bit v of the lane's mask), ranked by (key descending, expert
// ascending): the same set and order as token_topk<64, V>. Instead of k rounds of a wave-wide
// maximum, a radix select finds the k-th largest key with one ballot per bit (MSB first, stopping
// as soon as exactly k keys reach the prefix); equal keys at the threshold go to the lowest
// experts. Returns the lane's chosen-set bits; when out_e is given, the j-th chosen expert
// (j = its rank among the chosen) and its probability go to out_e[j], out_p[j]. With fewer than k
// eligible experts, all of them are chosen and the remaining out entries are left alone.
template <int V>
__device__ __forceinline__ unsigned wave_topk(const float (&key)[V], const float (&p)[V], unsigned allow, int E,
                                              int lane, int k, int* out_e, float* out_p) {
  uint32_t u[V];   // keys as unsigned integers of the same order
  bool el[V];
  int n = 0;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    u[v] = (uint32_t)float_order(key[v]) ^ 0x80000000u;
    el[v] = lane + v * 64 < E && ((allow >> v) & 1u);
    n += __popcll(__ballot(el[v]));
  }
  const int kq = min(k, n);
  if (kq <= 0) return 0;
  uint32_t T = 0;
  bool exact = false;   // exactly kq keys are >= T
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = T | (1u << b);
    int c = 0;
#pragma unroll
    for (int v = 0; v < V; ++v) c += __popcll(__ballot(el[v] && u[v] >= cand));
    if (c >= kq) T = cand;
    if (c == kq) {
      exact = true;
      break;
    }
  }
  unsigned taken = 0;
  if (exact) {
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (el[v] && u[v] >= T) taken |= 1u << v;
  } else {
    // T is the kq-th largest key: take the larger ones and the lowest experts holding T
    int need = kq;
#pragma unroll
    for (int v = 0; v < V; ++v) need -= __popcll(__ballot(el[v] && u[v] > T));
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const uint64_t eq = __ballot(el[v] && u[v] == T);
      const int r = __popcll(eq & lanemask_lt());
      if (el[v] && (u[v] > T || (u[v] == T && r < need))) taken |= 1u << v;
      need -= min(need, __popcll(eq));
    }
  }
  if (out_e) {
    // rank of each chosen expert: the chosen ones that come before it
    int rank[V];
#pragma unroll
    for (int v = 0; v < V; ++v) rank[v] = 0;
#pragma unroll
    for (int vc = 0; vc < V; ++vc) {
      uint64_t m = __ballot((taken >> vc) & 1u);
      while (m) {
        const int c = __ffsll((unsigned long long)m) - 1;
        m &= m - 1;
        const uint32_t tc = (uint32_t)__builtin_amdgcn_readlane((int)u[vc], c);
        const int ec = vc * 64 + c;
#pragma unroll
        for (int v = 0; v < V; ++v) rank[v] += (tc > u[v] || (tc == u[v] && ec < v * 64 + lane)) ? 1 : 0;
      }
    }
#pragma unroll
    for (int v = 0; v < V; ++v)
      if ((taken >> v) & 1u) {
        out_e[rank[v]] = v * 64 + lane;
        out_p[rank[v]] = p[v];
      }
  }
  return taken;
}

template <int LPT, int V, bool DES>
__global__ __launch_bounds__(kSmallThreads) void k_route_small(RouteArgs a, PermuteArgs q) {
  __shared__ float s_key[kSmallMaxSE];
  __shared__ float s_p[kSmallMaxSE];
  __shared__ float s_aux[DES ? kSmallMaxSE : 1];   // DES: filtered probabilities (DES-Seq: 1 per selection)
  __shared__ float s_votes[256];
  __shared__ int s_rank[256], s_core[256];
  __shared__ int s_ncore;
  __shared__ int s_idx[kSmallMaxPairs];
  __shared__ float s_w[kSmallMaxPairs];
  __shared__ uint8_t s_reuse[kSmallMaxS];
  __shared__ int s_wcnt[kSmallWaves][256];
  __shared__ int s_cnt[256], s_off[257], s_run[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = a.S, E = a.E_r, SE = S * E;
  // slot stride of the routing arrays: k (token choice, DES-Seq) or min(k, m_core) (DES-Vote); the
  // number of slots a token fills (kk) is the same except for DES-Seq, where it is min(k, |core|)
  // and only known after the core is formed
  const int ks = q.k;
  int M = a.m_core;
  int kk = DES ? min(a.k, max(M, 1)) : a.k;

  for (int i = tid; i < SE; i += kSmallThreads) s_key[i] = a.keys[i];
  for (int e = tid; e < 256; e += kSmallThreads) {
    s_cnt[e] = 0;
    s_run[e] = 0;
    s_rank[e] = 0;
  }
  for (int i = tid; i < kSmallWaves * 256; i += kSmallThreads) (&s_wcnt[0][0])[i] = 0;
  lds_barrier();

  // probabilities: LPT lanes per token (max-subtracted softmax, or the given probabilities); then,
  // DES: the filter (the top-vote_k experts of each token keep their probability); token choice:
  // the top-kk selection
  constexpr int tpb = kSmallThreads / LPT;
  const int sub = lane & (LPT - 1);
  for (int base = 0; base < S; base += tpb) {
    const int s = base + tid / LPT;
    const bool live = s < S;
    float key[V], p[V];
    token_probs<LPT, V>(s_key + min(s, S - 1) * E, live, E, sub, a.input_probs, key, p);
    float pm = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) pm = fmaxf(pm, p[v]);
    pm = group_max<LPT>(pm);
    int sel_e[kMaxK];
    float sel_p[kMaxK];
    const int kq = DES ? a.vote_k : kk;   // DES: the filter; token choice: the selection
    unsigned taken;
    if constexpr (LPT == 64)
      taken = wave_topk<V>(key, p, ~0u, E, lane, kq, (DES || !live) ? nullptr : s_idx + s * ks, s_w + s * ks);
    else
      taken = token_topk<LPT, V>(key, p, ~0u, E, sub, lane, kq, DES ? nullptr : sel_e, sel_p);
    if (live) {
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int e = sub + v * LPT;
        if (e < E) {
          s_p[s * E + e] = p[v];
          if constexpr (DES) s_aux[s * E + e] = ((taken >> v) & 1u) ? (a.seq ? 1.f : p[v]) : 0.f;
        }
      }
      if (sub == 0) {
        s_reuse[s] = (a.tau > 0.f && pm < a.tau) ? 1 : 0;
        if constexpr (!DES && LPT < 64) {
          for (int j = 0; j < kk; ++j) {
            s_idx[s * ks + j] = sel_e[j];
            s_w[s * ks + j] = sel_p[j];
          }
        }
      }
    }
  }
  lds_barrier();
  if (a.probs)
    for (int i = tid; i < SE; i += kSmallThreads) a.probs[i] = s_p[i];
  if (a.reuse)
    for (int s = tid; s < S; s += kSmallThreads) a.reuse[s] = s_reuse[s];

  if constexpr (DES) {
    // votes, summed over tokens in ascending order
    for (int e = tid; e < E; e += kSmallThreads) {
      float v = 0.f;
#pragma unroll 8
      for (int n = 0; n < S; ++n) v += s_aux[n * E + e];
      s_votes[e] = v;
      a.votes[e] = v;
    }
    lds_barrier();
    // core: DES-Vote: the M experts of largest vote (ties to the lower index). Expert e's rank is
    // the number of experts before it in that order; the E x E comparisons are split over all
    // threads (each expert gets kSmallThreads / E of them, adding partial counts into s_rank, zero
    // from the start). DES-Seq: the experts some token selected (vote > 0). The core is then
    // listed ascending by a prefix count over the membership flags.
    if (!a.seq) {
      const int per = max(1, kSmallThreads / E);   // threads per expert
      const int span = (E + per - 1) / per;        // rivals per thread
      for (int t = tid; t < E * per; t += kSmallThreads) {
        const int e = t / per, part = t - e * per;
        const float ve = s_votes[e];
        const int o0 = part * span, o1 = min(E, o0 + span);
        int r = 0;
        for (int o = o0; o < o1; ++o) {
          const float vo = s_votes[o];
          r += (vo > ve || (vo == ve && o < e)) ? 1 : 0;
        }
        if (r) atomicAdd(&s_rank[e], r);
      }
    }
    lds_barrier();
    if (wave == 0) {
      int cbase = 0;
      for (int e0 = 0; e0 < E; e0 += 64) {
        const int e = e0 + lane;
        const bool in = e < E && (a.seq ? s_votes[e] > 0.f : s_rank[e] < M);
        const uint64_t m = __ballot(in);
        if (in) {
          const int pos = cbase + __popcll(m & lanemask_lt());
          s_core[pos] = e;
          a.core[pos] = e;
        }
        cbase += __popcll(m);
      }
      if (a.seq)
        for (int j = cbase + lane; j < E; j += 64) a.core[j] = -1;
      if (lane == 0) s_ncore = cbase;
    }
    lds_barrier();
    M = s_ncore;
    kk = min(a.k, M);
    // selection: the top kk of each token inside the core. The keys of each token's core experts
    // are first gathered as order-preserving integers (s_aux, free again); lane (token s, core slot
    // c) then ranks its expert among them (key descending; the core is ascending, so ties go to the
    // lower slot) and, if the rank is below kk, writes the slot of that rank.
    int* s_ord = reinterpret_cast<int*>(s_aux);   // [S][M]
    for (int t = tid; t < S * M; t += kSmallThreads) {
      const int s = t / M, c = t - s * M;
      s_ord[t] = float_order(s_key[s * E + s_core[c]]);
    }
    lds_barrier();
    for (int t = tid; t < S * M; t += kSmallThreads) {
      const int s = t / M, c = t - s * M;
      const int* os = s_ord + s * M;
      const int oc = os[c];
      int r = 0;
#pragma unroll 8
      for (int c2 = 0; c2 < M; ++c2) {
        const int o2 = os[c2];
        r += (o2 > oc || (o2 == oc && c2 < c)) ? 1 : 0;
      }
      if (r < kk) {
        const int ec = s_core[c];
        s_idx[s * ks + r] = ec;
        s_w[s * ks + r] = s_p[s * E + ec];
      }
    }
    lds_barrier();
  }
  // weights: p, or p over the sum of the chosen p in slot order; DES-Seq slots past min(k, |core|)
  // hold expert -1 and weight 0. One thread per (token, slot) pair, each adding its token's chosen
  // p itself in slot order; every pair is read before any is rewritten (a token's slots may span
  // two rounds of the workgroup).
  {
    constexpr int RMAX = kSmallMaxPairs / kSmallThreads;
    const int P = S * ks;
    float wv[RMAX];
    int ev[RMAX];
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      const int p = r * kSmallThreads + tid;
      wv[r] = 0.f;
      ev[r] = -1;
      if (p < P) {
        const int s = p / ks, j = p - s * ks;
        if (j < kk) {
          ev[r] = s_idx[p];
          wv[r] = s_w[p];
          if (a.renorm) {
            float t = 0.f;
            for (int jj = 0; jj < kk; ++jj) t += s_w[s * ks + jj];
            wv[r] = wv[r] / t;
          }
        }
      }
    }
    lds_barrier();
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      const int p = r * kSmallThreads + tid;
      if (p < P) {
        s_idx[p] = ev[r];
        s_w[p] = wv[r];
        a.topk_idx[p] = ev[r];
        a.topk_w[p] = wv[r];
      }
    }
  }
  lds_barrier();

  // dispatch: pair p = s * ks + j goes to a row when its expert is heavy and s does not reuse
  const int P = S * ks;
  const bool use_reuse = q.reuse != nullptr;
  auto live_pair = [&](int p, int& e) -> bool {
    if (p >= P) {
      e = -1;
      return false;
    }
    e = s_idx[p];
    return e >= 0 && e < q.E_heavy && !(use_reuse && s_reuse[p / ks]);
  };
  for (int p = tid; p < P; p += kSmallThreads) {
    int e;
    if (live_pair(p, e)) atomicAdd(&s_cnt[e], 1);
  }
  lds_barrier();
  // offsets: exclusive scan of the counts over experts (light experts count 0), one wave
  if (wave == 0) {
    int base = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      const int c = (e < E && e < q.E_heavy) ? s_cnt[e] : 0;
      int incl = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      if (e < E) {
        s_off[e] = base + incl - c;
        q.offsets[e] = base + incl - c;
        q.counts[e] = c;
      }
      base += __shfl(incl, 63, 64);
    }
    if (lane == 0) {
      s_off[E] = base;
      q.offsets[E] = base;
      *q.n_rows = base;
    }
  }
  int nbits = 1;
  while ((1 << nbits) <= q.E_heavy) ++nbits;
  lds_barrier();
  for (int r0 = 0; r0 < P; r0 += kSmallThreads) {
    const int p = r0 + tid;
    int e;
    const bool ok = live_pair(p, e);
    const int key = ok ? e : q.E_heavy;
    uint64_t peers = ~0ull;
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (key >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const uint64_t lower = peers & lanemask_lt();
    if (ok && lower == 0) s_wcnt[wave][e] = __popcll(peers);
    lds_barrier();
    if (ok) {
      int base = s_off[e] + s_run[e];
      for (int o = 0; o < wave; ++o) base += s_wcnt[o][e];
      const int row = base + __popcll(lower);
      q.row_token[row] = p / ks;
      q.row_w[row] = s_w[p];
      q.token_rows[p] = row;
    } else if (p < P) {
      q.token_rows[p] = -1;
    }
    lds_barrier();
    for (int i = tid; i < q.E_heavy; i += kSmallThreads) {
      int add = 0;
      for (int o = 0; o < kSmallWaves; ++o) {
        add += s_wcnt[o][i];
        s_wcnt[o][i] = 0;
      }
      s_run[i] += add;
    }
    lds_barrier();
  }
}

template <int LPT, int V>
static void route_small_t(const RouteArgs& a, const PermuteArgs& q, bool des, hipStream_t st) {
  if (des) {
    auto kfn = k_route_small<LPT, V, true>;
    MOE_LAUNCH("route_small", kfn, 1, kSmallThreads, 0, st, a, q);
  } else {
    auto kfn = k_route_small<LPT, V, false>;
    MOE_LAUNCH("route_small", kfn, 1, kSmallThreads, 0, st, a, q);
  }
}

hipError_t launch_route_small(const RouteArgs& a, const PermuteArgs& q, bool des, hipStream_t st) {
  const int kk = des ? (a.seq ? a.k : std::min(a.k, a.m_core)) : a.k;
  if (!route_small_supported(a.S, a.E_r, kk) || q.E_heavy > 256 || q.k != kk) return hipErrorInvalidValue;
  const int E = a.E_r;   // the lane mapping of launch_route_topk
  if (E <= 8) route_small_t<8, 1>(a, q, des, st);
  else if (E <= 32) route_small_t<8, 4>(a, q, des, st);
  else if (E <= 64) route_small_t<64, 1>(a, q, des, st);
  else if (E <= 128) route_small_t<64, 2>(a, q, des, st);
  else route_small_t<64, 4>(a, q, des, st);
  return hipGetLastError();
}

// =============================================================================================
__global__ void k_fill_u32(uint32_t* __restrict__ p, uint32_t v, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t v, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 4096);
  auto kfn = k_fill_u32;
  MOE_LAUNCH("fill_u32", kfn, blocks, 256, 0, st, p, v, n);
  return hipGetLastError();
}

}  // namespace moe
