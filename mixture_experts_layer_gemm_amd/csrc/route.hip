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
// With nsplit > 1 (grid.z = nsplit) workgroup z takes the z-th of nsplit equal K ranges and writes
// its sums to out + z * S * E, without prev; the splits are added later in split order.
template <typename T, int ET, int TT>
__global__ __launch_bounds__(1024) void k_router(const T* __restrict__ x, const T* __restrict__ w,
                                                 const float* __restrict__ prev, float* __restrict__ logits,
                                                 int S, int d, int E, int nsplit) {
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
  const int ne = min(EW, E - e0);
  // the previous layer's logits for this thread's first PF outputs, loaded before the K loop so
  // that the epilogue does not wait a memory round trip for them (the rest are read there)
  constexpr int PF = 2;
  const bool add_prev = prev && nsplit == 1;
  float pre[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    const int o = threadIdx.x + i * blockDim.x;
    const int tr = o / ne, st = s0 + tr;
    pre[i] = add_prev && o < TW * ne && st < S ? prev[(size_t)st * E + e0 + (o - tr * ne)] : 0.f;
  }
  const int nsteps = d / STEP / nsplit;                    // K steps of this workgroup
  const size_t kz = (size_t)blockIdx.z * nsteps * STEP;   // start of its K range
  const T* xrow[TT];
#pragma unroll
  for (int p = 0; p < TT; ++p) xrow[p] = x + (size_t)min(s0 + p * 16 + r, S - 1) * d + kz + g * EPC;
  const T* wrow[ET];
  bool wok[ET];
  floatx4_t acc[TT][ET];
#pragma unroll
  for (int q = 0; q < ET; ++q) {
    const int e = e0 + q * 16 + r;
    wok[q] = e < E;
    wrow[q] = w + (size_t)min(e, E - 1) * d + kz + g * EPC;
#pragma unroll
    for (int p = 0; p < TT; ++p) acc[p][q] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  }
  // a wave takes about four K steps. It loads U of them before it multiplies any, so their loads
  // are in flight together (steps past the end load the last one again and are not multiplied):
  // 4 in the one-tile workgroup, 2 with 2 x 2 tiles; the widest tiles keep one step at a time, for
  // their registers. The accumulation order is step order whatever U is.
  constexpr int U = ET * TT == 1 ? 4 : (ET * TT <= 4 ? 2 : 1);
  if constexpr (U == 1) {
    // one step at a time, each weight fragment used as it arrives
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
  } else {
    for (int t0 = wave; t0 < nsteps; t0 += U * W) {
      uint4 xv[U][TT], wv[U][ET];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const size_t kk = (size_t)min(t0 + u * W, nsteps - 1) * STEP;
#pragma unroll
        for (int p = 0; p < TT; ++p) xv[u][p] = *reinterpret_cast<const uint4*>(xrow[p] + kk);
#pragma unroll
        for (int q = 0; q < ET; ++q) wv[u][q] = *reinterpret_cast<const uint4*>(wrow[q] + kk);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (t0 + u * W >= nsteps) break;   // uniform over the wave
#pragma unroll
        for (int q = 0; q < ET; ++q) {
          const uint4 w = wok[q] ? wv[u][q] : make_uint4(0, 0, 0, 0);
#pragma unroll
          for (int p = 0; p < TT; ++p) acc[p][q] = mfma16(w, xv[u][p], acc[p][q], T());
        }
      }
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
  float* out = logits + (size_t)blockIdx.z * S * E;
  auto finish = [&](int o, float pv, bool have) {
    const int tr = o / ne, el = o - tr * ne;
    const int st = s0 + tr, e = e0 + el;
    if (st >= S) return;
    float v = 0.f;
    for (int q = 0; q < W; ++q) v += s_part[((size_t)q * TW + tr) * EW + el];
    if (add_prev) v += have ? pv : prev[(size_t)st * E + e];
    out[(size_t)st * E + e] = v;
  };
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    const int o = threadIdx.x + i * blockDim.x;
    if (o < TW * ne) finish(o, pre[i], true);
  }
  for (int o = threadIdx.x + PF * blockDim.x; o < TW * ne; o += blockDim.x) finish(o, 0.f, false);
}

// logits = (sum over the K splits, in split order) + prev
__global__ void k_router_sum(const float* __restrict__ part, int nsplit, const float* __restrict__ prev,
                             float* __restrict__ logits, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float v = 0.f;
  for (int z = 0; z < nsplit; ++z) v += part[(size_t)z * n + i];
  if (prev) v += prev[i];
  logits[i] = v;
}

template <typename T, int ET, int TT>
static void router_t(const void* x, const void* w_router, const float* prev, float* out, int S, int d, int E,
                     int nsplit, hipStream_t st) {
  constexpr int STEP = 4 * Elem<T>::kPer16B;
  const int nsteps = d / STEP / nsplit;
  // about 4 K steps per wave; the partial sums of all waves fit in 64 KB of LDS
  const int W = std::max(1, std::min({16, nsteps / 4, 64 / (ET * TT)}));
  const size_t lds = (size_t)W * 16 * TT * ET * 16 * sizeof(float);
  const dim3 grid((S + 16 * TT - 1) / (16 * TT), (E + ET * 16 - 1) / (ET * 16), nsplit);
  auto kfn = k_router<T, ET, TT>;
  MOE_LAUNCH("router", kfn, grid, 64 * W, lds, st, (const T*)x, (const T*)w_router, prev, out, S, d, E, nsplit);
}

template <typename T>
static void router_dt(const void* x, const void* w_router, const float* prev, float* out, int S, int d, int E,
                      int nsplit, hipStream_t st) {
  // few tokens: one 16-expert tile per workgroup, for more workgroups; many tokens: all experts in
  // one workgroup, so x is read once, and 32 tokens per workgroup, so each W_r fragment read from
  // the cache serves two token tiles
  if (E <= 16 || S <= 1024) router_t<T, 1, 1>(x, w_router, prev, out, S, d, E, nsplit, st);
  else if (E <= 32) router_t<T, 2, 2>(x, w_router, prev, out, S, d, E, 1, st);
  else if (E <= 64) router_t<T, 4, 2>(x, w_router, prev, out, S, d, E, 1, st);
  else if (E <= 128) router_t<T, 8, 2>(x, w_router, prev, out, S, d, E, 1, st);
  else router_t<T, 16, 1>(x, w_router, prev, out, S, d, E, 1, st);   // two tiles would spill
}

// A workgroup of the one-tile router reads 16 rows of x and 16 of W_r over all of K (128 KB at
// d = 2048 in bf16), and its waves wait on that one compute unit's loads: with few tiles (a decode
// block: 2 x 4) most of the chip idles. Then K is split over 2 or 4 workgroups per tile (at most
// 128 workgroups, at least 8 K steps each).
int router_splits(int dtype, int S, int d, int E) {
  if (S <= 0 || !(E <= 16 || S <= 1024)) return 1;
  const int nsteps = d / (dtype == 0 ? 32 : 16);
  const int tiles = ((S + 15) / 16) * ((E + 15) / 16);
  int ks = 1;
  while (ks < 4 && tiles * ks * 2 <= 128 && nsteps % (ks * 2) == 0 && nsteps / (ks * 2) >= 8) ks *= 2;
  return ks;
}

hipError_t launch_router(int dtype, const void* x, const void* w_router, const float* prev, float* logits,
                         float* part, int nsplit, int S, int d, int E, hipStream_t st) {
  if (S <= 0) return hipSuccess;
  if (E < 1 || E > 256) return hipErrorInvalidValue;
  if (nsplit != 1 && (nsplit != router_splits(dtype, S, d, E) || !part)) return hipErrorInvalidValue;
  float* out = nsplit > 1 ? part : logits;
  if (dtype == 0) router_dt<bf16_t>(x, w_router, prev, out, S, d, E, nsplit, st);
  else router_dt<float>(x, w_router, prev, out, S, d, E, nsplit, st);
  return hipGetLastError();
}

hipError_t launch_router_sum(const float* part, int nsplit, const float* prev, float* logits, int n,
                             hipStream_t st) {
  if (n <= 0) return hipSuccess;
  auto kfn = k_router_sum;
  MOE_LAUNCH("router_sum", kfn, (n + 255) / 256, 256, 0, st, part, nsplit, prev, logits, n);
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

// Per-token probabilities from logits (softmax with the row max subtracted) or as given. Returns
// the token's largest probability, max(0, p): after the max subtraction the largest key's term is
// exp(0) = 1, so that is 1 / (sum of the terms), with no further reduction.
template <int LPT, int V>
__device__ __forceinline__ float token_probs(const float* keys_row, bool live, int E, int sub, int input_probs,
                                             float (&key)[V], float (&p)[V]) {
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int e = sub + v * LPT;
    key[v] = (live && e < E) ? keys_row[e] : -FLT_MAX;
  }
  if (input_probs) {
    float pm = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      p[v] = (sub + v * LPT < E) ? key[v] : 0.f;
      pm = fmaxf(pm, p[v]);
    }
    return group_max<LPT>(pm);
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
  return inv;
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
  const float pm = token_probs<LPT, V>(a.keys + (size_t)min(s, a.S - 1) * E, live, E, sub, a.input_probs, key, p);
  if (live && a.probs) {
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (sub + v * LPT < E) a.probs[(size_t)s * E + sub + v * LPT] = p[v];
  }
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
    const float pm =
        token_probs<LPT, V>(a.keys + (size_t)min(s, a.S - 1) * E, live, E, sub, a.input_probs, key, p);
    const unsigned taken = token_topk<LPT, V>(key, p, ~0u, E, sub, lane, a.vote_k, nullptr, nullptr);
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
// on the output order: per-chunk histograms, a scan, and a ranked scatter. When the chunk
// histograms are small (kPermFuseMax counts) every scatter workgroup sums them itself and the
// scan needs no launch of its own.
constexpr int kPermThreads = 256;
constexpr int kPermRounds = 4;
constexpr int kPermChunk = kPermThreads * kPermRounds;
constexpr int kPermMaxE = 1024;
constexpr int kPermFuseMax = 4096;   // chunk counts (chunks x heavy experts) a scatter workgroup reads
constexpr int kPermFuseLoads = kPermFuseMax / kPermThreads;

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

// The scan folded into the scatter (nblk * E_heavy <= kPermFuseMax): this workgroup's per-expert
// base (the counts of the chunks before it) and every expert's first row, from the chunk counts;
// workgroup 0 also writes offsets, counts and n_rows. Integer sums: the order does not matter.
__device__ __forceinline__ void perm_bases(const PermuteArgs& a, int nblk, int* s_base, int* s_off) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int EH = a.E_heavy, n = nblk * EH;
  int c[kPermFuseLoads];
#pragma unroll
  for (int j = 0; j < kPermFuseLoads; ++j) {
    const int t = tid + j * kPermThreads;
    c[j] = t < n ? a.blk_cnt[t] : 0;   // every load in flight before any is used
  }
  for (int i = tid; i < EH; i += kPermThreads) {
    s_base[i] = 0;
    s_off[i] = 0;   // the expert's total first
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPermFuseLoads; ++j) {
    const int t = tid + j * kPermThreads;
    if (t < n && c[j]) {
      const int bb = t / EH, e = t - bb * EH;
      atomicAdd(&s_off[e], c[j]);
      if (bb < (int)blockIdx.x) atomicAdd(&s_base[e], c[j]);
    }
  }
  __syncthreads();
  if (tid < 64) {
    // exclusive prefix of the totals over experts (light experts take no rows), 64 at a time
    int run = 0;
    for (int e0 = 0; e0 < a.E_r; e0 += 64) {
      const int e = e0 + lane;
      const int tot = e < EH ? s_off[e] : 0;
      int incl = tot;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
      }
      const int off = run + incl - tot;
      if (e < EH) s_off[e] = off;
      if (blockIdx.x == 0 && e < a.E_r) {
        a.offsets[e] = off;
        a.counts[e] = tot;
      }
      run += __shfl(incl, 63, 64);
    }
    if (blockIdx.x == 0 && lane == 0) {
      a.offsets[a.E_r] = run;
      *a.n_rows = run;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kPermThreads) void k_perm_scatter(PermuteArgs a, int nbits, int nblk, int fused) {
  __shared__ int wcnt[kPermThreads / 64][kPermMaxE];
  __shared__ int run[kPermMaxE];
  __shared__ int s_base[kPermMaxE];
  __shared__ int s_off[kPermMaxE];
  const int wave = threadIdx.x >> 6;
  if (fused) perm_bases(a, nblk, s_base, s_off);   // uniform over the workgroup
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
      const int row = fused ? s_off[e] + s_base[e] + base + rank : a.offsets[e] + bbase[e] + base + rank;
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
  // with few chunk counts the scatter workgroups sum them themselves; S = 0 (no chunks) still takes
  // the scan kernel, which writes the empty offsets
  const int fused = nblk > 0 && (int64_t)nblk * a.E_heavy <= kPermFuseMax ? 1 : 0;
  if (nblk > 0) {
    auto kfn = k_perm_count;
    MOE_LAUNCH("perm_count", kfn, nblk, kPermThreads, 0, st, a);
  }
  if (!fused) {
    auto kfn = k_perm_scan;
    MOE_LAUNCH("perm_scan", kfn, 1, kPermThreads, 0, st, a, nblk);
  }
  if (nblk > 0) {
    auto kfn = k_perm_scatter;
    MOE_LAUNCH("perm_scatter", kfn, nblk, kPermThreads, 0, st, a, nbits, nblk, fused);
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
constexpr int kSmallMaxSplits = 4;    // router K splits the kernel adds itself
static_assert(kSmallMaxPairs % kSmallThreads == 0, "whole rounds of pairs");

bool route_small_supported(int S, int E_r, int k) {
  return S >= 1 && S <= kSmallMaxS && (int64_t)S * E_r <= kSmallMaxSE && (int64_t)S * k <= kSmallMaxPairs &&
         E_r <= 256 && k <= kMaxK;
}

// Barrier for LDS data only: waits for this wave's LDS operations but not for its global stores,
// which a full __syncthreads would also wait for (their results are not read back here).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Integer with the order of the float (finite values); -0 and +0 are equal, as under a float
// comparison.
__device__ __forceinline__ int float_order(float f) {
  const int b = __float_as_int(f);
  return b >= 0 ? b : (b ^ 0x7fffffff) + 1;
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
  // keys as unsigned integers of the same order; every key maps to 1 or more, so the ineligible
  // entries take 0 and drop out of every count below (each candidate threshold is 1 or more)
  uint32_t u[V];
  bool el[V];
  int n = 0;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    el[v] = lane + v * 64 < E && ((allow >> v) & 1u);
    u[v] = el[v] ? (uint32_t)float_order(key[v]) ^ 0x80000000u : 0u;
    n += __popcll(__ballot(el[v]));
  }
  const int kq = min(k, n);
  if (kq <= 0) return 0;
  uint32_t T = 0;
  bool exact = false;   // exactly kq keys are >= T
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = T | (1u << b);
    int c = 0;
    // the comparison's lane mask straight from the compare instruction (35: unsigned >=)
#pragma unroll
    for (int v = 0; v < V; ++v) c += __popcll(__builtin_amdgcn_uicmp(u[v], cand, 35));
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
  // s_key holds the keys until the selections are made; the dispatch then keeps its per-(round,
  // wave) expert counts there
  __shared__ float s_key[kSmallMaxSE];
  __shared__ float s_p[kSmallMaxSE];
  __shared__ float s_aux[DES ? kSmallMaxSE : 1];   // DES: filtered probabilities (DES-Seq: 1 per selection)
  __shared__ float s_votes[256];
  __shared__ int s_core[256];
  __shared__ int s_ncore;
  __shared__ int s_counts[256];
  __shared__ int s_idx[kSmallMaxPairs];
  __shared__ float s_w[kSmallMaxPairs];
  __shared__ float s_wfin[kSmallMaxPairs];   // final weights (s_w is still read while they are formed)
  __shared__ uint8_t s_reuse[kSmallMaxS];
  __shared__ int s_off[257];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = a.S, E = a.E_r, SE = S * E;
  // slot stride of the routing arrays: k (token choice, DES-Seq) or min(k, m_core) (DES-Vote); the
  // number of slots a token fills (kk) is the same except for DES-Seq, where it is min(k, |core|)
  // and only known after the core is formed
  const int ks = q.k;
  int M = a.m_core;
  int kk = DES ? min(a.k, max(M, 1)) : a.k;

  {
    // every load in flight at once (the index is clamped rather than the load skipped, so that the
    // compiler does not wait for each one)
    constexpr int LR = kSmallMaxSE / kSmallThreads;
    float kv[LR];
    if (a.part) {
      // the router's K splits (at most kSmallMaxSplits) added in split order, then prev; the round
      // and split conditions are uniform over the workgroup
      const int ns = a.nsplit;
      float t[LR][kSmallMaxSplits], pv[LR];
#pragma unroll
      for (int r = 0; r < LR; ++r) {
        const int i = min(r * kSmallThreads + tid, SE - 1);
        if (r * kSmallThreads < SE) {
#pragma unroll
          for (int z = 0; z < kSmallMaxSplits; ++z)
            if (z < ns) t[r][z] = a.part[(size_t)z * SE + i];
          if (a.prev) pv[r] = a.prev[i];
        }
      }
#pragma unroll
      for (int r = 0; r < LR; ++r) {
        float v = 0.f;
        if (r * kSmallThreads < SE) {
#pragma unroll
          for (int z = 0; z < kSmallMaxSplits; ++z)
            if (z < ns) v += t[r][z];
          if (a.prev) v += pv[r];
        }
        kv[r] = v;
      }
    } else {
#pragma unroll
      for (int r = 0; r < LR; ++r) kv[r] = a.keys[min(r * kSmallThreads + tid, SE - 1)];
    }
#pragma unroll
    for (int r = 0; r < LR; ++r)
      if (r * kSmallThreads + tid < SE) s_key[r * kSmallThreads + tid] = kv[r];
    // every path waits here for all the loads, so that the compiler does not take the unused ones as
    // still in flight later on (its wait for them would also wait for the stores issued by then)
    wait_vmem<0>();
    if (a.part) {
#pragma unroll
      for (int r = 0; r < LR; ++r)
        if (r * kSmallThreads + tid < SE) a.logits[r * kSmallThreads + tid] = kv[r];
    }
  }
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
    const float pm = token_probs<LPT, V>(s_key + min(s, S - 1) * E, live, E, sub, a.input_probs, key, p);
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

  if constexpr (DES) {
    // votes and core, in one wave (expert e in lane e % 64, slot e / 64): the votes are summed over
    // tokens in ascending order; DES-Vote: the core is the M experts first under (vote desc, e asc),
    // found by the radix select of the token selections; DES-Seq: the experts some token selected
    // (vote > 0). The core is then listed ascending by a prefix count over the membership bits.
    if (wave == 0) {
      constexpr int VW = LPT == 64 ? V : 1;   // LPT < 64 only for E_r <= 32
      float vv[VW];
#pragma unroll
      for (int c = 0; c < VW; ++c) {
        const int e = lane + 64 * c;
        float v = 0.f;
        if (e < E) {
#pragma unroll 8
          for (int n = 0; n < S; ++n) v += s_aux[n * E + e];
          s_votes[e] = v;
        }
        vv[c] = v;
      }
      unsigned in_core = 0;
      if (!a.seq) {
        in_core = wave_topk<VW>(vv, vv, ~0u, E, lane, M, nullptr, nullptr);
      } else {
#pragma unroll
        for (int c = 0; c < VW; ++c)
          if (lane + 64 * c < E && vv[c] > 0.f) in_core |= 1u << c;
      }
      int cbase = 0;
#pragma unroll
      for (int c = 0; c < VW; ++c) {
        const int e = lane + 64 * c;
        const bool in = (in_core >> c) & 1u;
        const uint64_t m = __ballot(in);
        if (in) s_core[cbase + __popcll(m & lanemask_lt())] = e;
        cbase += __popcll(m);
      }
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
  // hold expert -1 and weight 0. Pair p = s * ks + j is handled by thread p % kSmallThreads here and
  // in the dispatch below, which therefore reads its own s_idx and s_wfin entries without a barrier.
  constexpr int RMAX = kSmallMaxPairs / kSmallThreads;
  const int P = S * ks;
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    const int p = r * kSmallThreads + tid;
    if (p < P) {
      const int s = p / ks, j = p - s * ks;
      int e = -1;
      float w = 0.f;
      if (j < kk) {
        e = s_idx[p];
        w = s_w[p];
        if (a.renorm) {
          float t = 0.f;
          for (int jj = 0; jj < kk; ++jj) t += s_w[s * ks + jj];
          w = w / t;
        }
      }
      s_idx[p] = e;
      s_wfin[p] = w;
    }
  }

  // dispatch: pair p goes to a row when its expert is heavy and its token does not reuse. Rows are
  // ordered by (expert, pair). Each wave counts, per round of kSmallThreads pairs, how many of its
  // pairs go to each expert (equal experts found with match-any ballots); one wave then turns the
  // counts into the experts' offsets and, per expert, the first row of each (round, wave); a pair's
  // row adds the lanes before it in its wave with the same expert.
  const int EH = q.E_heavy;
  const bool use_reuse = q.reuse != nullptr;
  int* s_cnt = reinterpret_cast<int*>(s_key);   // [round * kSmallWaves + wave][EH]
  int nbits = 1;
  while ((1 << nbits) <= EH) ++nbits;
  int pe[RMAX], plow[RMAX];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    const int p = r * kSmallThreads + tid;
    pe[r] = -1;
    plow[r] = 0;
    if (r * kSmallThreads >= P) continue;   // uniform over the workgroup
    int e = p < P ? s_idx[p] : -1;
    const bool ok = p < P && e >= 0 && e < EH && !(use_reuse && s_reuse[p / ks]);
    const int key = ok ? e : EH;
    uint64_t peers = ~0ull;
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (key >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const uint64_t lower = peers & lanemask_lt();
    int* row = s_cnt + (r * kSmallWaves + wave) * EH;
    for (int i = lane; i < EH; i += 64) row[i] = 0;
    // a wave's LDS writes take effect in order: the leader's count lands after the zeros
    if (ok && lower == 0) row[e] = __popcll(peers);
    if (ok) {
      pe[r] = e;
      plow[r] = __popcll(lower);
    }
  }
  lds_barrier();
  if (wave == 0) {
    const int nslot = ((P + kSmallThreads - 1) / kSmallThreads) * kSmallWaves;
    int base = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      int c = 0;
      if (e < EH) {
        // exclusive prefix over the (round, wave) slots, in place; c ends as the expert's count
        for (int s0 = 0; s0 < nslot; s0 += kSmallWaves) {
          int v[kSmallWaves];
#pragma unroll
          for (int w = 0; w < kSmallWaves; ++w) v[w] = s_cnt[(s0 + w) * EH + e];
#pragma unroll
          for (int w = 0; w < kSmallWaves; ++w) {
            s_cnt[(s0 + w) * EH + e] = c;
            c += v[w];
          }
        }
      }
      int incl = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      if (e < E) {
        s_off[e] = base + incl - c;
        s_counts[e] = c;
      }
      base += __shfl(incl, 63, 64);
    }
    if (lane == 0) s_off[E] = base;
  }
  lds_barrier();
  // every global store comes last: a wait that the compiler places for a load would otherwise
  // also wait for the stores issued before it
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    const int p = r * kSmallThreads + tid;
    if (p >= P) continue;
    const int e = pe[r];
    if (e >= 0) {
      const int row = s_off[e] + s_cnt[(r * kSmallWaves + wave) * EH + e] + plow[r];
      q.row_token[row] = p / ks;
      q.row_w[row] = s_wfin[p];
      q.token_rows[p] = row;
    } else {
      q.token_rows[p] = -1;
    }
  }
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    const int p = r * kSmallThreads + tid;
    if (p < P) {
      a.topk_idx[p] = s_idx[p];
      a.topk_w[p] = s_wfin[p];
    }
  }
  for (int e = tid; e <= E; e += kSmallThreads) {
    q.offsets[e] = s_off[e];
    if (e < E) q.counts[e] = s_counts[e];
    if (e == E) *q.n_rows = s_off[E];
  }
  if constexpr (DES) {
    const int nc = s_ncore;
    for (int e = tid; e < E; e += kSmallThreads) {
      a.votes[e] = s_votes[e];
      if (e < nc) a.core[e] = s_core[e];
      else if (a.seq) a.core[e] = -1;
    }
  }
  if (a.probs)
    for (int i = tid; i < SE; i += kSmallThreads) a.probs[i] = s_p[i];
  if (a.reuse)
    for (int s = tid; s < S; s += kSmallThreads) a.reuse[s] = s_reuse[s];
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
  if (!route_small_supported(a.S, a.E_r, kk) || q.E_heavy > a.E_r || q.k != kk) return hipErrorInvalidValue;
  if (a.part && (a.nsplit < 1 || a.nsplit > kSmallMaxSplits || !a.logits)) return hipErrorInvalidValue;
  // the dispatch's per-(round, wave) expert counts live in the key array (at most 4096 entries
  // within the limits above)
  if ((int64_t)((a.S * kk + kSmallThreads - 1) / kSmallThreads) * kSmallWaves * q.E_heavy > kSmallMaxSE)
    return hipErrorInvalidValue;
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
