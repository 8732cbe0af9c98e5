// C ABI of the MoE layer library: argument validation, workspace plan and launch sequence.
// The operations and their sources are described in include/moe.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "internal.hpp"
#include "moe.h"
#include "moe_prof.h"

// ---------------------------------------------------------------------------------------------
// Launch profiling: a fixed pool of events, handed out in launch order while enabled.
namespace moe {
namespace prof {
struct Rec {
  const char* name;
  hipEvent_t start, stop;
};
struct Entry {
  std::string name;
  double ms;
  int32_t launches;
};
static bool g_on = false;
static std::vector<hipEvent_t> g_pool;
static std::vector<Rec> g_recs;
static std::vector<Entry> g_entries;
constexpr size_t kPoolPairs = 4096;

bool enabled() { return g_on; }

bool take(const char* name, hipEvent_t* start, hipEvent_t* stop) {
  const size_t n = g_recs.size();
  if (2 * n + 2 > g_pool.size()) return false;
  *start = g_pool[2 * n];
  *stop = g_pool[2 * n + 1];
  g_recs.push_back({name, *start, *stop});
  return true;
}
}  // namespace prof
}  // namespace moe

namespace {

using namespace moe;

constexpr uint32_t kKnownFlags =
    MOE_F_INPUT_PROBS | MOE_F_SYNC_DEBUG | MOE_F_FORCE_TILED | MOE_F_FORCE_STREAM | MOE_F_ROUTE_MULTI;
constexpr int kMaxExperts = 256;
constexpr int kMaxK = 16;

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Everything derived from a validated descriptor.
struct Plan {
  int E_r = 0, k_eff = 0, C = 0;
  int64_t R_max = 0;
  bool streaming = false;     // heavy experts on the weight-streaming kernel
  size_t esz = 0;             // element size of dtype
  // workspace pieces (byte offsets)
  size_t o_blk = 0, o_filt = 0, o_pT = 0, o_tokrows = 0, o_tokcnt = 0;   // route scratch
  size_t o_logits = 0;                                                  // router output
  int nsplit = 1;                                                       // router K splits
  size_t o_rpart = 0;                                                   // their partial sums
  size_t o_rt = 0;                                                      // internal routing arrays
  size_t o_h = 0, o_hs = 0, o_yp = 0, o_ys = 0;                         // expert buffers
  size_t total = 0;
  // internal routing array offsets (relative to o_rt)
  size_t r_idx = 0, r_w = 0, r_cnt = 0, r_off = 0, r_rtok = 0, r_rw = 0, r_trow = 0, r_toff = 0, r_tlist = 0,
         r_core = 0, r_votes = 0, r_reuse = 0, r_nrows = 0, r_cap = 0, r_size = 0;
};

bool finite_nonneg(float v) { return std::isfinite(v) && v >= 0.f; }

// Upper bound on the experts a call can route rows to: the core of DES-Vote (m_core), the union of
// N top-k_seq sets for DES-Seq (at most S * k_seq experts), else every expert.
int64_t max_active_experts(const moe_desc* d) {
  const int64_t E_r = (int64_t)d->E_heavy + d->n_identity + d->n_zero + d->n_const;
  if (d->mode == MOE_DES_VOTE) return std::min<int64_t>(d->m_core, E_r);
  if (d->mode == MOE_DES_SEQ) return std::min<int64_t>((int64_t)d->S * d->vote_k, E_r);
  return E_r;
}

bool is_des(const moe_desc* d) { return d->mode == MOE_DES_VOTE || d->mode == MOE_DES_SEQ; }

moe_status make_plan(const moe_desc* d, Plan* p) {
  if (!d) return MOE_EINVAL;
  if (d->flags & ~kKnownFlags) return MOE_EINVAL;
  if (d->S < 0 || d->d < 1 || d->E_heavy < 0 || d->n_identity < 0 || d->n_zero < 0 || d->n_const < 0 ||
      d->n_shared < 0)
    return MOE_EINVAL;
  if (d->dtype != MOE_BF16 && d->dtype != MOE_F32) return MOE_EINVAL;
  if (d->act != MOE_ACT_GELU && d->act != MOE_ACT_GELU_TANH && d->act != MOE_ACT_SWIGLU) return MOE_EINVAL;
  if (d->mode != MOE_TOKEN_CHOICE && d->mode != MOE_EXPERT_CHOICE && d->mode != MOE_DES_VOTE &&
      d->mode != MOE_DES_SEQ)
    return MOE_EINVAL;
  const int64_t E_r = (int64_t)d->E_heavy + d->n_identity + d->n_zero + d->n_const;
  if (E_r < 1) return MOE_EINVAL;
  if ((d->E_heavy > 0 || d->n_shared > 0) && d->d_ff < 1) return MOE_EINVAL;
  if (!finite_nonneg(d->reuse_tau)) return MOE_EINVAL;
  if ((d->flags & MOE_F_FORCE_TILED) && (d->flags & MOE_F_FORCE_STREAM)) return MOE_EINVAL;
  p->E_r = (int)std::min<int64_t>(E_r, 1 << 30);
  p->esz = d->dtype == MOE_BF16 ? 2 : 4;
  if (d->mode == MOE_EXPERT_CHOICE) {
    if (!std::isfinite(d->capacity_factor) || d->capacity_factor <= 0.f) return MOE_EINVAL;
    const double c = std::floor((double)d->capacity_factor * (double)d->S / (double)E_r);
    const int64_t C = (int64_t)std::min<double>((double)d->S, c);
    if (C < 1 && d->S > 0) return MOE_EINVAL;   // no tokens: no capacity either
    p->C = (int)C;
    p->k_eff = 0;
    p->R_max = E_r * C;
  } else {
    if (d->k < 1 || d->k > E_r) return MOE_EINVAL;
    p->k_eff = d->k;
    if (d->mode == MOE_DES_VOTE) {
      if (d->m_core < 1 || d->m_core > E_r || d->vote_k < 1 || d->vote_k > E_r) return MOE_EINVAL;
      p->k_eff = std::min(d->k, d->m_core);
    }
    if (d->mode == MOE_DES_SEQ && (d->vote_k < 1 || d->vote_k > E_r)) return MOE_EINVAL;
    p->R_max = (int64_t)d->S * p->k_eff;
  }
  // What this library implements.
  if (E_r > kMaxExperts) return MOE_EUNSUPPORTED;
  if (p->k_eff > kMaxK) return MOE_EUNSUPPORTED;
  if (d->mode == MOE_EXPERT_CHOICE && (d->n_identity + d->n_zero + d->n_const > 0 || d->reuse_tau > 0.f))
    return MOE_EUNSUPPORTED;
  if (d->d % 8 != 0) return MOE_EUNSUPPORTED;
  if (d->d % (d->dtype == MOE_BF16 ? 32 : 16) != 0) return MOE_EUNSUPPORTED;   // router MFMA steps
  // kernels address rows of x, H, y_perm and one expert's weights with 32-bit byte offsets
  const int64_t lim = ((int64_t)1 << 31) - 1;
  const int64_t ff = std::max(d->d_ff, 0), es = d->dtype == MOE_BF16 ? 2 : 4;
  if ((int64_t)d->S * E_r > lim || p->R_max > lim || (int64_t)d->S * d->d * es > lim || p->R_max * ff * es > lim ||
      p->R_max * d->d * 4 > lim || (int64_t)d->S * d->n_shared * ff * es > lim || ff * d->d * es > lim)
    return MOE_EUNSUPPORTED;
  const int act = d->act;
  if (d->E_heavy > 0) {
    const int64_t per_expert = p->R_max / std::max<int64_t>(1, std::min<int64_t>(d->E_heavy, max_active_experts(d)));
    const bool stream_ok = stream_gemm_supported(d->dtype, GEMM_UP, act, d->d_ff, d->d) &&
                           stream_gemm_supported(d->dtype, GEMM_DOWN, act, d->d, d->d_ff);
    bool stream = per_expert <= 64 && stream_ok;
    if (d->flags & MOE_F_FORCE_TILED) stream = false;
    if (d->flags & MOE_F_FORCE_STREAM) stream = true;
    p->streaming = stream;
    if (stream) {
      if (!stream_gemm_supported(d->dtype, GEMM_UP, act, d->d_ff, d->d) ||
          !stream_gemm_supported(d->dtype, GEMM_DOWN, act, d->d, d->d_ff))
        return MOE_EUNSUPPORTED;
    } else {
      if (!grouped_gemm_supported(d->dtype, GEMM_UP, act, d->d_ff, d->d) ||
          !grouped_gemm_supported(d->dtype, GEMM_DOWN, act, d->d, d->d_ff))
        return MOE_EUNSUPPORTED;
    }
  }
  if (d->n_shared > 0) {
    if (!grouped_gemm_supported(d->dtype, GEMM_UP, act, d->d_ff, d->d) ||
        !grouped_gemm_supported(d->dtype, GEMM_DOWN, act, d->d, (int)std::min<int64_t>((int64_t)d->n_shared * d->d_ff, 1 << 30)))
      return MOE_EUNSUPPORTED;
  }

  // ---- workspace plan
  const size_t S = (size_t)d->S, Er = (size_t)E_r, R = (size_t)p->R_max;
  const size_t k = (size_t)std::max(p->k_eff, 1);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  const int nblk = permute_num_blocks(d->S, std::max(p->k_eff, 1));
  p->o_blk = take((size_t)nblk * std::max(d->E_heavy, 1) * 4);
  p->o_filt = take(is_des(d) ? S * Er * 4 : 0);
  p->o_pT = take(d->mode == MOE_EXPERT_CHOICE ? S * Er * 4 : 0);
  p->o_tokrows = take(d->mode == MOE_EXPERT_CHOICE ? S * Er * 4 : 0);
  p->o_tokcnt = take(d->mode == MOE_EXPERT_CHOICE ? S * 4 : 0);
  p->o_logits = take(S * Er * 4);
  // expert choice routes with its own kernels, which read finished logits
  p->nsplit = d->mode == MOE_EXPERT_CHOICE ? 1 : router_splits(d->dtype == MOE_BF16 ? 0 : 1, d->S, d->d, E_r);
  p->o_rpart = take(p->nsplit > 1 ? (size_t)p->nsplit * S * Er * 4 : 0);
  // internal routing arrays
  size_t r = 0;
  auto rt = [&](size_t bytes) {
    const size_t o = r;
    r += align256(bytes);
    return o;
  };
  p->r_idx = rt(S * k * 4);
  p->r_w = rt(S * k * 4);
  p->r_cnt = rt(Er * 4);
  p->r_off = rt((Er + 1) * 4);
  p->r_rtok = rt(R * 4);
  p->r_rw = rt(R * 4);
  p->r_trow = rt(S * k * 4);
  p->r_toff = rt((S + 1) * 4);
  p->r_tlist = rt(R * 4);
  p->r_core = rt((d->mode == MOE_DES_SEQ ? Er : (size_t)std::max(d->m_core, 1)) * 4);
  p->r_votes = rt(Er * 4);
  p->r_reuse = rt(S);
  p->r_nrows = rt(4);
  p->r_cap = rt(4);
  p->r_size = r;
  p->o_rt = take(r);
  const size_t f = (size_t)std::max(d->d_ff, 0);
  p->o_h = take(d->E_heavy > 0 ? R * f * p->esz : 0);
  p->o_hs = take(S * (size_t)d->n_shared * f * p->esz);
  p->o_yp = take(d->E_heavy > 0 ? R * (size_t)d->d * 4 : 0);
  p->o_ys = take(d->n_shared > 0 ? S * (size_t)d->d * 4 : 0);
  p->total = std::max<size_t>(off, 256);
  return MOE_OK;
}

moe_status check_ws(const Plan& p, const void* ws, size_t ws_bytes) {
  if (!ws) return MOE_EWORKSPACE;
  if (((uintptr_t)ws & 255) != 0) return MOE_EWORKSPACE;
  if (ws_bytes < p.total) return MOE_EWORKSPACE;
  return MOE_OK;
}

moe_status after_launch(hipError_t e, const moe_desc* d, hipStream_t st) {
  if (e != hipSuccess) return MOE_EHIP;
  if (d->flags & MOE_F_SYNC_DEBUG) {
    if (hipStreamSynchronize(st) != hipSuccess) return MOE_EHIP;
    if (hipGetLastError() != hipSuccess) return MOE_EHIP;
  }
  return MOE_OK;
}

#define MOE_TRY(expr)                   \
  do {                                  \
    const moe_status _s = (expr);       \
    if (_s != MOE_OK) return _s;        \
  } while (0)

moe_status check_routing(const moe_desc* d, const moe_routing* r) {
  if (!r) return MOE_EINVAL;
  if (!r->counts || !r->offsets || !r->row_token || !r->row_w || !r->n_rows) return MOE_EINVAL;
  if (d->mode == MOE_EXPERT_CHOICE) {
    if (!r->token_off || !r->token_list) return MOE_EINVAL;
  } else {
    if (!r->topk_idx || !r->topk_w || !r->token_rows) return MOE_EINVAL;
    if (d->reuse_tau > 0.f && !r->reuse) return MOE_EINVAL;
    if (is_des(d) && (!r->core || !r->votes)) return MOE_EINVAL;
  }
  return MOE_OK;
}

moe_routing internal_routing(const Plan& p, const moe_desc* d, void* ws) {
  uint8_t* b = (uint8_t*)ws + p.o_rt;
  moe_routing r{};
  r.topk_idx = (int32_t*)(b + p.r_idx);
  r.topk_w = (float*)(b + p.r_w);
  r.probs = nullptr;
  r.counts = (int32_t*)(b + p.r_cnt);
  r.offsets = (int32_t*)(b + p.r_off);
  r.row_token = (int32_t*)(b + p.r_rtok);
  r.row_w = (float*)(b + p.r_rw);
  r.token_rows = (int32_t*)(b + p.r_trow);
  r.token_off = (int32_t*)(b + p.r_toff);
  r.token_list = (int32_t*)(b + p.r_tlist);
  r.core = (int32_t*)(b + p.r_core);
  r.votes = (float*)(b + p.r_votes);
  r.reuse = d->reuse_tau > 0.f ? (uint8_t*)(b + p.r_reuse) : nullptr;
  r.n_rows = (int32_t*)(b + p.r_nrows);
  r.capacity = (int32_t*)(b + p.r_cap);
  return r;
}

// keys: the logits (or given probabilities). From the layer call with p.nsplit > 1 they are still to
// be formed from the router's partial sums (part) and prev, and written to keys.
moe_status do_route(const moe_desc* d, const Plan& p, const float* keys, bool input_probs, const moe_routing* r,
                    void* ws, hipStream_t st, const float* part = nullptr, const float* prev = nullptr) {
  uint8_t* w = (uint8_t*)ws;
  if (d->mode == MOE_EXPERT_CHOICE) {
    ECArgs a{};
    a.S = d->S;
    a.E = p.E_r;
    a.C = p.C;
    a.input_probs = input_probs;
    a.keys = keys;
    a.probs = r->probs;
    a.pT = (float*)(w + p.o_pT);
    a.tok_rows_tmp = (int32_t*)(w + p.o_tokrows);
    a.tok_cnt = (int32_t*)(w + p.o_tokcnt);
    a.counts = r->counts;
    a.offsets = r->offsets;
    a.row_token = r->row_token;
    a.row_w = r->row_w;
    a.token_off = r->token_off;
    a.token_list = r->token_list;
    a.n_rows = r->n_rows;
    a.capacity = r->capacity;
    return after_launch(launch_route_ec(a, st), d, st);
  }
  RouteArgs a{};
  a.S = d->S;
  a.E_r = p.E_r;
  a.E_heavy = d->E_heavy;
  a.k = p.k_eff;
  a.renorm = d->renorm != 0;
  a.input_probs = input_probs;
  a.n_identity = d->n_identity;
  a.n_zero = d->n_zero;
  a.n_const = d->n_const;
  a.tau = d->reuse_tau;
  a.vote_k = d->vote_k;
  a.m_core = d->mode == MOE_DES_SEQ ? 0 : d->m_core;
  a.seq = d->mode == MOE_DES_SEQ ? 1 : 0;
  a.keys = keys;
  a.probs = r->probs;
  a.topk_idx = r->topk_idx;
  a.topk_w = r->topk_w;
  a.reuse = r->reuse;
  a.votes = r->votes;
  a.core = r->core;
  const bool des = is_des(d);
  if (des) a.k = d->k;   // the kernels apply min(k, core size)
  PermuteArgs q{};
  q.S = d->S;
  q.k = p.k_eff;
  q.E_r = p.E_r;
  q.E_heavy = d->E_heavy;
  q.topk_idx = r->topk_idx;
  q.topk_w = r->topk_w;
  q.reuse = d->reuse_tau > 0.f ? r->reuse : nullptr;
  q.counts = r->counts;
  q.offsets = r->offsets;
  q.row_token = r->row_token;
  q.row_w = r->row_w;
  q.token_rows = r->token_rows;
  q.n_rows = r->n_rows;
  q.blk_cnt = (int32_t*)(w + p.o_blk);
  // small calls (a decode block, a tiny batch): routing and dispatch in one workgroup, which also
  // adds the router's K splits
  if (!(d->flags & MOE_F_ROUTE_MULTI) && route_small_supported(d->S, p.E_r, p.k_eff)) {
    if (part) {
      a.part = part;
      a.nsplit = p.nsplit;
      a.prev = prev;
      a.logits = const_cast<float*>(keys);
    }
    return after_launch(launch_route_small(a, q, des, st), d, st);
  }
  if (part)
    MOE_TRY(after_launch(launch_router_sum(part, p.nsplit, prev, const_cast<float*>(keys), d->S * p.E_r, st), d, st));
  if (des) MOE_TRY(after_launch(launch_route_des(a, (float*)(w + p.o_filt), st), d, st));
  else MOE_TRY(after_launch(launch_route_topk(a, st), d, st));
  return after_launch(launch_permute(q, st), d, st);
}

moe_status do_experts(const moe_desc* d, const Plan& p, const void* x, const void* x_perm, const moe_routing* r,
                      const moe_weights* wt, float* y_perm, float* y_shared, void* ws, hipStream_t st) {
  uint8_t* w = (uint8_t*)ws;
  const int64_t f = d->d_ff, dm = d->d;
  void* H = w + p.o_h;
  void* Hs = w + p.o_hs;
  GemmProblem up[2], dn[2];
  int64_t ub[2], mth[2] = {0, 0};
  int nup = 0;
  if (d->E_heavy > 0) {
    GemmProblem u{};
    u.A = x_perm ? x_perm : x;
    u.a_rows = x_perm ? nullptr : r->row_token;
    u.lda = dm;
    u.B = wt->w1;
    u.B3 = wt->w3;
    u.ldb = dm;
    u.b_gstride = f * dm;
    u.k_seg = dm;
    u.k_seg_stride = 0;
    u.C = H;
    u.ldc = f;
    u.c_gcol = 0;
    u.offsets = r->offsets;
    u.G = d->E_heavy;
    u.M_uni = 0;
    u.N = (int32_t)f;
    u.K = (int32_t)dm;
    GemmProblem v = u;
    v.A = H;
    v.a_rows = nullptr;
    v.lda = f;
    v.B = wt->w2;
    v.B3 = nullptr;
    v.ldb = f;
    v.b_gstride = dm * f;
    v.k_seg = f;
    v.C = y_perm;
    v.ldc = dm;
    v.N = (int32_t)dm;
    v.K = (int32_t)f;
    if (p.streaming) {
      const int max_active = (int)std::min<int64_t>({(int64_t)d->E_heavy, p.R_max, max_active_experts(d)});
      // Token rows per streaming pass: 64 when an expert can have more than 32 rows (a token takes an
      // expert at most once, so at most S) and the average active expert has more than 24; else 32.
      // A pass streams the expert's weights once; the wider pass costs more token-row loads.
      const int64_t rows_ub = std::min<int64_t>(p.R_max, d->mode == MOE_EXPERT_CHOICE ? (int64_t)p.C : (int64_t)d->S);
      const int pass_rows = (rows_ub > 32 && p.R_max > 24 * (int64_t)max_active) ? 64 : 32;
      MOE_TRY(after_launch(launch_stream_gemm(d->dtype, GEMM_UP, d->act, u, max_active, pass_rows, st), d, st));
      MOE_TRY(after_launch(launch_stream_gemm(d->dtype, GEMM_DOWN, d->act, v, max_active, pass_rows, st), d, st));
    } else {
      up[nup] = u;
      dn[nup] = v;
      ub[nup] = p.R_max;
      // expected 256-row tiles: expert choice fills every expert to C rows; otherwise about half a
      // ragged tile per expert on top of the rows
      mth[nup] = d->mode == MOE_EXPERT_CHOICE ? (int64_t)d->E_heavy * ((p.C + 255) / 256)
                                                : (p.R_max + 255) / 256 + d->E_heavy / 2;
      ++nup;
    }
  }
  if (d->n_shared > 0) {
    const int64_t ns = d->n_shared;
    GemmProblem u{};
    u.A = x;
    u.a_rows = nullptr;
    u.lda = dm;
    u.B = wt->s_w1;
    u.B3 = wt->s_w3;
    u.ldb = dm;
    u.b_gstride = f * dm;
    u.k_seg = dm;
    u.k_seg_stride = 0;
    u.C = Hs;
    u.ldc = ns * f;
    u.c_gcol = f;
    u.offsets = nullptr;
    u.G = (int32_t)ns;
    u.M_uni = d->S;
    u.N = (int32_t)f;
    u.K = (int32_t)dm;
    // down: one GEMM over the K-concatenation [H_1 | ... | H_ns] . [W2_1 | ... | W2_ns]^T
    GemmProblem v{};
    v.A = Hs;
    v.a_rows = nullptr;
    v.lda = ns * f;
    v.B = wt->s_w2;
    v.B3 = nullptr;
    v.ldb = f;
    v.b_gstride = 0;
    v.k_seg = f;
    v.k_seg_stride = dm * f;
    v.C = y_shared;
    v.ldc = dm;
    v.c_gcol = 0;
    v.offsets = nullptr;
    v.G = 1;
    v.M_uni = d->S;
    v.N = (int32_t)dm;
    v.K = (int32_t)(ns * f);
    up[nup] = u;
    dn[nup] = v;
    ub[nup] = d->S;
    ++nup;
  }
  if (nup > 0) {
    MOE_TRY(after_launch(launch_grouped_gemm(d->dtype, GEMM_UP, d->act, up, ub, mth, nup, st), d, st));
    MOE_TRY(after_launch(launch_grouped_gemm(d->dtype, GEMM_DOWN, d->act, dn, ub, mth, nup, st), d, st));
  }
  return MOE_OK;
}

moe_status do_combine(const moe_desc* d, const Plan& p, const void* x, const moe_routing* r, const float* y_perm,
                      const float* y_shared, const void* const_vec, void* cache, const void* residual, void* y,
                      hipStream_t st) {
  CombineArgs a{};
  a.dtype = d->dtype;
  a.mode = d->mode == MOE_EXPERT_CHOICE ? 1 : 0;
  a.S = d->S;
  a.d = d->d;
  a.k = p.k_eff;
  a.E_heavy = d->E_heavy;
  a.n_identity = d->n_identity;
  a.n_zero = d->n_zero;
  a.n_const = d->n_const;
  a.x = x;
  a.topk_idx = r->topk_idx;
  a.topk_w = r->topk_w;
  a.token_rows = r->token_rows;
  a.token_off = r->token_off;
  a.token_list = r->token_list;
  a.row_w = r->row_w;
  a.reuse = d->reuse_tau > 0.f ? r->reuse : nullptr;
  a.y_perm = y_perm;
  a.y_shared = d->n_shared > 0 ? y_shared : nullptr;
  a.const_vec = const_vec;
  a.cache = cache;
  a.residual = residual;
  a.y = y;
  return after_launch(launch_combine(a, st), d, st);
}

// A call with no tokens routes nothing: the per-expert counts and offsets, the row count and the
// capacity become 0, the DES votes 0 and the core slots -1. Arrays of S rows are not touched (they
// may be null).
moe_status empty_routing(const moe_desc* d, const Plan& p, const moe_routing* r, hipStream_t st) {
  if (!r) return MOE_OK;
  if (!r->counts || !r->offsets || !r->n_rows) return MOE_EINVAL;
  const size_t E = (size_t)p.E_r;
  MOE_TRY(after_launch(launch_fill_u32((uint32_t*)r->counts, 0u, E, st), d, st));
  MOE_TRY(after_launch(launch_fill_u32((uint32_t*)r->offsets, 0u, E + 1, st), d, st));
  MOE_TRY(after_launch(launch_fill_u32((uint32_t*)r->n_rows, 0u, 1, st), d, st));
  if (r->capacity) MOE_TRY(after_launch(launch_fill_u32((uint32_t*)r->capacity, 0u, 1, st), d, st));
  if (is_des(d)) {
    if (r->votes) MOE_TRY(after_launch(launch_fill_u32((uint32_t*)r->votes, 0u, E, st), d, st));
    const size_t ncore = d->mode == MOE_DES_SEQ ? E : (size_t)d->m_core;
    if (r->core) MOE_TRY(after_launch(launch_fill_u32((uint32_t*)r->core, 0xFFFFFFFFu, ncore, st), d, st));
  }
  return MOE_OK;
}

// Token rows, expert outputs and weights are read and written 16 bytes at a time (vector and
// global->LDS loads), so every such buffer must start on a 16-byte boundary (null: not used).
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

moe_status check_weights(const moe_desc* d, const moe_weights* w, bool need_router) {
  if (!w) return MOE_EINVAL;
  if (need_router && !w->w_router) return MOE_EINVAL;
  if (d->E_heavy > 0 && (!w->w1 || !w->w2 || (d->act == MOE_ACT_SWIGLU && !w->w3))) return MOE_EINVAL;
  if (d->n_shared > 0 && (!w->s_w1 || !w->s_w2 || (d->act == MOE_ACT_SWIGLU && !w->s_w3))) return MOE_EINVAL;
  if (d->n_const > 0 && !w->const_vec) return MOE_EINVAL;
  for (const void* p : {w->w_router, w->w1, w->w2, w->w3, w->s_w1, w->s_w2, w->s_w3, w->const_vec})
    if (!aligned16(p)) return MOE_EINVAL;
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_desc* desc) {
  Plan p;
  if (make_plan(desc, &p) != MOE_OK) return 0;
  return p.total;
}

moe_status moe_route(const moe_desc* desc, const float* logits, moe_routing* routing, void* ws, size_t ws_bytes,
                     void* stream) {
  Plan p;
  MOE_TRY(make_plan(desc, &p));
  if (desc->S == 0) return routing ? empty_routing(desc, p, routing, (hipStream_t)stream) : MOE_EINVAL;
  if (!logits) return MOE_EINVAL;
  MOE_TRY(check_routing(desc, routing));
  MOE_TRY(check_ws(p, ws, ws_bytes));
  return do_route(desc, p, logits, (desc->flags & MOE_F_INPUT_PROBS) != 0, routing, ws, (hipStream_t)stream);
}

moe_status moe_dispatch(const moe_desc* desc, const void* x, const moe_routing* routing, void* x_perm, void* stream) {
  Plan p;
  MOE_TRY(make_plan(desc, &p));
  if (desc->S == 0) return MOE_OK;
  if (!x || !x_perm || !routing || !routing->row_token || !routing->n_rows) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(x_perm)) return MOE_EINVAL;
  return after_launch(launch_gather(desc->dtype, x, routing->row_token, routing->n_rows, x_perm, (int)p.R_max,
                                    desc->d, (hipStream_t)stream),
                      desc, (hipStream_t)stream);
}

moe_status moe_expert_ffn(const moe_desc* desc, const void* x, const void* x_perm, const moe_routing* routing,
                          const moe_weights* weights, float* y_perm, float* y_shared, void* ws, size_t ws_bytes,
                          void* stream) {
  Plan p;
  MOE_TRY(make_plan(desc, &p));
  MOE_TRY(check_weights(desc, weights, false));
  if (desc->S == 0) return MOE_OK;
  if (!x) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(x_perm) || !aligned16(y_perm) || !aligned16(y_shared)) return MOE_EINVAL;
  if (desc->E_heavy > 0 && (!routing || !routing->offsets || !routing->row_token || !y_perm)) return MOE_EINVAL;
  if (desc->n_shared > 0 && !y_shared) return MOE_EINVAL;
  MOE_TRY(check_ws(p, ws, ws_bytes));
  return do_experts(desc, p, x, x_perm, routing, weights, y_perm, y_shared, ws, (hipStream_t)stream);
}

moe_status moe_combine(const moe_desc* desc, const void* x, const moe_routing* routing, const float* y_perm,
                       const float* y_shared, const void* const_vec, void* cache, const void* residual, void* y,
                       void* stream) {
  Plan p;
  MOE_TRY(make_plan(desc, &p));
  if (desc->S == 0) return MOE_OK;
  if (!x || !y || !routing) return MOE_EINVAL;
  for (const void* q : {x, (const void*)y_perm, (const void*)y_shared, const_vec, (const void*)cache, residual,
                        (const void*)y})
    if (!aligned16(q)) return MOE_EINVAL;
  if (desc->mode == MOE_EXPERT_CHOICE) {
    if (!routing->token_off || !routing->token_list || !routing->row_w) return MOE_EINVAL;
  } else {
    if (!routing->topk_idx || !routing->topk_w || !routing->token_rows) return MOE_EINVAL;
    if (desc->reuse_tau > 0.f && (!routing->reuse || !cache)) return MOE_EINVAL;
  }
  if (desc->E_heavy > 0 && !y_perm) return MOE_EINVAL;
  if (desc->n_shared > 0 && !y_shared) return MOE_EINVAL;
  if (desc->n_const > 0 && !const_vec) return MOE_EINVAL;
  return do_combine(desc, p, x, routing, y_perm, y_shared, const_vec, cache, residual, y, (hipStream_t)stream);
}

moe_status moe_layer_forward(const moe_desc* desc, const void* x, const moe_weights* weights, const float* prev_logits,
                             float* logits_out, moe_routing* routing, void* cache, const void* residual, void* y,
                             void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  MOE_TRY(make_plan(desc, &p));
  if (desc->flags & MOE_F_INPUT_PROBS) return MOE_EINVAL;
  MOE_TRY(check_weights(desc, weights, true));
  if (desc->S == 0) return empty_routing(desc, p, routing, (hipStream_t)stream);
  if (!x || !y) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(y) || !aligned16(cache) || !aligned16(residual)) return MOE_EINVAL;
  if (desc->reuse_tau > 0.f && !cache) return MOE_EINVAL;
  MOE_TRY(check_ws(p, ws, ws_bytes));
  moe_routing internal;
  if (routing) {
    MOE_TRY(check_routing(desc, routing));
  } else {
    internal = internal_routing(p, desc, ws);
    routing = &internal;
  }
  hipStream_t st = (hipStream_t)stream;
  uint8_t* w = (uint8_t*)ws;
  float* logits = logits_out ? logits_out : (float*)(w + p.o_logits);
  float* part = p.nsplit > 1 ? (float*)(w + p.o_rpart) : nullptr;
  MOE_TRY(after_launch(launch_router(desc->dtype == MOE_BF16 ? 0 : 1, x, weights->w_router, prev_logits, logits, part,
                                     p.nsplit, desc->S, desc->d, p.E_r, st),
                       desc, st));
  MOE_TRY(do_route(desc, p, logits, false, routing, ws, st, part, prev_logits));
  float* y_perm = (float*)(w + p.o_yp);
  float* y_shared = (float*)(w + p.o_ys);
  MOE_TRY(do_experts(desc, p, x, nullptr, routing, weights, y_perm, y_shared, ws, st));
  return do_combine(desc, p, x, routing, y_perm, y_shared, weights->const_vec, cache, residual, y, st);
}

moe_status moe_profile_begin(void) {
  if (prof::g_pool.empty()) {
    prof::g_pool.resize(2 * prof::kPoolPairs);
    for (auto& e : prof::g_pool)
      if (hipEventCreate(&e) != hipSuccess) {
        prof::g_pool.clear();
        return MOE_EHIP;
      }
  }
  prof::g_recs.clear();
  prof::g_entries.clear();
  prof::g_on = true;
  return MOE_OK;
}

int moe_profile_end(void) {
  prof::g_on = false;
  prof::g_entries.clear();
  for (const auto& r : prof::g_recs) {
    if (hipEventSynchronize(r.stop) != hipSuccess) return MOE_EHIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return MOE_EHIP;
    bool found = false;
    for (auto& e : prof::g_entries)
      if (e.name == r.name) {
        e.ms += ms;
        e.launches += 1;
        found = true;
        break;
      }
    if (!found) prof::g_entries.push_back({r.name, (double)ms, 1});
  }
  prof::g_recs.clear();
  return (int)prof::g_entries.size();
}

moe_status moe_profile_entry(int i, const char** name, double* total_ms, int32_t* launches) {
  if (i < 0 || i >= (int)prof::g_entries.size() || !name || !total_ms || !launches) return MOE_EINVAL;
  *name = prof::g_entries[i].name.c_str();
  *total_ms = prof::g_entries[i].ms;
  *launches = prof::g_entries[i].launches;
  return MOE_OK;
}

moe_status moe_attnres_aggregate(int32_t dtype, int32_t S, int32_t d, int32_t n, const void* const* states,
                                 const void* query, float eps, void* out, void* stream) {
  if (dtype != MOE_BF16 && dtype != MOE_F32) return MOE_EINVAL;
  if (S < 0 || d <= 0 || n < 1 || !states || !query || !out || !(eps >= 0.f) || !std::isfinite(eps))
    return MOE_EINVAL;
  if (n > kAttnMaxStates || !attnres_supported(dtype, d)) return MOE_EUNSUPPORTED;
  auto misaligned = [](const void* p) { return ((uintptr_t)p & 15u) != 0; };
  if (misaligned(query) || misaligned(out)) return MOE_EINVAL;
  AttnResArgs a{};
  for (int j = 0; j < n; ++j) {
    if (!states[j] || misaligned(states[j])) return MOE_EINVAL;
    a.states[j] = states[j];
  }
  a.query = query;
  a.out = out;
  a.n = n;
  a.S = S;
  a.d = d;
  a.eps = eps;
  return launch_attnres(dtype, a, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_EHIP;
}

const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported configuration";
    case MOE_EWORKSPACE: return "workspace too small or misaligned";
    case MOE_EHIP: return "HIP runtime or launch error";
    case MOE_ESCRATCH: return "the call needs more scratch than the no-allocation entry point's static buffer holds";
    default: return "unknown status";
  }
}

}  // extern "C"
