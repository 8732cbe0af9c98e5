// Internal launchers of the MoE layer library (host side). Not part of the C ABI.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------------------------------------
// Launch-time profiling (off by default). While on, every launch gets a start/stop event pair
// attached to its dispatch on the launch stream; the pairs are read back by moe_profile_end.
namespace prof {
bool enabled();
// Next free event pair for a launch named `name`; false when the pool is exhausted.
bool take(const char* name, hipEvent_t* start, hipEvent_t* stop);
}  // namespace prof

#define MOE_LAUNCH(name, kernel, grid, block, shmem, stream, ...)                                   \
  do {                                                                                              \
    hipEvent_t moe_ev0_, moe_ev1_;                                                                  \
    if (::moe::prof::enabled() && ::moe::prof::take((name), &moe_ev0_, &moe_ev1_))                  \
      hipExtLaunchKernelGGL((kernel), dim3(grid), dim3(block), (shmem), (stream), moe_ev0_, moe_ev1_, \
                            0, __VA_ARGS__);                                                        \
    else                                                                                            \
      hipLaunchKernelGGL((kernel), dim3(grid), dim3(block), (shmem), (stream), __VA_ARGS__);         \
  } while (0)

// ---------------------------------------------------------------------------------------------
// Router: logits[S, E] = x[S, d] . W_r[E, d]^T (+ prev[S, E]). With nsplit = router_splits(...) > 1
// the router writes nsplit partial sums over K to part[nsplit][S][E] instead; logits are then
// (their sum in split order) + prev, formed by launch_router_sum or by the one-workgroup routing.
int router_splits(int dtype, int S, int d, int E);
hipError_t launch_router(int dtype, const void* x, const void* w_router, const float* prev, float* logits,
                         float* part, int nsplit, int S, int d, int E, hipStream_t st);
hipError_t launch_router_sum(const float* part, int nsplit, const float* prev, float* logits, int n,
                             hipStream_t st);

// ---------------------------------------------------------------------------------------------
// Routing.
struct RouteArgs {
  int S, E_r, E_heavy, k, renorm, input_probs;
  int n_identity, n_zero, n_const;
  float tau;
  int vote_k, m_core;      // DES-Vote: filter K, core size; DES-Seq: vote_k = local count k_seq
  int seq;                 // 1: DES-Seq (core = union of the top-vote_k sets; its size is found here)
  const float* keys;       // logits [S,E_r] or probabilities (input_probs)
  float* probs;            // [S,E_r] out (nullable)
  int32_t* topk_idx;       // [S,k]
  float* topk_w;           // [S,k]
  uint8_t* reuse;          // [S] (nullable when tau == 0)
  float* votes;            // DES [E_r]: summed filtered probabilities (DES-Vote) or selection counts (DES-Seq)
  int32_t* core;           // DES-Vote [m_core]; DES-Seq [E_r], the union ascending then -1
  // one-workgroup routing only: with part set, keys = (sum of nsplit router partial sums, in split
  // order) + prev, written to logits
  const float* part;       // [nsplit][S][E_r] (nullable)
  int nsplit;
  const float* prev;       // [S][E_r] (nullable)
  float* logits;           // [S][E_r]
};
hipError_t launch_route_topk(const RouteArgs& a, hipStream_t st);
hipError_t launch_route_des(const RouteArgs& a, float* ws_filt /* [S,E_r] */, hipStream_t st);

// Counting sort of (token, slot) pairs to heavy experts (token choice / DES).
struct PermuteArgs {
  int S, k, E_r, E_heavy;
  const int32_t* topk_idx;
  const float* topk_w;
  const uint8_t* reuse;    // nullable
  int32_t* counts;         // [E_r]
  int32_t* offsets;        // [E_r+1]
  int32_t* row_token;      // [S*k]
  float* row_w;            // [S*k]
  int32_t* token_rows;     // [S*k]
  int32_t* n_rows;         // [1]
  int32_t* blk_cnt;        // scratch [nblk * E_heavy]
};
int permute_num_blocks(int S, int k);
hipError_t launch_permute(const PermuteArgs& a, hipStream_t st);

// Token choice or DES routing plus the dispatch of PermuteArgs, in one workgroup, for small calls
// (route_small_supported). For DES, a.k is the requested k (min(k, core size) is applied); the
// slot stride of topk_idx / topk_w / token_rows is q.k (min(k, m_core) for DES-Vote, k for DES-Seq).
bool route_small_supported(int S, int E_r, int k);
hipError_t launch_route_small(const RouteArgs& a, const PermuteArgs& q, bool des, hipStream_t st);

// Expert choice.
struct ECArgs {
  int S, E, C, input_probs;
  const float* keys;       // logits or probabilities [S,E]
  float* probs;            // [S,E] out (nullable)
  float* pT;               // scratch [E,S]
  int32_t* tok_rows_tmp;   // scratch [E,S]: the token's row for the expert, or -1
  int32_t* tok_cnt;        // scratch [S]: experts that took the token
  int32_t* counts;         // [E]
  int32_t* offsets;        // [E+1]
  int32_t* row_token;      // [E*C]
  float* row_w;            // [E*C]
  int32_t* token_off;      // [S+1]
  int32_t* token_list;     // [E*C]
  int32_t* n_rows;         // [1]
  int32_t* capacity;       // [1] (nullable)
};
hipError_t launch_route_ec(const ECArgs& a, hipStream_t st);

// ---------------------------------------------------------------------------------------------
// Dispatch / combine.
hipError_t launch_gather(int dtype, const void* x, const int32_t* row_token, const int32_t* n_rows, void* x_perm,
                         int R_max, int d, hipStream_t st);

struct CombineArgs {
  int dtype, mode, S, d, k, E_heavy, n_identity, n_zero, n_const;
  const void* x;
  const int32_t* topk_idx;
  const float* topk_w;
  const int32_t* token_rows;
  const int32_t* token_off;
  const int32_t* token_list;
  const float* row_w;
  const uint8_t* reuse;     // nullable
  const float* y_perm;
  const float* y_shared;    // nullable
  const void* const_vec;    // nullable
  void* cache;              // nullable
  const void* residual;     // nullable
  void* y;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t st);

// ---------------------------------------------------------------------------------------------
// Grouped GEMMs.
//
// One problem: groups g = 0..G-1 of rows. Group g's rows are [offsets[g], offsets[g+1]) of the
// output (offsets != null; data-dependent, read on the device), or rows [0, M_uni) (offsets == null).
//   A row of output row r: a_rows ? a_rows[r] : r      (row of A, length K, stride lda)
//   B: weights of group g at B + g*b_gstride, row n at + n*ldb; K split into segments of k_seg
//      elements placed k_seg_stride apart (a K-concatenation of several experts' weights).
//   C: row r, column g*c_gcol + n, stride ldc.
struct GemmProblem {
  const void* A; const int32_t* a_rows; int64_t lda;
  const void* B; const void* B3; int64_t ldb; int64_t b_gstride;
  int64_t k_seg, k_seg_stride;
  void* C; int64_t ldc; int64_t c_gcol;
  const int32_t* offsets; int32_t G, M_uni;
  int32_t N, K;            // N = output columns per group
};
enum { GEMM_UP = 0, GEMM_DOWN = 1 };
// kind GEMM_UP: C (dtype) = act(A.B^T) (SwiGLU: silu(A.B3^T) * (A.B^T)); GEMM_DOWN: C (fp32) = A.B^T.
// `rows_ub[i]` bounds the total rows of problem i (for the grid); `mt_hint[i]` (may be null) is the
// expected number of 256-row tiles of problem i, used to choose the tile width.
hipError_t launch_grouped_gemm(int dtype, int kind, int act, const GemmProblem* probs, const int64_t* rows_ub,
                               const int64_t* mt_hint, int nprob, hipStream_t st);
bool grouped_gemm_supported(int dtype, int kind, int act, int N, int K);

// Weight-streaming grouped GEMM for few rows per expert; grid.y = max_active bounds the number
// of experts with rows (offsets-based problems only); pass_rows (32 or 64) is the number of an
// expert's rows that one pass over its weights serves.
hipError_t launch_stream_gemm(int dtype, int kind, int act, const GemmProblem& p, int max_active, int pass_rows,
                              hipStream_t st);
bool stream_gemm_supported(int dtype, int kind, int act, int N, int K);

hipError_t launch_fill_u32(uint32_t* p, uint32_t v, size_t n, hipStream_t st);

// ---------------------------------------------------------------------------------------------
// Attention-residual aggregation: out[s] = sum_j softmax_j(q . v_j[s] / rms(v_j[s]))_j v_j[s] over
// n states of [S, d] (dtype), per token.
constexpr int kAttnMaxStates = 64;
struct AttnResArgs {
  const void* states[kAttnMaxStates];
  const void* query;   // [d]
  void* out;           // [S, d]
  int32_t n, S, d;
  float eps;
};
bool attnres_supported(int dtype, int d);
hipError_t launch_attnres(int dtype, const AttnResArgs& a, hipStream_t st);

}  // namespace moe
