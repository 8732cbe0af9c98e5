// Expert-choice routing: every expert takes the C tokens with the highest affinity.
//
// "EC-DiT: Scaling Diffusion Transformers with Adaptive Expert-Choice Routing", 三 技术架构 / 核心公式:
// A = softmax over experts of x' W_r, each expert picks its top tokens, which balances the load by
// construction and lets a token receive a variable number of experts; 容量因子: the capacity is
// f_c * S / E (rounded down here, clipped to S).
//
// Kernels: (1) per token, the probabilities, stored expert-major pT[E][S]; (2) one workgroup per
// expert: exact radix select of the C-th largest key (the fp32 bit pattern orders non-negative
// floats), then a stable compaction in token order (equal keys: lowest token first); (3) the
// per-token row lists (CSR, ascending expert) for the combine.
#include <float.h>

#include "common.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kECMaxE = 256;
constexpr int kSelThreads = 1024;

__global__ __launch_bounds__(256) void k_ec_probs(ECArgs a) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s >= a.S) return;
  const float* row = a.keys + (size_t)s * a.E;
  if (a.input_probs) {
    for (int e = 0; e < a.E; ++e) {
      const float p = row[e];
      a.pT[(size_t)e * a.S + s] = p;
      if (a.probs) a.probs[(size_t)s * a.E + e] = p;
    }
    return;
  }
  float m = -FLT_MAX;
  for (int e = 0; e < a.E; ++e) m = fmaxf(m, row[e]);
  float z = 0.f;
  for (int e = 0; e < a.E; ++e) z += expf(row[e] - m);
  const float inv = 1.0f / z;
  for (int e = 0; e < a.E; ++e) {
    const float p = expf(row[e] - m) * inv;
    a.pT[(size_t)e * a.S + s] = p;
    if (a.probs) a.probs[(size_t)s * a.E + e] = p;
  }
}

// Exclusive prefix of a 0/1 flag over the workgroup (threads in order), and the total.
__device__ __forceinline__ int block_flag_scan(bool f, int* s_w, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const uint64_t m = __ballot(f);
  const int in_wave = __popcll(m & lanemask_lt());
  if (lane == 0) s_w[wave] = __popcll(m);
  __syncthreads();
  int before = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    const int c = s_w[w];
    before += (w < wave) ? c : 0;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return before + in_wave;
}

__global__ __launch_bounds__(kSelThreads) void k_ec_select(ECArgs a) {
  __shared__ int hist[256];
  __shared__ int s_sel, s_rem;
  __shared__ int s_w[kSelThreads / 64];
  const int e = blockIdx.x;
  const uint32_t* keys = reinterpret_cast<const uint32_t*>(a.pT + (size_t)e * a.S);
  uint32_t prefix = 0, pmask = 0;
  int remaining = a.C;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    for (int s = threadIdx.x; s < a.S; s += kSelThreads) {
      const uint32_t u = keys[s];
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int cum = 0, sel = 0;
      for (int b = 255; b >= 0; --b) {
        if (cum + hist[b] >= remaining) { sel = b; break; }
        cum += hist[b];
      }
      s_sel = sel;
      s_rem = remaining - cum;
    }
    __syncthreads();
    prefix |= (uint32_t)s_sel << shift;
    pmask |= 255u << shift;
    remaining = s_rem;
    __syncthreads();
  }
  const uint32_t T = prefix;      // the C-th largest key
  const int need_eq = remaining;  // keys equal to T still to take (lowest tokens first)
  const int mw = (a.E + 31) >> 5;
  int eq_base = 0, take_base = 0;
  for (int base = 0; base < a.S; base += kSelThreads) {
    const int s = base + threadIdx.x;
    const uint32_t u = s < a.S ? keys[s] : 0u;
    const bool gt = s < a.S && u > T;
    const bool eq = s < a.S && u == T;
    int eq_tot, take_tot;
    const int eq_rank = eq_base + block_flag_scan(eq, s_w, eq_tot);
    const bool take = gt || (eq && eq_rank < need_eq);
    const int pos = take_base + block_flag_scan(take, s_w, take_tot);
    if (take) {
      const int row = e * a.C + pos;
      a.row_token[row] = s;
      a.row_w[row] = __uint_as_float(u);
      a.tok_rows_tmp[(size_t)s * a.E + e] = row;
      atomicOr(&a.tok_mask[(size_t)s * mw + (e >> 5)], 1u << (e & 31));
    }
    eq_base += eq_tot;
    take_base += take_tot;
  }
}

// One workgroup: CSR offsets of every token's rows, plus the fixed per-expert counts/offsets.
__global__ __launch_bounds__(kSelThreads) void k_ec_csr_scan(ECArgs a) {
  __shared__ int s_w[kSelThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int mw = (a.E + 31) >> 5;
  int run = 0;
  for (int base = 0; base < a.S; base += kSelThreads) {
    const int s = base + threadIdx.x;
    int c = 0;
    if (s < a.S)
      for (int w = 0; w < mw; ++w) c += __popc(a.tok_mask[(size_t)s * mw + w]);
    // inclusive wave scan
    int v = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(v, o, 64);
      if (lane >= o) v += t;
    }
    if (lane == 63) s_w[wave] = v;
    __syncthreads();
    int before = 0, tot = 0;
    for (int w = 0; w < kSelThreads / 64; ++w) {
      before += (w < wave) ? s_w[w] : 0;
      tot += s_w[w];
    }
    __syncthreads();
    if (s < a.S) a.token_off[s] = run + before + v - c;
    run += tot;
  }
  if (threadIdx.x == 0) a.token_off[a.S] = run;
  for (int e = threadIdx.x; e < a.E; e += kSelThreads) {
    a.counts[e] = a.C;
    a.offsets[e] = e * a.C;
  }
  if (threadIdx.x == 0) {
    a.offsets[a.E] = a.E * a.C;
    *a.n_rows = a.E * a.C;
    if (a.capacity) *a.capacity = a.C;
  }
}

__global__ __launch_bounds__(256) void k_ec_csr_fill(ECArgs a) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s >= a.S) return;
  const int mw = (a.E + 31) >> 5;
  int pos = a.token_off[s];
  for (int w = 0; w < mw; ++w) {
    uint32_t m = a.tok_mask[(size_t)s * mw + w];
    while (m) {
      const int b = __ffs(m) - 1;
      m &= m - 1;
      const int e = w * 32 + b;
      a.token_list[pos++] = a.tok_rows_tmp[(size_t)s * a.E + e];
    }
  }
}

hipError_t launch_route_ec(const ECArgs& a, hipStream_t st) {
  const int mw = (a.E + 31) >> 5;
  hipError_t err = launch_fill_u32(a.tok_mask, 0u, (size_t)a.S * mw, st);
  if (err != hipSuccess) return err;
  auto k1 = k_ec_probs;
  MOE_LAUNCH("ec_probs", k1, (a.S + 255) / 256, 256, 0, st, a);
  auto k2 = k_ec_select;
  MOE_LAUNCH("ec_select", k2, a.E, kSelThreads, 0, st, a);
  auto k3 = k_ec_csr_scan;
  MOE_LAUNCH("ec_csr_scan", k3, 1, kSelThreads, 0, st, a);
  auto k4 = k_ec_csr_fill;
  MOE_LAUNCH("ec_csr_fill", k4, (a.S + 255) / 256, 256, 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
