// Expert-choice routing: every expert takes the C tokens with the highest affinity.
//
// "EC-DiT: Scaling Diffusion Transformers with Adaptive Expert-Choice Routing", 三 技术架构 / 核心公式:
// A = softmax over experts of x' W_r, each expert picks its top tokens, which balances the load by
// construction and lets a token receive a variable number of experts; 容量因子: the capacity is
// f_c * S / E (rounded down here, clipped to S).
//
// Kernels: (1) per block of 64 tokens (4 lanes per token), the probabilities, staged through LDS so
// that both the token-major output and the expert-major copy pT[E][S] are written with coalesced
// stores; (2) one workgroup per expert: exact radix select of the C-th largest key (the fp32 bit
// pattern orders non-negative floats; 8-bit digits from the highest bit in which the expert's keys
// differ, one LDS histogram atomic per key), then a
// stable compaction in token order (equal keys: lowest token first) from one workgroup-wide scan;
// every token's row for the expert (or -1) goes to rowsT[E][S] and the token's expert count is
// incremented; (3) the per-token row lists (CSR, ascending expert) for the combine.
#include <float.h>

#include "common.hpp"
#include "internal.hpp"

extern "C" __device__ __attribute__((const)) unsigned int __ockl_wfred_and_u32(unsigned int);
extern "C" __device__ __attribute__((const)) unsigned int __ockl_wfred_or_u32(unsigned int);

namespace moe {

constexpr int kProbTok = 64;       // tokens per probability workgroup
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

constexpr int kProbLanes = 4;   // lanes per token (expert e handled by lane e % 4 of its group)

__global__ __launch_bounds__(kProbTok * kProbLanes) void k_ec_probs(ECArgs a) {
  __shared__ float s_blk[kProbTok * 257];   // [token][expert], row stride E + 1
  constexpr int NT = kProbTok * kProbLanes;
  const int E = a.E, ld = E + 1;
  const int s0 = blockIdx.x * kProbTok;
  const int ns = min(kProbTok, a.S - s0);
  const float* kb = a.keys + (size_t)s0 * E;
  // eight loads in flight per thread (the index is clamped rather than the load skipped, so that the
  // compiler does not wait for each one before its LDS store)
  const int n = ns * E;
  for (int i0 = threadIdx.x; i0 < n; i0 += 8 * NT) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = kb[min(i0 + j * NT, n - 1)];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + j * NT;
      if (i < n) s_blk[(i / E) * ld + i % E] = v[j];
    }
  }
  __syncthreads();
  const int t = threadIdx.x / kProbLanes, q = threadIdx.x % kProbLanes;
  if (!a.input_probs) {   // uniform: all lanes of a group take part in the shuffles
    float* row = s_blk + min(t, ns - 1) * ld;
    float m = -FLT_MAX;
    for (int e = q; e < E; e += kProbLanes) m = fmaxf(m, row[e]);
    m = fmaxf(m, __shfl_xor(m, 1, 64));
    m = fmaxf(m, __shfl_xor(m, 2, 64));
    float z = 0.f;
    for (int e = q; e < E; e += kProbLanes) z += expf(row[e] - m);
    z += __shfl_xor(z, 1, 64);
    z += __shfl_xor(z, 2, 64);
    const float inv = 1.0f / z;
    __syncthreads();
    if (t < ns)
      for (int e = q; e < E; e += kProbLanes) row[e] = expf(row[e] - m) * inv;
    __syncthreads();
  }
  if (a.probs) {
    float* pb = a.probs + (size_t)s0 * E;
    for (int i = threadIdx.x; i < ns * E; i += NT) pb[i] = s_blk[(i / E) * ld + i % E];
  }
  for (int i = threadIdx.x; i < E * kProbTok; i += NT) {
    const int e = i / kProbTok, tt = i % kProbTok;
    if (tt < ns) a.pT[(size_t)e * a.S + s0 + tt] = s_blk[tt * ld + e];
  }
  if ((int)threadIdx.x < ns) a.tok_cnt[s0 + threadIdx.x] = 0;   // experts per token, counted by k_ec_select
}

// Exclusive prefix over the workgroup (threads in order) of two counts, and their totals.
__device__ __forceinline__ void block_scan2(int x, int y, int* s_w, int& xb, int& yb, int& xt, int& yt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int vx = x, vy = y;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int tx = __shfl_up(vx, o, 64), ty = __shfl_up(vy, o, 64);
    if (lane >= o) {
      vx += tx;
      vy += ty;
    }
  }
  if (lane == 63) {
    s_w[2 * wave] = vx;
    s_w[2 * wave + 1] = vy;
  }
  __syncthreads();
  int bx = 0, by = 0, tx = 0, ty = 0;
  for (int w = 0; w < kSelWaves; ++w) {
    const int cx = s_w[2 * w], cy = s_w[2 * w + 1];
    if (w < wave) {
      bx += cx;
      by += cy;
    }
    tx += cx;
    ty += cy;
  }
  __syncthreads();
  xb = bx + vx - x;
  yb = by + vy - y;
  xt = tx;
  yt = ty;
}

// Thread t owns the tokens [t * per, (t + 1) * per), per = ceil(S / kSelThreads). With REG, per <=
// kSelRegs and the keys stay in registers across the radix passes.
constexpr int kSelRegs = 16;

template <bool REG>
__global__ __launch_bounds__(kSelThreads) void k_ec_select(ECArgs a) {
  __shared__ int hist[256];
  __shared__ int s_sel, s_rem;
  __shared__ int s_w[2 * kSelWaves];
  __shared__ uint32_t s_bits[2 * kSelWaves];
  const int e = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const uint32_t* keys = reinterpret_cast<const uint32_t*>(a.pT + (size_t)e * a.S);
  const int per = (a.S + kSelThreads - 1) / kSelThreads;
  const int s_beg = min(a.S, (int)threadIdx.x * per), s_end = min(a.S, s_beg + per);
  uint32_t ureg[REG ? kSelRegs : 1];
  if constexpr (REG) {
#pragma unroll
    for (int j = 0; j < kSelRegs; ++j) ureg[j] = (j < per && s_beg + j < s_end) ? keys[s_beg + j] : 0u;
  }
  auto key = [&](int j) -> uint32_t {
    if constexpr (REG) return ureg[j];
    else return keys[s_beg + j];
  };
  // Bits in which every key of the expert agrees (where the AND and the OR of the keys are equal)
  // hold the same value in the C-th largest key. The 8-bit digits therefore start just below the
  // highest bit in which keys differ: with probabilities of one magnitude the top byte is the same
  // for every key, and a first histogram over it would send every LDS atomic to one bin, where
  // they serialise. Later digits may overlap bits already fixed; keys that pass the prefix test
  // agree there, so the bins stay exact.
  uint32_t k_and = ~0u, k_or = 0u;
#pragma unroll
  for (int j = 0; j < (REG ? kSelRegs : 1); ++j) {
    for (int jj = REG ? j : 0; jj < (REG ? j + 1 : per); ++jj) {
      if (REG && j >= per) break;
      if (s_beg + jj < s_end) {
        const uint32_t u = key(jj);
        k_and &= u;
        k_or |= u;
      }
    }
  }
  k_and = __ockl_wfred_and_u32(k_and);
  k_or = __ockl_wfred_or_u32(k_or);
  const int wave = threadIdx.x >> 6;
  if (lane == 0) {
    s_bits[2 * wave] = k_and;
    s_bits[2 * wave + 1] = k_or;
  }
  __syncthreads();
  k_and = ~0u;
  k_or = 0u;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    k_and &= s_bits[2 * w];
    k_or |= s_bits[2 * w + 1];
  }
  const uint32_t diff = k_and ^ k_or;   // 0: every key is the same (S >= C >= 1 keys exist)
  const int hb = diff ? 31 - __clz((int)diff) : -1;
  // bits above the highest differing one (all of them when every key is the same)
  const uint32_t fixed = hb < 0 ? ~0u : hb >= 31 ? 0u : ~((2u << hb) - 1u);
  uint32_t prefix = k_and & fixed, pmask = fixed;
  int remaining = a.C;
  for (int shift = max(hb - 7, 0); hb >= 0; shift = max(shift - 8, 0)) {
    for (int i = threadIdx.x; i < 256; i += kSelThreads) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < (REG ? kSelRegs : 1); ++j) {
      for (int jj = REG ? j : 0; jj < (REG ? j + 1 : per); ++jj) {
        if (REG && j >= per) break;
        const bool valid = s_beg + jj < s_end;
        const uint32_t u = valid ? key(jj) : 0u;
        // one LDS atomic per key: lanes that hit the same bin serialise in the LDS, which costs less
        // than matching equal bins over the wave first (30 against 18 us on 32 x 8192 keys)
        if (valid && (u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1);
      }
    }
    __syncthreads();
    // the bin holding the remaining-th largest key: wave 0 scans the bins from the top
    if (threadIdx.x < 64) {
      int v[4], run = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] = hist[255 - 4 * lane - j];
        run += v[j];
      }
      int incl = run;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      int above = incl - run;   // keys in bins above this lane's first bin
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (above < remaining && above + v[j] >= remaining) {
          s_sel = 255 - 4 * lane - j;
          s_rem = remaining - above;
        }
        above += v[j];
      }
    }
    __syncthreads();
    prefix |= (uint32_t)s_sel << shift;
    pmask |= 255u << shift;
    remaining = s_rem;
    __syncthreads();
    if (shift == 0) break;
  }
  const uint32_t T = prefix;      // the C-th largest key
  const int need_eq = remaining;  // keys equal to T to take, lowest tokens first
  int n_gt = 0, n_eq = 0;
  for (int j = 0; j < s_end - s_beg; ++j) {
    const uint32_t u = key(j);
    n_gt += u > T ? 1 : 0;
    n_eq += u == T ? 1 : 0;
  }
  int gt_before, eq_before, gt_tot, eq_tot;
  block_scan2(n_gt, n_eq, s_w, gt_before, eq_before, gt_tot, eq_tot);
  int eq_rank = eq_before;
  int pos = gt_before + min(eq_before, need_eq);
  int32_t* rows_e = a.tok_rows_tmp + (size_t)e * a.S;
  for (int j = 0; j < s_end - s_beg; ++j) {
    const int s = s_beg + j;
    const uint32_t u = key(j);
    bool take = u > T;
    if (u == T) take = eq_rank++ < need_eq;
    int row = -1;
    if (take) {
      row = e * a.C + pos++;
      a.row_token[row] = s;
      a.row_w[row] = __uint_as_float(u);
      atomicAdd(&a.tok_cnt[s], 1);
    }
    rows_e[s] = row;
  }
}

// Every token's rows in ascending expert order (CSR), kCsrTok tokens per workgroup: the offset of
// the workgroup's first token is the sum of the counts before it (read directly: S ints), then a
// workgroup scan; the first workgroup also writes the fixed per-expert counts / offsets.
constexpr int kCsrTok = 256;
constexpr int kCsrPre = 32;   // experts whose row entries a thread loads before anything else

__global__ __launch_bounds__(kCsrTok) void k_ec_csr(ECArgs a) {
  __shared__ int s_w[2 * (kCsrTok / 64)];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int s0 = blockIdx.x * kCsrTok;
  // this token's rows of the first kCsrPre experts go out first, with the count loads below
  const int sc = min(s0 + (int)threadIdx.x, a.S - 1);
  int pre[kCsrPre];
#pragma unroll
  for (int j = 0; j < kCsrPre; ++j) pre[j] = a.tok_rows_tmp[(size_t)min(j, a.E - 1) * a.S + sc];
  const int s = s0 + threadIdx.x;
  const int c_raw = a.tok_cnt[sc];
  int before = 0;
  // 32 loads in flight per round (s0 is a multiple of kCsrTok, so the masks are uniform over the
  // workgroup; the masked ones read a valid count and add nothing)
  for (int i0 = 0; i0 < s0; i0 += 32 * kCsrTok) {
    int v[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = a.tok_cnt[min(i0 + j * kCsrTok, s0 - kCsrTok) + threadIdx.x];
#pragma unroll
    for (int j = 0; j < 32; ++j) before += i0 + j * kCsrTok < s0 ? v[j] : 0;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) before += __shfl_xor(before, o, 64);
  const int c = s < a.S ? c_raw : 0;
  int incl = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 0) s_w[wave] = before;
  if (lane == 63) s_w[kCsrTok / 64 + wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < kCsrTok / 64; ++w) base += s_w[w];   // the prefix before s0, summed by all waves
  for (int w = 0; w < wave; ++w) base += s_w[kCsrTok / 64 + w];
  int pos = base + incl - c;
  if (s < a.S) {
    a.token_off[s] = pos;
#pragma unroll
    for (int j = 0; j < kCsrPre; ++j)
      if (j < a.E && pre[j] >= 0) a.token_list[pos++] = pre[j];
    for (int e0 = kCsrPre; e0 < a.E; e0 += 8) {   // eight loads in flight, then the writes in expert order
      int r[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) r[j] = e0 + j < a.E ? a.tok_rows_tmp[(size_t)(e0 + j) * a.S + s] : -1;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (r[j] >= 0) a.token_list[pos++] = r[j];
    }
    if (s == a.S - 1) a.token_off[a.S] = pos;
  }
  if (blockIdx.x == 0) {
    for (int e = threadIdx.x; e < a.E; e += kCsrTok) {
      a.counts[e] = a.C;
      a.offsets[e] = e * a.C;
    }
    if (threadIdx.x == 0) {
      a.offsets[a.E] = a.E * a.C;
      *a.n_rows = a.E * a.C;
      if (a.capacity) *a.capacity = a.C;
    }
  }
}

hipError_t launch_route_ec(const ECArgs& a, hipStream_t st) {
  if (a.E > 256) return hipErrorInvalidValue;
  auto k1 = k_ec_probs;
  MOE_LAUNCH("ec_probs", k1, (a.S + kProbTok - 1) / kProbTok, kProbTok * kProbLanes, 0, st, a);
  if ((a.S + kSelThreads - 1) / kSelThreads <= kSelRegs) {
    auto k2 = k_ec_select<true>;
    MOE_LAUNCH("ec_select", k2, a.E, kSelThreads, 0, st, a);
  } else {
    auto k2 = k_ec_select<false>;
    MOE_LAUNCH("ec_select", k2, a.E, kSelThreads, 0, st, a);
  }
  auto k3 = k_ec_csr;
  MOE_LAUNCH("ec_csr", k3, (a.S + kCsrTok - 1) / kCsrTok, kCsrTok, 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
