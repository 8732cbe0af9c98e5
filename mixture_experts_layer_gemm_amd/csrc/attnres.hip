// Attention-residual aggregation over block states.
//
// "MMOE: Modernizing Diffusion Transformers with Efficient Expert Design", 方法论: before a
// sub-layer, a learned pseudo-query aggregates the completed block states (kept, with the current
// partial state, as the forward's recurrent state). Per token s, with the states v_j in the order
// given (the completed ones, then the partial one):
//   z_j = q . v_j / sqrt(mean(v_j^2) + eps),  alpha = softmax_j(z),  out_s = sum_j alpha_j v_j.
//
// HBM-bound: every state row is read once. One wave per token streams the states in order with
// an online softmax (running maximum m and sum l; the fp32 accumulator is rescaled by e^(m_old -
// m_new) when the maximum grows), so nothing is read twice; the next state's row is loaded before
// the current one is reduced. Lane l holds the 16-byte chunks l, l + 64, ... of the row (1 KB
// contiguous per wave-wide load); the two per-state sums (q . v and v . v) are wave reductions.
#include "common.hpp"
#include "internal.hpp"

// Wave-wide sum of the device library (DPP based; every lane of the wave must be active).
extern "C" __device__ __attribute__((const)) float __ockl_wfred_add_f32(float);

namespace moe {

constexpr int kAttnTokPerBlock = 4;   // one wave per token

template <typename T, int MAXC>
__global__ __launch_bounds__(64 * kAttnTokPerBlock) void k_attnres(AttnResArgs a) {
  constexpr int EPC = Elem<T>::kPer16B;
  const int lane = threadIdx.x & 63;
  const int s = blockIdx.x * kAttnTokPerBlock + (int)(threadIdx.x >> 6);
  if (s >= a.S) return;   // the whole wave: s is uniform over it
  const int nch = a.d / EPC;
  const size_t row_off = (size_t)s * a.d;

  float q[MAXC][EPC], acc[MAXC][EPC], cur[MAXC][EPC];
  uint4 nxt[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) unpack16(*reinterpret_cast<const uint4*>((const T*)a.query + (size_t)c * EPC), q[i], T());
    else
#pragma unroll
      for (int e = 0; e < EPC; ++e) q[i][e] = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[i][e] = 0.f;
  }
  auto load_row = [&](int j) {
    const T* row = (const T*)a.states[j] + row_off;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int c = lane + 64 * i;
      nxt[i] = c < nch ? *reinterpret_cast<const uint4*>(row + (size_t)c * EPC) : make_uint4(0, 0, 0, 0);
    }
  };
  const float inv_d = 1.0f / (float)a.d;
  float m = -INFINITY, l = 0.f;
  load_row(0);
  for (int j = 0; j < a.n; ++j) {
#pragma unroll
    for (int i = 0; i < MAXC; ++i) unpack16(nxt[i], cur[i], T());
    if (j + 1 < a.n) load_row(j + 1);
    float dot = 0.f, ss = 0.f;
#pragma unroll
    for (int i = 0; i < MAXC; ++i)
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        dot = fmaf(q[i][e], cur[i][e], dot);
        ss = fmaf(cur[i][e], cur[i][e], ss);
      }
    dot = __ockl_wfred_add_f32(dot);
    ss = __ockl_wfred_add_f32(ss);
    const float z = dot / sqrtf(fmaf(ss, inv_d, a.eps));
    const float m_new = fmaxf(m, z);
    const float scale = fast_exp(m - m_new);   // 0 for the first state (m = -inf)
    const float p = fast_exp(z - m_new);
    l = fmaf(l, scale, p);
#pragma unroll
    for (int i = 0; i < MAXC; ++i)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[i][e] = fmaf(acc[i][e], scale, p * cur[i][e]);
    m = m_new;
  }
  const float inv_l = 1.0f / l;
  T* out = (T*)a.out + row_off;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = lane + 64 * i;
    if (c >= nch) continue;
    float o[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) o[e] = acc[i][e] * inv_l;
    *reinterpret_cast<uint4*>(out + (size_t)c * EPC) = pack16(o, T());
  }
}

template <typename T, int MAXC>
static void attnres_t(const AttnResArgs& a, hipStream_t st) {
  const int grid = (a.S + kAttnTokPerBlock - 1) / kAttnTokPerBlock;
  auto kfn = k_attnres<T, MAXC>;
  MOE_LAUNCH("attnres", kfn, grid, 64 * kAttnTokPerBlock, 0, st, a);
}

// Chunks per lane: the smallest of 1, 2, 3, 4, 8, 16 that covers the row (registers scale with it).
template <typename T>
static hipError_t attnres_dt(const AttnResArgs& a, hipStream_t st) {
  const int per = (a.d / Elem<T>::kPer16B + 63) / 64;
  if (per <= 1) attnres_t<T, 1>(a, st);
  else if (per <= 2) attnres_t<T, 2>(a, st);
  else if (per <= 3) attnres_t<T, 3>(a, st);
  else if (per <= 4) attnres_t<T, 4>(a, st);
  else if (per <= 8) attnres_t<T, 8>(a, st);
  else if (per <= 16) attnres_t<T, 16>(a, st);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

bool attnres_supported(int dtype, int d) {
  const int epc = dtype == 0 ? 8 : 4;
  return d > 0 && d % epc == 0 && (d / epc + 63) / 64 <= (dtype == 0 ? 8 : 16);
}

hipError_t launch_attnres(int dtype, const AttnResArgs& a, hipStream_t st) {
  if (a.S <= 0) return hipSuccess;
  if (a.n < 1 || a.n > kAttnMaxStates || !attnres_supported(dtype, a.d)) return hipErrorInvalidValue;
  return dtype == 0 ? attnres_dt<bf16_t>(a, st) : attnres_dt<float>(a, st);
}

}  // namespace moe
