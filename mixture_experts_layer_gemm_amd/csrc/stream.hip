// Weight-streaming grouped GEMM for experts that receive only a few rows.
//
// In a DES decode block each active expert serves ~N*k/M_core rows (8-32), so its time is the
// fetch of its weights from HBM: "Dynamic Expert Sharing: Decoupling Memory from Parallelism in
// Mixture-of-Experts Diffusion LLMs", 2.1 (per-expert latency a*c + b, b the HBM weight fetch;
// the block latency is dominated by b times the number of distinct experts loaded). This kernel
// reads every weight byte of an active expert exactly once and keeps the MFMA work beside it.
//
// Layout: workgroup (x = 64-column slice, y = active-expert slot), 4 waves, each wave owns 16
// output columns (16 weight rows; 32 for SwiGLU gate+up) and the full K. Weight rows are MFMA
// operand P streamed straight from HBM (16-byte loads, 8 steps in flight); the expert's token rows
// (operand Q, gathered through row_token) come from L2, 32 rows per pass. Experts with no rows are
// skipped, so bytes = (active experts) x (weight bytes per expert).
#include "common.hpp"
#include "internal.hpp"

namespace moe {

// The slot-th expert (ascending id) with at least one row, or -1.
__device__ __forceinline__ int locate_active(const GemmProblem& P, int slot) {
  __shared__ int s_e;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int carry = 0, found = -1;
    for (int g0 = 0; g0 < P.G && found < 0; g0 += 64) {
      const int gi = g0 + lane;
      const bool act = gi < P.G && P.offsets[gi + 1] > P.offsets[gi];
      const uint64_t m = __ballot(act);
      const int before = carry + __popcll(m & lanemask_lt());
      const uint64_t hit = __ballot(act && before == slot);
      if (hit) found = g0 + __ffsll((unsigned long long)hit) - 1;
      carry += __popcll(m);
    }
    if (lane == 0) s_e = found;
  }
  __syncthreads();
  return s_e;
}

template <typename T, int KIND, int ACT>
__global__ __launch_bounds__(256) void k_stream_gemm(GemmProblem la_p) {
  constexpr int EPC = Elem<T>::kPer16B;
  constexpr bool SWIGLU = (ACT == ACT_SWIGLU) && (KIND == GEMM_UP);
  const GemmProblem& P = la_p;
  const int e = locate_active(P, blockIdx.y);
  if (e < 0) return;
  const int beg = P.offsets[e];
  const int cnt = P.offsets[e + 1] - beg;
  if (cnt <= 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int fr = lane & 15, fg = lane >> 4;
  const int n0 = blockIdx.x * 64 + wave * 16;
  const T* wrow = (const T*)P.B + (size_t)e * P.b_gstride + (size_t)(n0 + fr) * P.ldb + fg * EPC;
  const T* grow = SWIGLU ? (const T*)P.B3 + (size_t)e * P.b_gstride + (size_t)(n0 + fr) * P.ldb + fg * EPC : nullptr;
  const T* A = (const T*)P.A;
  const int K = P.K;
  for (int t0 = 0; t0 < cnt; t0 += 32) {
    const T* xr[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = beg + min(t0 + j * 16 + fr, cnt - 1);
      const int src = P.a_rows ? P.a_rows[r] : r;
      xr[j] = A + (size_t)src * P.lda + fg * EPC;
    }
    floatx4_t acc[2], accg[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
      accg[j] = acc[j];
    }
    const bool two = t0 + 16 < cnt;
#pragma unroll 8
    for (int k = 0; k < K; k += 4 * EPC) {
      const uint4 w = load_nt16(wrow + k);
      uint4 wg;
      if (SWIGLU) wg = load_nt16(grow + k);
      const uint4 x0 = *reinterpret_cast<const uint4*>(xr[0] + k);
      acc[0] = mfma16(w, x0, acc[0], T());
      if (SWIGLU) accg[0] = mfma16(wg, x0, accg[0], T());
      if (two) {
        const uint4 x1 = *reinterpret_cast<const uint4*>(xr[1] + k);
        acc[1] = mfma16(w, x1, acc[1], T());
        if (SWIGLU) accg[1] = mfma16(wg, x1, accg[1], T());
      }
    }
    // lane holds columns n0 + 4*fg + t of row t0 + j*16 + fr
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int rl = t0 + j * 16 + fr;
      if (rl >= cnt) continue;
      const int64_t orow = beg + rl;
      const int n = n0 + 4 * fg;
      if (KIND == GEMM_UP) {
        float h[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float u = acc[j][t];
          if (SWIGLU) h[t] = silu(accg[j][t]) * u;
          else if (ACT == ACT_GELU_TANH) h[t] = gelu_tanh(u);
          else h[t] = gelu_erf(u);
        }
        T* c = (T*)P.C + orow * P.ldc + n;
        if (sizeof(T) == 2) {
          uint2 v;
          v.x = (uint32_t)f32_to_bf16(h[0]) | ((uint32_t)f32_to_bf16(h[1]) << 16);
          v.y = (uint32_t)f32_to_bf16(h[2]) | ((uint32_t)f32_to_bf16(h[3]) << 16);
          *reinterpret_cast<uint2*>(c) = v;
        } else {
          *reinterpret_cast<float4*>(c) = make_float4(h[0], h[1], h[2], h[3]);
        }
      } else {
        float* c = (float*)P.C + orow * P.ldc + n;
        *reinterpret_cast<float4*>(c) = make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
      }
    }
  }
}

bool stream_gemm_supported(int dtype, int kind, int act, int N, int K) {
  const int step = dtype == 0 ? 32 : 16;
  (void)kind;
  (void)act;
  return N > 0 && N % 64 == 0 && K > 0 && K % step == 0;
}

template <typename T, int KIND, int ACT>
static void stream_t(const GemmProblem& la, dim3 grid, hipStream_t st) {
  auto kfn = k_stream_gemm<T, KIND, ACT>;
  MOE_LAUNCH(KIND == GEMM_UP ? "stream_up" : "stream_down", kfn, grid, 256, 0, st, la);
}

template <typename T>
static void launch_stream_t(const GemmProblem& la, int kind, int act, dim3 grid, hipStream_t st) {
  if (kind == GEMM_DOWN) stream_t<T, GEMM_DOWN, ACT_GELU>(la, grid, st);
  else if (act == ACT_SWIGLU) stream_t<T, GEMM_UP, ACT_SWIGLU>(la, grid, st);
  else if (act == ACT_GELU_TANH) stream_t<T, GEMM_UP, ACT_GELU_TANH>(la, grid, st);
  else stream_t<T, GEMM_UP, ACT_GELU>(la, grid, st);
}

hipError_t launch_stream_gemm(int dtype, int kind, int act, const GemmProblem& p, int max_active, hipStream_t st) {
  if (max_active <= 0 || !p.offsets) return hipSuccess;
  dim3 grid(p.N / 64, max_active);
  if (dtype == 0) launch_stream_t<bf16_t>(p, kind, act, grid, st);
  else launch_stream_t<float>(p, kind, act, grid, st);
  return hipGetLastError();
}

}  // namespace moe
