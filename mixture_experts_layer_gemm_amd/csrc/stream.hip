// Weight-streaming grouped GEMMs for experts that receive only a few rows.
//
// In a DES decode block each active expert serves ~N*k/M_core rows (8-32), so its time is the
// fetch of its weights from HBM: "Dynamic Expert Sharing: Decoupling Memory from Parallelism in
// Mixture-of-Experts Diffusion LLMs", 2.1 (per-expert latency a*c + b, b the HBM weight fetch;
// the block latency is dominated by b times the number of distinct experts loaded). These kernels
// read every weight byte of an active expert once per pass over its rows and keep the MFMA work
// beside the loads. Experts with no rows are skipped, so bytes = (active experts) x (weight bytes
// per expert) per pass.
//
// k_stream_ring (bf16, the usual path; described at its definition) streams weight and token rows
// through per-wave LDS rings with direct global->LDS loads. k_stream_gemm covers fp32 and the
// shapes the ring does not take:
// workgroup (x = slice of 16 * G columns, y = active-expert slot) of G * SL waves. Wave w owns 16
// output columns (16 weight rows; 32 for SwiGLU gate+up): column group w % G, K slice w / G. The
// slices take blocks of 4 MFMA steps (256 bytes of each row) in turn; each load instruction reads
// 64 contiguous bytes of each of 16 rows. Weight rows are MFMA operand P, streamed from HBM with
// non-temporal loads into registers; the expert's token rows (operand Q, gathered through
// row_token) come from L2, 32 rows per pass. The K slices are added in LDS in slice order.
#include "common.hpp"
#include "internal.hpp"

namespace moe {

// The slot-th expert (ascending id) with at least one row, with its first row and row count
// (e = -1, cnt = 0 past the last one). The offsets read to find it give those too, so the
// workgroup waits for one round of memory latency, not two. sh: three ints of LDS to pass them on.
struct ActiveExpert {
  int e, beg, cnt;
};
__device__ __forceinline__ ActiveExpert locate_active(const GemmProblem& P, int slot, int* sh) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int carry = 0, found = -1, beg = 0, cnt = 0;
    for (int g0 = 0; g0 < P.G && found < 0; g0 += 64) {
      const int gi = g0 + lane;
      const int o0 = gi < P.G ? P.offsets[gi] : 0;
      const int o1 = gi < P.G ? P.offsets[gi + 1] : 0;
      const bool act = gi < P.G && o1 > o0;
      const uint64_t m = __ballot(act);
      const int before = carry + __popcll(m & lanemask_lt());
      const uint64_t hit = __ballot(act && before == slot);
      if (hit) {
        const int l = __ffsll((unsigned long long)hit) - 1;
        found = g0 + l;
        beg = __shfl(o0, l, 64);
        cnt = __shfl(o1, l, 64) - beg;
      }
      carry += __popcll(m);
    }
    if (lane == 0) {
      sh[0] = found;
      sh[1] = beg;
      sh[2] = cnt;
    }
  }
  __syncthreads();
  return ActiveExpert{sh[0], sh[1], sh[2]};
}

// G (16-column groups) x SL (K slices) waves per workgroup
template <typename T, int KIND, int ACT, int G, int SL>
__global__ __launch_bounds__(64 * G * SL) void k_stream_gemm(GemmProblem la_p) {
  constexpr int COLS = 16 * G;
  constexpr int EPC = Elem<T>::kPer16B;
  constexpr int KB = 16 * EPC;   // K elements per block (4 MFMA steps)
  constexpr bool SWIGLU = (ACT == ACT_SWIGLU) && (KIND == GEMM_UP);
  constexpr int NACC = SWIGLU ? 4 : 2;   // floatx4 accumulators per lane: 2 token groups (x gate)
  __shared__ floatx4_t s_red[SL - 1][G][NACC][64];
  __shared__ int s_act[3];
  const GemmProblem& P = la_p;
  const ActiveExpert ae = locate_active(P, blockIdx.y, s_act);
  const int e = ae.e, beg = ae.beg, cnt = ae.cnt;
  if (e < 0 || cnt <= 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cg = wave % G, ks = wave / G;
  const int fr = lane & 15, fg = lane >> 4;
  const int n0 = blockIdx.x * COLS + cg * 16;
  const int lane_k = fg * EPC;   // this lane's 16 bytes inside each MFMA step
  const T* wrow = (const T*)P.B + (size_t)e * P.b_gstride + (size_t)(n0 + fr) * P.ldb + lane_k;
  const T* grow = SWIGLU ? (const T*)P.B3 + (size_t)e * P.b_gstride + (size_t)(n0 + fr) * P.ldb + lane_k : nullptr;
  const T* A = (const T*)P.A;
  const int nblk = P.K / KB;
  for (int t0 = 0; t0 < cnt; t0 += 32) {
    const T* xr[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = beg + min(t0 + j * 16 + fr, cnt - 1);
      const int src = P.a_rows ? P.a_rows[r] : r;
      xr[j] = A + (size_t)src * P.lda + lane_k;
    }
    floatx4_t acc[NACC];
#pragma unroll
    for (int j = 0; j < NACC; ++j) acc[j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    const bool two = t0 + 16 < cnt;
    for (int b = ks; b < nblk; b += SL) {
      const size_t k = (size_t)b * KB;
      uint4 w[4], wg[4], x0[4], x1[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = load_nt16(wrow + k + i * 4 * EPC);
      if (SWIGLU) {
#pragma unroll
        for (int i = 0; i < 4; ++i) wg[i] = load_nt16(grow + k + i * 4 * EPC);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) x0[i] = *reinterpret_cast<const uint4*>(xr[0] + k + i * 4 * EPC);
      if (two) {
#pragma unroll
        for (int i = 0; i < 4; ++i) x1[i] = *reinterpret_cast<const uint4*>(xr[1] + k + i * 4 * EPC);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[0] = mfma16(w[i], x0[i], acc[0], T());
        if (SWIGLU) acc[2] = mfma16(wg[i], x0[i], acc[2], T());
        if (two) {
          acc[1] = mfma16(w[i], x1[i], acc[1], T());
          if (SWIGLU) acc[3] = mfma16(wg[i], x1[i], acc[3], T());
        }
      }
    }
    // add the K slices in slice order
    if (ks > 0) {
#pragma unroll
      for (int j = 0; j < NACC; ++j) s_red[ks - 1][cg][j][lane] = acc[j];
    }
    __syncthreads();
    if (ks == 0) {
#pragma unroll
      for (int q = 0; q < SL - 1; ++q)
#pragma unroll
        for (int j = 0; j < NACC; ++j) {
          const floatx4_t o = s_red[q][cg][j][lane];
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[j][t] += o[t];
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
            if (SWIGLU) h[t] = silu(acc[2 + j][t]) * u;
            else if (ACT == ACT_GELU_TANH) h[t] = gelu_tanh(u);
            else h[t] = gelu_erf(u);
          }
          T* c = (T*)P.C + orow * P.ldc + n;
          if (sizeof(T) == 2) {
            uint2 v;
            v.x = pack2_bf16(h[0], h[1]);
            v.y = pack2_bf16(h[2], h[3]);
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
    __syncthreads();   // s_red is reused by the next pass
  }
}

// ---------------------------------------------------------------------------------------------
// Ring streaming (bf16). A workgroup of 4 waves owns 64 weight rows (64 more gate rows with SwiGLU)
// of one active expert; wave w takes the K stages w, w + 4, w + 8, ... (one MFMA K step, 64 bytes
// of every row, per stage), so the four waves read neighbouring 64-byte pieces of each row at the
// same time. Each wave streams its stages, weight rows and the 16 * GRP token rows of the pass
// alike, through a private ring of D LDS slots (3 or 4) with direct global->LDS loads,
// D - 1 stages in flight while one is multiplied: no barrier inside the loop and no
// register staging. The four partial sums are added in LDS in wave order at the end. GRP (2 or 4
// groups of 16 token rows per pass) comes from the host: an expert with more rows than a pass
// serves streams its weights once per pass.
constexpr int kRingRows = 64;    // weight rows per workgroup (x 2 with SwiGLU)
constexpr int kRingSlots = 3;    // fewest stages per wave ring
constexpr int kRingRowB = 64;    // bytes of one row per stage
constexpr int kRingStageK = 4 * kRingRowB / 2;   // K elements per round of the 4 waves (bf16)

bool stream_ring_supported(int dtype, int N, int K) {
  return dtype == 0 && N > 0 && N % kRingRows == 0 && K % kRingStageK == 0 &&
         K / kRingStageK >= kRingSlots - 1;
}

// One 16-byte global->LDS load per lane from a per-lane 64-bit address; lane l writes
// LDS[lds + 16 * l].
__device__ __forceinline__ void gload_lds16_va(const void* addr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(addr), "s"(lds)
               : "memory", "m0");
}

// D: ring slots per wave (D - 1 stages in flight)
template <int KIND, int ACT, int GRP, int D>
__global__ __launch_bounds__(256) void k_stream_ring(GemmProblem la_p) {
  using T = bf16_t;
  constexpr int EPC = Elem<T>::kPer16B;
  constexpr int BK = kRingRowB / (int)sizeof(T);               // K elements per stage
  constexpr bool SWIGLU = (ACT == ACT_SWIGLU) && (KIND == GEMM_UP);
  constexpr int RW = SWIGLU ? 2 * kRingRows : kRingRows;       // weight rows per stage
  constexpr int TR = 16 * GRP;                                  // token rows per pass
  constexpr int SLOT = (RW + TR) * kRingRowB;
  constexpr int LPS = RW / 16;                                  // weight loads per stage
  constexpr int PER = LPS + GRP;                                // loads per stage
  constexpr int NT = kRingRows / 16;                            // 16-column subtiles (= waves)
  constexpr int NB = SWIGLU ? 2 * NT : NT;                      // weight fragments per stage
  static_assert(NT == 4, "one subtile per wave in the epilogue");
  static_assert(D >= 3 && (D - 2) * PER < 64, "stages in flight within the wait counter");
  static_assert(4 * GRP * NB * 64 * 16 <= 4 * D * SLOT, "reduction fits in the ring");
  __shared__ __attribute__((aligned(16))) uint8_t ring[4][D][SLOT];
  const GemmProblem& P = la_p;
  // the expert comes through the ring's first words (the ring may fill all of LDS); every thread
  // has read them before any load into the ring is issued
  const ActiveExpert ae = locate_active(P, blockIdx.y, reinterpret_cast<int*>(&ring[0][0][0]));
  __syncthreads();
  const int e = __builtin_amdgcn_readfirstlane(ae.e);
  const int beg = __builtin_amdgcn_readfirstlane(ae.beg);
  const int cnt = __builtin_amdgcn_readfirstlane(ae.cnt);
  if (e < 0 || cnt <= 0) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int fr = lane & 15, fg = lane >> 4;
  const int n0 = blockIdx.x * kRingRows;
  // a load fills 16 rows of a slot: lane l writes row l/4 at position l%4, which holds the row's
  // 16-byte chunk (l%4) ^ ((row/4)%4); readers undo the swizzle with swz()
  const int rr = lane >> 2;
  const int cc = (lane & 3) ^ ((rr >> 2) & 3);
  const uint32_t lane_off = (uint32_t)(((size_t)rr * P.ldb + cc * EPC) * sizeof(T));
  const T* Wb = (const T*)P.B + (size_t)e * P.b_gstride + (size_t)n0 * P.ldb;
  const T* W3b = SWIGLU ? (const T*)P.B3 + (size_t)e * P.b_gstride + (size_t)n0 * P.ldb : Wb;
  const int ns = P.K / kRingStageK;   // stages of every wave
  uint8_t* myring = &ring[wave][0][0];
  const uint32_t ring_lds = lds_addr(myring);
  auto swz = [](int row, int chunk) { return row * kRingRowB + ((chunk ^ ((row >> 2) & 3)) << 4); };
  const T* A = (const T*)P.A;

  for (int t0 = 0; t0 < cnt; t0 += TR) {
    const T* xr[GRP];   // this lane's token row (clamped to the expert's rows) and chunk, per group
#pragma unroll
    for (int g = 0; g < GRP; ++g) {
      const int r = beg + min(t0 + g * 16 + rr, cnt - 1);
      const int src = P.a_rows ? P.a_rows[r] : r;
      xr[g] = A + (size_t)src * P.lda + cc * EPC + (size_t)wave * BK;
    }
    auto issue = [&](int s) {
      const int sl = s % D;
      const size_t k = (size_t)(s * 4 + wave) * BK;
      const uint32_t dst = ring_lds + sl * SLOT;
#pragma unroll
      for (int i = 0; i < LPS; ++i) {
        const T* base = (i < NT ? Wb : W3b) + (size_t)(i % NT) * 16 * P.ldb + k;
        gload_lds16(base, lane_off, dst + i * 16 * kRingRowB);
      }
#pragma unroll
      for (int g = 0; g < GRP; ++g)
        gload_lds16_va(xr[g] + (size_t)s * 4 * BK, dst + (RW + g * 16) * kRingRowB);
    };
    floatx4_t acc[GRP][NB];
#pragma unroll
    for (int g = 0; g < GRP; ++g)
#pragma unroll
      for (int i = 0; i < NB; ++i) acc[g][i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int s) {
      const uint8_t* sp = myring + (s % D) * SLOT;
      uint4 bf[NB], xv[GRP];
#pragma unroll
      for (int i = 0; i < NB; ++i) bf[i] = *reinterpret_cast<const uint4*>(sp + swz(i * 16 + fr, fg));
#pragma unroll
      for (int g = 0; g < GRP; ++g) xv[g] = *reinterpret_cast<const uint4*>(sp + swz(RW + g * 16 + fr, fg));
#pragma unroll
      for (int g = 0; g < GRP; ++g)
#pragma unroll
        for (int i = 0; i < NB; ++i) acc[g][i] = mfma16(bf[i], xv[g], acc[g][i], T());
    };
    // ns >= D - 1 (stream_ring_supported and the launcher's choice of D)
    static_for<D - 1>([&](auto Sc) { issue(decltype(Sc)::value); });
    // stage s: wait for it (stages s + 1 .. s + D - 2 stay in flight) and for the LDS reads of
    // stage s - 1, refill that slot with stage s + D - 1, multiply
    constexpr int INF = (D - 2) * PER;
    for (int s = 0; s + D - 1 < ns; ++s) {
      __builtin_amdgcn_s_waitcnt((INF & 15) | (((INF >> 4) & 3) << 14) | (7 << 4));   // + lgkmcnt(0)
      asm volatile("" ::: "memory");
      issue(s + D - 1);
      compute(s);
    }
    // drain: the last D - 1 stages, each once the stages after it are the only ones in flight
    static_for<D - 1>([&](auto Jc) {
      constexpr int left = D - 2 - decltype(Jc)::value;   // stages still in flight after this one
      wait_vmem<left * PER>();
      asm volatile("" ::: "memory");
      compute(ns - 1 - left);
    });
    // add the four waves' partial sums in wave order; wave w finishes subtile w
    __syncthreads();
    floatx4_t* red = reinterpret_cast<floatx4_t*>(&ring[0][0][0]);   // [wave][g][NB][64]
#pragma unroll
    for (int g = 0; g < GRP; ++g)
#pragma unroll
      for (int i = 0; i < NB; ++i) red[((wave * GRP + g) * NB + i) * 64 + lane] = acc[g][i];
    __syncthreads();
    const int nt = wave;
#pragma unroll
    for (int g = 0; g < GRP; ++g) {
      floatx4_t u = floatx4_t{0.f, 0.f, 0.f, 0.f}, gt = u;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const floatx4_t a = red[((w * GRP + g) * NB + nt) * 64 + lane];
#pragma unroll
        for (int t = 0; t < 4; ++t) u[t] += a[t];
        if (SWIGLU) {
          const floatx4_t b = red[((w * GRP + g) * NB + NT + nt) * 64 + lane];
#pragma unroll
          for (int t = 0; t < 4; ++t) gt[t] += b[t];
        }
      }
      // lane holds columns n0 + nt*16 + 4*fg + t of row t0 + g*16 + fr
      const int rl = t0 + g * 16 + fr;
      if (rl >= cnt) continue;
      const int64_t orow = beg + rl;
      const int n = n0 + nt * 16 + 4 * fg;
      if (KIND == GEMM_UP) {
        float h[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (SWIGLU) h[t] = silu(gt[t]) * u[t];
          else if (ACT == ACT_GELU_TANH) h[t] = gelu_tanh(u[t]);
          else h[t] = gelu_erf(u[t]);
        }
        uint2 v;
        v.x = pack2_bf16(h[0], h[1]);
        v.y = pack2_bf16(h[2], h[3]);
        *reinterpret_cast<uint2*>((T*)P.C + orow * P.ldc + n) = v;
      } else {
        *reinterpret_cast<float4*>((float*)P.C + orow * P.ldc + n) = make_float4(u[0], u[1], u[2], u[3]);
      }
    }
    __syncthreads();   // the ring is reused by the next pass
  }
}

// Ring depth: the SwiGLU up projection with 32-row passes (10 KB stages, a whole compute unit per
// workgroup) takes a fourth slot, which fills the 160 KB of LDS: three stages in flight per wave
// instead of two. The other shapes keep three slots, which lets two workgroups share a compute unit
// (GELU and down projections: 6 KB stages).
template <int KIND, int ACT>
static void ring_t(const GemmProblem& la, int max_active, int pass_rows, hipStream_t st) {
  const dim3 grid(la.N / kRingRows, max_active);
  const char* name = KIND == GEMM_UP ? "stream_up" : "stream_down";
  if (pass_rows > 32) {
    auto kfn = k_stream_ring<KIND, ACT, 4, 3>;
    MOE_LAUNCH(name, kfn, grid, 256, 0, st, la);
    return;
  }
  if constexpr (KIND == GEMM_UP && ACT == ACT_SWIGLU) {
    if (la.K / kRingStageK >= 3) {
      auto kfn = k_stream_ring<KIND, ACT, 2, 4>;
      MOE_LAUNCH(name, kfn, grid, 256, 0, st, la);
      return;
    }
  }
  auto kfn = k_stream_ring<KIND, ACT, 2, 3>;
  MOE_LAUNCH(name, kfn, grid, 256, 0, st, la);
}

bool stream_gemm_supported(int dtype, int kind, int act, int N, int K) {
  const int step = dtype == 0 ? 128 : 64;   // K elements per block
  (void)kind;
  (void)act;
  return N > 0 && N % 64 == 0 && K > 0 && K % step == 0;
}

template <typename T, int KIND, int ACT, int G, int SL>
static void stream_shape(const GemmProblem& la, int max_active, hipStream_t st) {
  const dim3 grid(la.N / (16 * G), max_active);
  auto kfn = k_stream_gemm<T, KIND, ACT, G, SL>;
  MOE_LAUNCH(KIND == GEMM_UP ? "stream_up" : "stream_down", kfn, grid, 64 * G * SL, 0, st, la);
}

// Shape: 16 waves per workgroup by default (4 column groups x 4 K slices). When that gives fewer
// workgroups than compute units, 2 x 8 (twice the workgroups); when each K slice would get fewer
// than 4 blocks of K, 4 x 2.
template <typename T, int KIND, int ACT>
static void stream_t(const GemmProblem& la, int max_active, hipStream_t st) {
  constexpr int KB = 16 * Elem<T>::kPer16B;
  const int nblk = la.K / KB;
  if ((la.N / 64) * max_active < 256) stream_shape<T, KIND, ACT, 2, 8>(la, max_active, st);
  else if (nblk < 16) stream_shape<T, KIND, ACT, 4, 2>(la, max_active, st);
  else stream_shape<T, KIND, ACT, 4, 4>(la, max_active, st);
}

template <typename T>
static void launch_stream_t(const GemmProblem& la, int kind, int act, int max_active, hipStream_t st) {
  if (kind == GEMM_DOWN) stream_t<T, GEMM_DOWN, ACT_GELU>(la, max_active, st);
  else if (act == ACT_SWIGLU) stream_t<T, GEMM_UP, ACT_SWIGLU>(la, max_active, st);
  else if (act == ACT_GELU_TANH) stream_t<T, GEMM_UP, ACT_GELU_TANH>(la, max_active, st);
  else stream_t<T, GEMM_UP, ACT_GELU>(la, max_active, st);
}

hipError_t launch_stream_gemm(int dtype, int kind, int act, const GemmProblem& p, int max_active, int pass_rows,
                              hipStream_t st) {
  if (max_active <= 0 || !p.offsets) return hipSuccess;
  if (stream_ring_supported(dtype, p.N, p.K) && p.k_seg == p.K) {
    if (kind == GEMM_DOWN) ring_t<GEMM_DOWN, ACT_GELU>(p, max_active, pass_rows, st);
    else if (act == ACT_SWIGLU) ring_t<GEMM_UP, ACT_SWIGLU>(p, max_active, pass_rows, st);
    else if (act == ACT_GELU_TANH) ring_t<GEMM_UP, ACT_GELU_TANH>(p, max_active, pass_rows, st);
    else ring_t<GEMM_UP, ACT_GELU>(p, max_active, pass_rows, st);
    return hipGetLastError();
  }
  if (dtype == 0) launch_stream_t<bf16_t>(p, kind, act, max_active, st);
  else launch_stream_t<float>(p, kind, act, max_active, st);
  return hipGetLastError();
}

}  // namespace moe
