// Dispatch gather and the weighted combine.
//
// Combine: y_s = residual_s + shared_s + sum over the token's slots of w * expert output, with
// zero-computation experts inline ("MMOE: Modernizing Diffusion Transformers with Efficient Expert
// Design", 方法论 / MoE++: identity copies x, zero gives 0, constant gives its learned vector; the
// shared expert always adds with weight 1), expert choice summing A_{s,i} * FFN_i over the experts
// that chose the token ("EC-DiT ...", 核心公式), and cached routed parts for low-score tokens
// ("DICE: Staleness-Centric Optimizations for Parallel Diffusion MoE Inference", 条件通信; only the
// combine result is cached, 交织并行).
//
// HBM-bound: one thread per (token, 8 consecutive columns); every access is a 16-byte (bf16) or
// 32-byte (fp32) contiguous run; accumulation in fp32 in a fixed order (shared, then slots in slot
// order / experts ascending, then the residual) so repeated calls are bit-identical.
#include "common.hpp"
#include "internal.hpp"

namespace moe {

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* v);
template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float* v) {
  unpack16(*reinterpret_cast<const uint4*>(p), v, bf16_t());
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* v) {
  unpack16(*reinterpret_cast<const uint4*>(p), v, float());
  unpack16(*reinterpret_cast<const uint4*>(p + 4), v + 4, float());
}
template <typename T>
__device__ __forceinline__ void store8(T* p, const float* v);
template <>
__device__ __forceinline__ void store8<bf16_t>(bf16_t* p, const float* v) {
  *reinterpret_cast<uint4*>(p) = pack16(v, bf16_t());
}
template <>
__device__ __forceinline__ void store8<float>(float* p, const float* v) {
  *reinterpret_cast<uint4*>(p) = pack16(v, float());
  *reinterpret_cast<uint4*>(p + 4) = pack16(v + 4, float());
}

template <typename T>
__global__ __launch_bounds__(256) void k_gather(const T* __restrict__ x, const int32_t* __restrict__ row_token,
                                                const int32_t* __restrict__ n_rows, T* __restrict__ xp, int R_max,
                                                int d) {
  constexpr int EPC = Elem<T>::kPer16B;
  const int cpr = d / EPC;
  const int n = min(*n_rows, R_max);
  const size_t total = (size_t)n * cpr;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i / cpr;
    const int c = (int)(i - r * cpr) * EPC;
    const int tok = row_token[r];
    *reinterpret_cast<uint4*>(xp + r * d + c) = *reinterpret_cast<const uint4*>(x + (size_t)tok * d + c);
  }
}

hipError_t launch_gather(int dtype, const void* x, const int32_t* row_token, const int32_t* n_rows, void* x_perm,
                         int R_max, int d, hipStream_t st) {
  const size_t chunks = (size_t)R_max * d / (dtype == 0 ? 8 : 4);
  const int blocks = (int)std::max<size_t>(1, std::min<size_t>((chunks + 255) / 256, 8192));
  if (dtype == 0) {
    auto kfn = k_gather<bf16_t>;
    MOE_LAUNCH("gather", kfn, blocks, 256, 0, st, (const bf16_t*)x, row_token, n_rows, (bf16_t*)x_perm, R_max, d);
  } else {
    auto kfn = k_gather<float>;
    MOE_LAUNCH("gather", kfn, blocks, 256, 0, st, (const float*)x, row_token, n_rows, (float*)x_perm, R_max, d);
  }
  return hipGetLastError();
}

// KM: an upper bound on k (2, 4, 8 or 16), which sizes the per-slot registers
template <typename T, bool EC, int KM>
__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  constexpr int GRP = KM < 4 ? KM : 4;   // slots whose rows are loaded together
  const int cpr = a.d >> 3;
  const size_t total = (size_t)a.S * cpr;
  const T* x = (const T*)a.x;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int s = (int)(i / cpr);
    const int c0 = (int)(i - (size_t)s * cpr) * 8;
    float routed[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float v[8];
    const bool reused = a.reuse && a.reuse[s];
    if (reused) {
      load8<T>((const T*)a.cache + (size_t)s * a.d + c0, routed);
    } else if (!EC) {
      // the slots' metadata first, then their rows GRP at a time, added in slot order: the loads of
      // a group are in flight together instead of one dependent pair per slot
      int src_kind[KM], src_row[KM];
      float src_w[KM];
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        src_kind[j] = 0;   // 0: nothing (also an empty slot), 1: routed row, 2: x, 3: constant row
        src_row[j] = 0;
        src_w[j] = 0.f;
        if (j < a.k) {
          const int e = a.topk_idx[(size_t)s * a.k + j];   // -1: an empty DES-Seq slot
          src_w[j] = a.topk_w[(size_t)s * a.k + j];
          int l = e - a.E_heavy;
          if (e < 0) {
            // nothing
          } else if (l < 0) {
            src_kind[j] = 1;
            src_row[j] = a.token_rows[(size_t)s * a.k + j];
          } else if (l < a.n_identity) {
            src_kind[j] = 2;
          } else if ((l -= a.n_identity) >= a.n_zero) {
            src_kind[j] = 3;
            src_row[j] = l - a.n_zero;
          }
        }
      }
#pragma unroll
      for (int j0 = 0; j0 < KM; j0 += GRP) {
        if (j0 < a.k) {
          float vv[GRP][8];
#pragma unroll
          for (int jj = 0; jj < GRP; ++jj) {
            const int j = j0 + jj;
            if (src_kind[j] == 1) load8<float>(a.y_perm + (size_t)src_row[j] * a.d + c0, vv[jj]);
            else if (src_kind[j] == 2) load8<T>(x + (size_t)s * a.d + c0, vv[jj]);
            else if (src_kind[j] == 3) load8<T>((const T*)a.const_vec + (size_t)src_row[j] * a.d + c0, vv[jj]);
          }
#pragma unroll
          for (int jj = 0; jj < GRP; ++jj) {
            if (src_kind[j0 + jj] != 0) {
#pragma unroll
              for (int q = 0; q < 8; ++q) routed[q] += src_w[j0 + jj] * vv[jj][q];
            }
          }
        }
      }
    } else {
      const int q0 = a.token_off[s], q1 = a.token_off[s + 1];
      for (int qq = q0; qq < q1; ++qq) {
        const int r = a.token_list[qq];
        const float w = a.row_w[r];
        load8<float>(a.y_perm + (size_t)r * a.d + c0, v);
#pragma unroll
        for (int q = 0; q < 8; ++q) routed[q] += w * v[q];
      }
    }
    if (a.cache && !reused) store8<T>((T*)a.cache + (size_t)s * a.d + c0, routed);
    float out[8];
    if (a.y_shared) {
      load8<float>(a.y_shared + (size_t)s * a.d + c0, out);
#pragma unroll
      for (int q = 0; q < 8; ++q) out[q] += routed[q];
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) out[q] = routed[q];
    }
    if (a.residual) {
      load8<T>((const T*)a.residual + (size_t)s * a.d + c0, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) out[q] += v[q];
    }
    store8<T>((T*)a.y + (size_t)s * a.d + c0, out);
  }
}

template <typename T, bool EC>
static void combine_t(const CombineArgs& a, int blocks, hipStream_t st) {
  if (EC || a.k <= 2) {   // expert choice reads its rows through the token CSR: no slot registers
    auto kfn = k_combine<T, EC, 2>;
    MOE_LAUNCH("combine", kfn, blocks, 256, 0, st, a);
    return;
  }
  if constexpr (EC) return;
  if (a.k <= 4) {
    auto kfn = k_combine<T, EC, 4>;
    MOE_LAUNCH("combine", kfn, blocks, 256, 0, st, a);
  } else if (a.k <= 8) {
    auto kfn = k_combine<T, EC, 8>;
    MOE_LAUNCH("combine", kfn, blocks, 256, 0, st, a);
  } else {
    auto kfn = k_combine<T, EC, 16>;
    MOE_LAUNCH("combine", kfn, blocks, 256, 0, st, a);
  }
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t st) {
  const size_t items = (size_t)a.S * (a.d / 8);
  const int blocks = (int)std::max<size_t>(1, std::min<size_t>((items + 255) / 256, 16384));
  const bool ec = a.mode == 1;
  if (a.dtype == 0) {
    if (ec) combine_t<bf16_t, true>(a, blocks, st);
    else combine_t<bf16_t, false>(a, blocks, st);
  } else {
    if (ec) combine_t<float, true>(a, blocks, st);
    else combine_t<float, false>(a, blocks, st);
  }
  return hipGetLastError();
}

}  // namespace moe
