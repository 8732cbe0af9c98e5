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

// KM: an upper bound on k (2, 4, 8 or 16), which sizes the per-slot registers.
// Latency: every load that does not depend on another one is issued first, together (the reuse
// flag, the slots' expert / weight / row, the shared-expert and residual rows), then the rows the
// slots name, all of them together; so a call with few tokens (a decode block) waits for two
// rounds of memory latency instead of one or two per slot.
template <typename T, bool EC, int KM>
__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  const int cpr = a.d >> 3;
  const size_t total = (size_t)a.S * cpr;
  const T* x = (const T*)a.x;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int s = (int)(i / cpr);
    const int c0 = (int)(i - (size_t)s * cpr) * 8;
    const size_t row = (size_t)s * a.d + c0;
    // independent loads. The reuse flag comes first, so waiting for it leaves the others in flight.
    // Without a reuse mask, a byte of another array this call reads stands in: a load with no
    // branch around it is not waited for until its value is used.
    const uint8_t* fl = a.reuse ? a.reuse + s : reinterpret_cast<const uint8_t*>(EC ? a.token_off : a.topk_idx);
    const uint8_t rflag = *fl;
    int e[KM], tr[KM];
    float w[KM];
    int q0 = 0, q1 = 0;   // expert choice: the token's entries in the token CSR
    if (EC) {
      q0 = a.token_off[s];
      q1 = a.token_off[s + 1];
    } else {
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        const size_t o = (size_t)s * a.k + min(j, a.k - 1);   // slots past k re-read the last one
        e[j] = a.topk_idx[o];                                 // -1: an empty DES-Seq slot
        w[j] = a.topk_w[o];
        tr[j] = a.token_rows[o];
      }
    }
    // the shared-expert and residual rows as raw 16-byte pieces, converted at the end
    constexpr int LW = sizeof(T) == 4 ? 2 : 1;   // 16-byte pieces of 8 elements of T
    uint4 rsh[2], rres[LW];
    if (a.y_shared) {
      const uint4* p = reinterpret_cast<const uint4*>(a.y_shared + row);
      rsh[0] = p[0];
      rsh[1] = p[1];
    }
    if (a.residual) {
      const uint4* p = reinterpret_cast<const uint4*>((const T*)a.residual + row);
#pragma unroll
      for (int h = 0; h < LW; ++h) rres[h] = p[h];
    }
    const bool reused = a.reuse && rflag != 0;

    float routed[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (reused) {
      load8<T>((const T*)a.cache + row, routed);
    } else if (!EC) {
      // each slot's source row: 0 nothing (a slot past k, an empty slot, a zero expert), 1 a routed
      // row of y_perm, 2 x (identity), 3 a constant expert's vector
      int kind[KM];
      const T* src[KM];
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        const int l = e[j] - a.E_heavy;
        const int lc = l - a.n_identity - a.n_zero;   // constant expert index
        kind[j] = j >= a.k || e[j] < 0 ? 0 : l < 0 ? 1 : l < a.n_identity ? 2 : lc >= 0 ? 3 : 0;
        src[j] = kind[j] == 3 ? (const T*)a.const_vec + (size_t)lc * a.d + c0 : x + row;
      }
      // raw 16-byte pieces first, into registers of their own per kind of source (a load whose
      // destination another branch also writes would have to wait for that one), converted after
      uint4 rp[KM][2], rx[KM][LW];
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        if (kind[j] == 1) {
          const uint4* p = reinterpret_cast<const uint4*>(a.y_perm + (size_t)tr[j] * a.d + c0);
          rp[j][0] = p[0];
          rp[j][1] = p[1];
        }
        if (kind[j] >= 2) {
          const uint4* p = reinterpret_cast<const uint4*>(src[j]);
#pragma unroll
          for (int h = 0; h < LW; ++h) rx[j][h] = p[h];
        }
      }
      // added in slot order
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        if (kind[j] != 0) {
          float vv[8];
          if (kind[j] == 1) {
            unpack16(rp[j][0], vv, float());
            unpack16(rp[j][1], vv + 4, float());
          } else if (sizeof(T) == 4) {
            unpack16(rx[j][0], vv, float());
            unpack16(rx[j][LW - 1], vv + 4, float());
          } else {
            unpack16(rx[j][0], vv, bf16_t());
          }
#pragma unroll
          for (int q = 0; q < 8; ++q) routed[q] += w[j] * vv[q];
        }
      }
    } else {
      // the experts that chose the token, four entries at a time: their rows are in flight together
      constexpr int U = 4;
      for (int qb = q0; qb < q1; qb += U) {
        int r[U];
#pragma unroll
        for (int u = 0; u < U; ++u) r[u] = a.token_list[min(qb + u, q1 - 1)];
        float wr[U];
        uint4 rp[U][2];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          wr[u] = a.row_w[r[u]];
          const uint4* p = reinterpret_cast<const uint4*>(a.y_perm + (size_t)r[u] * a.d + c0);
          rp[u][0] = p[0];
          rp[u][1] = p[1];
        }
        // (the scheduler would otherwise interleave the loads with their uses to save registers)
        __builtin_amdgcn_sched_barrier(0);
        // entries past the last re-read it and add it with weight 0 (no branch around the use, so
        // the compiler keeps the four loads together)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float wu = qb + u < q1 ? wr[u] : 0.f;
          float v[8];
          unpack16(rp[u][0], v, float());
          unpack16(rp[u][1], v + 4, float());
#pragma unroll
          for (int q = 0; q < 8; ++q) routed[q] += wu * v[q];
        }
      }
    }
    if (a.cache && !reused) store8<T>((T*)a.cache + row, routed);
    float out[8];
    if (a.y_shared) {
      float sh[8];
      unpack16(rsh[0], sh, float());
      unpack16(rsh[1], sh + 4, float());
#pragma unroll
      for (int q = 0; q < 8; ++q) out[q] = sh[q] + routed[q];
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) out[q] = routed[q];
    }
    if (a.residual) {
      float res[8];
      if (sizeof(T) == 4) {
        unpack16(rres[0], res, float());
        unpack16(rres[LW - 1], res + 4, float());
      } else {
        unpack16(rres[0], res, bf16_t());
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) out[q] += res[q];
    }
    store8<T>((T*)a.y + row, out);
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
