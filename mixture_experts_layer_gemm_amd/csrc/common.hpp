// Device-side helpers shared by the gfx950 kernels of the MoE layer library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load that bypasses cache retention (for data read exactly once).
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Storage element of a bf16 tensor: its 16-bit encoding.
typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// fp32 -> bf16, round to nearest, ties to even (finite inputs).
// fp32 -> bf16, round to nearest even: the hardware conversion (v_cvt_pk_bf16_f32 on gfx950)
typedef __bf16 hw_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float hw_f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  const hw_f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, hw_bf16x2_t));
}
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return (bf16_t)(pack2_bf16(f, 0.f) & 0xFFFFu); }

template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
  static constexpr int kPer16B = 8;   // elements in one 16-byte chunk
  static constexpr int kMfmaPerStep = 1;   // MFMA instructions per 16x16 product over 16 bytes of K
  __device__ static __forceinline__ float to_f(bf16_t v) { return bf16_to_f32(v); }
  __device__ static __forceinline__ bf16_t from_f(float v) { return f32_to_bf16(v); }
};
template <> struct Elem<float> {
  static constexpr int kPer16B = 4;
  static constexpr int kMfmaPerStep = 4;
  __device__ static __forceinline__ float to_f(float v) { return v; }
  __device__ static __forceinline__ float from_f(float v) { return v; }
};

// Unpack a 16-byte chunk into floats (8 for bf16, 4 for fp32).
__device__ __forceinline__ void unpack16(const uint4 v, float* out, bf16_t) {
  out[0] = __uint_as_float(v.x << 16); out[1] = __uint_as_float(v.x & 0xFFFF0000u);
  out[2] = __uint_as_float(v.y << 16); out[3] = __uint_as_float(v.y & 0xFFFF0000u);
  out[4] = __uint_as_float(v.z << 16); out[5] = __uint_as_float(v.z & 0xFFFF0000u);
  out[6] = __uint_as_float(v.w << 16); out[7] = __uint_as_float(v.w & 0xFFFF0000u);
}
__device__ __forceinline__ void unpack16(const uint4 v, float* out, float) {
  out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
  out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
}
__device__ __forceinline__ uint4 pack16(const float* in, bf16_t) {
  uint4 v;
  v.x = pack2_bf16(in[0], in[1]);
  v.y = pack2_bf16(in[2], in[3]);
  v.z = pack2_bf16(in[4], in[5]);
  v.w = pack2_bf16(in[6], in[7]);
  return v;
}
__device__ __forceinline__ uint4 pack16(const float* in, float) {
  return make_uint4(__float_as_uint(in[0]), __float_as_uint(in[1]), __float_as_uint(in[2]), __float_as_uint(in[3]));
}

// One MFMA step on a 16-byte chunk per lane, for a 16x16 output tile.
// The lane layout (verified on gfx950): operand P supplies rows i = lane % 16 of the first
// matrix, operand Q rows j = lane % 16 of the second; lane group g = lane / 16 supplies a slice
// of the reduction index (the same slice in P and Q, so the slice order does not matter);
// acc[t] of lane l is D[i = 4*(l/16) + t][j = l % 16], D = sum_k P[i][k] * Q[j][k].
__device__ __forceinline__ floatx4_t mfma16(const uint4 p, const uint4 q, floatx4_t acc, bf16_t) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, p), __builtin_bit_cast(bf16x8_t, q),
                                                 acc, 0, 0, 0);
}
__device__ __forceinline__ floatx4_t mfma16(const uint4 p, const uint4 q, floatx4_t acc, float) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(p.x), __uint_as_float(q.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(p.y), __uint_as_float(q.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(p.z), __uint_as_float(q.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(p.w), __uint_as_float(q.w), acc, 0, 0, 0);
  return acc;
}

// Activations (MLP hidden layer).
enum { ACT_GELU = 0, ACT_GELU_TANH = 1, ACT_SWIGLU = 2 };

// e^x through the hardware base-2 exponential (about 1 ulp).
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// erf GELU, z * Phi(z), written as max(z, 0) - |z| * Q(|z|) with Q(u) = 1 - Phi(u) = erfc(u / sqrt 2) / 2
// (for z >= 0 that is z - z Q; for z < 0 it is z Phi(z) = z Q(|z|)). erfc comes from the
// approximation of Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.28
// (|error| <= 3e-7 for x >= 0): erfc(x) = (1 + a1 x + ... + a6 x^6)^-16, so Q(u) = q(u)^-16 with
// q(u) = 2^(1/16) (1 + a1 u/sqrt2 + ... + a6 (u/sqrt2)^6). The coefficients of q are those of the
// formula rescaled by 2^(1/16) and powers of 1/sqrt 2 (exact in double, rounded once to float).
// Twelve VALU operations and one reciprocal; |error| <= 8e-7 over all z.
__device__ __forceinline__ float gelu_erf(float z) {
  constexpr double c = 1.0442737824274138;   // 2^(1/16)
  constexpr double s = 0.70710678118654752;  // 1/sqrt(2)
  constexpr float b0 = (float)c;
  constexpr float b1 = (float)(c * 0.0705230784 * s);
  constexpr float b2 = (float)(c * 0.0422820123 * s * s);
  constexpr float b3 = (float)(c * 0.0092705272 * s * s * s);
  constexpr float b4 = (float)(c * 0.0001520143 * s * s * s * s);
  constexpr float b5 = (float)(c * 0.0002765672 * s * s * s * s * s);
  constexpr float b6 = (float)(c * 0.0000430638 * s * s * s * s * s * s);
  const float u = fabsf(z);
  float q = fmaf(b6, u, b5);
  q = fmaf(q, u, b4);
  q = fmaf(q, u, b3);
  q = fmaf(q, u, b2);
  q = fmaf(q, u, b1);
  q = fmaf(q, u, b0);
  q = q * q;
  q = q * q;
  q = q * q;
  q = q * q;   // q^16; overflows to inf for large |z|, whose reciprocal is 0
  // max(z, 0) as a median of three (z, 0, the largest float): for finite z the same value, in one
  // instruction where fmaxf takes two (it first quiets a possible signalling NaN)
  return fmaf(-u, fast_rcp(q), __builtin_amdgcn_fmed3f(z, 0.0f, 3.402823466e38f));
}
// tanh form: 0.5 z (1 + tanh(u)) = z - z / (1 + e^{2u}), u = sqrt(2/pi) (z + 0.044715 z^3)
__device__ __forceinline__ float gelu_tanh(float z) {
  const float u = 0.79788456080286536f * fmaf(0.044715f * z, z * z, z);
  return z - z * fast_rcp(1.0f + fast_exp(2.0f * u));
}
__device__ __forceinline__ float silu(float z) { return z * fast_rcp(1.0f + fast_exp(-z)); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = __lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// ---------------------------------------------------------------------------------------------
// Direct global -> LDS loads and their waits (grouped GEMM and weight streaming).
// Compile-time loop over 0..N-1 (every index a constant, so register arrays stay in registers).
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

typedef __attribute__((address_space(3))) uint8_t lds_u8_t;

// 16 bytes per lane from global memory (wave-uniform base + per-lane byte offset) straight into
// LDS: lane l of the wave writes LDS[lds_addr + 16*l]; lds_addr is the same for the whole wave (M0). Completion is tracked by
// the wave's vmcnt, which the K loop waits on explicitly (wait_vmem) before a stage is read. The
// instruction is issued from inline assembly so the compiler does not add its own wait for every
// LDS DMA in flight before each LDS read (it cannot tell the ring's stages apart). Nothing else
// in these kernels uses M0.
__device__ __forceinline__ void gload_lds16(const void* base, uint32_t lane_off, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(lane_off), "s"(base),
               "s"(lds_addr)
               : "memory", "m0");
}
// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(size_t)(const lds_u8_t*)p; }
// Wait until at most N of this wave's global loads (including loads into LDS) are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | (7 << 4) | (15 << 8));
}
// Workgroup barrier for the LDS ring. Every wave has already waited for its own loads of the
// stage it needs (wait_vmem) and for its LDS reads (lgkmcnt 0), so no memory fence is needed (a
// fence would also wait for the stages still in flight). The empty asm statements keep the
// compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace moe
