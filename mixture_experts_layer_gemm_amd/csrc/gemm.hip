// Grouped expert GEMMs on gfx950 matrix cores (bf16 -> fp32 MFMA 16x16x32, or fp32 MFMA 16x16x4).
//
// Heavy experts are standard MLPs ("MMOE: Modernizing Diffusion Transformers with Efficient Expert
// Design", 方法论 / MoE++ heavy experts; GELU or SwiGLU), run as one grouped GEMM per projection:
//   up:   H[r, :] = act(A[r] . W1_e^T)    (SwiGLU: silu(A[r] . W3_e^T) * (A[r] . W1_e^T))
//   down: Y[r, :] = H[r] . W2_e^T          (fp32 out)
// over the rows r of each expert e, whose count is only known on the device (offsets[]). Shared
// experts are extra problems in the same launch (all S rows; their down projections are one GEMM
// over the K-concatenation of their hidden activations).
//
// Design (one workgroup = 4 waves = one 256 x BN output tile, BN in {128, 256}):
//   * K advances 128 bytes per stage (64 bf16 / 32 fp32); A and B stages are double-buffered in
//     LDS (2 x (32 KB + BN*128 B)) and filled by direct global->LDS loads (no staging registers),
//     one barrier per stage; stage k+1's loads are in flight while stage k feeds the MFMAs.
//   * LDS rows are 128 B; 16-byte chunk c of row r sits at slot c ^ ((r >> 1) & 7), so the
//     16-byte fragment reads of 16 consecutive rows hit distinct banks.
//   * Weights are MFMA operand P and tokens operand Q, so each lane ends with 4 consecutive output
//     columns of one row: 8-byte (bf16) / 16-byte (fp32) stores.
//   * Gather fused into the A loads: row r reads x[row_token[r]].
//   * Tile order: workgroup b runs on XCD b % 8; tiles are renumbered so each XCD owns a
//     contiguous range, swept as 8 m-tiles x all n-tiles, which keeps an expert's weight panels and
//     token panels in one XCD's L2.
//   * The expert of an m-tile comes from a wave-wide scan of ceil(count_e / 256) over experts.
#include "common.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kBM = 256;
constexpr int kRowB = 128;          // bytes of one tile row per stage
constexpr int kThreads = 256;
constexpr int kGM = 8;              // m-tiles per sweep group

struct GemmLaunch {
  GemmProblem p0, p1;
  int32_t tiles_n0, tiles_n1;
  int32_t mt_ub0, mt_ub1;
  int32_t tile_begin1;
  int32_t nprob;
  int32_t total_tiles;
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowB + ((chunk ^ ((row >> 1) & 7)) << 4); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 16 bytes per lane from global memory straight into LDS: lane l of the wave writes
// LDS[dst + 16*l]. dst must be the same for the whole wave.
__device__ __forceinline__ void gload_lds16(const void* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)dst, 16, 0, 0);
}
// Wait until this wave's outstanding global loads (including loads into LDS) have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Map m-tile `mt` of problem P to (group, first row, rows). Returns false for a tile past the end.
__device__ __forceinline__ bool locate_mtile(const GemmProblem& P, int mt, int& g, int& row0, int& rows) {
  if (!P.offsets) {
    const int mpg = (P.M_uni + kBM - 1) / kBM;
    if (mpg == 0) return false;
    g = mt / mpg;
    if (g >= P.G) return false;
    const int lm = mt - g * mpg;
    row0 = lm * kBM;
    rows = min(kBM, P.M_uni - row0);
    return true;
  }
  __shared__ int s_res[3];
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int carry = 0;
    int found = 0, fg = -1, frow0 = 0, frows = 0;
    for (int g0 = 0; g0 < P.G && !found; g0 += 64) {
      const int gi = g0 + lane;
      int beg = 0, cnt = 0;
      if (gi < P.G) {
        beg = P.offsets[gi];
        cnt = P.offsets[gi + 1] - beg;
      }
      const int mts = (cnt + kBM - 1) / kBM;
      int incl = mts;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      const int excl = carry + incl - mts;
      const bool hit = gi < P.G && mt >= excl && mt < excl + mts;
      const uint64_t m = __ballot(hit);
      if (m) {
        const int src = __ffsll((unsigned long long)m) - 1;
        const int lm = __shfl(mt - excl, src, 64);
        fg = g0 + src;
        frow0 = __shfl(beg, src, 64) + lm * kBM;
        frows = min(kBM, __shfl(beg + cnt, src, 64) - frow0);
        found = 1;
      }
      carry += __shfl(incl, 63, 64);
    }
    if (lane == 0) {
      s_res[0] = found ? fg : -1;
      s_res[1] = frow0;
      s_res[2] = frows;
    }
  }
  __syncthreads();
  g = s_res[0];
  row0 = s_res[1];
  rows = s_res[2];
  return g >= 0;
}

template <typename T, int KIND, int ACT, int BN>
__global__ __launch_bounds__(kThreads, 1) void k_grouped_gemm(GemmLaunch args) {
  constexpr int EPC = Elem<T>::kPer16B;        // elements per 16-byte chunk
  constexpr int BK = kRowB / sizeof(T);        // K elements per stage
  constexpr bool SWIGLU = (ACT == ACT_SWIGLU) && (KIND == GEMM_UP);
  constexpr int NI = BN / 32;                  // 16-row n-subtiles per wave (wave covers BN/2 B rows)
  constexpr int MJ = 8;                        // 16-row m-subtiles per wave (wave covers 128 rows)
  constexpr int A_BYTES = kBM * kRowB;
  constexpr int B_BYTES = BN * kRowB;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int A_LD = kBM / 32;               // wave load instructions per stage (8 rows x 128 B each)
  constexpr int B_LD = BN / 32;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  // ---- tile decode (XCD-contiguous renumbering)
  const int nb = gridDim.x;
  const int L = (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3);
  if (L >= args.total_tiles) return;
  const bool second = args.nprob > 1 && L >= args.tile_begin1;
  const GemmProblem& P = second ? args.p1 : args.p0;
  const int Lq = second ? L - args.tile_begin1 : L;
  const int tn = second ? args.tiles_n1 : args.tiles_n0;
  const int mt_ub = second ? args.mt_ub1 : args.mt_ub0;
  const int grp = Lq / (kGM * tn);
  const int rem = Lq - grp * kGM * tn;
  const int gsz = min(kGM, mt_ub - grp * kGM);
  const int mt = grp * kGM + rem % gsz;
  const int nt = rem / gsz;
  int g, row0, rows;
  if (!locate_mtile(P, mt, g, row0, rows)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- per-lane source offsets. Load instruction i of wave w fills tile rows i*32 + 8w .. +8;
  // lane l writes row r = i*32 + 8w + l/8 at slot l%8, i.e. chunk (l%8) ^ ((r >> 1) & 7).
  const T* __restrict__ Ab = (const T*)P.A;
  const T* __restrict__ Bb = (const T*)P.B + (size_t)g * P.b_gstride;
  const T* __restrict__ B3b = SWIGLU ? (const T*)P.B3 + (size_t)g * P.b_gstride : nullptr;
  uint32_t a_off[A_LD], b_off[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int r = i * 32 + wave * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const int orow = row0 + min(r, rows - 1);
    const int arow = P.a_rows ? P.a_rows[orow] : orow;
    a_off[i] = (uint32_t)((size_t)arow * P.lda + c * EPC);
  }
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int r = i * 32 + wave * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const bool gate = SWIGLU && (i >= B_LD / 2);
    const int brow = SWIGLU ? nt * (BN / 2) + (gate ? r - BN / 2 : r) : nt * BN + r;
    b_off[i] = (uint32_t)((size_t)brow * P.ldb + c * EPC);
  }

  const int nk = P.K / BK;
  auto issue_stage = [&](int kt, int buf) {
    const int64_t k0 = (int64_t)kt * BK;
    const int64_t seg = k0 / P.k_seg;
    const int64_t boff = seg * P.k_seg_stride + (k0 - seg * P.k_seg);
    uint8_t* sa = smem + buf * STAGE + wave * 8 * kRowB;
    uint8_t* sb = smem + buf * STAGE + A_BYTES + wave * 8 * kRowB;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) gload_lds16(Ab + k0 + a_off[i], sa + i * 32 * kRowB);
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const bool gate = SWIGLU && (i >= B_LD / 2);
      gload_lds16((gate ? B3b : Bb) + boff + b_off[i], sb + i * 32 * kRowB);
    }
  };

  // B-tile row of n-subtile i for this wave.
  auto brow_of = [&](int i) -> int {
    if (SWIGLU) {
      constexpr int H = NI / 2;
      return i < H ? wn * (BN / 4) + i * 16 : BN / 2 + wn * (BN / 4) + (i - H) * 16;
    }
    return wn * (BN / 2) + i * 16;
  };

  floatx4_t acc[NI][MJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < MJ; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  issue_stage(0, 0);
  const int fr = lane & 15, fg = lane >> 4;
  for (int kt = 0; kt < nk; ++kt) {
    wait_vmem();
    __syncthreads();                       // stage kt is in LDS; stage kt-1's buffer is free
    if (kt + 1 < nk) issue_stage(kt + 1, (kt + 1) & 1);
    const uint8_t* sa = smem + (kt & 1) * STAGE;
    const uint8_t* sb = sa + A_BYTES;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ch = ks * 4 + fg;
      uint4 af[MJ], bfr[NI];
#pragma unroll
      for (int j = 0; j < MJ; ++j) af[j] = *reinterpret_cast<const uint4*>(sa + swz(wm * 128 + j * 16 + fr, ch));
#pragma unroll
      for (int i = 0; i < NI; ++i) bfr[i] = *reinterpret_cast<const uint4*>(sb + swz(brow_of(i) + fr, ch));
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < MJ; ++j) acc[i][j] = mfma16(bfr[i], af[j], acc[i][j], T());
    }
  }

  // ---- epilogue: lane holds rows (m) = wm*128 + j*16 + fr, columns 4*fg + t of n-subtile i
  const int64_t col_base = (int64_t)g * P.c_gcol;
#pragma unroll
  for (int j = 0; j < MJ; ++j) {
    const int ml = wm * 128 + j * 16 + fr;
    if (ml >= rows) continue;
    const int64_t orow = row0 + ml;
    if (KIND == GEMM_UP) {
      T* crow = (T*)P.C + orow * P.ldc + col_base;
      constexpr int NO = SWIGLU ? NI / 2 : NI;
#pragma unroll
      for (int i = 0; i < NO; ++i) {
        float h[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float u = acc[i][j][t];
          if (SWIGLU) h[t] = silu(acc[i + NI / 2][j][t]) * u;
          else if (ACT == ACT_GELU_TANH) h[t] = gelu_tanh(u);
          else h[t] = gelu_erf(u);
        }
        const int n = SWIGLU ? nt * (BN / 2) + wn * (BN / 4) + i * 16 + 4 * fg : nt * BN + wn * (BN / 2) + i * 16 + 4 * fg;
        if (sizeof(T) == 2) {
          uint2 v;
          v.x = (uint32_t)f32_to_bf16(h[0]) | ((uint32_t)f32_to_bf16(h[1]) << 16);
          v.y = (uint32_t)f32_to_bf16(h[2]) | ((uint32_t)f32_to_bf16(h[3]) << 16);
          *reinterpret_cast<uint2*>(crow + n) = v;
        } else {
          *reinterpret_cast<float4*>(crow + n) = make_float4(h[0], h[1], h[2], h[3]);
        }
      }
    } else {
      float* crow = (float*)P.C + orow * P.ldc + col_base;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int n = nt * BN + wn * (BN / 2) + i * 16 + 4 * fg;
        *reinterpret_cast<float4*>(crow + n) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      }
    }
  }
}

static int out_cols_per_tile(int kind, int act, int BN) { return (kind == GEMM_UP && act == ACT_SWIGLU) ? BN / 2 : BN; }

static int pick_bn(int kind, int act, int N) {
  if (N % out_cols_per_tile(kind, act, 256) == 0) return 256;
  if (N % out_cols_per_tile(kind, act, 128) == 0) return 128;
  return 0;
}

bool grouped_gemm_supported(int dtype, int kind, int act, int N, int K) {
  const int bk = dtype == 0 ? 64 : 32;
  return N > 0 && K > 0 && K % bk == 0 && pick_bn(kind, act, N) != 0;
}

template <typename T, int KIND, int ACT, int BN>
static void launch_t(const GemmLaunch& la, int grid, hipStream_t st) {
  auto kfn = k_grouped_gemm<T, KIND, ACT, BN>;
  MOE_LAUNCH(KIND == GEMM_UP ? "gemm_up" : "gemm_down", kfn, grid, kThreads, 0, st, la);
}

template <typename T, int KIND, int ACT>
static void launch_bn(const GemmLaunch& la, int bn, int grid, hipStream_t st) {
  if (bn == 256) launch_t<T, KIND, ACT, 256>(la, grid, st);
  else launch_t<T, KIND, ACT, 128>(la, grid, st);
}

template <typename T>
static void launch_kind(const GemmLaunch& la, int kind, int act, int bn, int grid, hipStream_t st) {
  if (kind == GEMM_DOWN) {
    launch_bn<T, GEMM_DOWN, ACT_GELU>(la, bn, grid, st);
  } else if (act == ACT_SWIGLU) {
    launch_bn<T, GEMM_UP, ACT_SWIGLU>(la, bn, grid, st);
  } else if (act == ACT_GELU_TANH) {
    launch_bn<T, GEMM_UP, ACT_GELU_TANH>(la, bn, grid, st);
  } else {
    launch_bn<T, GEMM_UP, ACT_GELU>(la, bn, grid, st);
  }
}

hipError_t launch_grouped_gemm(int dtype, int kind, int act, const GemmProblem* probs, const int64_t* rows_ub,
                               int nprob, hipStream_t st) {
  if (nprob < 1 || nprob > 2) return hipErrorInvalidValue;
  const int bn = pick_bn(kind, act, probs[0].N);
  if (bn == 0) return hipErrorInvalidValue;
  GemmLaunch la{};
  la.nprob = nprob;
  int64_t total = 0;
  for (int i = 0; i < nprob; ++i) {
    if (pick_bn(kind, act, probs[i].N) != bn) return hipErrorInvalidValue;
    const int32_t tiles_n = probs[i].N / out_cols_per_tile(kind, act, bn);
    int64_t mt;
    if (probs[i].offsets) mt = (rows_ub[i] + kBM - 1) / kBM + probs[i].G;   // sum of ceil() over groups
    else mt = (int64_t)probs[i].G * ((probs[i].M_uni + kBM - 1) / kBM);
    if (i == 0) {
      la.p0 = probs[0];
      la.tiles_n0 = tiles_n;
      la.mt_ub0 = (int32_t)mt;
    } else {
      la.p1 = probs[1];
      la.tiles_n1 = tiles_n;
      la.mt_ub1 = (int32_t)mt;
      la.tile_begin1 = (int32_t)total;
    }
    total += mt * tiles_n;
  }
  if (total == 0) return hipSuccess;
  if (total > (int64_t)1 << 30) return hipErrorInvalidValue;
  la.total_tiles = (int32_t)total;
  const int grid = (int)((total + 7) / 8 * 8);
  if (dtype == 0) launch_kind<bf16_t>(la, kind, act, bn, grid, st);
  else launch_kind<float>(la, kind, act, bn, grid, st);
  return hipGetLastError();
}

}  // namespace moe
