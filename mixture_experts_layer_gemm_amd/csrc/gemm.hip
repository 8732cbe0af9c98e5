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
// Design (one workgroup = 4 waves, one per SIMD, = one 256 x BN tile, BN in {128, 192, 256}; each wave
// owns 128 token rows x BN/2 weight rows, the 2 x 2 split with the fewest LDS reads per MFMA):
//   * K advances one MFMA K step (64 bytes of every tile row) per stage. Stages go through a ring
//     of five LDS slots, filled by direct global->LDS loads (no staging registers): four stages
//     are in flight while one feeds the MFMAs, which hides L2-miss latency; one barrier per stage.
//   * The loads of a stage and the LDS fragment reads of the next one are spread between the
//     MFMAs of the current one (sched_group_barrier regions), so issue never stalls on a full queue.
//   * LDS rows are 64 B; 16-byte chunk c of row r sits at slot c ^ ((r >> 2) & 3), so the 16-byte
//     fragment reads of 16 consecutive rows cover all banks once.
//   * Weights are MFMA operand P and tokens operand Q, so each lane ends with 4 consecutive output
//     columns of one row: 8-byte (bf16) / 16-byte (fp32) stores.
//   * Gather fused into the A loads: row r reads x[row_token[r]].
//   * Tile order: workgroup b runs on XCD b % 8; tiles are renumbered so each XCD owns a
//     contiguous range, swept as 8 m-tiles x all n-tiles, which keeps an expert's weight panels and
//     token panels in one XCD's L2.
//   * The expert of an m-tile comes from a wave-wide scan of ceil(count_e / 256) over experts.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kBM = 256;
constexpr int kRowB = 64;           // bytes of one tile row per stage (one MFMA K-step)
constexpr int kStages = 5;          // LDS ring: four stages in flight while one is consumed
constexpr int kRowsPerLoad = 1024 / kRowB;   // rows one wave-wide 16-byte-per-lane load fills
constexpr int kWaves = 4;           // 2 x 2 wave grid, one wave per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kGM = 8;              // m-tiles per sweep group

struct GemmLaunch {
  GemmProblem p0, p1;
  int32_t tiles_n0, tiles_n1;
  int32_t slots0, slots1;   // workgroups per XCD reserved for each problem (from upper bounds)
};

// 16-byte chunk c (0..3) of tile row r sits at slot c ^ ((r >> 2) & 3): the 16-byte fragment reads
// of 16 consecutive rows then cover all 64 banks once.
__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowB + ((chunk ^ ((row >> 2) & 3)) << 4); }

// m-tiles of a problem: groups in order, ceil(rows_g / 256) tiles each. The group offsets are read
// with scalar loads (constant address space: the kernel never writes them), so finding a tile's
// group takes no vector registers and no vector-memory wait (those would also wait for the ring's
// loads in flight).
typedef const __attribute__((address_space(4))) int32_t* scalar_i32_ptr;

__device__ __forceinline__ int mtile_total(const GemmProblem& P) {
  if (!P.offsets) return P.G * ((P.M_uni + kBM - 1) / kBM);
  const scalar_i32_ptr o = (scalar_i32_ptr)P.offsets;
  int tot = 0, prev = o[0];
  for (int g = 0; g < P.G; ++g) {
    const int nx = o[g + 1];
    tot += (nx - prev + kBM - 1) / kBM;
    prev = nx;
  }
  return tot;
}

// Group, first row and row count of m-tile `mt` (uniform). False past the end.
__device__ __forceinline__ bool mtile_locate(const GemmProblem& P, int mt, int& g, int& row0, int& rows) {
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
  const scalar_i32_ptr o = (scalar_i32_ptr)P.offsets;
  int acc = 0, prev = o[0];
  for (int gi = 0; gi < P.G; ++gi) {
    const int nx = o[gi + 1];
    const int mts = (nx - prev + kBM - 1) / kBM;
    if (mt < acc + mts) {
      g = gi;
      row0 = prev + (mt - acc) * kBM;
      rows = min(kBM, nx - row0);
      return true;
    }
    acc += mts;
    prev = nx;
  }
  return false;
}

// Placement of the work of one K step: NM MFMAs; NF LDS reads, read q right before MFMA
// read_pos(q); LPS global->LDS loads, load d right before MFMA (d * NM) / LPS. An "MFMA" here is
// one 16x16 product step, MPC instructions. region<M0, M1>() pins the order of the LDS reads and
// MFMAs of MFMAs [M0, M1) (loads bound the regions).
template <int NM, int NF, int LPS, int MPC>
struct step_sched {
  static constexpr int load_pos(int d) { return d < 0 ? 0 : (d * NM) / LPS; }
  static constexpr int load_at(int m) {
    for (int d = 0; d < LPS; ++d)
      if (load_pos(d) == m) return d;
    return -1;
  }
  // the reads are spread over the first 3/4 of the MFMAs, so that they have landed when the next
  // step starts
  static constexpr int RSPAN = NM - NM / 4;
  static_assert(RSPAN >= NF, "one read per MFMA slot at most");
  static constexpr int read_pos(int q) { return (q * RSPAN) / NF; }
  static constexpr int read_at_q(int m) {
    for (int q = 0; q < NF; ++q)
      if (read_pos(q) == m) return q;
    return -1;
  }
  static constexpr bool read_at(int m) { return read_at_q(m) >= 0; }
  // MFMAs from m up to (not including) the next read position or m1
  static constexpr int run(int m, int m1) {
    int e = m + 1;
    while (e < m1 && !read_at(e)) ++e;
    return e - m;
  }
  template <int M0, int M1>
  __device__ static __forceinline__ void region() {
    if constexpr (M0 < M1) {
      constexpr int n = run(M0, M1);
      if constexpr (read_at(M0)) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, n * MPC, 0);                       // MFMA
      region<M0 + n, M1>();
    }
  }
};

template <typename T, int KIND, int ACT, int BN>
__global__ __launch_bounds__(kThreads, 1) void k_grouped_gemm(GemmLaunch args) {
  constexpr int EPC = Elem<T>::kPer16B;        // elements per 16-byte chunk
  constexpr int BK = kRowB / sizeof(T);        // K elements per stage
  constexpr bool SWIGLU = (ACT == ACT_SWIGLU) && (KIND == GEMM_UP);
  constexpr int NI = BN / 32;                  // 16-row n-subtiles per wave (wave covers BN/2 B rows)
  constexpr int MJ = 8;                        // 16-row m-subtiles per wave (wave covers 128 rows)
  constexpr int NF = MJ + NI;                  // fragments per K step
  constexpr int A_BYTES = kBM * kRowB;
  constexpr int B_BYTES = BN * kRowB;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int A_LD = kBM / (kRowsPerLoad * kWaves);   // wave load instructions per stage
  constexpr int B_LD = BN / (kRowsPerLoad * kWaves);
  constexpr int LPS = A_LD + B_LD;                       // loads per wave per stage
  // One array per ring stage: with the K loop unrolled every LDS access names its stage at compile
  // time. Five 32 KB slots are all of LDS; nothing else in the kernel uses LDS.
  static_assert(kStages == 5, "the ring below is written for five stages");
  __shared__ __attribute__((aligned(16))) uint8_t smem0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t smem1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t smem2[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t smem3[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t smem4[STAGE];

  // ---- tile decode. Workgroups are dealt to the 8 XCDs round robin (workgroup b to XCD b % 8), in
  // order. The tiles of each problem that exist (m-tiles counted from the offsets) are cut into 8
  // contiguous chunks, one per XCD, swept as kGM m-tiles x all n-tiles, which keeps an expert's
  // weight panels and token panels in one L2. An XCD runs its chunk of problem 0 (the one with the
  // longer K, placed there by the host) and then its chunk of problem 1; workgroups beyond both
  // chunks (the grid is sized from upper bounds on the row counts) exit at once.
  const int mtl0 = mtile_total(args.p0), mtl1 = args.slots1 ? mtile_total(args.p1) : 0;
  const int live0 = mtl0 * args.tiles_n0, live1 = mtl1 * args.tiles_n1;
  const int c0 = (live0 + 7) >> 3, c1 = (live1 + 7) >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const bool second = slot >= c0;
  const int Lq = second ? xcd * c1 + (slot - c0) : xcd * c0 + slot;
  if (second ? (slot - c0 >= c1 || Lq >= live1) : Lq >= live0) return;
  const GemmProblem P = second ? args.p1 : args.p0;   // a copy: kept in scalar registers
  const int tn = second ? args.tiles_n1 : args.tiles_n0;
  const int mt_live = second ? mtl1 : mtl0;
  const int grp = Lq / (kGM * tn);
  const int rem = Lq - grp * kGM * tn;
  const int gsz = min(kGM, mt_live - grp * kGM);
  const int mt = grp * kGM + rem % gsz;
  const int nt = rem / gsz;
  int g, row0, rows;
  if (!mtile_locate(P, mt, g, row0, rows)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // ---- per-lane source offsets. Load instruction i of wave w fills tile rows
  // i*16*kWaves + 16w .. +16; lane l writes row r = i*16*kWaves + 16w + l/4 at slot l%4, i.e. the
  // chunk (l%4) ^ ((r >> 2) & 3) of that row.
  const T* __restrict__ Ab = (const T*)P.A;
  const T* __restrict__ Bb = (const T*)P.B + (size_t)g * P.b_gstride;
  const T* __restrict__ B3b = SWIGLU ? (const T*)P.B3 + (size_t)g * P.b_gstride : nullptr;
  // byte offsets of this lane's 16 bytes in the A and B tiles, constant over K
  uint32_t a_off[A_LD], b_off[B_LD];
  bool b_gate[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int r = i * kRowsPerLoad * kWaves + wave * kRowsPerLoad + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    const int orow = row0 + min(r, rows - 1);
    const int arow = P.a_rows ? P.a_rows[orow] : orow;
    a_off[i] = (uint32_t)(((size_t)arow * P.lda + c * EPC) * sizeof(T));
  }
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int r = i * kRowsPerLoad * kWaves + wave * kRowsPerLoad + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    const bool gate = SWIGLU && r >= BN / 2;   // the same for the whole wave
    b_gate[i] = gate;
    // rows past N (a ragged last column tile) re-read row N-1; their columns are not stored
    const int brow = min(SWIGLU ? nt * (BN / 2) + (gate ? r - BN / 2 : r) : nt * BN + r, P.N - 1);
    b_off[i] = (uint32_t)(((size_t)brow * P.ldb + c * EPC) * sizeof(T));
  }

  const int nk = P.K / BK;
  // Source positions of the next stage to load: K offset into A, and into B (whose K axis may be
  // split into segments of k_seg elements placed k_seg_stride apart). Stages are issued in order,
  // one per K step; stages past the end re-load the last stage (valid memory that the load just
  // before brought into the caches; never read).
  const int k_seg = (int)P.k_seg;
  const int64_t k_skip = P.k_seg_stride - P.k_seg;
  int64_t a_k = 0, b_k = 0;
  int b_within = 0, issued = 0;
  const uint32_t wave_off = (uint32_t)(wave * kRowsPerLoad * kRowB);
  struct Dma {
    const T* a;
    const T* b;
    const T* b3;
    uint32_t lds;
  };
  auto next_dma = [&](uint32_t stage) -> Dma {
    Dma d;
    d.a = Ab + a_k;
    d.b = Bb + b_k;
    d.b3 = SWIGLU ? B3b + b_k : nullptr;
    d.lds = stage + wave_off;
    if (++issued < nk) {   // past the end the position stays on the last stage
      a_k += BK;
      b_k += BK;
      b_within += BK;
      if (b_within == k_seg) {
        b_within = 0;
        b_k += k_skip;
      }
    }
    return d;
  };
  // load instruction q (0..LPS) of a stage: A loads first, then B
  auto dma_one = [&](const Dma& d, auto Qc) {
    constexpr int q = decltype(Qc)::value;
    if constexpr (q < A_LD) {
      gload_lds16(d.a, a_off[q], d.lds + q * kRowsPerLoad * kWaves * kRowB);
    } else {
      constexpr int i = q - A_LD;
      gload_lds16(b_gate[i] ? d.b3 : d.b, b_off[i], d.lds + A_BYTES + i * kRowsPerLoad * kWaves * kRowB);
    }
  };
  auto issue_all = [&](const Dma& d) {
    dma_one(d, std::integral_constant<int, 0>{});
    if constexpr (LPS > 1) dma_one(d, std::integral_constant<int, 1>{});
    if constexpr (LPS > 2) dma_one(d, std::integral_constant<int, 2>{});
    if constexpr (LPS > 3) dma_one(d, std::integral_constant<int, 3>{});
    if constexpr (LPS > 4) dma_one(d, std::integral_constant<int, 4>{});
    if constexpr (LPS > 5) dma_one(d, std::integral_constant<int, 5>{});
    if constexpr (LPS > 6) dma_one(d, std::integral_constant<int, 6>{});
    if constexpr (LPS > 7) dma_one(d, std::integral_constant<int, 7>{});
    static_assert(LPS <= 8, "at most 8 loads per stage");
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

  const int fr = lane & 15, fg = lane >> 4;
  // Fragments of one K step: f[0..MJ) token rows (operand Q), f[MJ..) weight rows (operand P).
  auto read_frags = [&](const uint8_t* stage, uint4 (&f)[NF]) {
#pragma unroll
    for (int j = 0; j < MJ; ++j) f[j] = *reinterpret_cast<const uint4*>(stage + swz(wm * 128 + j * 16 + fr, fg));
#pragma unroll
    for (int i = 0; i < NI; ++i)
      f[MJ + i] = *reinterpret_cast<const uint4*>(stage + A_BYTES + swz(brow_of(i) + fr, fg));
  };

  // One K step t, after the barrier: MFMAs on the fragments of stage t (cur) with, spread between
  // them, the LDS reads of stage t + 1 (into nxt) and the loads of stage t + 5 (into the LDS slot
  // of stage t, free once every wave has passed the barrier). Issued as blocks, the LDS reads would
  // fill the LDS queue and the loads the memory queue, stalling the wave before its MFMAs (issue is
  // in order). Loads are inline assembly, which the scheduler does not move, so the step is a chain
  // of regions separated by loads, each with its own sched_group_barrier pattern. The body is
  // generated by compile-time recursion so that every accumulator index is a constant.
  constexpr int NM = NI * MJ;   // MFMAs per step
  using SS = step_sched<NM, NF, LPS, Elem<T>::kMfmaPerStep>;
  auto read_frag = [&](const uint8_t* stage, auto Qc) -> uint4 {
    constexpr int q = decltype(Qc)::value;
    if constexpr (q < MJ) return *reinterpret_cast<const uint4*>(stage + swz(wm * 128 + q * 16 + fr, fg));
    else return *reinterpret_cast<const uint4*>(stage + A_BYTES + swz(brow_of(q - MJ) + fr, fg));
  };
  auto body = [&](auto self, auto Mc, const uint8_t* next, const Dma& dma, uint4 (&cur)[NF],
                  uint4 (&nxt)[NF]) -> void {
    constexpr int m = decltype(Mc)::value;
    if constexpr (m < NM) {
      constexpr int d = SS::load_at(m);
      if constexpr (d >= 0) {
        SS::template region<SS::load_pos(d - 1), m>();
        dma_one(dma, std::integral_constant<int, d>{});
      }
      constexpr int q = SS::read_at_q(m);   // the read that belongs right before MFMA m, if any
      if constexpr (q >= 0) nxt[q] = read_frag(next, std::integral_constant<int, q>{});
      constexpr int i = m / MJ, j = m % MJ;
      acc[i][j] = mfma16(cur[MJ + i], cur[j], acc[i][j], T());
      self(self, std::integral_constant<int, m + 1>{}, next, dma, cur, nxt);
    } else {
      SS::template region<SS::load_pos(LPS - 1), NM>();
    }
  };
  // step t: wait for stage t + 1 (stages t + 2 .. t + 4 may stay in flight), synchronise, then the
  // body.
  auto step = [&](const uint8_t* next, uint32_t refill, uint4 (&cur)[NF], uint4 (&nxt)[NF]) {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): cur is in registers
    wait_vmem<3 * LPS>();
    ring_barrier();
    const Dma dma = next_dma(refill);
    body(body, std::integral_constant<int, 0>{}, next, dma, cur, nxt);
  };

  uint4 fa[NF], fb[NF];
  const uint32_t l0 = lds_addr(smem0), l1 = lds_addr(smem1), l2 = lds_addr(smem2), l3 = lds_addr(smem3),
                 l4 = lds_addr(smem4);
  issue_all(next_dma(l0));
  issue_all(next_dma(l1));
  issue_all(next_dma(l2));
  issue_all(next_dma(l3));
  issue_all(next_dma(l4));
  wait_vmem<4 * LPS>();
  ring_barrier();
  read_frags(smem0, fa);
  // stage t sits in slot t % 5; the fragment buffers alternate, so ten steps bring both back
  for (int kt = 0; kt < nk; kt += 2 * kStages) {
    step(smem1, l0, fa, fb);
    if (kt + 1 < nk) step(smem2, l1, fb, fa);
    if (kt + 2 < nk) step(smem3, l2, fa, fb);
    if (kt + 3 < nk) step(smem4, l3, fb, fa);
    if (kt + 4 < nk) step(smem0, l4, fa, fb);
    if (kt + 5 < nk) step(smem1, l0, fb, fa);
    if (kt + 6 < nk) step(smem2, l1, fa, fb);
    if (kt + 7 < nk) step(smem3, l2, fb, fa);
    if (kt + 8 < nk) step(smem4, l3, fa, fb);
    if (kt + 9 < nk) step(smem0, l4, fb, fa);
  }
  wait_vmem<0>();   // no load into LDS may still be in flight when the workgroup ends

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
        if (n >= P.N) continue;
        if (sizeof(T) == 2) {
          uint2 v;
          v.x = pack2_bf16(h[0], h[1]);
          v.y = pack2_bf16(h[2], h[3]);
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
        if (n >= P.N) continue;
        *reinterpret_cast<float4*>(crow + n) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      }
    }
  }
}

static int out_cols_per_tile(int kind, int act, int BN) { return (kind == GEMM_UP && act == ACT_SWIGLU) ? BN / 2 : BN; }

// Tile width. The time of a launch is modelled as (rounds of one tile per compute unit) x (time of
// one tile), with the time of a tile proportional to BN / eff(BN): the wider tile reads fewer LDS
// bytes per MFMA (measured dense rates: eff = 1, 0.9, 0.74 for BN = 256, 192, 128), the narrower
// ones make more tiles, which can fill the last round better. A problem's tiles count K / K_min
// rounds each, K_min the shortest K of the launch.
static int tile_cost(int bn) { return bn == 256 ? 256 : bn == 192 ? 213 : 173; }

static int compute_units() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// m-tiles of a problem: exact for uniform groups; for offsets-based groups the caller's hint, else
// the count for rows_ub rows plus half a ragged tile per group.
static int64_t est_mtiles(const GemmProblem& p, int64_t rows_ub, const int64_t* hint) {
  if (!p.offsets) return (int64_t)p.G * ((p.M_uni + kBM - 1) / kBM);
  if (hint && *hint > 0) return *hint;
  return std::max<int64_t>(1, (rows_ub + kBM - 1) / kBM + p.G / 2);
}

static int pick_bn(int kind, int act, const GemmProblem* probs, const int64_t* rows_ub, const int64_t* mt_hint,
                   int nprob) {
  for (int i = 0; i < nprob; ++i)
    if (probs[i].N <= 0 || probs[i].N % 64 != 0) return 0;
  int kmin = probs[0].K;
  for (int i = 0; i < nprob; ++i) kmin = std::min(kmin, probs[i].K);
  kmin = std::max(kmin, 1);
  const int64_t cus = compute_units();
  int best = 0;
  double best_t = 0.0;
  for (int bn : {256, 192, 128}) {
    const int c = out_cols_per_tile(kind, act, bn);
    double units = 0.0;   // tiles, weighted by K / kmin (a round is one tile of the shortest K)
    for (int i = 0; i < nprob; ++i)
      units += (double)est_mtiles(probs[i], rows_ub[i], mt_hint ? mt_hint + i : nullptr) *
               ((probs[i].N + c - 1) / c) * probs[i].K / kmin;
    const double t = std::ceil(units / (double)cus - 1e-9) * tile_cost(bn);
    if (best == 0 || t < best_t) {
      best = bn;
      best_t = t;
    }
  }
  return best;
}

bool grouped_gemm_supported(int dtype, int kind, int act, int N, int K) {
  (void)kind;
  (void)act;
  const int bk = kRowB / (dtype == 0 ? 2 : 4);
  return N > 0 && N % 64 == 0 && K > 0 && K % bk == 0;
}

template <typename T, int KIND, int ACT, int BN>
static void launch_t(const GemmLaunch& la, int grid, hipStream_t st) {
  auto kfn = k_grouped_gemm<T, KIND, ACT, BN>;
  MOE_LAUNCH(KIND == GEMM_UP ? "gemm_up" : "gemm_down", kfn, grid, kThreads, 0, st, la);
}

template <typename T, int KIND, int ACT>
static void launch_bn(const GemmLaunch& la, int bn, int grid, hipStream_t st) {
  if (bn == 256) launch_t<T, KIND, ACT, 256>(la, grid, st);
  else if (bn == 192) launch_t<T, KIND, ACT, 192>(la, grid, st);
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
                               const int64_t* mt_hint, int nprob, hipStream_t st) {
  if (nprob < 1 || nprob > 2) return hipErrorInvalidValue;
  const int bn = pick_bn(kind, act, probs, rows_ub, mt_hint, nprob);
  if (bn == 0) return hipErrorInvalidValue;
  // the problem with the longer K goes first (see the tile decode in the kernel)
  const int first = (nprob == 2 && probs[1].K > probs[0].K) ? 1 : 0;
  GemmLaunch la{};
  int64_t total = 0;
  for (int n = 0; n < nprob; ++n) {
    const int i = n == 0 ? first : 1 - first;
    const int c = out_cols_per_tile(kind, act, bn);
    const int64_t tiles_n = (probs[i].N + c - 1) / c;
    int64_t mt;
    if (probs[i].offsets) mt = (rows_ub[i] + kBM - 1) / kBM + probs[i].G;   // sum of ceil() over groups
    else mt = (int64_t)probs[i].G * ((probs[i].M_uni + kBM - 1) / kBM);
    const int64_t tiles = mt * tiles_n;
    if (tiles > (int64_t)1 << 28) return hipErrorInvalidValue;
    const int32_t slots = (int32_t)((tiles + 7) / 8);
    if (n == 0) {
      la.p0 = probs[i];
      la.tiles_n0 = (int32_t)tiles_n;
      la.slots0 = slots;
    } else {
      la.p1 = probs[i];
      la.tiles_n1 = (int32_t)tiles_n;
      la.slots1 = slots;
    }
    total += slots;
  }
  if (total == 0) return hipSuccess;
  const int grid = (int)(8 * total);
  if (dtype == 0) launch_kind<bf16_t>(la, kind, act, bn, grid, st);
  else launch_kind<float>(la, kind, act, bn, grid, st);
  return hipGetLastError();
}

}  // namespace moe
