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
// Design (one workgroup = one 256 x BN tile, BN in {128, 192, 256}, of 4 waves, one per SIMD, each
// owning 128 token rows x BN/2 weight rows, the 2 x 2 split with the fewest LDS reads per MFMA; the
// GELU up projections use 8 waves, two per SIMD, each owning 128 x BN/4):
//   * K advances in blocks of two MFMA K steps: 128 bytes of every tile row, one whole cache line,
//     so every 16-byte-per-lane load instruction reads 8 full lines (reading 64-byte halves made
//     twice the L2 requests for the same bytes, and the L2 request rate was the limit).
//   * The A block (256 token rows) and the B block (BN weight rows) of a K block each fill one
//     32 KB unit of a five-unit LDS ring, by direct global->LDS loads (no staging registers). The
//     loads of one operand (L) start three MFMA steps before its first read, those of the other
//     (S) two; the up projections give the weights the long lead, the down projections the
//     tokens. Each step carries one unit's loads; one barrier per block.
//   * The loads of a block and the LDS fragment reads of the next step are spread between the
//     MFMAs of the current one (sched_group_barrier regions), so issue never stalls on a full queue.
//   * LDS rows are 128 B; 16-byte chunk c of row r sits at slot c ^ ((r >> 1) & 7), so the 16-byte
//     fragment reads of 16 consecutive rows cover all banks once.
//   * Weights are MFMA operand P and tokens operand Q, so each lane ends with 4 consecutive output
//     columns of one row: 8-byte (bf16) / 16-byte (fp32) stores. With 256-wide tiles the SwiGLU up
//     and the fp32 down outputs are staged through the freed LDS ring first, so that each store
//     instruction writes whole 128-byte lines.
//   * Gather fused into the A loads: row r reads x[row_token[r]].
//   * Tile order: workgroup b runs on XCD b % 8; tiles are renumbered so each XCD owns a
//     contiguous range, swept as 4 m-tiles x all n-tiles, which keeps an expert's weight panels and
//     token panels in one XCD's L2.
//   * The expert of an m-tile comes from a scalar scan of ceil(count_e / 256) over experts.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kBM = 256;
constexpr int kRowB = 128;          // bytes of one tile row per LDS unit: one cache line, two MFMA K steps
constexpr int kStepB = 64;          // bytes of one tile row per MFMA K step
constexpr int kUnits = 5;           // LDS ring of 32 KB units; the A and B units of the K blocks alternate
constexpr int kUnitB = 32768;
constexpr int kRowsPerLoad = 1024 / kRowB;   // rows one wave-wide 16-byte-per-lane load fills
constexpr int kGM = 4;              // m-tiles per sweep group

struct GemmLaunch {
  GemmProblem p0, p1;
  int32_t tiles_n0, tiles_n1;
  int32_t slots0, slots1;   // workgroups per XCD reserved for each problem (from upper bounds)
};

// 16-byte chunk c (0..7) of tile row r sits at slot c ^ ((r >> 1) & 7): the 16-byte fragment reads
// of 16 consecutive rows (one chunk each) then cover all 64 banks once (the even rows fill one half
// of the 256-byte bank cycle, the odd rows the other).
__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowB + ((chunk ^ ((row >> 1) & 7)) << 4); }

// m-tiles of a problem: groups in order, ceil(rows_g / 256) tiles each. The group offsets are read
// with scalar loads (constant address space: the kernel never writes them), so finding a tile's
// group takes no vector registers and no vector-memory wait (those would also wait for the ring's
// loads in flight). They are read kOffChunk + 1 at a time, every load of a chunk issued before any
// is used, so a chunk costs one scalar round trip; one load per group, each waited for before the
// next, made the decode about 6% of a GELU up-projection tile.
typedef const __attribute__((address_space(4))) int32_t* scalar_i32_ptr;
constexpr int kOffChunk = 16;

__device__ __forceinline__ int tiles_of(int rows) { return (int)(((unsigned)rows + (kBM - 1)) / kBM); }

// offsets[g0 .. g0 + kOffChunk] into v, for g0 < G. A whole chunk in bounds is read at immediate
// offsets from one base (one instruction per entry, no address arithmetic); in the last, partial
// chunk entries past G are not read and are set to offsets[G], so that their groups have no rows.
__device__ __forceinline__ void load_chunk(scalar_i32_ptr o, int g0, int G, int (&v)[kOffChunk + 1]) {
  const scalar_i32_ptr b = o + g0;
  const int n = G - g0;
  if (n >= kOffChunk) {
#pragma unroll
    for (int j = 0; j <= kOffChunk; ++j) v[j] = b[j];
  } else {
#pragma unroll
    for (int j = 0; j <= kOffChunk; ++j) v[j] = j <= n ? b[j] : 0;
#pragma unroll
    for (int j = 1; j <= kOffChunk; ++j)
      if (j > n) v[j] = v[j - 1];
  }
}

__device__ __forceinline__ int mtile_total(const GemmProblem& P) {
  if (!P.offsets) return P.G * tiles_of(P.M_uni);
  const scalar_i32_ptr o = (scalar_i32_ptr)P.offsets;
  int tot = 0;
  for (int g0 = 0; g0 < P.G; g0 += kOffChunk) {
    int v[kOffChunk + 1];
    load_chunk(o, g0, P.G, v);
#pragma unroll
    for (int j = 0; j < kOffChunk; ++j) tot += tiles_of(v[j + 1] - v[j]);   // 0 past G: equal entries
  }
  return tot;
}

// Group, first row and row count of m-tile `mt` (uniform). False past the end.
__device__ __forceinline__ bool mtile_locate(const GemmProblem& P, int mt, int& g, int& row0, int& rows) {
  if (!P.offsets) {
    const int mpg = tiles_of(P.M_uni);
    if (mpg == 0) return false;
    g = mt / mpg;
    if (g >= P.G) return false;
    const int lm = mt - g * mpg;
    row0 = lm * kBM;
    rows = min(kBM, P.M_uni - row0);
    return true;
  }
  const scalar_i32_ptr o = (scalar_i32_ptr)P.offsets;
  int acc = 0;
  for (int g0 = 0; g0 < P.G; g0 += kOffChunk) {
    int v[kOffChunk + 1];
    load_chunk(o, g0, P.G, v);
#pragma unroll
    for (int j = 0; j < kOffChunk; ++j) {
      const int mts = tiles_of(v[j + 1] - v[j]);
      if (mt < acc + mts) {   // never past G: groups there have no tiles
        g = g0 + j;
        row0 = v[j] + (mt - acc) * kBM;
        rows = min(kBM, v[j + 1] - row0);
        return true;
      }
      acc += mts;
    }
  }
  return false;
}

// Placement of the work of one K step: NM MFMAs; NF LDS reads, read q right before MFMA
// read_pos(q); LPS global->LDS loads, load d right before MFMA (d * NM) / LPS. An "MFMA" here is
// one 16x16 product step, MPC instructions. region<M0, M1>() pins the order of the LDS reads and
// MFMAs of MFMAs [M0, M1) (loads bound the regions).
template <int NM, int NF, int LPS, int MPC>
struct step_sched {
  static constexpr int load_pos(int d) { return d < 0 || LPS == 0 ? 0 : (d * NM) / LPS; }
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

// The LDS ring: five 32 KB units, one array per unit, so that with the K loop unrolled every LDS
// access names its unit at compile time. They are all of LDS; nothing else in the GEMM kernels uses
// LDS, and each kernel that uses them gets its own copy.
static_assert(kUnits == 5, "the ring below is written for five units");
__shared__ __attribute__((aligned(16))) uint8_t smem0[kUnitB];
__shared__ __attribute__((aligned(16))) uint8_t smem1[kUnitB];
__shared__ __attribute__((aligned(16))) uint8_t smem2[kUnitB];
__shared__ __attribute__((aligned(16))) uint8_t smem3[kUnitB];
__shared__ __attribute__((aligned(16))) uint8_t smem4[kUnitB];

// One 256 x BN tile of problem P: m-tile rows [row0, row0 + rows) of group g, n-tile nt.
template <typename T, int KIND, int ACT, int BN, int WV>
__device__ __forceinline__ void gemm_tile(const GemmProblem& P, const int g, const int row0, const int rows,
                                          const int nt) {
  constexpr int EPC = Elem<T>::kPer16B;        // elements per 16-byte chunk
  constexpr int BK = kStepB / sizeof(T);       // K elements per MFMA step
  constexpr int BU = 2 * BK;                   // K elements per unit (one K block)
  constexpr bool SWIGLU = (ACT == ACT_SWIGLU) && (KIND == GEMM_UP);
  constexpr int WN = WV / 2;                   // wave grid: 2 rows of WN waves
  constexpr int NI = BN / (16 * WN);           // 16-row n-subtiles per wave (wave covers BN/WN B rows)
  constexpr int MJ = 8;                        // 16-row m-subtiles per wave (wave covers 128 rows)
  constexpr int NF = MJ + NI;                  // fragments per K step
  constexpr int A_LD = kBM / (kRowsPerLoad * WV);   // wave load instructions per A unit
  constexpr int B_LD = BN / (kRowsPerLoad * WV);    // per B unit
  static_assert(BN % (16 * WN) == 0 && (!SWIGLU || NI % 2 == 0), "whole n-subtiles per wave (gate and up halves)");
  static_assert(A_LD * kRowsPerLoad * WV == kBM && B_LD * kRowsPerLoad * WV == BN, "whole loads per unit");
  static_assert(kBM * kRowB <= kUnitB && BN * kRowB <= kUnitB, "a unit holds one K block of A or of B");


  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // ---- per-lane source offsets. Load instruction i of wave w fills the 128-byte rows
  // i*8*WV + 8w .. +8 of a unit; lane l writes row r = i*8*WV + 8w + l/8 at slot l%8, i.e. the
  // chunk (l%8) ^ ((r >> 1) & 7) of that row. Eight lanes read one whole cache line.
  const T* __restrict__ Ab = (const T*)P.A;
  const T* __restrict__ Bb = (const T*)P.B + (size_t)g * P.b_gstride;
  const T* __restrict__ B3b = SWIGLU ? (const T*)P.B3 + (size_t)g * P.b_gstride : nullptr;
  // byte offsets of this lane's 16 bytes in the A and B tiles, constant over K
  uint32_t a_off[A_LD], b_off[B_LD];
  bool b_gate[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int r = i * kRowsPerLoad * WV + wave * kRowsPerLoad + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const int orow = row0 + min(r, rows - 1);
    const int arow = P.a_rows ? P.a_rows[orow] : orow;
    a_off[i] = (uint32_t)(((size_t)arow * P.lda + c * EPC) * sizeof(T));
  }
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int r = i * kRowsPerLoad * WV + wave * kRowsPerLoad + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const bool gate = SWIGLU && r >= BN / 2;   // the same for the whole wave
    b_gate[i] = gate;
    // rows past N (a ragged last column tile) re-read row N-1; their columns are not stored
    const int brow = min(SWIGLU ? nt * (BN / 2) + (gate ? r - BN / 2 : r) : nt * BN + r, P.N - 1);
    b_off[i] = (uint32_t)(((size_t)brow * P.ldb + c * EPC) * sizeof(T));
  }

  const int nu = P.K / BU;   // K blocks (two MFMA steps each)
  // Source positions of the next A and B units to load: K offset into A, and into B (whose K axis
  // may be split into segments of k_seg elements placed k_seg_stride apart). Units of each kind are
  // issued in order; past the end the position stays on the last block (valid memory that the load
  // just before brought into the caches; never read).
  const int k_seg = (int)P.k_seg;
  const int64_t k_skip = P.k_seg_stride - P.k_seg;
  int64_t a_k = 0, b_k = 0;
  int b_within = 0, a_issued = 0, b_issued = 0;
  const uint32_t wave_off = (uint32_t)(wave * kRowsPerLoad * kRowB);
  struct Dma {
    const T* p;    // A, or B (W1) rows
    const T* p3;   // SwiGLU gate rows (W3)
    uint32_t lds;
  };
  auto next_a = [&](uint32_t unit) -> Dma {
    Dma d;
    d.p = Ab + a_k;
    d.p3 = nullptr;
    d.lds = unit + wave_off;
    if (++a_issued < nu) a_k += BU;
    return d;
  };
  auto next_b = [&](uint32_t unit) -> Dma {
    Dma d;
    d.p = Bb + b_k;
    d.p3 = SWIGLU ? B3b + b_k : nullptr;
    d.lds = unit + wave_off;
    if (++b_issued < nu) {
      b_k += BU;
      b_within += BU;
      if (b_within == k_seg) {
        b_within = 0;
        b_k += k_skip;
      }
    }
    return d;
  };
  constexpr uint32_t kLoadStride = kRowsPerLoad * WV * kRowB;   // LDS bytes between a wave's loads
  auto dma_a = [&](const Dma& d, auto Qc) {
    constexpr int q = decltype(Qc)::value;
    gload_lds16(d.p, a_off[q], d.lds + q * kLoadStride);
  };
  auto dma_b = [&](const Dma& d, auto Qc) {
    constexpr int i = decltype(Qc)::value;
    gload_lds16(b_gate[i] ? d.p3 : d.p, b_off[i], d.lds + i * kLoadStride);
  };
  auto issue_a = [&](const Dma& d) { static_for<A_LD>([&](auto Qc) { dma_a(d, Qc); }); };
  // The ring alternates the units of two operands: L, whose loads start three MFMA steps before
  // it is first read, and S, two steps (below). The up projections give the weights the longer
  // lead, the down projections the tokens (measured on the dense SwiGLU up and long-K down shapes).
  constexpr bool B_LONG = KIND == GEMM_UP;
  constexpr int L_LD = B_LONG ? B_LD : A_LD, S_LD = B_LONG ? A_LD : B_LD;
  auto issue_b = [&](const Dma& d) { static_for<B_LD>([&](auto Qc) { dma_b(d, Qc); }); };

  // B-tile row of n-subtile i for this wave.
  auto brow_of = [&](int i) -> int {
    if (SWIGLU) {
      constexpr int H = NI / 2;
      return i < H ? wn * (BN / (2 * WN)) + i * 16 : BN / 2 + wn * (BN / (2 * WN)) + (i - H) * 16;
    }
    return wn * (BN / WN) + i * 16;
  };

  floatx4_t acc[NI][MJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < MJ; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  const int fr = lane & 15, fg = lane >> 4;
  // Fragment q of K step s of a block: q < MJ token rows (operand Q, from the A unit ua), else
  // weight rows (operand P, from the B unit ub); 16-byte chunk 4s + fg of the 128-byte row.
  auto read_frag = [&](const uint8_t* ua, const uint8_t* ub, auto Sc, auto Qc) -> uint4 {
    constexpr int st = decltype(Sc)::value, q = decltype(Qc)::value;
    if constexpr (q < MJ) return *reinterpret_cast<const uint4*>(ua + swz(wm * 128 + q * 16 + fr, st * 4 + fg));
    else return *reinterpret_cast<const uint4*>(ub + swz(brow_of(q - MJ) + fr, st * 4 + fg));
  };
  auto read_all = [&](auto self, auto Qc, const uint8_t* ua, const uint8_t* ub, uint4 (&f)[NF]) -> void {
    constexpr int q = decltype(Qc)::value;
    if constexpr (q < NF) {
      f[q] = read_frag(ua, ub, std::integral_constant<int, 0>{}, Qc);
      self(self, std::integral_constant<int, q + 1>{}, ua, ub, f);
    }
  };

  // One K step: MFMAs on the fragments in registers (cur) with, spread between them, the LDS reads
  // of the next step's fragments (into nxt) and, on the second step of a block, the loads of two
  // units. Issued as blocks, the LDS reads would fill the LDS queue and the loads the memory queue,
  // stalling the wave before its MFMAs (issue is in order). Loads are inline assembly, which the
  // scheduler does not move, so the step is a chain of regions separated by loads, each with its
  // own sched_group_barrier pattern. The body is generated by compile-time recursion so that every
  // accumulator index is a constant.
  constexpr int NM = NI * MJ;   // MFMAs per step
  auto body = [&](auto self, auto Lc, auto Sc, auto Mc, const uint8_t* ua, const uint8_t* ub, const Dma& ds,
                  const Dma& dl, uint4 (&cur)[NF], uint4 (&nxt)[NF]) -> void {
    constexpr int KL = decltype(Lc)::value;   // -1: the loads of an L unit; -2: of an S unit
    constexpr int NL = KL == -1 ? L_LD : S_LD;
    using SS = step_sched<NM, NF, NL, Elem<T>::kMfmaPerStep>;
    constexpr int m = decltype(Mc)::value;
    if constexpr (m < NM) {
      constexpr int d = SS::load_at(m);
      if constexpr (d >= 0) {
        SS::template region<SS::load_pos(d - 1), m>();
        if constexpr (KL == -2) {
          if constexpr (B_LONG) dma_a(ds, std::integral_constant<int, d>{});
          else dma_b(ds, std::integral_constant<int, d>{});
        } else {
          if constexpr (B_LONG) dma_b(dl, std::integral_constant<int, d>{});
          else dma_a(dl, std::integral_constant<int, d>{});
        }
      }
      constexpr int q = SS::read_at_q(m);   // the read that belongs right before MFMA m, if any
      if constexpr (q >= 0) nxt[q] = read_frag(ua, ub, Sc, std::integral_constant<int, q>{});
      constexpr int i = m / MJ, j = m % MJ;
      acc[i][j] = mfma16(cur[MJ + i], cur[j], acc[i][j], T());
      self(self, Lc, Sc, std::integral_constant<int, m + 1>{}, ua, ub, ds, dl, cur, nxt);
    } else {
      SS::template region<SS::load_pos(NL - 1), NM>();
    }
  };
  // Ring: unit u (L_p = 2p, S_p = 2p + 1) sits in slot u % 5. During block p the slots hold L_p and
  // S_p (being read), L_{p+1}, S_{p+1} and L_{p+2}.
  // First step of block p: its second step's fragments come from L_p and S_p, which every wave has
  // seen since the previous barrier, so there is no wait for memory and no barrier; it loads
  // L_{p+2} into the slot of S_{p-1}, free since that barrier.
  auto step0 = [&](const uint8_t* ul, const uint8_t* us, uint32_t slot_sprev, uint4 (&cur)[NF], uint4 (&nxt)[NF]) {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): cur is in registers
    const Dma dl = B_LONG ? next_b(slot_sprev) : next_a(slot_sprev);
    body(body, std::integral_constant<int, -1>{}, std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{},
         B_LONG ? us : ul, B_LONG ? ul : us, dl, dl, cur, nxt);
  };
  // Second step of block p: wait for L_{p+1} and S_{p+1} (L_{p+2}, issued after them, may stay in
  // flight), synchronise (L_p and S_p are then free: every wave has read its fragments of block p),
  // load S_{p+2} into the slot of L_p, and read the first step's fragments of block p + 1.
  auto step1 = [&](const uint8_t* nul, const uint8_t* nus, uint32_t slot_lp, uint4 (&cur)[NF], uint4 (&nxt)[NF]) {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    wait_vmem<L_LD>();
    ring_barrier();
    const Dma ds = B_LONG ? next_a(slot_lp) : next_b(slot_lp);
    body(body, std::integral_constant<int, -2>{}, std::integral_constant<int, 0>{},
         std::integral_constant<int, 0>{}, B_LONG ? nus : nul, B_LONG ? nul : nus, ds, ds, cur, nxt);
  };

  uint4 fa[NF], fb[NF];
  const uint32_t l0 = lds_addr(smem0), l1 = lds_addr(smem1), l2 = lds_addr(smem2), l3 = lds_addr(smem3),
                 l4 = lds_addr(smem4);
  auto issue_l = [&](uint32_t slot) {
    if constexpr (B_LONG) issue_b(next_b(slot));
    else issue_a(next_a(slot));
  };
  auto issue_s = [&](uint32_t slot) {
    if constexpr (B_LONG) issue_a(next_a(slot));
    else issue_b(next_b(slot));
  };
  issue_l(l0);   // L_0
  issue_s(l1);   // S_0
  issue_l(l2);   // L_1
  issue_s(l3);   // S_1 (L_2 comes with the first step)
  wait_vmem<L_LD + S_LD>();   // L_0 and S_0
  ring_barrier();
  if constexpr (B_LONG) read_all(read_all, std::integral_constant<int, 0>{}, smem1, smem0, fa);
  else read_all(read_all, std::integral_constant<int, 0>{}, smem0, smem1, fa);
  // block p reads L_p, S_p from slots (2p) % 5, (2p + 1) % 5, and S_{p-1} sat in slot (2p - 1) % 5:
  // five blocks bring the pattern back
  for (int pb = 0; pb < nu; pb += kUnits) {
    step0(smem0, smem1, l4, fa, fb);
    step1(smem2, smem3, l0, fb, fa);
    if (pb + 1 < nu) {
      step0(smem2, smem3, l1, fa, fb);
      step1(smem4, smem0, l2, fb, fa);
    }
    if (pb + 2 < nu) {
      step0(smem4, smem0, l3, fa, fb);
      step1(smem1, smem2, l4, fb, fa);
    }
    if (pb + 3 < nu) {
      step0(smem1, smem2, l0, fa, fb);
      step1(smem3, smem4, l1, fb, fa);
    }
    if (pb + 4 < nu) {
      step0(smem3, smem4, l2, fa, fb);
      step1(smem0, smem1, l3, fb, fa);
    }
  }
  wait_vmem<0>();   // no load into LDS may still be in flight when the workgroup ends

  // ---- epilogue: lane holds rows (m) = wm*128 + j*16 + fr, columns 4*fg + t of n-subtile i
  const int64_t col_base = (int64_t)g * P.c_gcol;
  if constexpr (SWIGLU && BN == 256 && sizeof(T) == 2 && WV == 4) {
    // SwiGLU with 256-wide tiles: each wave's 128 x 64 bf16 outputs (128 bytes per row) go through
    // LDS, so that every store instruction writes 8 whole 128-byte lines instead of 16 rows x 32
    // bytes. 16-byte chunk c of staged row r sits at slot c ^ (r & 7). The ring is free once every
    // wave has passed this barrier (their last fragment reads are done).
    ring_barrier();
    uint8_t* stage = (wave < 2 ? smem0 : smem1) + (wave & 1) * (128 * 128);
#pragma unroll
    for (int j = 0; j < MJ; ++j)
#pragma unroll
      for (int i = 0; i < NI / 2; ++i) {
        float h[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) h[t] = silu(acc[i + NI / 2][j][t]) * acc[i][j][t];
        uint2 v;
        v.x = pack2_bf16(h[0], h[1]);
        v.y = pack2_bf16(h[2], h[3]);
        const int r = j * 16 + fr, c = 2 * i + (fg >> 1);
        *reinterpret_cast<uint2*>(stage + r * 128 + ((c ^ (r & 7)) << 4) + (fg & 1) * 8) = v;
      }
    asm volatile("" ::: "memory");   // the wave's LDS accesses run in order; keep the compiler's too
    const int c = lane & 7;
    const int n = nt * (BN / 2) + wn * (BN / 4) + c * 8;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int r = q * 8 + (lane >> 3);
      const uint4 v = *reinterpret_cast<const uint4*>(stage + r * 128 + ((c ^ (r & 7)) << 4));
      const int ml = wm * 128 + r;
      if (ml >= rows || n >= P.N) continue;
      *reinterpret_cast<uint4*>((T*)P.C + (row0 + ml) * P.ldc + col_base + n) = v;
    }
    return;
  }
  if constexpr (KIND == GEMM_UP && !SWIGLU && BN == 256 && WV == 8 && sizeof(T) == 2) {
    // GELU with 256-wide tiles and 8 waves: each wave's 128 x 64 bf16 outputs (128 bytes per row, one
    // cache line) go through its own 16 KB of the freed ring, so that every store instruction writes 8
    // whole lines instead of 16 rows x 32 bytes. 16-byte chunk c of staged row r sits at slot c ^ (r & 7).
    ring_barrier();
    uint8_t* stage = (wave < 2 ? smem0 : wave < 4 ? smem1 : wave < 6 ? smem2 : smem3) + (wave & 1) * (128 * 128);
#pragma unroll
    for (int j = 0; j < MJ; ++j)
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float h[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) h[t] = ACT == ACT_GELU_TANH ? gelu_tanh(acc[i][j][t]) : gelu_erf(acc[i][j][t]);
        uint2 v;
        v.x = pack2_bf16(h[0], h[1]);
        v.y = pack2_bf16(h[2], h[3]);
        const int r = j * 16 + fr, c = 2 * i + (fg >> 1);
        *reinterpret_cast<uint2*>(stage + r * 128 + ((c ^ (r & 7)) << 4) + (fg & 1) * 8) = v;
      }
    asm volatile("" ::: "memory");   // the wave's LDS accesses run in order; keep the compiler's too
    const int c = lane & 7;
    const int n = nt * BN + wn * (BN / WN) + c * 8;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int r = q * 8 + (lane >> 3);
      const uint4 v = *reinterpret_cast<const uint4*>(stage + r * 128 + ((c ^ (r & 7)) << 4));
      const int ml = wm * 128 + r;
      if (ml >= rows || n >= P.N) continue;
      *reinterpret_cast<uint4*>((T*)P.C + (row0 + ml) * P.ldc + col_base + n) = v;
    }
    return;
  }
  if constexpr (KIND == GEMM_DOWN && BN == 256 && WV == 4) {
    // fp32 outputs with 256-wide tiles: each wave's 128 x 128 outputs go through its own 32 KB unit
    // in two halves of 64 rows (512 bytes per row), 16-byte chunk c of row r at slot c ^ (r & 15);
    // each store instruction then writes 2 rows x 512 bytes (8 whole lines) instead of 16 rows x
    // 64 bytes.
    ring_barrier();
    uint8_t* stage = wave == 0 ? smem0 : wave == 1 ? smem1 : wave == 2 ? smem2 : smem3;
    const int c = lane & 31;
    const int n = nt * BN + wn * (BN / 2) + c * 4;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int jj = 0; jj < MJ / 2; ++jj)
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int j = hf * (MJ / 2) + jj;
          const int r = jj * 16 + fr, ch = 4 * i + fg;
          *reinterpret_cast<float4*>(stage + r * 512 + ((ch ^ (r & 15)) << 4)) =
              make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
      asm volatile("" ::: "memory");
#pragma unroll
      for (int q = 0; q < 32; ++q) {
        const int r = q * 2 + (lane >> 5);
        const float4 v = *reinterpret_cast<const float4*>(stage + r * 512 + ((c ^ (r & 15)) << 4));
        const int ml = wm * 128 + hf * 64 + r;
        if (ml >= rows || n >= P.N) continue;
        *reinterpret_cast<float4*>((float*)P.C + (row0 + ml) * P.ldc + col_base + n) = v;
      }
      asm volatile("" ::: "memory");   // the second half overwrites what the first half read
    }
    return;
  }
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
        const int n = SWIGLU ? nt * (BN / 2) + wn * (BN / (2 * WN)) + i * 16 + 4 * fg
                             : nt * BN + wn * (BN / WN) + i * 16 + 4 * fg;
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
        const int n = nt * BN + wn * (BN / WN) + i * 16 + 4 * fg;
        if (n >= P.N) continue;
        *reinterpret_cast<float4*>(crow + n) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      }
    }
  }
}

// WV waves per workgroup: 4 (one per SIMD, each wave 128 x BN/2 outputs) or 8 (two per SIMD, each
// 128 x BN/4: a wave that stalls on a load, an LDS read or the barrier leaves the matrix core to the
// other wave of its SIMD).
template <typename T, int KIND, int ACT, int BN, int WV>
__global__ __launch_bounds__(64 * WV, 1) void k_grouped_gemm(GemmLaunch args) {
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
  // A last column tile that is at most half used (N = 1152 with 256-wide tiles: 4.5 tiles) runs the
  // 128-wide body: the same columns at about two thirds of the time, where the 256-wide body would
  // multiply a half tile of repeated weight rows (for the fp32 down projection).
  if constexpr (KIND == GEMM_DOWN && BN == 256 && WV == 4 && sizeof(T) == 2) {
    if (nt == tn - 1 && P.N - nt * BN <= BN / 2) {
      gemm_tile<T, KIND, ACT, BN / 2, WV>(P, g, row0, rows, 2 * nt);
      return;
    }
  }
  gemm_tile<T, KIND, ACT, BN, WV>(P, g, row0, rows, nt);
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

// Column tiles of one m-tile, in units of a tile of width bn; a last 256-wide tile that is at most half
// used runs the 128-wide body (bf16 down projection) and counts at that body's cost.
static double col_tiles(int N, int c, int bn, bool half_tile) {
  if (half_tile && bn == 256 && N % 256 != 0 && N % 256 <= 128)
    return N / 256 + (double)tile_cost(128) / tile_cost(256);
  return (N + c - 1) / c;
}

static int pick_bn(int kind, int act, bool half_tile, const GemmProblem* probs, const int64_t* rows_ub,
                   const int64_t* mt_hint, int nprob) {
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
               col_tiles(probs[i].N, c, bn, half_tile) * probs[i].K / kmin;
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
  const int bu = kRowB / (dtype == 0 ? 2 : 4);   // K elements per unit
  return N > 0 && N % 64 == 0 && K > 0 && K % bu == 0;
}

template <typename T, int KIND, int ACT, int BN, int WV>
static void launch_t(const GemmLaunch& la, int grid, hipStream_t st) {
  auto kfn = k_grouped_gemm<T, KIND, ACT, BN, WV>;
  MOE_LAUNCH(KIND == GEMM_UP ? "gemm_up" : "gemm_down", kfn, grid, 64 * WV, 0, st, la);
}

// Waves per workgroup. Eight (two per SIMD) for the bf16 GELU up projections with 256-wide tiles:
// their long activation epilogue and the main loop's issue stalls then share each SIMD with a
// second wave (mmoe: 537 -> 516 us per layer on one box). Four everywhere else: with eight, the
// waves read 1.5x the LDS fragments per MFMA and the down projections lose the LDS-staged store
// (mmoe down 431 -> 475 us, dit_moe_xl down 313 -> 354 us); the SwiGLU up projection was unchanged.
template <typename T, int KIND, int ACT>
static void launch_bn(const GemmLaunch& la, int bn, int grid, hipStream_t st) {
  constexpr bool W8 = sizeof(T) == 2 && KIND == GEMM_UP && ACT != ACT_SWIGLU;
  if (bn == 256) launch_t<T, KIND, ACT, 256, W8 ? 8 : 4>(la, grid, st);
  else if (bn == 192) launch_t<T, KIND, ACT, 192, 4>(la, grid, st);
  else launch_t<T, KIND, ACT, 128, 4>(la, grid, st);
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
  const int bu = kRowB / (dtype == 0 ? 2 : 4);   // K elements per unit: a unit never straddles a K segment
  for (int i = 0; i < nprob; ++i)
    if (probs[i].K <= 0 || probs[i].K % bu != 0 || probs[i].k_seg <= 0 || probs[i].k_seg % bu != 0)
      return hipErrorInvalidValue;
  const int bn = pick_bn(kind, act, kind == GEMM_DOWN && dtype == 0, probs, rows_ub, mt_hint, nprob);
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
