// FP32 SGEMM on the CDNA4 matrix cores (v_mfma_f32_32x32x2_f32).
//
// C = alpha*op(A)*op(B) + beta*C, row-major ("GEMM 优化之路", problem
// statement), where op(A) = A (stored M x K) or A^T (A stored K x M), and
// op(B) = B (stored K x N) or B^T (B stored N x K) -- the transposed cases of
// the gsyq.cn guide (section 6.4, step 8).  The structure keeps the page's
// data-reuse ladder -- block tile staged in LDS, per-wave register tile, LDS
// stages with one barrier per K step, fused alpha/beta update -- with each
// level shaped for gfx950:
//
// * Block tile BM x BN, K step BK (16, 32 or 64) per K group; a stage holds
//   BKS = KG * BK values of k.  Each wave owns a WM x WN sub-tile of 32x32
//   MFMA blocks (16 accumulators per lane per block).
// * An operand tile in LDS has one of two unpadded layouts, chosen by how the
//   operand is stored, with 16-byte units XOR-swizzled instead of padding:
//   - K-contiguous (A as stored, or B^T): rows of the outer index (m or n)
//     holding BKS/4 units of four consecutive k; unit c of row r sits at
//     c ^ ((r / (64/BKS)) & (BKS/4 - 1)), so the 16-byte reads of 16
//     consecutive rows at one column group hit 16 distinct bank groups.
//   - outer-contiguous (B as stored, or A^T): rows of k holding the outer
//     index; the second k half of every K step has its 32-float halves
//     exchanged, so the two MFMA lane halves read different banks.
// * Lane l of a wave moves 16-byte unit (v*WAVES + wave)*64 + l of a stage.
//   Its global source is the inverse of the swizzle, so consecutive lanes
//   read consecutive 16-byte pieces of a stored row: loads stay coalesced.
// * Loader, aligned and edge kernels: global_load_lds_dwordx4, which
//   writes lane l's 16 bytes to LDS at M0 + 16*l with no register staging.
//   Two stages: the loads of step t+1 go out before the MFMAs of step t and
//   are waited for (vmcnt) before the barrier that ends step t.  The LDS
//   holds the A tiles of both stages, then the B tiles, and the K loop is
//   unrolled by stage, so fragment reads take the stage in their immediate
//   offsets.  The 64x64 tile also reads step t+1's fragments into a second
//   register set during step t (its steps are short), and its loads run two
//   steps ahead.
// * Three modes per tile shape:
//   - aligned (MODE 0): M, N and K are whole multiples of the tile and of the
//     stage's K range; every load is a direct load.
//   - edge (MODE 1): any M, N, K.  Whole K steps still use direct loads.  A
//     unit that lies past the last row or column of an operand is loaded from
//     the last valid row or column instead: it only feeds outputs outside
//     M x N, which are never stored, so clamping the address is enough and no
//     zero fill is needed.  The partial K step at the end (K not a multiple of
//     the stage's K range) goes through registers with zero fill, since there
//     both operands must be exactly zero past K.  A unit that runs along M or
//     N (B as stored, or A^T) may straddle the edge when that extent is not a
//     multiple of 4: its elements past the edge again only feed outputs that
//     are never stored, and the 16-byte read stays inside the operand as long
//     as the row is not the last one (the read ends at most 3 floats into the
//     next row).  In that case the last K row always goes through the
//     zero-filled register step, which then covers the last partial or whole
//     K step.  This mode needs that extent to be at least 4.
//   - guarded (MODE 2): every unit through registers, 16-byte loads where the
//     whole unit is inside the operand, element loads with zero fill elsewhere
//     ("GEMM 优化之路", exercise 2: out-of-range loads become zeros; no thread
//     leaves before the barriers).
//   16-byte global loads (plain and direct-to-LDS) need only 4-byte aligned
//   addresses on gfx950 (checked with an in-bounds probe), so neither the
//   leading dimensions nor the base pointers of A and B have to be multiples
//   of 4 floats.
// * MFMA operands are swapped (B block as the first operand): the 32x32
//   result is then the transpose of the C block, and each lane holds four
//   consecutive columns of one C row per register quad.  The epilogue reads C
//   (only when beta != 0) and writes it with 16-byte accesses when ldc and C
//   allow, one 32x32 block at a time.
// * Which k an MFMA lane half uses is free as long as A and B agree: lanes
//   0-31 take k in [0, BK/2) of the K step and lanes 32-63 take [BK/2, BK).
//   A K-contiguous fragment is then one 16-byte LDS read per four MFMAs; an
//   outer-contiguous one is one 4-byte read per MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tile_map.hpp"

namespace sgemm {

typedef float f32x4 __attribute__((ext_vector_type(4)));
// a 16-byte operand piece that may be only 4-byte aligned
typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

template <int BM_, int BN_, int WM_, int WN_, int OCC_, int S_ = 2, int BK_ = 16,
          int KG_ = 1, int PF_ = 0>
struct MfmaTile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
  static constexpr int OCC = OCC_;  // waves per SIMD the registers are sized for
  // LDS stages: two, so the direct loads run one K step ahead of the MFMAs
  // (three and four stages measured slower on every tile).
  static constexpr int S = S_;
  // K groups: KG groups of waves split every stage's K range (KG*BK values)
  // and their partial sums are added through LDS at the end, group 1 first.
  // This multiplies the waves per tile for problems with few tiles without a
  // workspace or a second pass.
  static constexpr int KG = KG_;
  // Fragment prefetch (two stages only): each wave reads the next K step's
  // fragments from LDS into a second register set while its MFMAs run on
  // the current step's, so after a barrier the MFMAs start at once instead
  // of waiting for LDS reads.  Pays where a step is short (few MFMAs per
  // wave between barriers) and the registers are there.
  static constexpr bool PF = PF_ != 0;
  static constexpr int BKS = KG * BK;  // K values per LDS stage
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int WAVES_MN = WAVES_M * WAVES_N;  // waves of one K group
  static constexpr int WAVES = WAVES_MN * KG;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int FM = WM / 32, FN = WN / 32;  // 32x32 blocks per wave
  static constexpr int A_ELEMS = BM * BKS, B_ELEMS = BKS * BN;
  static constexpr int STAGE = A_ELEMS + B_ELEMS;  // floats per LDS stage
  static constexpr int LDS_BYTES = S * STAGE * 4;
  static constexpr int A_UNITS = BM * BKS / 4, B_UNITS = BKS * BN / 4;
  static constexpr int A_VEC = A_UNITS / THREADS;  // 16-byte units per lane
  static constexpr int B_VEC = B_UNITS / THREADS;
  static constexpr int KH = BK / 2;    // k values per MFMA lane half per K step
  static constexpr int QN = KH / 4;    // four-k fragments per lane half
  static constexpr int UPR = BKS / 4;  // 16-byte units per K-contiguous row
  static constexpr int RPG = 16 / UPR; // such rows per 256-byte bank sweep
  static_assert(BM % WM == 0 && BN % WN == 0, "wave grid");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "32x32 MFMA blocks");
  static_assert(BM >= 32 && (BM & (BM - 1)) == 0, "tile rows");
  static_assert(BN >= 64 && (BN & (BN - 1)) == 0, "outer-contiguous B swizzle");
  static_assert(A_VEC >= 1 && A_VEC * THREADS == A_UNITS, "A loader");
  static_assert(B_VEC >= 1 && B_VEC * THREADS == B_UNITS, "B loader");
  static_assert(LDS_BYTES <= 160 * 1024, "gfx950 LDS");
  static_assert(S == 2, "two LDS stages");
  static_assert(A_VEC + B_VEC <= 63, "vmcnt range");
  static_assert(BK == 16 || BK == 32 || BK == 64, "K step");
  static_assert(BKS <= 64, "K-contiguous rows of at most 16 units");
  static_assert(KG == 1 || KG == 2 || KG == 4, "K groups");
  // floats the K groups 1..KG-1 leave in LDS for group 0
  static constexpr int RED_ELEMS = (KG - 1) * WAVES_MN * 64 * 16 * FM * FN;
  static_assert(RED_ELEMS <= 2 * STAGE, "reduction fits in LDS");
  // Stream-K: workgroups per CU in the persistent grid (one when a
  // workgroup already has 8 waves or more, so the kernel keeps the
  // registers of two waves per SIMD or more), and the waves per SIMD the
  // stream-K kernel's registers are sized for.
  static constexpr int SK_PER_CU = WAVES >= 8 ? 1 : 2;
  static constexpr int SK_OCC = (WAVES * SK_PER_CU + 3) / 4;
};

// K-contiguous tile: float offset of unit c (four k) of outer row r.
template <class T>
__device__ __forceinline__ int kc_unit_off(int r, int c) {
  return 4 * (T::UPR * r + (c ^ ((r / T::RPG) & (T::UPR - 1))));
}
// Outer-contiguous tile of width X: float offset of element (k, x).
template <class T, int X>
__device__ __forceinline__ int oc_elem_off(int k, int x) {
  return k * X + (x ^ (((k / T::KH) & 1) << 5));
}

// Tile-relative coordinates of 16-byte unit u of an operand tile with outer
// size X: the unit covers (outer, k..k+3) in a K-contiguous tile and
// (outer..outer+3, k) in an outer-contiguous one.
template <class T, int X, bool KCONTIG>
__device__ __forceinline__ void unit_coords(int u, int& outer, int& k) {
  if (KCONTIG) {
    outer = u / T::UPR;
    k = 4 * ((u % T::UPR) ^ ((outer / T::RPG) & (T::UPR - 1)));
  } else {
    k = u / (X / 4);
    outer = 4 * ((u % (X / 4)) ^ (((k / T::KH) & 1) << 3));
  }
}

// One global_load_lds_dwordx4: this lane's 16 bytes at `base` + `voff`
// bytes go to LDS at `lds_base` + 16 * lane.  `base` (scalar registers) and
// `lds_base` must be the same for the whole wave; `voff` is the lane's byte
// offset.  Writing M0 and then issuing a load that writes LDS through M0
// needs one wait state in between.  A wave-uniform base keeps the per-step
// address update scalar: the lanes' offsets stay fixed for the whole loop.
__device__ __forceinline__ void dma16(const float* base, unsigned voff,
                                      unsigned lds_base) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(lds_base), "v"(voff), "s"(base)
      : "memory", "m0");
}

enum { MODE_ALIGNED = 0, MODE_EDGE = 1, MODE_GUARDED = 2 };

// The operation's arguments, as the C ABI receives them.
struct GemmArgs {
  int M, N, K;
  float alpha, beta;
  const float* A;
  int lda;
  const float* B;
  int ldb;
  float* C;
  int ldc;
};

// LDS floats a kernel of tile T in mode MODE uses (two stages).
template <class T, int MODE>
struct TileLds {
  static constexpr int NST = T::S;
  static constexpr int FLOATS = NST * T::STAGE;
};

// K steps of one tile: ceil(K / (K values per stage)).  The direct loads
// cover the first ones; a partial last step (and, when a 16-byte piece can
// straddle the edge, the step holding the last K row) goes through registers.
template <class T>
__host__ __device__ inline int tile_k_steps(int K) {
  return (K + T::BKS - 1) / T::BKS;
}

// Lane layout of a wave's tile (the same in every kernel of tile T).
template <class T>
struct WaveCoords {
  int lane, wave, kg, wmn, wm, wn, li, lh;
  __device__ __forceinline__ WaveCoords() {
    lane = threadIdx.x & 63;
    wave = threadIdx.x >> 6;
    kg = wave / T::WAVES_MN;
    wmn = wave % T::WAVES_MN;
    wm = wmn / T::WAVES_N;
    wn = wmn % T::WAVES_N;
    li = lane & 31;
    lh = lane >> 5;
  }
};

// Whether a tile's C accesses need bounds checks (guarded kernels, and edge
// tiles of edge kernels), and whether they can be 16 bytes wide.
template <class T, int MODE>
__device__ __forceinline__ bool c_masked(const GemmArgs& g, int m0, int n0) {
  return MODE == MODE_GUARDED ||
         (MODE == MODE_EDGE && (m0 + T::BM > g.M || n0 + T::BN > g.N));
}
__device__ __forceinline__ bool c_vector(const GemmArgs& g) {
  return (g.ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(g.C) & 15u) == 0);
}

// Read C at this wave's blocks of the tile at (m0, n0) (callers do so only
// when beta != 0): block (i, j), register 4q + e of lane (li, lh) is
// C(row, col) with row = li and col = 8q + 4lh + e inside the block, the
// accumulators' layout.  Each group of four columns is one 16-byte read when
// it lies wholly inside M x N (and C allows 16-byte accesses), else element
// reads of the columns inside; nothing outside M x N is read.
template <class T, int MODE>
__device__ __forceinline__ void load_c(const GemmArgs& g, int m0, int n0,
                                       f32x16 (&cin)[T::FM][T::FN]) {
  const WaveCoords<T> w;
  const bool masked = c_masked<T, MODE>(g, m0, n0);
  const bool vec = c_vector(g);
  const float* __restrict__ C = g.C;
  const int crow = m0 + w.wm * T::WM + w.li;
  const int ccol = n0 + w.wn * T::WN + w.lh * 4;
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j) {
      const int row = crow + i * 32, col = ccol + j * 32;
      const float* p = C + (size_t)row * g.ldc + (masked && row >= g.M ? 0 : col);
      const bool row_in = !masked || row < g.M;
      // the block is built in a register vector and stored whole, so that
      // it stays in registers
      f32x16 v;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (row_in && vec && (!masked || col + 8 * q + 3 < g.N)) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(p + 8 * q);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[4 * q + e] = x[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[4 * q + e] = row_in && (!masked || col + 8 * q + e < g.N) ? p[8 * q + e] : 0.0f;
        }
      }
      cin[i][j] = v;
    }
}

// TA: A stored K x M (op(A) = A^T).  TB: B stored N x K (op(B) = B^T).
// Accumulate the output tile at (m0, n0) over K steps [s0, s1) into acc (the
// caller zeroes it).  On return the first K group's waves (kg == 0) hold the
// tile's partial sum over those steps; the LDS is still in use by the K-group
// reduction, so a caller that reuses it must pass a barrier first.  With
// LOADC (tiles with K groups, whose registers have room for it), the first
// group's waves also read their C blocks into cv (when beta != 0) before the
// K loop: every workgroup otherwise reads C in one burst after the loop,
// with nothing left to overlap it.  Without LOADC cv is not touched.
template <class T, int MODE, bool TA, bool TB, bool LOADC = false>
__device__ __forceinline__ void tile_accumulate(
    const GemmArgs& g, float* lds, int m0, int n0, int s0, int s1,
    f32x16 (&acc)[T::FM][T::FN], f32x16 (&cv)[T::FM][T::FN]) {
  constexpr bool A_KC = !TA;  // A tile K-contiguous
  constexpr bool B_KC = TB;   // B tile K-contiguous
  // the outer-contiguous swizzle exchanges 32-float halves of a row
  static_assert(A_KC || T::BM >= 64, "A stored K x M needs tiles of 64 rows or more");
  constexpr bool GUARD = MODE == MODE_GUARDED;  // no direct loads
  constexpr bool EDGE = MODE == MODE_EDGE;
  constexpr int NST = TileLds<T, MODE>::NST;
  const int M = g.M, N = g.N, K = g.K;
  const float* __restrict__ A = g.A;
  const float* __restrict__ B = g.B;
  const int lda = g.lda, ldb = g.ldb;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int kg = wave / T::WAVES_MN;  // K group
  const int wmn = wave % T::WAVES_MN;
  const int wm = wmn / T::WAVES_N, wn = wmn % T::WAVES_N;
  const int li = lane & 31, lh = lane >> 5;
  // LDS: the A tiles of all stages, then the B tiles, so that a stage's
  // offset from the first stage of its operand stays below 64 KiB and can
  // ride in a read's immediate offset when the stage is known at compile
  // time (the loops below are unrolled by stage).
  auto a_stage_off = [](int stage) { return stage * T::A_ELEMS; };
  auto b_stage_off = [](int stage) { return NST * T::A_ELEMS + stage * T::B_ELEMS; };

  // Tile coordinates of the units this lane moves.
  int a_o[T::A_VEC], a_k[T::A_VEC], b_o[T::B_VEC], b_k[T::B_VEC];
#pragma unroll
  for (int v = 0; v < T::A_VEC; ++v)
    unit_coords<T, T::BM, A_KC>((v * T::WAVES + wave) * 64 + lane, a_o[v], a_k[v]);
#pragma unroll
  for (int v = 0; v < T::B_VEC; ++v)
    unit_coords<T, T::BN, B_KC>((v * T::WAVES + wave) * 64 + lane, b_o[v], b_k[v]);

  // Address of a stored element: (outer, k) of A or B at K offset k0.
  auto a_addr = [&](int o, int k) -> const float* {
    return TA ? A + (size_t)k * lda + (m0 + o) : A + (size_t)(m0 + o) * lda + k;
  };
  auto b_addr = [&](int o, int k) -> const float* {
    return TB ? B + (size_t)(n0 + o) * ldb + k : B + (size_t)k * ldb + (n0 + o);
  };

  // Direct loads: a wave-uniform base per operand (the tile's origin at K
  // step 0, advanced by a fixed stride per step) and per-lane byte offsets
  // that stay fixed; LDS destinations are wave-uniform.  The host keeps every
  // offset below 2^32, and no offset may be negative (it would wrap).  Edge
  // kernels move a unit wholly past the last row (K-contiguous) onto the last
  // valid row, and one wholly past the last column (outer-contiguous, extent
  // at least 4) onto the last four columns, or onto the tile's first column
  // when those start left of the tile (extent not a multiple of 4: that unit
  // then straddles the edge, which the K-row limit below allows); a unit that
  // straddles the last column is read as it is.
  const float* a_base = TA ? A + m0 : A + (size_t)m0 * lda;
  const float* b_base = TB ? B + (size_t)n0 * ldb : B + n0;
  unsigned a_voff[T::A_VEC], b_voff[T::B_VEC];
  if (!GUARD) {
#pragma unroll
    for (int v = 0; v < T::A_VEC; ++v) {
      int o = a_o[v];
      if (EDGE && m0 + o >= M) o = A_KC ? M - 1 - m0 : (M - 4 > m0 ? M - 4 - m0 : 0);
      a_voff[v] = 4u * (TA ? (unsigned)a_k[v] * (unsigned)lda + (unsigned)o
                           : (unsigned)o * (unsigned)lda + (unsigned)a_k[v]);
    }
#pragma unroll
    for (int v = 0; v < T::B_VEC; ++v) {
      int o = b_o[v];
      if (EDGE && n0 + o >= N) o = B_KC ? N - 1 - n0 : (N - 4 > n0 ? N - 4 - n0 : 0);
      b_voff[v] = 4u * (TB ? (unsigned)o * (unsigned)ldb + (unsigned)b_k[v]
                           : (unsigned)b_k[v] * (unsigned)ldb + (unsigned)o);
    }
  }
  const size_t a_step = TA ? (size_t)T::BKS * lda : (size_t)T::BKS;
  const size_t b_step = TB ? (size_t)T::BKS : (size_t)T::BKS * ldb;
  const unsigned lds_u = (unsigned)(uintptr_t)(lds_void_t*)lds;

  // Direct load d of K step kt (the A units first, then the B units).
  auto issue_one = [&](int d, int kt, int stage) {
    if (d < T::A_VEC)
      dma16(a_base + (size_t)kt * a_step, a_voff[d],
            lds_u + 4u * (unsigned)a_stage_off(stage) +
                1024u * (unsigned)(d * T::WAVES + wave_u));
    else
      dma16(b_base + (size_t)kt * b_step, b_voff[d - T::A_VEC],
            lds_u + 4u * (unsigned)b_stage_off(stage) +
                1024u * (unsigned)((d - T::A_VEC) * T::WAVES + wave_u));
  };
  auto issue_dma = [&](int kt, int stage) {
#pragma unroll
    for (int d = 0; d < T::A_VEC + T::B_VEC; ++d) issue_one(d, kt, stage);
  };

  // Register-staged loads (guarded kernels, and the partial last K step of
  // edge kernels): 16-byte loads where the whole unit is inside the operand,
  // element loads with zero fill elsewhere.
  constexpr bool STAGED = GUARD || EDGE;
  f32x4 ra[STAGED ? T::A_VEC : 1], rb[STAGED ? T::B_VEC : 1];
  // Load one unit: KCONTIG runs over k (bounds: outer < OUTER, k < K), else
  // over the outer index (bounds: k < K, outer < OUTER).
  auto load_unit = [&](const float* p, bool kcontig, int outer, int outer_n,
                       int k) -> f32x4 {
    f32x4 x;
    if (kcontig) {
      if (outer < outer_n && k + 3 < K) {
        const f32x4u v = *reinterpret_cast<const f32x4u*>(p);
        return f32x4{v[0], v[1], v[2], v[3]};
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (outer < outer_n && k + e < K) ? p[e] : 0.0f;
    } else {
      if (k < K && outer + 3 < outer_n) {
        const f32x4u v = *reinterpret_cast<const f32x4u*>(p);
        return f32x4{v[0], v[1], v[2], v[3]};
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (k < K && outer + e < outer_n) ? p[e] : 0.0f;
    }
    return x;
  };
  auto load_regs = [&](int kt) {
    const int k0 = kt * T::BKS;
#pragma unroll
    for (int v = 0; v < T::A_VEC; ++v)
      ra[v] = load_unit(a_addr(a_o[v], k0 + a_k[v]), A_KC, m0 + a_o[v], M,
                        k0 + a_k[v]);
#pragma unroll
    for (int v = 0; v < T::B_VEC; ++v)
      rb[v] = load_unit(b_addr(b_o[v], k0 + b_k[v]), B_KC, n0 + b_o[v], N,
                        k0 + b_k[v]);
  };
  auto store_regs = [&](int stage) {
#pragma unroll
    for (int v = 0; v < T::A_VEC; ++v)
      *reinterpret_cast<f32x4*>(lds + a_stage_off(stage) + 256 * (v * T::WAVES + wave) +
                                4 * lane) = ra[v];
#pragma unroll
    for (int v = 0; v < T::B_VEC; ++v)
      *reinterpret_cast<f32x4*>(lds + b_stage_off(stage) + 256 * (v * T::WAVES + wave) +
                                4 * lane) = rb[v];
  };

  // Wait until none of this wave's LDS-bound loads is still in flight
  // (vmcnt(0); the other counters are left at their maxima).
  auto wait_all = [] { __builtin_amdgcn_s_waitcnt(0x0F70); };

  // Fragments of four k (one per MFMA lane half) of LDS stage `stage`.  They
  // are kept as separate floats, not 4-vectors: an outer-contiguous fragment
  // is gathered by 4-byte reads that the compiler pairs, and a 4-vector would
  // force register copies of the pairs (and waits for them) when two
  // fragment sets alternate.
  auto read_q = [&](int stage, int q, float (&a)[T::FM][4], float (&b)[T::FN][4]) {
    const float* As = lds + a_stage_off(stage);
    const float* Bs = lds + b_stage_off(stage);
    // lane half lh of K group kg covers k = kg*BK + lh*KH + 4q .. +3
    const int kq = kg * T::BK + lh * T::KH + q * 4;
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      const int m = wm * T::WM + i * 32 + li;
      if (A_KC) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(As + kc_unit_off<T>(m, kq / 4));
#pragma unroll
        for (int u = 0; u < 4; ++u) a[i][u] = v[u];
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) a[i][u] = As[oc_elem_off<T, T::BM>(kq + u, m)];
      }
    }
#pragma unroll
    for (int j = 0; j < T::FN; ++j) {
      const int n = wn * T::WN + j * 32 + li;
      if (B_KC) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(Bs + kc_unit_off<T>(n, kq / 4));
#pragma unroll
        for (int u = 0; u < 4; ++u) b[j][u] = v[u];
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) b[j][u] = Bs[oc_elem_off<T, T::BN>(kq + u, n)];
      }
    }
  };
  auto mma_q = [&](const float (&a)[T::FM][4], const float (&b)[T::FN][4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(b[j][u], a[i][u],
                                                          acc[i][j], 0, 0, 0);
  };
  // MFMAs of one LDS stage.
  auto compute = [&](int stage) {
#pragma unroll
    for (int q = 0; q < T::QN; ++q) {
      float a[T::FM][4], b[T::FN][4];
      read_q(stage, q, a, b);
      mma_q(a, b);
    }
  };
  // A whole stage's fragments, for the prefetching loop.
  struct Frags {
    float a[T::QN][T::FM][4], b[T::QN][T::FN][4];
  };
  auto read_frags = [&](int stage, Frags& f) {
#pragma unroll
    for (int q = 0; q < T::QN; ++q) read_q(stage, q, f.a[q], f.b[q]);
  };
  auto mma_frags = [&](const Frags& f) {
#pragma unroll
    for (int q = 0; q < T::QN; ++q) mma_q(f.a[q], f.b[q]);
  };


  // K steps: all of them for guarded kernels; the whole ones for the direct
  // loads (aligned kernels have no partial step).  When a unit can straddle
  // the last column of an outer-contiguous operand, the direct loads stop
  // short of the last K row (see the edge mode above).
  const bool straddle = EDGE && ((!A_KC && (M & 3) != 0) || (!B_KC && (N & 3) != 0));
  // direct-load steps: [0, kd); guarded kernels load every step through
  // registers
  const int kd = GUARD      ? tile_k_steps<T>(K)
                 : straddle ? (K > 0 ? (K - 1) / T::BKS : 0)
                            : K / T::BKS;
  // No scalar load may be in flight inside the K loop.  The epilogue's kernel
  // arguments are otherwise fetched just before the loop, and scalar loads
  // complete out of order, so one still pending there turns every LDS-read
  // wait inside the loop into a full lgkmcnt(0) (measured: 4096^3 at 89% of
  // peak instead of 92%).  Make them live here and wait once.
  asm volatile("" ::"s"(g.C), "s"(g.ldc), "s"(g.alpha), "s"(g.beta), "s"(M), "s"(N));
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  // C for the epilogue, read now so that it arrives during the K loop
  if (LOADC && kg == 0 && g.beta != 0.0f) load_c<T, MODE>(g, m0, n0, cv);
  if (GUARD) {
    if (s0 < s1) {
      load_regs(s0);
      store_regs(0);
    }
    __syncthreads();
    for (int kt = s0; kt < s1; ++kt) {
      const int stage = (kt - s0) & 1;
      const bool more = kt + 1 < s1;
      if (more) load_regs(kt + 1);
      compute(stage);
      if (more) store_regs(stage ^ 1);
      __syncthreads();
    }
  } else if (T::PF) {
    // Two stages and two register sets.  Step kt's fragments are read during
    // step kt-1; step kt+2's direct loads go into step kt's stage as soon as
    // the barrier after those reads has passed (the barrier also waits for
    // the wave's LDS reads), and must have landed by the next barrier.
    const int e = s1 < kd ? s1 : kd;  // direct-load steps [s0, e)
    if (s0 < e) issue_dma(s0, 0);
    if (s0 + 1 < e) issue_dma(s0 + 1, 1);
    wait_all();
    __syncthreads();
    Frags f0, f1;
    if (s0 < e) read_frags(0, f0);
    // Every wave's reads of stage 0 must be done before the first step's
    // direct loads overwrite it.
    __syncthreads();
    // One step: MFMAs on `cur` (stage `st`'s data), the next step's
    // fragments into `nxt`, the step after next into stage `st`.  The
    // scheduling barriers keep the MFMAs between the loads and the wait:
    // MFMAs touch no memory, and the compiler would otherwise move most of
    // them past the wait and the barrier, leaving the direct loads nothing
    // to hide behind.
    auto step = [&](int kt, int st, const Frags& cur, Frags& nxt) {
      if (kt + 1 < e) read_frags(st ^ 1, nxt);
      if (kt + 2 < e) issue_dma(kt + 2, st);
      __builtin_amdgcn_sched_barrier(0);
      mma_frags(cur);
      __builtin_amdgcn_sched_barrier(0);
      wait_all();
      __syncthreads();
    };
    int kt = s0;
    for (; kt + 1 < e; kt += 2) {
      step(kt, 0, f0, f1);
      step(kt + 1, 1, f1, f0);
    }
    if (kt < e) step(kt, 0, f0, f1);
  } else {
    const int e = s1 < kd ? s1 : kd;  // direct-load steps [s0, e)
    // Prologue: K step s0 into stage 0.
    if (s0 < e) issue_dma(s0, 0);
    wait_all();
    __syncthreads();
    // One K step from `stage`, loading step kt+1 into `next`, whose previous
    // contents (step kt-1) were read before the last barrier; step kt+1 must
    // be in LDS at the barrier that ends the step.
    auto step = [&](int kt, int stage, int next) {
      if (kt + 1 < e) issue_dma(kt + 1, next);
      compute(stage);
      wait_all();
      __syncthreads();
    };
    int kt = s0;
    for (; kt + 1 < e; kt += 2) {
      step(kt, 0, 1);
      step(kt + 1, 1, 0);
    }
    if (kt < e) step(kt, 0, 1);
  }
  // Edge kernels: the last step through registers, zero-filled past K, when
  // it is partial or holds the last K row of a straddling operand.  The
  // stages are free after the direct-load loop's last barrier.
  if (EDGE && kd * T::BKS < K && s0 <= kd && kd < s1) {
    load_regs(kd);
    store_regs(0);
    __syncthreads();
    // a K group whose whole k range in this step lies past K holds only
    // zeros there: its waves skip the MFMAs
    if (kg * T::BK < K - kd * T::BKS) compute(0);
    if (T::KG > 1) __syncthreads();  // the K-group reduction reuses the LDS
  }


  // K groups 1..KG-1 hand their partial sums to group 0 through LDS (the
  // stages are free after the last barrier); group 0 adds them in order.
  if (T::KG > 1) {
    f32x4* red = reinterpret_cast<f32x4*>(lds);
    constexpr int PER_WAVE = 4 * T::FM * T::FN;  // float4 per lane
    if (kg > 0) {
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int e4 = (i * T::FN + j) * 4 + gq;
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * gq + e];
            red[(((kg - 1) * T::WAVES_MN + wmn) * PER_WAVE + e4) * 64 + lane] = v;
          }
    }
    __syncthreads();
    if (kg == 0) {
#pragma unroll
    for (int src = 1; src < T::KG; ++src)
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int e4 = (i * T::FN + j) * 4 + gq;
            const f32x4 v =
                red[(((src - 1) * T::WAVES_MN + wmn) * PER_WAVE + e4) * 64 + lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][4 * gq + e] += v[e];
          }
    }
  }
}

// C = alpha*acc + beta*C for the tile at (m0, n0), by the waves of the first
// K group.  Block (i, j), register 4g + e of lane (li, lh) holds C(row, col)
// with row = li and col = 8g + 4lh + e inside the block.  C is read here,
// one block at a time, unless HAVE_C: then cv holds it already (load_c).
template <class T, int MODE, bool HAVE_C = false>
__device__ __forceinline__ void store_tile(const GemmArgs& g, int m0, int n0,
                                           const f32x16 (&acc)[T::FM][T::FN],
                                           const f32x16 (&cv)[T::FM][T::FN]) {
  const WaveCoords<T> w;
  const int M = g.M, N = g.N, ldc = g.ldc;
  const float alpha = g.alpha, beta = g.beta;
  float* __restrict__ C = g.C;
  const int crow = m0 + w.wm * T::WM + w.li;
  const int ccol = n0 + w.wn * T::WN + w.lh * 4;
  const bool c_vec = c_vector(g);
  // stores need bounds checks: guarded kernels, and edge tiles of edge kernels
  const bool masked = c_masked<T, MODE>(g, m0, n0);
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j) {
      const int row = crow + i * 32;
      const int col = ccol + j * 32;
      float* p = C + (size_t)row * ldc + col;
      if (masked && row >= M) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // a group of four columns wholly inside M x N: 16-byte accesses
        if (c_vec && (!masked || col + 8 * q + 3 < N)) {
          f32x4 cin = {0.0f, 0.0f, 0.0f, 0.0f};
          if (beta != 0.0f) {
            if (HAVE_C) {
#pragma unroll
              for (int e = 0; e < 4; ++e) cin[e] = cv[i][j][4 * q + e];
            } else {
              cin = *reinterpret_cast<const f32x4*>(p + 8 * q);
            }
          }
          f32x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[e] = alpha * acc[i][j][4 * q + e];
            if (beta != 0.0f) o[e] = fmaf(beta, cin[e], o[e]);
          }
          *reinterpret_cast<f32x4*>(p + 8 * q) = o;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (masked && col + 8 * q + e >= N) continue;
            float o = alpha * acc[i][j][4 * q + e];
            if (beta != 0.0f)
              o = fmaf(beta, HAVE_C ? cv[i][j][4 * q + e] : p[8 * q + e], o);
            p[8 * q + e] = o;
          }
        }
      }
      // keep one block's C traffic in registers at a time
      __builtin_amdgcn_sched_barrier(0);
    }
}

// The same epilogue staged through LDS, one 32x32 block per wave at a time
// (the stages are free; the caller has passed a barrier after the last LDS
// read): a store of the MFMA register layout writes 32 rows x 32 bytes, one
// piece of each 128-byte line it touches, and the lines' other pieces come
// in three more instructions.  Staged and read back row by row, each wave
// instruction reads or writes eight whole rows of the block, i.e. eight
// whole lines.  A staged row is 32 floats, eight 16-byte units, unit u of
// row r at u ^ (r % 8).  On gfx950 a 16-byte LDS write serves 8 lanes at a
// time over 32 banks and a 16-byte read 16 lanes over 64 banks (measured
// with the bank-conflict counter on single-wave patterns): the register
// layout's writes (8 rows of one unit per 8 lanes) then fall on 8 distinct
// units and the row reads (two rows of eight units per 16 lanes) on 16
// distinct bank groups.  Rows past M and columns past N are
// skipped; C that is not 16-byte aligned, or whose ldc is not a multiple of
// 4, takes element accesses.  With HAVE_C, cv holds C in the register
// layout (read before the K loop) and the update is applied before staging.
template <class T, int MODE, bool HAVE_C = false>
__device__ __forceinline__ void store_tile_lds(const GemmArgs& g, int m0, int n0,
                                               const f32x16 (&acc)[T::FM][T::FN],
                                               const f32x16 (&cv)[T::FM][T::FN],
                                               float* lds) {
  constexpr int LD = 32;  // a staged row
  static_assert(T::WAVES_MN * 32 * LD * 4 <= TileLds<T, MODE>::FLOATS * 4, "staging area");
  const WaveCoords<T> w;
  float* reg = lds + w.wmn * 32 * LD;
  const int M = g.M, N = g.N, ldc = g.ldc;
  const float alpha = g.alpha, beta = g.beta;
  const int rr = w.lane >> 3, cc = 4 * (w.lane & 7);  // row (of 8) and column read back
  const bool c_vec = c_vector(g);
  // the swizzle folded into per-lane constants: the lane writes unit
  // (2q + lh) ^ (li % 8) = 2q ^ xw of row li and reads unit
  // (cc/4) ^ ((8t + rr) % 8) = xr of row 8t + rr
  float* const wrow = reg + w.li * LD;
  float* const rrow = reg + rr * LD;
  const int xw = w.lh ^ (w.li & 7);
  const int xr = (cc >> 2) ^ rr;
  const size_t rstep = (size_t)8 * ldc;  // rows between a lane's accesses
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j) {
      const int row0 = m0 + w.wm * T::WM + i * 32 + rr;  // the lane's first row
      const int col = n0 + w.wn * T::WN + j * 32 + cc;
      const bool vec = c_vec && col + 3 < N;
      float* p = g.C + (size_t)row0 * ldc + col;
      f32x4 cin[4];
      if (!HAVE_C && beta != 0.0f) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          cin[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
          if (row0 + 8 * t < M) {
            if (vec) {
              cin[t] = *reinterpret_cast<const f32x4*>(p + t * rstep);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (col + e < N) cin[t][e] = p[t * rstep + e];
            }
          }
        }
      }
      // register 4q + e of lane (li, lh): row li, column 8q + 4lh + e
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = acc[i][j][4 * q + e];
          if (HAVE_C) {
            v[e] *= alpha;
            if (beta != 0.0f) v[e] = fmaf(beta, cv[i][j][4 * q + e], v[e]);
          }
        }
        *reinterpret_cast<f32x4*>(wrow + 4 * ((2 * q) ^ xw)) = v;
      }
      // the wave reads back its own writes: one wave's LDS operations
      // complete in issue order
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const f32x4 v =
            *reinterpret_cast<const f32x4*>(rrow + 8 * t * LD + 4 * xr);
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] = v[e];
          if (!HAVE_C) {
            o[e] *= alpha;
            if (beta != 0.0f) o[e] = fmaf(beta, cin[t][e], o[e]);
          }
        }
        if (row0 + 8 * t < M) {
          if (vec) {
            *reinterpret_cast<f32x4*>(p + t * rstep) = o;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (col + e < N) p[t * rstep + e] = o[e];
          }
        }
      }
      // one block's C traffic at a time
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_wave_barrier();
    }
}

template <class T>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[T::FM][T::FN]) {
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j) acc[i][j] = f32x16(0.0f);
}

// Clock stamps (diagnostic): the shader cycle counter (s_memtime) at p[0]
// and the constant-rate wall clock (s_memrealtime) at p[2], written by the
// calling lane with vector stores.
__device__ __forceinline__ void clock_stamp(long long* p) {
  const long long c = (long long)__builtin_amdgcn_s_memtime();
  const long long w = (long long)__builtin_amdgcn_s_memrealtime();
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): both readings are in
  p[0] = c;
  p[2] = w;
}

// One tile per workgroup: workgroup -> tile through the XCD-aware order.
// With `stamps` (a diagnostic; null in every product call) the first lane
// records {cycles, cycles, wall, wall} at stamps[4*workgroup]: the counters
// when the workgroup starts and after all its waves are done, so cycles over
// wall ticks is the shader clock the tile ran at.
template <class T, int MODE, bool TA, bool TB>
__global__ void __launch_bounds__(T::THREADS, T::OCC)
    mfma_sgemm_kernel(GemmArgs g, int tiles_m, int tiles_n, int band,
                      long long* __restrict__ stamps) {
  __shared__ __attribute__((aligned(1024))) float lds[TileLds<T, MODE>::FLOATS];
  if (stamps != nullptr && threadIdx.x == 0) clock_stamp(stamps + 4 * blockIdx.x);
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, band, tm, tn);
  f32x16 acc[T::FM][T::FN];
  zero_acc<T>(acc);
  // Tiles with K groups read C before their K loop (see tile_accumulate)
  // when the 16 registers per block fit their budget: at 6 waves per SIMD
  // (85 registers a lane) they do; at 8 (the 64x64 tile's 64) they spill.
  constexpr bool LOADC = T::KG > 1 && T::OCC <= 6;
  f32x16 cv[T::FM][T::FN];
  tile_accumulate<T, MODE, TA, TB, LOADC>(g, lds, tm * T::BM, tn * T::BN, 0,
                                          tile_k_steps<T>(g.K), acc, cv);
  __syncthreads();  // every wave is done with the LDS (stages, K-group sums)
  if (threadIdx.x / 64 / T::WAVES_MN == 0)
    store_tile_lds<T, MODE, LOADC>(g, tm * T::BM, tn * T::BN, acc, cv, lds);
  if (stamps != nullptr) {
    __syncthreads();
    if (threadIdx.x == 0) clock_stamp(stamps + 4 * blockIdx.x + 1);
  }
}

// ---- stream-K ------------------------------------------------------------
//
// A persistent grid of G workgroups.  Tiles [0, D) of the band walk (D a
// multiple of G, from sk_dp_tiles) are whole-tile work: the workgroup at
// position h (xcd_position: one XCD's workgroups hold consecutive
// positions) computes tiles h, h+G, ... and stores them.  The iteration
// space of the other tiles times their K steps (W = (tiles-D) * steps,
// tile-major) is cut into G equal contiguous ranges: workgroup h owns
// iterations [b(h), b(h+1)) with b(h) = floor(h*W/G), iteration i being
// step i % steps of tile D + i / steps, so an XCD works on a compact block
// of C in both parts.  It
// walks them tile by tile; a tile it covers whole is stored at once, a part
// of a tile is a partial sum written to the workspace.  A workgroup writes
// at most two partials: slot 2h for a part that starts at b(h) (its first
// part) and slot 2h+1 for a part that ends at b(h+1) inside a tile (its
// last).  The fixup kernel then adds each split tile's partials in K order
// and stores the tile, so the result does not depend on timing.
//
// Slot layout: the first K group's accumulators as the waves hold them,
// f32x4 per lane, (wave, block, quad) major -- BM*BN floats per slot.

__host__ __device__ inline long long sk_bound(long long W, int G, int h) {
  return W * h / G;
}

// Whole tiles before the split ones.  Splitting only the last, partial
// round keeps the partial sums few; when that round is so small that each
// workgroup's share would be under a quarter of a tile's K steps (or two
// steps), the round before it is split too.  No whole rounds: every tile
// is split; no partial round: no tile is.
__host__ __device__ inline int sk_dp_tiles(int tiles, int G, int steps) {
  const int full = tiles / G, rem = tiles % G;
  if (full == 0) return 0;
  if (rem == 0) return tiles;
  const int min_share = steps / 4 > 2 ? steps / 4 : 2;
  if ((long long)rem * steps >= (long long)G * min_share) return full * G;
  return (full - 1) * G;
}

template <class T>
__device__ __forceinline__ void store_partial(float* slot,
                                              const f32x16 (&acc)[T::FM][T::FN]) {
  const WaveCoords<T> w;
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
        *reinterpret_cast<f32x4*>(
            slot + (((w.wmn * T::FM + i) * T::FN + j) * 4 + q) * 256 + 4 * w.lane) = v;
      }
}

template <class T, int MODE, bool TA, bool TB>
__global__ void __launch_bounds__(T::THREADS, T::SK_OCC)
    mfma_sgemm_sk_kernel(GemmArgs g, int tiles_m, int tiles_n, int band,
                         int steps, int dp, float* __restrict__ ws) {
  __shared__ __attribute__((aligned(1024))) float lds[TileLds<T, MODE>::FLOATS];
  const int tiles = tiles_m * tiles_n;
  const long long W = (long long)(tiles - dp) * steps;
  const int G = gridDim.x, h = xcd_position(blockIdx.x, gridDim.x);
  const long long b0 = sk_bound(W, G, h), b1 = sk_bound(W, G, h + 1);
  const bool first_group = threadIdx.x / 64 / T::WAVES_MN == 0;
  // One loop over this workgroup's work items (its whole tiles, then the
  // parts of its range), so the K loop is inlined once.
  int next_whole = h;
  long long i = b0;
  while (true) {
    int t, s0, s1, slot = -1;  // slot < 0: the item covers its whole tile
    if (next_whole < dp) {
      t = next_whole;
      s0 = 0;
      s1 = steps;
      next_whole += G;
    } else if (i < b1) {
      const int ti = (int)(i / steps);
      const long long ts = (long long)ti * steps;
      s0 = (int)(i - ts);
      s1 = (int)(b1 - ts < steps ? b1 - ts : steps);
      if (s0 != 0 || s1 != steps) slot = 2 * h + (i == b0 ? 0 : 1);
      t = dp + ti;
      i = ts + s1;
    } else {
      break;
    }
    int tm, tn;
    band_walk(t, tiles_m, tiles_n, band, tm, tn);
    f32x16 acc[T::FM][T::FN];
    zero_acc<T>(acc);
    tile_accumulate<T, MODE, TA, TB>(g, lds, tm * T::BM, tn * T::BN, s0, s1, acc, acc);
    if (first_group) {
      if (slot < 0)
        store_tile<T, MODE>(g, tm * T::BM, tn * T::BN, acc, acc);
      else
        store_partial<T>(ws + (size_t)slot * (T::BM * T::BN), acc);
    }
    __syncthreads();  // the next item reuses the LDS
  }
}

// Elementwise fixup of the split tiles: each thread takes 16-byte pieces
// (chunk c of a slot: the four floats at 4c) of split tiles, adds the
// partials of that piece from every owner of the tile in K order, applies
// alpha and beta and stores.  The owners of split tile u (iterations
// [u*steps, (u+1)*steps)) run from owner(u*steps) to owner((u+1)*steps - 1),
// owner(i) = floor(((i+1)*G - 1) / W); a tile with a single owner was stored
// by it.  Owner o's part of the tile is in its first slot (2o) when o's
// range starts inside the tile, else in its last (2o+1).
template <class T, int MODE>
__global__ void __launch_bounds__(256)
    mfma_sgemm_fixup_kernel(GemmArgs g, int tiles_m, int tiles_n, int band,
                            int steps, int dp, int G,
                            const float* __restrict__ ws) {
  constexpr int CHUNKS = T::BM * T::BN / 4;
  constexpr bool EDGE = MODE == MODE_EDGE;
  const int tiles = tiles_m * tiles_n;
  const long long W = (long long)(tiles - dp) * steps;
  const long long total = (long long)(tiles - dp) * CHUNKS;
  const int M = g.M, N = g.N, ldc = g.ldc;
  const float alpha = g.alpha, beta = g.beta;
  float* __restrict__ C = g.C;
  const bool c_vec = (ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(C) & 15u) == 0);
  for (long long x = (long long)blockIdx.x * 256 + threadIdx.x; x < total;
       x += (long long)gridDim.x * 256) {
    const int u = (int)(x / CHUNKS), c = (int)(x - (long long)u * CHUNKS);
    const long long ts = (long long)u * steps;
    const int first = (int)(((ts + 1) * G - 1) / W);
    const int last = (int)(((ts + steps) * G - 1) / W);
    if (first == last) continue;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int o = first; o <= last; ++o) {
      const long long bo = sk_bound(W, G, o);
      if (bo >= sk_bound(W, G, o + 1)) continue;  // empty range
      acc += *reinterpret_cast<const f32x4*>(
          ws + (size_t)(2 * o + (bo >= ts ? 0 : 1)) * (T::BM * T::BN) + 4 * c);
    }
    // chunk c = (((wmn * FM + i) * FN + j) * 4 + q) * 64 + lane: four
    // consecutive columns of one row of the tile
    const int lane = c & 63, q = (c >> 6) & 3;
    const int j = (c >> 8) % T::FN, i = (c >> 8) / T::FN % T::FM;
    const int wmn = (c >> 8) / (T::FN * T::FM);
    int tm, tn;
    band_walk(dp + u, tiles_m, tiles_n, band, tm, tn);
    const int row = tm * T::BM + (wmn / T::WAVES_N) * T::WM + i * 32 + (lane & 31);
    const int col = tn * T::BN + (wmn % T::WAVES_N) * T::WN + j * 32 + (lane >> 5) * 4 + 8 * q;
    if (EDGE && row >= M) continue;
    float* p = C + (size_t)row * ldc + col;
    if (c_vec && (!EDGE || col + 3 < N)) {
      f32x4 o;
      const f32x4 cin = beta != 0.0f ? *reinterpret_cast<const f32x4*>(p) : f32x4{};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = alpha * acc[e];
        if (beta != 0.0f) o[e] = fmaf(beta, cin[e], o[e]);
      }
      *reinterpret_cast<f32x4*>(p) = o;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (EDGE && col + e >= N) continue;
        float o = alpha * acc[e];
        if (beta != 0.0f) o = fmaf(beta, p[e], o);
        p[e] = o;
      }
    }
  }
}

}  // namespace sgemm
