// Products with 16-bit A and B (bfloat16 or IEEE binary16) or 8-bit A and B
// (OCP E4M3 or E5M2) and FP32 C on the CDNA4 matrix cores
// (v_mfma_f32_32x32x16_bf16 / _f16, v_mfma_scale_f32_32x32x64_f8f6f4).
//
// C = alpha*op(A)*op(B) + beta*C with op(A), op(B) as in the FP32 kernels and
// C, alpha, beta in FP32: the mixed-precision matrix-unit product of the
// gsyq.cn guide, section 5.1 (16-bit inputs, FP32 accumulation).  The
// structure is the FP32 kernels' -- block tile staged in LDS, per-wave
// register tile of 32x32 MFMA blocks, one barrier per K step, fused
// alpha/beta update -- with the operand tiles reshaped for the 16-bit
// instructions:
//
// * A K step is 64 values of k.  Each lane of a 32x32x16 MFMA supplies eight
//   consecutive k of one row of A and of one column of B (lanes 0-31 one half
//   of the 16, lanes 32-63 the other; which half is free as long as A and B
//   agree).
// * An operand stored K-contiguous (A as stored, B stored N x K) sits in LDS
//   as one 128-byte row of 64 k per row of A or column of B, eight 16-byte
//   units per row, unit c of row r at c ^ ((r / 2) & 7): a fragment is one
//   ds_read_b128, and the reads of 16 consecutive rows at one unit hit 16
//   distinct 16-byte bank groups.
// * Aligned kernels: an operand stored outer-contiguous (B stored K x N, A
//   stored K x M) keeps that layout in LDS -- rows of k holding the tile's
//   outer indices, units XOR-swizzled per row (lp_oc_swz) -- and its
//   fragments come from pairs of transposing reads (ds_read_b64_tr_b16), which
//   hand each lane four k of one column.  Every operand tile then arrives by
//   direct global-to-LDS loads (global_load_lds_dwordx4, as in the FP32
//   kernels): lane l's 16 bytes land in slot 64*i + l of the tile, and the
//   lane reads the global piece that the swizzle puts in that slot.
// * Aligned kernels keep S LDS stages (two for the 256x256 tile, four for the
//   smaller ones); the loads of step k+S go out after step k's barrier, over
//   the step's second half, and have about S-1 steps to land.  The barrier
//   sits halfway through a step's groups of MFMAs, the fragment reads run
//   half a step ahead, and every group issues its MFMAs one at a time with
//   reads and loads in the slots between them, in a fixed order: one wave
//   per SIMD keeps the matrix pipe busy without another wave to hide its
//   reads and loads.
// * Edge kernels (any sizes; M at least one 16-byte piece -- 8 elements of a
//   16-bit format, 16 of an 8-bit one -- when A is stored K x M, N likewise
//   when B is stored K x N) run the whole K steps on the aligned kernels'
//   schedule, with what lies past M or N clamped (a K-contiguous row past the
//   edge reads the last valid row, an outer-contiguous piece wholly past the
//   edge the last piece's worth of valid indices, a piece that straddles the
//   edge is read as it is and runs into the next k row -- so, when one can
//   straddle, the step holding the last K row is left out); those values
//   only feed outputs that are never stored.  The rest of K goes through
//   registers, zero-filled, in the register-staged layout below, and stores
//   are masked on edge tiles.
// * Guarded kernels (any sizes and strides) load every operand through
//   registers, one step ahead, with zero fill past the edges (no lane leaves
//   before the barriers): K-contiguous pieces go to LDS as they are; 16-bit
//   outer-contiguous ones are transposed in registers -- each lane loads an
//   8 x 8 block (eight 16-byte loads of k rows) and writes eight 16-byte units
//   of eight k, built by v_perm; lanes with odd block column write their rows
//   pair-swapped, so one LDS write of 16 lanes covers all 16 bank groups (only
//   the v_perm byte selector differs).  The edge kernels' register step uses
//   the same loads.  Their stores are masked.
// * Global loads of both kinds, direct-to-LDS ones included, take any byte
//   address on gfx950 (checked with in-bounds probes at 1- and 2-byte
//   offsets): no kernel needs aligned leading dimensions or base pointers.
// * 8-bit operands use the same kernels with the element size halved: a
//   16-byte unit holds 16 elements, a K step is 128 k (K-contiguous LDS rows
//   stay 128 bytes, same swizzle), and each lane hands the 8-bit instruction
//   32 consecutive bytes of k per operand (two units), with unit block
//   scales; a step has two groups of 64 k in place of four of 16.  An 8-bit
//   operand stored outer-contiguous keeps its stored layout in LDS in every
//   mode (rows of k, units swizzled by lp_oc_swz8; register-staged steps
//   load whole 16-byte pieces into the same layout, zero-filled past the
//   edges) and its fragments come from transposing reads
//   (ds_read_b64_tr_b8, four per fragment).  That instruction sums each block of 64 products in a
//   fixed-point window below the block's largest product before adding it
//   to the FP32 accumulator (measured), so its sums carry more rounding
//   error than an FP32 accumulation of the same products.
// * MFMA operands are swapped (the B fragment first), so a 32x32 result is
//   the transpose of its C block and the FP32 kernels' epilogue applies as it
//   is: lane (li, lh) holds row li and columns 8g + 4lh + e of the block.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "mfma_sgemm.hpp"
#include "skinny_sgemm.hpp"  // skinny_ws_stride: the split-K partial-sum rows
#include "tile_map.hpp"

namespace sgemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Element formats of A and B: 16-bit (bfloat16, binary16) and 8-bit (OCP
// E4M3, E5M2).
enum { LP_BF16 = 1, LP_F16 = 2, LP_E4M3 = 3, LP_E5M2 = 4 };

// What a format changes.  An LDS row is always 128 bytes of k, eight 16-byte
// units; a K step is one such row: 64 k of a 16-bit format, 128 of an 8-bit
// one.  A 16-bit MFMA (32x32x16) takes eight k per lane, one unit; an 8-bit
// one (32x32x64) takes 32 k per lane, two units, so a K step holds four
// groups of 16-bit MFMAs or two of 8-bit ones.
template <int DT>
struct LpFmt {
  static constexpr int ESZ = DT >= LP_E4M3 ? 1 : 2;  // bytes per element
  static constexpr int UE = 16 / ESZ;                // elements per unit
  static constexpr int BKE = 128 / ESZ;              // k per K step
  static constexpr int FU = 3 - ESZ;                 // units per lane per fragment
  static constexpr int QG = ESZ == 2 ? 4 : 2;        // MFMA groups per K step
  typedef typename std::conditional<ESZ == 1, uint8_t, uint16_t>::type E;
};

// The operation's arguments: A and B as bit patterns of the format.
struct LpArgs {
  int M, N, K;
  float alpha, beta;
  const void* A;
  int lda;
  const void* B;
  int ldb;
  float* C;
  int ldc;
};

// Block tile BM x BN, wave tile WM x WN of 32x32 blocks, registers sized for
// OCC waves per SIMD.  The member names the FP32 epilogue (store_tile) and
// WaveCoords read are the same as MfmaTile's (one K group).
template <int BM_, int BN_, int WM_, int WN_, int OCC_, int S_ = 2>
struct LpTile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, OCC = OCC_;
  // LDS stages of the aligned kernels: their direct loads run S-1 K steps
  // ahead (guarded kernels use two stages).
  static constexpr int S = S_;
  static constexpr int BK = 64;  // k per K step: one 128-byte LDS row
  static constexpr int KG = 1;
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int WAVES_MN = WAVES_M * WAVES_N, WAVES = WAVES_MN;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;  // one stage
  static constexpr int LDS_BYTES = S * (A_BYTES + B_BYTES);
  // K-contiguous loader: 16-byte units per lane per K step
  static constexpr int A_VEC = BM * 8 / THREADS, B_VEC = BN * 8 / THREADS;
  // transposing loader: waves that move the operand (64 outer indices each)
  static constexpr int A_TW = BM / 64, B_TW = BN / 64;
  static_assert(BM % WM == 0 && BN % WN == 0, "wave grid");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "32x32 MFMA blocks");
  static_assert(A_VEC >= 1 && A_VEC * THREADS == BM * 8, "A loader");
  static_assert(B_VEC >= 1 && B_VEC * THREADS == BN * 8, "B loader");
  static_assert(BM % 64 == 0 && BN % 64 == 0, "transposing loader regions");
  static_assert(A_TW <= WAVES && B_TW <= WAVES, "transposing loader waves");
  // the stages plus the 1 KB that look-ahead loads past the end land in
  static constexpr int LDS_ALIGNED = LDS_BYTES + 1024;
  static_assert(LDS_ALIGNED <= 160 * 1024, "gfx950 LDS");
  static_assert(S >= 2, "stages");
  static_assert((S - 1) * (A_VEC + B_VEC) <= 63, "vmcnt range");
};

// f(std::integral_constant<int, i>) for i = 0 .. N-1, in order.
template <class F, int... I>
__device__ __forceinline__ void lp_static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void lp_static_for(F&& f) {
  lp_static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Outer-contiguous tiles (aligned mode): rows of k holding X outer indices,
// X / 8 units of 16 bytes per row; unit p of row k sits at p ^ lp_oc_swz.
// A transposing read of 16 lanes touches four consecutive rows (k & 3 = 0..3)
// at the same units.  Rows of at least 16 units map every row onto the same
// 16 bank groups, so the XOR takes bits 2-3 of the unit from k & 3; rows of
// 8 units (X = 64) alternate between two halves of the bank groups by k & 1,
// so the XOR takes bit 2 from k & 2 (and stays inside the row).
template <int X>
__device__ __forceinline__ int lp_oc_swz(int k) {
  static_assert(X == 64 || X % 128 == 0, "outer-contiguous tile width");
  return X >= 128 ? 4 * (k & 3) : 4 * ((k >> 1) & 1);
}

// Outer-contiguous tiles of 8-bit elements: rows of k holding X outer
// indices in X / 16 units of 16 bytes; unit p of row k sits at p ^
// lp_oc_swz8<X>(k).  Half a wave of a transposing read (ds_read_b64_tr_b8)
// touches eight consecutive rows (k & 7 = 0..7) at two units c and c ^ 1 (c
// even), so the sixteen (row, unit) pairs must land on distinct 16-byte bank
// groups: the XOR takes even values only (c and c ^ 1 then fill complementary
// groups) that differ between rows starting on the same group -- rows of 256
// bytes all start on one group (2 * (k & 7)), rows of 128 bytes on two
// (2 * (k / 2 & 3)), rows of 64 bytes on four (2 * (k / 4 & 1)); each XOR
// stays inside its row.
template <int X>
__device__ __forceinline__ int lp_oc_swz8(int k) {
  static_assert(X == 64 || X == 128 || X == 256, "8-bit outer-contiguous tile width");
  return 2 * (X == 256 ? (k & 7) : X == 128 ? ((k >> 1) & 3) : ((k >> 2) & 1));
}

// The unit swizzle of an outer-contiguous tile of ESZ-byte elements.
template <int ESZ, int X>
__device__ __forceinline__ int lp_oc_unit_swz(int k) {
  if constexpr (ESZ == 2)
    return lp_oc_swz<X>(k);
  else
    return lp_oc_swz8<X>(k);
}

// Byte offset of 16-byte unit c (k = 8c .. 8c+7) of row r in an operand tile.
__device__ __forceinline__ int lp_unit_off(int r, int c) {
  return r * 128 + 16 * (c ^ ((r >> 1) & 7));
}

// One MFMA on fragments x (first operand) and y of FU units each.  8-bit
// formats use the scaled 32x32x64 instruction with both E8M0 scales 127
// (2^0), i.e. unscaled; its format fields select E4M3 (0) or E5M2 (1).
template <int DT>
__device__ __forceinline__ f32x16 lp_mfma(const u32x4* x, const u32x4* y, f32x16 acc) {
  if constexpr (DT == LP_BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        __builtin_bit_cast(bf16x8, x[0]), __builtin_bit_cast(bf16x8, y[0]), acc, 0, 0, 0);
  } else if constexpr (DT == LP_F16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(
        __builtin_bit_cast(f16x8, x[0]), __builtin_bit_cast(f16x8, y[0]), acc, 0, 0, 0);
  } else {
    constexpr int fmt = DT == LP_E4M3 ? 0 : 1;
    const i32x8 xa = {(int)x[0][0], (int)x[0][1], (int)x[0][2], (int)x[0][3],
                      (int)x[1][0], (int)x[1][1], (int)x[1][2], (int)x[1][3]};
    const i32x8 ya = {(int)y[0][0], (int)y[0][1], (int)y[0][2], (int)y[0][3],
                      (int)y[1][0], (int)y[1][1], (int)y[1][2], (int)y[1][3]};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(xa, ya, acc, fmt, fmt, 0, 127, 0,
                                                           127);
  }
}

// A 16-byte piece at any byte address: 16-byte global loads on gfx950 take
// any alignment (checked with in-bounds probes at 1- and 2-byte offsets).
typedef unsigned u32x4u1 __attribute__((ext_vector_type(4), aligned(1)));

// One 16-byte unit of elements of type E at p: one 16-byte load when all
// 16 / sizeof(E) elements are wanted, else element loads of the first n (n
// may be <= 0) with zeros after them.  The element loads are unconditional
// -- element t reads p[min(t, n-1)], inside the n wanted -- and masked
// afterwards: loads under per-element branches were each waited for before
// the next was issued (one memory round trip per element of a partial
// piece).
template <class E>
__device__ __forceinline__ u32x4 lp_load_unit(const E* p, int n) {
  constexpr int UE = 16 / sizeof(E), BITS = 8 * sizeof(E);
  if (n >= UE) {
    const u32x4u1 v = *reinterpret_cast<const u32x4u1*>(p);
    return u32x4{v[0], v[1], v[2], v[3]};
  }
  u32x4 out = {0u, 0u, 0u, 0u};
  if (n <= 0) return out;
  unsigned h[UE];
#pragma unroll
  for (int t = 0; t < UE; ++t) h[t] = (unsigned)p[t < n ? t : n - 1];
#pragma unroll
  for (int t = 0; t < UE; ++t)
    if (t < n) out[t / (32 / BITS)] |= h[t] << (BITS * (t % (32 / BITS)));
  return out;
}

// Accumulate the output tile at (m0, n0) over all of K into acc (zeroed by
// the caller).  TA: A stored K x M; TB: B stored N x K.
template <class T, int DT, int MODE, bool TA, bool TB>
__device__ __forceinline__ void lp_tile_accumulate(const LpArgs& g, char* lds,
                                                   int m0, int n0,
                                                   f32x16 (&acc)[T::FM][T::FN]) {
  typedef LpFmt<DT> F;
  typedef typename F::E E;
  constexpr int ESZ = F::ESZ, UE = F::UE, BKE = F::BKE, FU = F::FU, QG = F::QG;
  constexpr bool GUARD = MODE == MODE_GUARDED;
  constexpr bool EDGE = MODE == MODE_EDGE;
  constexpr bool A_KC = !TA;  // A stored K-contiguous
  constexpr bool B_KC = TB;   // B stored K-contiguous
  const int M = g.M, N = g.N, K = g.K;
  const E* __restrict__ A = static_cast<const E*>(g.A);
  const E* __restrict__ B = static_cast<const E*>(g.B);
  const int lda = g.lda, ldb = g.ldb;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;
  const int li = lane & 31, lh = lane >> 5;
  const int kb = lane & 7, ob = lane >> 3;  // transposing loader block
  const int nk = (K + BKE - 1) / BKE;

  // LDS: the A tiles of all stages, then the B tiles.
  auto a_off = [](int st) { return st * T::A_BYTES; };
  constexpr int NST = GUARD ? 2 : T::S;  // stages in use
  auto b_off = [](int st) { return NST * T::A_BYTES + st * T::B_BYTES; };

  // ---- K-contiguous operands: slot u of the tile holds (row, unit) ------
  int a_r[T::A_VEC], a_c[T::A_VEC], b_r[T::B_VEC], b_c[T::B_VEC];
#pragma unroll
  for (int v = 0; v < T::A_VEC; ++v) {
    const int u = (v * T::WAVES + wave) * 64 + lane;
    a_r[v] = u >> 3;
    a_c[v] = (u & 7) ^ ((a_r[v] >> 1) & 7);
  }
#pragma unroll
  for (int v = 0; v < T::B_VEC; ++v) {
    const int u = (v * T::WAVES + wave) * 64 + lane;
    b_r[v] = u >> 3;
    b_c[v] = (u & 7) ^ ((b_r[v] >> 1) & 7);
  }
  // Direct loads (aligned and edge modes): a wave-uniform base at the tile's
  // origin, advanced one K step per step, and fixed per-lane byte offsets
  // (the host keeps them below 2^32).  An operand stored outer-contiguous
  // keeps that layout in these modes (rows of k, units swizzled by
  // lp_oc_swz): slot u of such a tile is row u / (X/8), physical unit
  // u % (X/8).
  const unsigned lds_u = (unsigned)(uintptr_t)(lds_void_t*)lds;
  unsigned a_voff[T::A_VEC], b_voff[T::B_VEC];
  // Edge kernels clamp what lies past M or N: a K-contiguous row past the
  // edge reads the last valid row; an outer-contiguous piece wholly past the
  // edge reads the last eight valid indices (or the tile's first eight when
  // fewer remain), and one that straddles the edge is read as it is (its
  // elements past the edge come from the next k row).  Either kind only feeds
  // outputs that are never stored.
  if (!GUARD) {
#pragma unroll
    for (int v = 0; v < T::A_VEC; ++v) {
      if (A_KC) {
        int r = a_r[v];
        if (EDGE && m0 + r >= M) r = M - 1 - m0;
        a_voff[v] = ESZ * ((unsigned)r * (unsigned)lda + UE * (unsigned)a_c[v]);
      } else {
        const int u = (v * T::WAVES + wave) * 64 + lane;
        constexpr int UPR = T::BM * ESZ / 16;  // units per row of k
        const int k = u / UPR, c = (u % UPR) ^ lp_oc_unit_swz<ESZ, T::BM>(k);
        int o = UE * c;
        if (EDGE && m0 + o >= M) o = M - UE > m0 ? M - UE - m0 : 0;
        a_voff[v] = ESZ * ((unsigned)k * (unsigned)lda + (unsigned)o);
      }
    }
#pragma unroll
    for (int v = 0; v < T::B_VEC; ++v) {
      if (B_KC) {
        int r = b_r[v];
        if (EDGE && n0 + r >= N) r = N - 1 - n0;
        b_voff[v] = ESZ * ((unsigned)r * (unsigned)ldb + UE * (unsigned)b_c[v]);
      } else {
        const int u = (v * T::WAVES + wave) * 64 + lane;
        constexpr int UPR = T::BN * ESZ / 16;  // units per row of k
        const int k = u / UPR, c = (u % UPR) ^ lp_oc_unit_swz<ESZ, T::BN>(k);
        int o = UE * c;
        if (EDGE && n0 + o >= N) o = N - UE > n0 ? N - UE - n0 : 0;
        b_voff[v] = ESZ * ((unsigned)k * (unsigned)ldb + (unsigned)o);
      }
    }
  }
  // Tile origins and the advance per K step of the direct loads.
  const E* a_dbase = A_KC ? A + (size_t)m0 * lda : A + m0;
  const E* b_dbase = B_KC ? B + (size_t)n0 * ldb : B + n0;
  const size_t a_dstep = A_KC ? (size_t)BKE : (size_t)BKE * lda;
  const size_t b_dstep = B_KC ? (size_t)BKE : (size_t)BKE * ldb;
  // ---- register-staged operands --------------------------------------------
  // K-contiguous operands in guarded and edge mode: one unit per slot.
  constexpr int A_RK = ((GUARD || EDGE) && A_KC) ? T::A_VEC : 1;
  constexpr int B_RK = ((GUARD || EDGE) && B_KC) ? T::B_VEC : 1;
  u32x4 ra_kc[A_RK], rb_kc[B_RK];
  // Outer-contiguous operands: 16-bit ones as one 8 x 8 block per lane of the
  // loading waves, transposed in registers to the K-contiguous layout; 8-bit
  // ones as 16-byte units in their own layout (read by transposing reads).
  constexpr bool A_T16 = TA && ESZ == 2, B_T16 = !TB && ESZ == 2;
  constexpr bool A_O8 = TA && ESZ == 1, B_O8 = !TB && ESZ == 1;
  u32x4 ra_t[A_T16 ? 8 : 1], rb_t[B_T16 ? 8 : 1];
  u32x4 ra_o[A_O8 ? T::A_VEC : 1], rb_o[B_O8 ? T::B_VEC : 1];
  // (every wave when the tile has as many 64-wide regions as waves)
  const bool a_tw = T::A_TW >= T::WAVES || wave < T::A_TW;
  const bool b_tw = T::B_TW >= T::WAVES || wave < T::B_TW;
  const int a_to = 64 * wave + 8 * ob;  // tile-relative outer index of the block
  const int b_to = 64 * wave + 8 * ob;

  // Register loads of K step kt (guarded mode; the last step of edge mode).
  // ops: 1 = A, 2 = B, 3 = both.
  auto load_regs = [&](int kt, int ops = 3) {
    const int k0 = kt * BKE;
    if ((GUARD || EDGE) && A_KC && (ops & 1)) {
#pragma unroll
      for (int v = 0; v < T::A_VEC; ++v) {
        const int row = m0 + a_r[v], k = k0 + UE * a_c[v];
        ra_kc[v] = lp_load_unit(A + (size_t)(row < M ? row : 0) * lda + k,
                                row < M ? K - k : 0);
      }
    }
    if ((GUARD || EDGE) && B_KC && (ops & 2)) {
#pragma unroll
      for (int v = 0; v < T::B_VEC; ++v) {
        const int row = n0 + b_r[v], k = k0 + UE * b_c[v];
        rb_kc[v] = lp_load_unit(B + (size_t)(row < N ? row : 0) * ldb + k,
                                row < N ? K - k : 0);
      }
    }
    if constexpr (A_O8) {
      if (ops & 1) {
#pragma unroll
        for (int v = 0; v < T::A_VEC; ++v) {
          constexpr int UPR = T::BM / 16;
          const int u = (v * T::WAVES + wave) * 64 + lane;
          const int kr = u / UPR, k = k0 + kr;
          const int o = m0 + 16 * ((u % UPR) ^ lp_oc_swz8<T::BM>(kr));
          const bool in = k < K && o < M;
          ra_o[v] = lp_load_unit(A + (in ? (size_t)k * lda + o : (size_t)0), in ? M - o : 0);
        }
      }
    }
    if constexpr (B_O8) {
      if (ops & 2) {
#pragma unroll
        for (int v = 0; v < T::B_VEC; ++v) {
          constexpr int UPR = T::BN / 16;
          const int u = (v * T::WAVES + wave) * 64 + lane;
          const int kr = u / UPR, k = k0 + kr;
          const int o = n0 + 16 * ((u % UPR) ^ lp_oc_swz8<T::BN>(kr));
          const bool in = k < K && o < N;
          rb_o[v] = lp_load_unit(B + (in ? (size_t)k * ldb + o : (size_t)0), in ? N - o : 0);
        }
      }
    }
    if constexpr (A_T16) {
      if (a_tw && (ops & 1)) {
        const int o = m0 + a_to;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int k = k0 + 8 * kb + j;
          ra_t[j] = lp_load_unit(A + (size_t)(k < K ? k : 0) * lda + o, k < K ? M - o : 0);
        }
      }
    }
    if constexpr (B_T16) {
      if (b_tw && (ops & 2)) {
        const int o = n0 + b_to;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int k = k0 + 8 * kb + j;
          rb_t[j] = lp_load_unit(B + (size_t)(k < K ? k : 0) * ldb + o, k < K ? N - o : 0);
        }
      }
    }
  };
  // Direct load d of K step kt into stage st (aligned mode: the A units,
  // then the B units, whatever their storage).
  constexpr int ND_A = T::A_VEC;
  constexpr int ND = T::A_VEC + T::B_VEC;
  // Look-ahead loads past the last direct-load step repeat that step (in
  // bounds, so that the loop's slots carry no branches); `live` false sends
  // them to a scratch KB past the stages that nothing reads, so the stages
  // are free for the epilogue once the loop's last barrier has passed.
  const unsigned lds_dummy = lds_u + (unsigned)T::LDS_BYTES;
  auto direct_one = [&](int kt, int st, int d, bool live) {
    if (d < ND_A)
      dma16(reinterpret_cast<const float*>(a_dbase + (size_t)kt * a_dstep), a_voff[d],
            live ? lds_u + (unsigned)a_off(st) + 1024u * (unsigned)(d * T::WAVES + wave_u)
                 : lds_dummy);
    else
      dma16(reinterpret_cast<const float*>(b_dbase + (size_t)kt * b_dstep), b_voff[d - ND_A],
            live ? lds_u + (unsigned)b_off(st) +
                       1024u * (unsigned)((d - ND_A) * T::WAVES + wave_u)
                 : lds_dummy);
  };

  // Output row e of a block (its outer index 8ob + e, eight k) from the eight
  // loaded k rows: dword d packs k = 2d (low half) and 2d + 1 (high half),
  // each the half e & 1 of dword e / 2 of its row.  Lanes with odd ob write
  // row i ^ 1 when asked for row i (pair-swapped order).
  const unsigned sel_even = 0x05040100u, sel_odd = 0x07060302u;
  auto store_row = [&](char* tile, const u32x4 (&in)[8], int to, int i) {
    const int e = i ^ (ob & 1);
    const unsigned sel = ((i ^ ob) & 1) ? sel_odd : sel_even;
    u32x4 out;
#pragma unroll
    for (int d = 0; d < 4; ++d)
      out[d] = __builtin_amdgcn_perm(in[2 * d + 1][i >> 1], in[2 * d][i >> 1], sel);
    *reinterpret_cast<u32x4*>(tile + lp_unit_off(to + e, kb)) = out;
  };
  // Transposed row r of the step's register blocks (A's rows first) into
  // stage st.
  constexpr int NS = (A_T16 ? 8 : 0) + (B_T16 ? 8 : 0);
  auto store_t_row = [&](int st, int r) {
    if (A_T16 && r < 8) {
      if constexpr (A_T16) {
        if (a_tw) store_row(lds + a_off(st), ra_t, a_to, r);
      }
    } else {
      if constexpr (B_T16) {
        if (b_tw) store_row(lds + b_off(st), rb_t, b_to, A_T16 ? r - 8 : r);
      }
    }
  };
  auto store_regs = [&](int st, int ops = 3) {  // what load_regs loaded
    if ((GUARD || EDGE) && A_KC && (ops & 1)) {
#pragma unroll
      for (int v = 0; v < T::A_VEC; ++v)
        *reinterpret_cast<u32x4*>(lds + a_off(st) + 16 * ((v * T::WAVES + wave) * 64 + lane)) =
            ra_kc[v];
    }
    if ((GUARD || EDGE) && B_KC && (ops & 2)) {
#pragma unroll
      for (int v = 0; v < T::B_VEC; ++v)
        *reinterpret_cast<u32x4*>(lds + b_off(st) + 16 * ((v * T::WAVES + wave) * 64 + lane)) =
            rb_kc[v];
    }
#pragma unroll
    for (int r = 0; r < NS; ++r)
      if ((A_T16 && r < 8) ? (ops & 1) : (ops & 2)) store_t_row(st, r);
    if constexpr (A_O8) {
      if (ops & 1) {
#pragma unroll
        for (int v = 0; v < T::A_VEC; ++v)
          *reinterpret_cast<u32x4*>(lds + a_off(st) + 16 * ((v * T::WAVES + wave) * 64 + lane)) =
              ra_o[v];
      }
    }
    if constexpr (B_O8) {
      if (ops & 2) {
#pragma unroll
        for (int v = 0; v < T::B_VEC; ++v)
          *reinterpret_cast<u32x4*>(lds + b_off(st) + 16 * ((v * T::WAVES + wave) * 64 + lane)) =
              rb_o[v];
      }
    }
  };

  // ---- fragments and MFMAs: four groups of 16 k per K step ------------------
  struct Frag {
    u32x4 a[T::FM][FU], b[T::FN][FU];
  };
  constexpr int NF = T::FM + T::FN;  // fragment reads per group
  constexpr int SL = T::FM * T::FN;  // MFMAs per group
  // A fragment of 32 outer indices from an outer-contiguous tile of width X
  // (aligned mode), by two transposing reads (ds_read_b64_tr_b16).  In each
  // group of 16 lanes such a read hands lane i, element e, element i % 4 of
  // the four that lane 4e + i / 4 points at.  So lane 4e + r points at row
  // k + e and outer indices 4r .. 4r+3 of the lane group's 16 (lanes 0-15
  // and 32-47 the block's first 16, the others the next 16; lanes 32-63 the
  // k half 8 .. 15), and lane i receives k + 0 .. 3 of outer index i: the
  // same k order as a K-contiguous fragment.  With the unit swizzle the four
  // rows of a lane group fall on distinct bank groups.
  const int tr_e = (lane & 15) >> 2, tr_r = lane & 3;
  const int tr_o = 16 * ((lane >> 4) & 1) + 4 * tr_r;  // outer index in the block
  auto read_tr = [&](const char* tile, auto x_c, int o_block, int q) -> u32x4 {
    constexpr int X = decltype(x_c)::value;
    const int k = 16 * q + 8 * lh + tr_e;
    const int o = o_block + tr_o;
    // (rows k and k + 4 share the swizzle)
    const int off = k * 2 * X + 16 * ((o >> 3) ^ lp_oc_swz<X>(k)) + 2 * (o & 7);
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16*)(lds_void_t*)(tile + off));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16*)(lds_void_t*)(tile + off + 4 * 2 * X));
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
  };
  // A fragment of 32 outer indices of an 8-bit outer-contiguous tile of width
  // X (every mode), by four transposing reads (ds_read_b64_tr_b8).  In each
  // group of 16 lanes such a read hands lane i, as byte e, byte i % 8 of the
  // eight that lane 2e + i / 8 points at (measured on the device with an
  // in-bounds probe).  So lane 2e + h points at row k + e and outer indices
  // 8h .. 8h+7 of the lane group's 16 (lanes 0-15 and 32-47 the block's first
  // 16, the others the next 16; lanes 32-63 the k half 32 .. 63 of group q's
  // 64), and lane i receives eight consecutive k of outer index i; read j
  // gives k 8j .. 8j+7 of the lane's 32, the K-contiguous fragment's order.
  const int t8_e = (lane & 15) >> 1;
  const int t8_o = 16 * ((lane >> 4) & 1) + 8 * (lane & 1);  // outer index in the block
  auto read_tr8 = [&](const char* tile, auto x_c, int o_block, int q, u32x4 (&out)[FU]) {
    constexpr int X = decltype(x_c)::value;
    typedef int v2i32 __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) v2i32 lds_v2i32;
    const int o = o_block + t8_o;
#pragma unroll
    for (int u = 0; u < FU; ++u) {
      v2i32 part[2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int k = 64 * q + 32 * lh + 8 * (2 * u + jj) + t8_e;
        const int off = k * X + 16 * ((o >> 4) ^ lp_oc_swz8<X>(k)) + (o & 15);
        part[jj] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32*)(lds_void_t*)(tile + off));
      }
      out[u] = u32x4{(unsigned)part[0][0], (unsigned)part[0][1], (unsigned)part[1][0],
                     (unsigned)part[1][1]};
    }
  };
  // Read r of a group, in the order the MFMAs (i-major) first need them:
  // a[0], b[0 .. FN-1], then a[1 .. FM-1].
  // K-contiguous fragment units: lane half lh of group q holds units
  // FU*(2q + lh) .. +FU-1 of its row (8 k of a 16-bit format, 32 of an 8-bit
  // one).
  auto kc_frag = [&](const char* tile, int row, int q, u32x4 (&out)[FU]) {
#pragma unroll
    for (int u = 0; u < FU; ++u)
      out[u] = *reinterpret_cast<const u32x4*>(tile + lp_unit_off(row, FU * (2 * q + lh) + u));
  };
  auto read_one = [&](int st, int q, int r, Frag& f) {
    if (r >= 1 && r <= T::FN) {
      const int j = r - 1;
      if constexpr (B_O8)
        read_tr8(lds + b_off(st), std::integral_constant<int, T::BN>{}, wn * T::WN + j * 32,
                 q, f.b[j]);
      else if constexpr (!GUARD && !B_KC)
        f.b[j][0] = read_tr(lds + b_off(st), std::integral_constant<int, T::BN>{},
                            wn * T::WN + j * 32, q);
      else
        kc_frag(lds + b_off(st), wn * T::WN + j * 32 + li, q, f.b[j]);
    } else {
      const int i = r == 0 ? 0 : r - T::FN;
      if constexpr (A_O8)
        read_tr8(lds + a_off(st), std::integral_constant<int, T::BM>{}, wm * T::WM + i * 32,
                 q, f.a[i]);
      else if constexpr (!GUARD && !A_KC)
        f.a[i][0] = read_tr(lds + a_off(st), std::integral_constant<int, T::BM>{},
                            wm * T::WM + i * 32, q);
      else
        kc_frag(lds + a_off(st), wm * T::WM + i * 32 + li, q, f.a[i]);
    }
  };
  auto read_frag = [&](int st, int q, Frag& f) {
#pragma unroll
    for (int r = 0; r < NF; ++r) read_one(st, q, r, f);
  };
  // Fragments of a register-staged stage (guarded kernels; the last step of
  // edge kernels): the K-contiguous layout, into which 16-bit outer-contiguous
  // operands are transposed in registers; 8-bit ones keep their own layout.
  auto read_frag_kc = [&](int st, int q, Frag& f) {
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      if constexpr (A_O8)
        read_tr8(lds + a_off(st), std::integral_constant<int, T::BM>{}, wm * T::WM + i * 32,
                 q, f.a[i]);
      else
        kc_frag(lds + a_off(st), wm * T::WM + i * 32 + li, q, f.a[i]);
    }
#pragma unroll
    for (int j = 0; j < T::FN; ++j) {
      if constexpr (B_O8)
        read_tr8(lds + b_off(st), std::integral_constant<int, T::BN>{}, wn * T::WN + j * 32,
                 q, f.b[j]);
      else
        kc_frag(lds + b_off(st), wn * T::WN + j * 32 + li, q, f.b[j]);
    }
  };
  auto mma_one = [&](const Frag& f, int m) {
    const int i = m / T::FN, j = m % T::FN;
    acc[i][j] = lp_mfma<DT>(f.b[j], f.a[i], acc[i][j]);
  };

  auto wait_all = [] { __builtin_amdgcn_s_waitcnt(0x0F70); };  // vmcnt(0)
  auto wait_lds = [] { __builtin_amdgcn_s_waitcnt(0xC07F); };  // lgkmcnt(0)
  // No scalar load may be in flight inside the K loop (the epilogue's
  // arguments would otherwise be fetched just before it, and a pending
  // scalar load turns every LDS-read wait into a full lgkmcnt(0)).
  asm volatile("" ::"s"(g.C), "s"(g.ldc), "s"(g.alpha), "s"(g.beta), "s"(M), "s"(N));
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)

  if constexpr (GUARD) {
    // Guarded mode: every load through registers, one step ahead.
    if (nk > 0) {
      load_regs(0);
      store_regs(0);
      wait_lds();
      __syncthreads();
    }
    auto step = [&](int kt, int st) {
      const bool more = kt + 1 < nk;
      if (more) load_regs(kt + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < QG; ++q) {
        Frag f;
        read_frag_kc(st, q, f);
#pragma unroll
        for (int m = 0; m < SL; ++m) mma_one(f, m);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (more) store_regs(st ^ 1);
      wait_lds();
      __syncthreads();
    };
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      step(kt, 0);
      step(kt + 1, 1);
    }
    if (kt < nk) step(kt, 0);
  } else {
    // Aligned mode: every operand tile arrives by direct loads.  Every group
    // of MFMAs is issued one MFMA at a time with other work in the slots
    // between them, in a fixed order (scheduling barriers), so that with one
    // wave per SIMD the matrix pipe is not left idle while the wave issues
    // reads or loads.  Each group q has a fragment set of its own, and the
    // reads run H = QG/2 groups ahead:
    //   groups 0 .. H-1 of step kt: reads of groups H .. QG-1 of step kt;
    //   barrier of step kt: every wave has read all of stage kt (lgkmcnt(0))
    //     and seen its direct loads of step kt+1 land (vmcnt(0));
    //   groups H .. QG-1: reads of groups 0 .. H-1 of step kt+1, now
    //     visible, and step kt+2's direct loads into stage kt, now free,
    //     spread over those groups' slots.
    // The LDS so takes the loads' writes over half a step: with 16-bit
    // operands (four groups of 32-cycle MFMAs) the loads and reads that had
    // shared the last group asked the LDS for 1.5 times the group's length
    // (4096^3 bfloat16: 124 -> 114 us).  A barrier before group 1, with the
    // loads over three groups, measured no better: the last loads then have
    // a quarter step to land instead of half a step.
    auto issue_step = [&](int kt, int st, bool live) {
#pragma unroll
      for (int o = 0; o < ND; ++o) direct_one(kt, st, o, live);
    };
    // Group q of step kt (stage st) on fragments cur; fills the slots as
    // described.  kl = step kt+S clamped to the last step: past the end of K
    // the same (in-bounds) loads are repeated into a stage that is never read
    // again, and step kt+1's first fragments are read even at the last step,
    // which keeps the slots free of branches.
    constexpr int S = T::S;
    // Direct-load steps: all of them (aligned), the whole ones (edge), and
    // not the one holding the last K row when an outer-contiguous piece can
    // straddle the M or N edge (its read runs into the next k row).
    int kd = nk;
    if (EDGE) {
      const bool straddle = (!A_KC && (M & (UE - 1)) != 0) || (!B_KC && (N & (UE - 1)) != 0);
      kd = straddle ? (K - 1) / BKE : K / BKE;
    }
    constexpr int H = QG / 2;  // groups the reads run ahead (the barrier precedes group H)
    Frag fr[QG];
    auto group = [&](int kl, bool live, auto st_c, auto q_c) {
      constexpr int st = decltype(st_c)::value, q = decltype(q_c)::value;
      constexpr int st1 = st + 1 == S ? 0 : st + 1;
      // the group read in this one's slots, and the stage it comes from
      constexpr int rq = (q + H) % QG;
      constexpr int rst = q + H < QG ? st : st1;
#pragma unroll
      for (int m = 0; m < SL; ++m) {
        mma_one(fr[q], m);
#pragma unroll
        for (int r = 0; r < NF; ++r)
          if (r * SL / NF == m) read_one(rst, rq, r, fr[rq]);
        if (q >= H) {
          constexpr int SLOTS = (QG - H) * SL;
#pragma unroll
          for (int o = 0; o < ND; ++o)
            if (o * SLOTS / ND == (q - H) * SL + m) direct_one(kl, st, o, live);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // vmcnt(N) before a barrier: step kt+1's loads have landed once at most
    // the S-2 later steps' loads are still in flight.
    constexpr int AHEAD = (S - 2) * ND;
    constexpr int WAIT_AHEAD = 0x0F70 | (AHEAD & 15) | ((AHEAD >> 4) << 14);
    auto step = [&](int kt, auto st_c) {
      const bool live = kt + S < kd;
      const int kl = live ? kt + S : kd - 1;
      lp_static_for<H>([&](auto q_c) { group(kl, live, st_c, q_c); });
      wait_lds();
      __builtin_amdgcn_s_waitcnt(WAIT_AHEAD);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      lp_static_for<QG - H>([&](auto i) {
        group(kl, live, st_c, std::integral_constant<int, H + decltype(i)::value>{});
      });
    };
    if (!EDGE || kd > 0) {  // (aligned kernels run with K >= 64)
      // Steps 0 .. S-1 go out first; step 0 must have landed before the
      // first barrier.
      lp_static_for<S>([&](auto i) {
        constexpr int st = decltype(i)::value;
        issue_step(st < kd ? st : kd - 1, st, st < kd);
      });
      constexpr int FIRST = (S - 1) * ND;
      __builtin_amdgcn_s_waitcnt(0x0F70 | (FIRST & 15) | ((FIRST >> 4) << 14));
      wait_lds();
      __syncthreads();
      lp_static_for<H>([&](auto q_c) {
        read_frag(0, decltype(q_c)::value, fr[decltype(q_c)::value]);
      });
      int kt = 0;
      for (; kt + S <= kd; kt += S)
        lp_static_for<S>([&](auto i) { step(kt + decltype(i)::value, i); });
      lp_static_for<S - 1>([&](auto i) {
        if (kt + decltype(i)::value < kd) step(kt + decltype(i)::value, i);
      });
    }
    if (EDGE && kd < nk) {
      // The rest of K (at most one step) through registers, zero-filled past
      // K, M and N, in the K-contiguous layout.  The loop's clamped
      // look-ahead loads may still be landing: every wave waits for its own
      // and for every other wave's reads before the stage is rewritten.
      // Both operands' loads go out first and share one wait with the
      // look-ahead loads.
      load_regs(kd, 3);
      wait_all();
      wait_lds();
      __syncthreads();
      store_regs(0, 3);
      wait_lds();
      __syncthreads();
#pragma unroll
      for (int q = 0; q < QG; ++q) {
        Frag f;
        read_frag_kc(0, q, f);
#pragma unroll
        for (int m = 0; m < SL; ++m) mma_one(f, m);
      }
    }
  }
}

// Epilogue through LDS, for tiles whose wave tiles are at least 64 columns
// wide: a store of the MFMA register layout writes 32 rows x 32 bytes, one
// piece of every 128-byte line it touches, and the lines' other pieces come
// in three more instructions.  Here each wave stages one 32-row block row of
// its tile at a time in LDS (rows padded by 16 bytes) and reads it back row
// by row, so every C read and write of a wave instruction covers whole rows
// of the wave tile (WN floats), i.e. whole lines.  Rows past M and columns
// past N are skipped (edge tiles), and C that is not 16-byte aligned or
// whose ldc is not a multiple of 4 takes element accesses.  Measured at
// 4096 x 4096 with one K step (256x256 tiles): 27.1 us with beta 0.5 and
// 16.6 us with beta 0, against 28.4 and 20.0 us through the register layout
// (a plain device copy of the same 128 MB takes 19.6 us, a fill of the 64 MB
// 11.2 us); 4096^3: bfloat16 114 -> 113 us, E4M3 66.8 -> 64.2 us.
template <class T>
__device__ __forceinline__ void lp_store_tile_lds(const GemmArgs& g, int m0, int n0,
                                                  const f32x16 (&acc)[T::FM][T::FN],
                                                  char* lds) {
  constexpr int WN = T::WN, LD = WN + 4;  // LDS row: the wave tile's row + 16 bytes
  constexpr int LPR = WN / 4;             // lanes per row, 16 bytes each
  constexpr int RPI = 64 / LPR;           // rows per wave instruction
  constexpr int NI = 32 / RPI;            // instructions per 32-row block row
  static_assert(WN % 64 == 0 && T::WAVES * 32 * LD * 4 <= T::LDS_BYTES, "staging area");
  const WaveCoords<T> w;
  float* reg = reinterpret_cast<float*>(lds) + w.wave * 32 * LD;
  const float alpha = g.alpha, beta = g.beta;
  const int M = g.M, N = g.N, ldc = g.ldc;
  const int rr = w.lane / LPR, cc = 4 * (w.lane % LPR);
  const int col = n0 + w.wn * WN + cc;  // the lane's first column
  const bool vec = c_vector(g) && col + 3 < N;
  const size_t rstep = (size_t)RPI * ldc;  // rows between a lane's accesses
  __syncthreads();  // every wave is done reading the stages
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
    const int row0 = m0 + w.wm * T::WM + 32 * i + rr;  // the lane's first row
    float* p = g.C + (size_t)row0 * ldc + col;
    f32x4 cin[NI];
    if (beta != 0.0f) {
#pragma unroll
      for (int t = 0; t < NI; ++t) {
        cin[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (row0 + t * RPI < M) {
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
    // block (i, j), register 4q + e of lane (li, lh): row li, column
    // 32j + 8q + 4lh + e of the block row
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(reg + w.li * LD + 32 * j + 8 * q + 4 * w.lh) =
            f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                  acc[i][j][4 * q + 3]};
    // the wave reads back its own writes: one wave's LDS operations complete
    // in issue order
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int t = 0; t < NI; ++t) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(reg + (t * RPI + rr) * LD + cc);
      f32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = alpha * v[e];
        if (beta != 0.0f) o[e] = fmaf(beta, cin[t][e], o[e]);
      }
      if (row0 + t * RPI < M) {
        if (vec) {
          *reinterpret_cast<f32x4*>(p + t * rstep) = o;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < N) p[t * rstep + e] = o[e];
        }
      }
    }
    // one block row's C traffic at a time (reading the next block row's C
    // before this one's stores measured slower: 4096^2 with one K step and
    // beta 0.5, 32.5 against 27.1 us)
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_wave_barrier();
  }
}

template <class T, int DT, int MODE, bool TA, bool TB>
__global__ void __launch_bounds__(T::THREADS, T::OCC)
    lp_gemm_kernel(LpArgs g, int tiles_m, int tiles_n, int band) {
  // guarded kernels use two stages
  __shared__ __attribute__((aligned(1024)))
  char lds[MODE == MODE_GUARDED ? 2 * (T::A_BYTES + T::B_BYTES) : T::LDS_ALIGNED];
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, band, tm, tn);
  f32x16 acc[T::FM][T::FN];
  zero_acc<T>(acc);
  lp_tile_accumulate<T, DT, MODE, TA, TB>(g, lds, tm * T::BM, tn * T::BN, acc);
  GemmArgs e;
  e.M = g.M;
  e.N = g.N;
  e.K = g.K;
  e.alpha = g.alpha;
  e.beta = g.beta;
  e.A = nullptr;
  e.lda = 0;
  e.B = nullptr;
  e.ldb = 0;
  e.C = g.C;
  e.ldc = g.ldc;
  const int m0 = tm * T::BM, n0 = tn * T::BN;
  if constexpr (MODE != MODE_GUARDED && T::WN >= 64)
    lp_store_tile_lds<T>(e, m0, n0, acc, lds);
  else
    store_tile<T, MODE>(e, m0, n0, acc, acc);
  // The K loop's last steps issue look-ahead loads into LDS that nothing
  // waits for: they must land before the workgroup's LDS is released.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
}

// Split K (products with a few rows of A): workgroup b takes tile
// b % tiles (tn = tile % tiles_n, tm = tile / tiles_n) over the K range
// [s*kps, min((s+1)*kps, K)) of split s = b / tiles, kps a multiple of the K
// step.  That range is the whole K of a sub-problem whose A and B start kps*s
// values of k in, so lp_tile_accumulate runs on it unchanged (the last
// split takes the ragged end of K, if any).  The workgroup writes its
// partial sums, rows < M and columns < N, to ws[s][m][n] (rows of
// skinny_ws_stride(N) floats); skinny_reduce_kernel adds the splits in split
// order and applies alpha and beta.
template <class T, int DT, int MODE, bool TA, bool TB>
__global__ void __launch_bounds__(T::THREADS, T::OCC)
    lp_splitk_kernel(LpArgs g, int tiles_m, int tiles_n, int kps,
                     float* __restrict__ ws) {
  __shared__ __attribute__((aligned(1024)))
  char lds[MODE == MODE_GUARDED ? 2 * (T::A_BYTES + T::B_BYTES) : T::LDS_ALIGNED];
  typedef typename LpFmt<DT>::E E;
  const int tiles = tiles_m * tiles_n;
  const int split = blockIdx.x / tiles, tile = blockIdx.x - split * tiles;
  const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
  const int k0 = split * kps;
  LpArgs sub = g;
  sub.K = g.K - k0 < kps ? g.K - k0 : kps;
  sub.A = static_cast<const E*>(g.A) + (TA ? (size_t)k0 * g.lda : (size_t)k0);
  sub.B = static_cast<const E*>(g.B) + (TB ? (size_t)k0 : (size_t)k0 * g.ldb);
  f32x16 acc[T::FM][T::FN];
  zero_acc<T>(acc);
  lp_tile_accumulate<T, DT, MODE, TA, TB>(sub, lds, tm * T::BM, tn * T::BN, acc);
  // block (i, j), register 4q + e of lane (li, lh): row li, column
  // 8q + 4lh + e of the block (the epilogue's layout)
  const WaveCoords<T> w;
  const int stride = skinny_ws_stride(g.N);
  float* part = ws + (size_t)split * g.M * stride;
  const int crow = tm * T::BM + w.wm * T::WM + w.li;
  const int ccol = tn * T::BN + w.wn * T::WN + w.lh * 4;
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j) {
      const int row = crow + i * 32;
      if (row >= g.M) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = ccol + j * 32 + 8 * q;
        float* p = part + (size_t)row * stride + col;
        if (col + 3 < g.N) {
          *reinterpret_cast<f32x4*>(p) =
              f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                    acc[i][j][4 * q + 3]};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < g.N) p[e] = acc[i][j][4 * q + e];
        }
      }
    }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // the K loop's look-ahead loads into LDS
}

// Tile shapes: LpTile<BM, BN, WM, WN, OCC>.
// 4 waves of 128x128 (256 accumulators per lane), one workgroup per CU,
// 128 KB of LDS for the two stages.
typedef LpTile<256, 256, 128, 128, 1> L256x256;
// 4 waves of 64x64, four LDS stages (128 KB): problems with fewer than one
// 256x256 tile per CU.
typedef LpTile<128, 128, 64, 64, 2, 4> L128x128;
// 4 waves of 32x32, four LDS stages (64 KB): small problems, whose K steps
// are short, so the loads run three steps ahead.
typedef LpTile<64, 64, 32, 32, 2, 4> L64x64;

}  // namespace sgemm
