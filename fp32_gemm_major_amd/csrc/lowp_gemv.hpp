// Products with a few rows of A (M <= 16), 16- or 8-bit A and B with B
// stored N x K, and FP32 C, in one pass on the matrix cores with no LDS
// tiles.
//
// Row n of B (column n of C) is then contiguous along K, and a 16 x 16 MFMA
// block's operands can come straight from memory: the instruction's first
// operand is 16 rows of B (lane l supplies row l % 16), its second the rows of
// A as columns (lane l supplies row l % 16 of A, zero past M), and lane group
// q = l / 16 supplies one quarter of the block's k -- the same k for both
// operands, which is all an MFMA's k assignment needs.  A 16-bit block is
// v_mfma_f32_16x16x32_{bf16,f16} (one 16-byte piece per lane, k = 8q..8q+7),
// an 8-bit one v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales (two
// pieces per lane, k = 16q.. and 64 + 16q.., so that one load instruction of
// a wave reads 64 contiguous bytes of each of 16 rows).  The result block D
// holds C(m, n0 + i) at row i, column m: lane l's register r is
// C(l % 16, n0 + 4(l / 16) + r).
//
// A workgroup takes 16 columns of C over all of K: its LPV_WAVES waves split
// K into contiguous runs of blocks, with the loads of V::BATCH blocks (eight
// 16-byte pieces of B per lane) in flight at a time, and add their partial
// blocks through LDS in wave order (a fixed order), after which the first
// wave applies alpha and beta.  No workspace, no second pass, and B is read
// once in whole 64-byte runs.
#pragma once

#include "lowp_gemm.hpp"

namespace sgemm {

constexpr int LPV_WAVES = 8;
constexpr int LPV_THREADS = 64 * LPV_WAVES;
constexpr int LPV_COLS = 16;  // columns of C (rows of B) per workgroup
constexpr int LPV_MT = 16;    // the most rows of A

template <int DT>
struct LpvFmt {
  static constexpr int KB = DT >= LP_E4M3 ? 128 : 32;  // k per MFMA block
  static constexpr int PC = DT >= LP_E4M3 ? 2 : 1;     // 16-byte pieces per lane
  // blocks per wave whose loads are in flight together: eight pieces of B
  // per lane
  static constexpr int BATCH = 8 / PC;
  // first element of piece p of lane group q, inside a block
  static __device__ __forceinline__ int piece_k(int q, int p) {
    return DT >= LP_E4M3 ? 16 * q + 64 * p : 8 * q;
  }
};

template <int DT>
__device__ __forceinline__ f32x4 lpv_mfma(const u32x4 (&x)[LpvFmt<DT>::PC],
                                          const u32x4 (&y)[LpvFmt<DT>::PC], f32x4 acc) {
  if constexpr (DT == LP_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        __builtin_bit_cast(bf16x8, x[0]), __builtin_bit_cast(bf16x8, y[0]), acc, 0, 0, 0);
  } else if constexpr (DT == LP_F16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(
        __builtin_bit_cast(f16x8, x[0]), __builtin_bit_cast(f16x8, y[0]), acc, 0, 0, 0);
  } else {
    constexpr int fmt = DT == LP_E4M3 ? 0 : 1;
    const i32x8 xa = {(int)x[0][0], (int)x[0][1], (int)x[0][2], (int)x[0][3],
                      (int)x[1][0], (int)x[1][1], (int)x[1][2], (int)x[1][3]};
    const i32x8 ya = {(int)y[0][0], (int)y[0][1], (int)y[0][2], (int)y[0][3],
                      (int)y[1][0], (int)y[1][1], (int)y[1][2], (int)y[1][3]};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(xa, ya, acc, fmt, fmt, 0, 127, 0,
                                                            127);
  }
}

// TA: A stored K x M.  Workgroup b takes columns [16b, 16b + 16) of C.
template <int DT, bool TA>
__global__ void __launch_bounds__(LPV_THREADS) lp_gemv_kernel(LpArgs g) {
  typedef LpFmt<DT> F;
  typedef LpvFmt<DT> V;
  typedef typename F::E E;
  constexpr int UE = F::UE, BITS = 8 * F::ESZ, KB = V::KB, PC = V::PC, BATCH = V::BATCH;
  __shared__ f32x4 red[LPV_WAVES * 64];
  const int M = g.M, N = g.N, K = g.K;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, q = lane >> 4;
  const int n = blockIdx.x * LPV_COLS + i;  // this lane's row of B
  const E* __restrict__ A = static_cast<const E*>(g.A);
  const E* __restrict__ B = static_cast<const E*>(g.B);
  const int lda = g.lda, ldb = g.ldb;
  const bool b_in = n < N, a_in = i < M;
  const E* __restrict__ brow = B + (size_t)(b_in ? n : 0) * ldb;

  // this wave's blocks: a contiguous run
  const int nblk = (K + KB - 1) / KB;
  const int per = (nblk + LPV_WAVES - 1) / LPV_WAVES;
  const int b0 = wave * per, b1 = b0 + per < nblk ? b0 + per : nblk;

  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int blk = b0; blk < b1; blk += BATCH) {
    u32x4 x[BATCH][PC], y[BATCH][PC];
    if (blk + BATCH <= b1 && (blk + BATCH) * KB <= K && !TA) {
      // whole blocks (the wave-uniform common case): plain 16-byte loads,
      // all issued before the first MFMA
#pragma unroll
      for (int j = 0; j < BATCH; ++j)
#pragma unroll
        for (int p = 0; p < PC; ++p) {
          const int k = (blk + j) * KB + V::piece_k(q, p);
          x[j][p] = u32x4{0u, 0u, 0u, 0u};
          y[j][p] = u32x4{0u, 0u, 0u, 0u};
          if (b_in) {
            const u32x4u1 v = *reinterpret_cast<const u32x4u1*>(brow + k);
            x[j][p] = u32x4{v[0], v[1], v[2], v[3]};
          }
          if (a_in) {
            const u32x4u1 v = *reinterpret_cast<const u32x4u1*>(A + (size_t)i * lda + k);
            y[j][p] = u32x4{v[0], v[1], v[2], v[3]};
          }
        }
#pragma unroll
      for (int j = 0; j < BATCH; ++j) acc = lpv_mfma<DT>(x[j], y[j], acc);
      continue;
    }
#pragma unroll
    for (int j = 0; j < BATCH; ++j)
#pragma unroll
      for (int p = 0; p < PC; ++p) {
        const int k = (blk + j) * KB + V::piece_k(q, p);
        const bool live = blk + j < b1;
        x[j][p] = live && b_in ? lp_load_unit(brow + k, K - k) : u32x4{0u, 0u, 0u, 0u};
        u32x4 v = {0u, 0u, 0u, 0u};
        if (live && a_in) {
          if (!TA) {
            v = lp_load_unit(A + (size_t)i * lda + k, K - k);
          } else if (k < K) {  // A(i, k) = A[k*lda + i]: one element per k
            // unconditional loads (k clamped to K - 1), masked afterwards, so
            // that they are all in flight at once
            unsigned h[UE];
#pragma unroll
            for (int e = 0; e < UE; ++e)
              h[e] = (unsigned)A[(size_t)(k + e < K ? k + e : K - 1) * lda + i];
#pragma unroll
            for (int e = 0; e < UE; ++e)
              if (k + e < K) v[e / (32 / BITS)] |= h[e] << (BITS * (e % (32 / BITS)));
          }
        }
        y[j][p] = v;
      }
#pragma unroll
    for (int j = 0; j < BATCH; ++j)
      if (blk + j < b1) acc = lpv_mfma<DT>(x[j], y[j], acc);
  }

  red[wave * 64 + lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  f32x4 s = red[lane];
#pragma unroll
  for (int w = 1; w < LPV_WAVES; ++w) {
    const f32x4 v = red[w * 64 + lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] += v[r];
  }
  if (!a_in) return;
  const int col = blockIdx.x * LPV_COLS + 4 * q;
  const float alpha = g.alpha, beta = g.beta;
  float* p = g.C + (size_t)i * g.ldc + col;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (col + r < N) {
      float o = alpha * s[r];
      if (beta != 0.0f) o = fmaf(beta, p[r], o);
      p[r] = o;
    }
  }
}

}  // namespace sgemm
