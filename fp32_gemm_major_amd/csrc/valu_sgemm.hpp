// FP32 SGEMM on the vector ALUs: per-lane register outer products.
//
// This is the gfx950 form of the page's most tuned CUDA-core kernel
// ("GEMM 优化之路", sections on 2-D register tiling and vectorised access):
// a BM x BN block tile, each lane accumulating a TM x TN = 8 x 8 sub-tile,
// A stored transposed in LDS ([k][m]) so a lane's eight A values for one k
// are two 16-byte reads, B stored [k][n], 16-byte global loads, and two LDS
// stages with one barrier per K step.  A lane's 8 rows are split into two
// runs of 4 (at ty*4 and BM/2 + ty*4), and likewise its columns, so the 16
// lanes of a row group read one contiguous 256-byte span of B per run.
//
// It exists to be measured against the MFMA kernel.  Each multiply-add is one
// unpacked v_fmac_f32: the library is compiled with packed FP32 arithmetic
// turned off (-packed-fp32-ops), so the compiler makes no v_pk_fma_f32.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mfma_sgemm.hpp"  // f32x4
#include "tile_map.hpp"

namespace sgemm {

template <int BM_, int BN_, int BK_>
struct ValuTile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int TM = 8, TN = 8;
  static constexpr int TX = BN / TN, TY = BM / TM;
  static constexpr int THREADS = TX * TY;
  static constexpr int AS = BM + 4;  // LDS row stride of transposed A ([k][m])
  static constexpr int BS = BN + 4;  // LDS row stride of B ([k][n])
  static constexpr int A_ELEMS = BK * AS;
  static constexpr int B_ELEMS = BK * BS;
  static constexpr int STAGE = A_ELEMS + B_ELEMS;
  static constexpr int LDS_BYTES = 2 * STAGE * 4;
  static constexpr int A_VEC = BM * BK / 4 / THREADS;
  static constexpr int B_VEC = BK * BN / 4 / THREADS;
  static_assert(A_VEC >= 1 && A_VEC * THREADS * 4 == BM * BK, "A loader");
  static_assert(B_VEC >= 1 && B_VEC * THREADS * 4 == BK * BN, "B loader");
  static_assert(BK % 4 == 0, "");
};

template <class T, bool GUARD>
__global__ void __launch_bounds__(T::THREADS)
    valu_sgemm_kernel(int M, int N, int K, float alpha,
                      const float* __restrict__ A, int lda,
                      const float* __restrict__ B, int ldb, float beta,
                      float* __restrict__ C, int ldc, int tiles_m,
                      int tiles_n, int band) {
  __shared__ __attribute__((aligned(16))) float lds[2 * T::STAGE];

  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, band, tm, tn);
  const int m0 = tm * T::BM, n0 = tn * T::BN;
  const int tid = threadIdx.x;
  const int ty = tid / T::TX, tx = tid % T::TX;

  constexpr int A_PER_ROW = T::BK / 4, B_PER_ROW = T::BN / 4;
  constexpr int A_ROWS_PER_PASS = T::THREADS / A_PER_ROW;
  constexpr int B_ROWS_PER_PASS = T::THREADS / B_PER_ROW;
  const int a_row0 = tid / A_PER_ROW, a_col = (tid % A_PER_ROW) * 4;
  const int b_row0 = tid / B_PER_ROW, b_col = (tid % B_PER_ROW) * 4;

  float acc[T::TM][T::TN];
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j) acc[i][j] = 0.0f;

  f32x4 ra[T::A_VEC], rb[T::B_VEC];

  // Guarded kernels still use 16-byte loads for pieces that lie wholly inside
  // the operand and start on a 16-byte boundary (every piece starts at a
  // multiple of 4 elements from the tile corner, so row alignment decides).
  const bool a_vec_ok =
      (lda % 4 == 0) && ((reinterpret_cast<uintptr_t>(A) & 15u) == 0);
  const bool b_vec_ok =
      (ldb % 4 == 0) && ((reinterpret_cast<uintptr_t>(B) & 15u) == 0);

  auto load_tile = [&](int k0) {
#pragma unroll
    for (int v = 0; v < T::A_VEC; ++v) {
      const int gm = m0 + a_row0 + v * A_ROWS_PER_PASS;
      const int gk = k0 + a_col;
      const float* p = A + (size_t)gm * lda + gk;
      if (!GUARD || (a_vec_ok && gm < M && gk + 3 < K)) {
        ra[v] = *reinterpret_cast<const f32x4*>(p);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          ra[v][e] = (gm < M && gk + e < K) ? p[e] : 0.0f;
      }
    }
#pragma unroll
    for (int v = 0; v < T::B_VEC; ++v) {
      const int gk = k0 + b_row0 + v * B_ROWS_PER_PASS;
      const int gn = n0 + b_col;
      const float* p = B + (size_t)gk * ldb + gn;
      if (!GUARD || (b_vec_ok && gk < K && gn + 3 < N)) {
        rb[v] = *reinterpret_cast<const f32x4*>(p);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          rb[v][e] = (gk < K && gn + e < N) ? p[e] : 0.0f;
      }
    }
  };

  auto store_tile = [&](int stage) {
    float* As = lds + stage * T::STAGE;
    float* Bs = As + T::A_ELEMS;
#pragma unroll
    for (int v = 0; v < T::A_VEC; ++v) {
      const int m = a_row0 + v * A_ROWS_PER_PASS;
#pragma unroll
      for (int e = 0; e < 4; ++e) As[(a_col + e) * T::AS + m] = ra[v][e];
    }
#pragma unroll
    for (int v = 0; v < T::B_VEC; ++v)
      *reinterpret_cast<f32x4*>(Bs + (b_row0 + v * B_ROWS_PER_PASS) * T::BS +
                                b_col) = rb[v];
  };

  auto compute_tile = [&](int stage) {
    const float* As = lds + stage * T::STAGE;
    const float* Bs = As + T::A_ELEMS;
#pragma unroll
    for (int k = 0; k < T::BK; ++k) {
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(As + k * T::AS + ty * 4);
      const f32x4 a1 =
          *reinterpret_cast<const f32x4*>(As + k * T::AS + T::BM / 2 + ty * 4);
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(Bs + k * T::BS + tx * 4);
      const f32x4 b1 =
          *reinterpret_cast<const f32x4*>(Bs + k * T::BS + T::BN / 2 + tx * 4);
      float a[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      float b[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
  };

  const int ktiles = (K + T::BK - 1) / T::BK;
  // The epilogue's kernel arguments are fetched here, not inside the K loop:
  // a scalar load in flight in the loop forces full LDS waits there.
  asm volatile("" ::"s"(C), "s"(ldc), "s"(alpha), "s"(beta), "s"(M), "s"(N));
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  if (ktiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int kt = 0; kt < ktiles; ++kt) {
    const int stage = kt & 1;
    const bool more = kt + 1 < ktiles;
    if (more) load_tile((kt + 1) * T::BK);
    compute_tile(stage);
    if (more) store_tile(stage ^ 1);
    __syncthreads();
  }

  // Epilogue: lane rows ty*4+i and BM/2+ty*4+i, column runs tx*4..+3 and
  // BN/2+tx*4..+3; C is read only when beta != 0.
  const bool c_vec =
      (ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(C) & 15u) == 0);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = m0 + (i < 4 ? ty * 4 + i : T::BM / 2 + ty * 4 + (i - 4));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int col = n0 + h * (T::BN / 2) + tx * 4;
      float* p = C + (size_t)row * ldc + col;
      if (!GUARD && c_vec) {
        f32x4 o;
        f32x4 cin = beta != 0.0f ? *reinterpret_cast<const f32x4*>(p) : f32x4(0.0f);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] = alpha * acc[i][4 * h + e];
          if (beta != 0.0f) o[e] = fmaf(beta, cin[e], o[e]);
        }
        *reinterpret_cast<f32x4*>(p) = o;
      } else if (!GUARD || row < M) {
        float cin[4];
        if (beta != 0.0f) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (!GUARD || col + e < N) cin[e] = p[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (GUARD && col + e >= N) continue;
          float o = alpha * acc[i][4 * h + e];
          if (beta != 0.0f) o = fmaf(beta, cin[e], o);
          p[e] = o;
        }
      }
    }
  }
}

}  // namespace sgemm
