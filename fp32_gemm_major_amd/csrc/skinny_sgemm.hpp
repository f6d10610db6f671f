// Small-M SGEMM (M <= 16) on the vector ALUs.
//
// With a handful of rows in A the product is bound by reading B once from
// HBM (2*M flops per 4 bytes of B, far under the MFMA ridge), so the matrix
// cores do not help and an output tile of 64 or more rows would waste most
// of their work; what matters is streaming B with wide, coalesced loads and
// enough of them in flight.  The problem definition is the pages' ("GEMM
// 优化之路", problem statement): C = alpha * op(A) * B + beta * C.
//
// A workgroup of 8 waves takes 256 columns of C (64 lanes x 4 adjacent
// columns, one 16-byte load of a B row per lane) and one K range of a
// split-K decomposition.  Its waves take the range's rows of B in turn
// (wave w: rows w, w+8, ...), eight rows in flight per wave, and multiply
// each with the matching column of A, which the workgroup stages in LDS as
// [k][m] so one 16-byte broadcast read gives four rows' values.  The waves'
// partial sums are added through LDS in a fixed tree, and the workgroup then
// either applies alpha and beta (one K range) or writes its partial sums to
// the workspace as [split][m][n] (row stride N rounded up to 4); a second
// kernel adds the splits in order and applies alpha and beta.  Every sum is
// taken in a fixed order, so results do not depend on timing.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mfma_sgemm.hpp"  // f32x4, f32x4u, GemmArgs

namespace sgemm {

constexpr int SKINNY_COLS = 256;    // columns of C per workgroup
constexpr int SKINNY_WAVES = 8;     // waves per workgroup, interleaved over k
constexpr int SKINNY_THREADS = 64 * SKINNY_WAVES;
constexpr int SKINNY_UNROLL = 8;    // rows of B in flight per wave
constexpr int SKINNY_KC = 256;      // rows of A staged in LDS at a time

// Row stride of a partial-sum row in the workspace: N rounded up to 4, so
// every 4-column group starts 16-byte aligned.
__host__ __device__ inline int skinny_ws_stride(int N) { return (N + 3) & ~3; }

template <int MT>
struct SkinnyLds {
  // the A chunk ([k][m]) and, after the K loop, the waves' partial sums
  static constexpr int A_FLOATS = SKINNY_KC * MT;
  static constexpr int RED_FLOATS = (SKINNY_WAVES / 2) * MT * 64 * 4;
  static constexpr int FLOATS = A_FLOATS > RED_FLOATS ? A_FLOATS : RED_FLOATS;
};

// 16 bytes of a row of B at column n (any 4-byte alignment), zero past N.
__device__ __forceinline__ f32x4 skinny_load_b(const float* p, int n, int N) {
  if (n + 3 < N) {
    const f32x4u v = *reinterpret_cast<const f32x4u*>(p);
    return f32x4{v[0], v[1], v[2], v[3]};
  }
  f32x4 x;
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = n + e < N ? p[e] : 0.0f;
  return x;
}

// Grid: splits * column blocks; split s covers rows [s*kps, min(K, (s+1)*kps))
// of B.  MT >= M (rows of A past M are zero in LDS and never stored).  TA: A
// stored K x M.  ws: the workspace when splits > 1, else unused.
template <int MT, bool TA>
__global__ void __launch_bounds__(SKINNY_THREADS)
    skinny_sgemm_kernel(GemmArgs g, int col_blocks, int kps, float* __restrict__ ws) {
  __shared__ __attribute__((aligned(16))) float lds[SkinnyLds<MT>::FLOATS];
  const int M = g.M, N = g.N, K = g.K;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int s = blockIdx.x / col_blocks, cb = blockIdx.x - s * col_blocks;
  const int splits = gridDim.x / col_blocks;
  const int k0 = s * kps, k1 = k0 + kps < K ? k0 + kps : K;
  const int n = cb * SKINNY_COLS + 4 * lane;
  const float* __restrict__ A = g.A;
  const float* __restrict__ B = g.B;
  const int lda = g.lda, ldb = g.ldb;

  float acc[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[m][e] = 0.0f;

  constexpr int STEP = SKINNY_WAVES * SKINNY_UNROLL;
  for (int kc = k0; kc < k1; kc += SKINNY_KC) {
    const int kn = k1 - kc < SKINNY_KC ? k1 - kc : SKINNY_KC;
    const float* bp = B + (size_t)kc * ldb + n;
    // rows kk + u*SKINNY_WAVES of the chunk, loaded together, then multiplied
    auto load = [&](int kk, f32x4 (&b)[SKINNY_UNROLL]) {
#pragma unroll
      for (int u = 0; u < SKINNY_UNROLL; ++u) {
        const int k = kk + u * SKINNY_WAVES;
        b[u] = k < kn ? skinny_load_b(bp + (size_t)k * ldb, n, N) : f32x4{};
      }
    };
    auto multiply = [&](int kk, const f32x4 (&b)[SKINNY_UNROLL]) {
#pragma unroll
      for (int u = 0; u < SKINNY_UNROLL; ++u) {
        const int k = kk + u * SKINNY_WAVES;
        if (k < kn) {
#pragma unroll
          for (int m4 = 0; m4 < MT; m4 += 4) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(&lds[k * MT + m4]);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                acc[m4 + mi][e] = fmaf(a[mi], b[u][e], acc[m4 + mi][e]);
          }
        }
      }
    };
    // the chunk's first rows of B are requested before A is staged, so their
    // latency overlaps the staging and its barrier
    f32x4 b[SKINNY_UNROLL];
    load(wave, b);
    // stage A(0..MT-1, kc..kc+kn) as lds[k][m], zero past M and past kn
    for (int i = threadIdx.x; i < SKINNY_KC * MT; i += SKINNY_THREADS) {
      int k, m;
      if (TA) {  // A(m, k) = A[k*lda + m]: m fastest reads a row of A^T
        k = i / MT;
        m = i - k * MT;
      } else {   // A(m, k) = A[m*lda + k]: k fastest reads a row of A
        m = i / SKINNY_KC;
        k = i - m * SKINNY_KC;
      }
      float v = 0.0f;
      if (m < M && k < kn)
        v = TA ? A[(size_t)(kc + k) * lda + m] : A[(size_t)m * lda + (kc + k)];
      lds[k * MT + m] = v;
    }
    __syncthreads();
    for (int kk = wave; kk < kn; kk += STEP) {
      if (kk != wave) load(kk, b);
      multiply(kk, b);
    }
    __syncthreads();  // the next chunk, or the reduction, reuses the LDS
  }

  // waves [h, 2h) hand their sums to waves [0, h), h = 4, 2, 1
  f32x4* red = reinterpret_cast<f32x4*>(lds);
#pragma unroll
  for (int h = SKINNY_WAVES / 2; h >= 1; h /= 2) {
    if (wave >= h && wave < 2 * h) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
        red[((wave - h) * MT + m) * 64 + lane] =
            f32x4{acc[m][0], acc[m][1], acc[m][2], acc[m][3]};
    }
    __syncthreads();
    if (wave < h) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const f32x4 v = red[(wave * MT + m) * 64 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[m][e] += v[e];
      }
    }
    __syncthreads();
  }
  if (wave != 0 || n >= N) return;

  if (splits > 1) {
    const int stride = skinny_ws_stride(N);
#pragma unroll
    for (int m = 0; m < MT; ++m)
      if (m < M)
        *reinterpret_cast<f32x4*>(ws + ((size_t)s * M + m) * stride + n) =
            f32x4{acc[m][0], acc[m][1], acc[m][2], acc[m][3]};
    return;
  }
  const float alpha = g.alpha, beta = g.beta;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m < M) {
      float* p = g.C + (size_t)m * g.ldc + n;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (n + e < N) {
          float o = alpha * acc[m][e];
          if (beta != 0.0f) o = fmaf(beta, p[e], o);
          p[e] = o;
        }
      }
    }
  }
}

// Adds the splits' partial sums in split order and applies alpha and beta:
// one thread per 4-column group of one row of C.  The partial sums are a few
// MB that the first kernel has just written, so the kernel is bound by load
// latency: workgroups of one wave spread it over every CU, and each thread
// has C and up to 16 splits' loads in flight at once (1 x 4096 and 16 x 4096
// products: 3.9 us with 256-thread workgroups and 8 loads at a time).
constexpr int SKINNY_REDUCE_THREADS = 64;

__global__ void __launch_bounds__(SKINNY_REDUCE_THREADS)
    skinny_reduce_kernel(GemmArgs g, int splits, const float* __restrict__ ws) {
  const int M = g.M, N = g.N;
  const int stride = skinny_ws_stride(N);
  const int groups = stride / 4;
  const long long x = (long long)blockIdx.x * SKINNY_REDUCE_THREADS + threadIdx.x;
  if (x >= (long long)M * groups) return;
  const int m = (int)(x / groups), n = 4 * (int)(x - (long long)m * groups);
  const float alpha = g.alpha, beta = g.beta;
  float* p = g.C + (size_t)m * g.ldc + n;
  float c[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (beta != 0.0f) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (n + e < N) c[e] = p[e];
  }
  // sixteen independent loads at a time, added in split order
  const float* p0 = ws + (size_t)m * stride + n;
  const size_t split_stride = (size_t)M * stride;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s = 0; s < splits; s += 16) {
    f32x4 v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (s + j < splits)
        v[j] = *reinterpret_cast<const f32x4*>(p0 + (size_t)(s + j) * split_stride);
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (s + j < splits) acc += v[j];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (n + e >= N) break;
    float o = alpha * acc[e];
    if (beta != 0.0f) o = fmaf(beta, c[e], o);
    p[e] = o;
  }
}

// ---- small M, B stored N x K, in one pass -----------------------------------
//
// Row n of B is then contiguous along K, so one load instruction of a wave
// can read 1 KB of one row (64 lanes x 16 bytes, k = 256p + 4*lane ..): whole
// cache lines, with no LDS and no workspace.  A workgroup of SKINNY_NT_WAVES
// waves takes R rows of B (R columns of C) over all of K; its waves split K
// into contiguous runs of 256-k pieces, and each lane multiplies its 16 bytes
// of the R rows with the same 16 bytes of every row of A, which it loads
// itself (A is small and read from the caches), keeping MT x R sums.  The
// lanes' sums meet by recursive halving (each exchange step halves the sums a
// lane holds, so MT*R sums take MT*R exchanges rather than 6*MT*R), the
// waves' through LDS in wave order, and one thread per output applies alpha
// and beta: every sum is taken in a fixed order.  R shrinks as MT grows so
// that the sums, the pieces in flight and the A pieces fit 128 registers
// (four waves per SIMD, two workgroups per CU).

constexpr int SKINNY_NT_WAVES = 8;
constexpr int SKINNY_NT_THREADS = 64 * SKINNY_NT_WAVES;
constexpr int SKINNY_NT_PIECE = 256;  // k per wave load instruction

// rows of B per workgroup for MT rows of A (measured on MI355X, 4096 x 4096
// and 11008 x 4096: 8 rows for MT <= 2, 4 rows for MT = 4 and 8)
__host__ __device__ constexpr int skinny_nt_rows(int mt) { return mt <= 2 ? 8 : 4; }

// 16 bytes at p (any 4-byte alignment) holding n elements of the row (n <= 0:
// none; n < 4: the rest are zero).  The partial case loads from clamped,
// in-bounds addresses and masks afterwards, so its loads do not wait on
// per-element branches.
__device__ __forceinline__ f32x4 skinny_nt_load(const float* p, int n) {
  if (n >= 4) {
    const f32x4u v = *reinterpret_cast<const f32x4u*>(p);
    return f32x4{v[0], v[1], v[2], v[3]};
  }
  f32x4 x = {0.0f, 0.0f, 0.0f, 0.0f};
  if (n <= 0) return x;
  float h[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) h[e] = p[e < n ? e : n - 1];
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = e < n ? h[e] : 0.0f;
  return x;
}

// Recursive halving of V partial sums per lane over the lane bits from 32
// down to LOWEST: at the exchange with lane l ^ off, the lane whose bit `off`
// is set keeps the upper half of its current sums and sends the lower half
// (its partner the reverse) and adds what it receives, so V sums take V
// exchanges rather than log2(64 / LOWEST) per sum.  Once a lane holds one sum
// the remaining exchanges add whole sums.  Afterwards acc[0 .. max(1, V >> n))
// (n = the exchanges that halved) hold sums number base, base + 1, ..., each
// added over the lanes that differ from this one in the exchanged bits;
// returns base.  Every lane adds in the same fixed order.
template <int V, int LOWEST>
__device__ __forceinline__ int skinny_halve(float (&acc)[V], int lane) {
  int cnt = V, base = 0;
#pragma unroll
  for (int off = 32; off >= LOWEST; off >>= 1) {
    const bool up = (lane & off) != 0;
    if (cnt > 1) {
      const int half = cnt >> 1;
#pragma unroll
      for (int i = 0; i < V / 2; ++i) {
        if (i < half) {
          // bitwise selects: a select between two elements of the array
          // becomes an indexed read of the whole array
          const unsigned lo = __float_as_uint(acc[i]), hi = __float_as_uint(acc[i + half]);
          const unsigned msk = up ? 0xFFFFFFFFu : 0u;
          const float send = __uint_as_float((lo & msk) | (hi & ~msk));
          const float keep = __uint_as_float((hi & msk) | (lo & ~msk));
          acc[i] = keep + __shfl_xor(send, off);
        }
      }
      if (up) base += half;
      cnt = half;
    } else {
      acc[0] += __shfl_xor(acc[0], off);
    }
  }
  return base;
}

// Grid: ceil(N / R) workgroups, workgroup b taking rows [R*b, R*b + R) of B.
// MT >= M >= 1; N >= 1; K <= INT_MAX - 256.  TA: A stored K x M.
template <int MT, bool TA>
__global__ void __launch_bounds__(SKINNY_NT_THREADS, 4) skinny_nt_kernel(GemmArgs g) {
  constexpr int R = skinny_nt_rows(MT);
  constexpr int V = MT * R;  // sums per lane, a power of two up to 64
  static_assert((V & (V - 1)) == 0 && V <= 64, "sums per lane");
  constexpr int LOGV = V == 1 ? 0 : V == 2 ? 1 : V == 4 ? 2 : V == 8 ? 3 : V == 16 ? 4
                     : V == 32 ? 5 : 6;
  __shared__ float red[SKINNY_NT_WAVES * V];
  const int M = g.M, N = g.N, K = g.K;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * R;
  const float* __restrict__ A = g.A;
  const int lda = g.lda;
  // rows of B past N and of A past M are clamped to the last one: their
  // loads stay in bounds and their sums are never stored
  const float* brow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) brow[r] = g.B + (size_t)(n0 + r < N ? n0 + r : N - 1) * g.ldb;
  int am[MT];
  const float* arow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    am[m] = m < M ? m : M - 1;
    arow[m] = A + (size_t)am[m] * lda;
  }
  // this wave's pieces: a contiguous run
  const int np = K / SKINNY_NT_PIECE + (K % SKINNY_NT_PIECE != 0);
  const int per = (np + SKINNY_NT_WAVES - 1) / SKINNY_NT_WAVES;
  const int p0 = wave * per, p1 = p0 + per < np ? p0 + per : np;

  float acc[V];  // acc[m * R + r]
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = 0.0f;
  for (int p = p0; p < p1; ++p) {
    const int k = p * SKINNY_NT_PIECE + 4 * lane;
    f32x4 b[R], a[MT];
    if ((p + 1) * SKINNY_NT_PIECE <= K) {
      // a whole piece (wave-uniform): plain loads, all issued before the
      // first multiply-add
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const f32x4u v = *reinterpret_cast<const f32x4u*>(brow[r] + k);
        b[r] = f32x4{v[0], v[1], v[2], v[3]};
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (!TA) {
          const f32x4u v = *reinterpret_cast<const f32x4u*>(arow[m] + k);
          a[m] = f32x4{v[0], v[1], v[2], v[3]};
        } else {  // A(m, k) = A[k*lda + m]: one element per k
#pragma unroll
          for (int e = 0; e < 4; ++e) a[m][e] = A[(size_t)(k + e) * lda + am[m]];
        }
      }
    } else {  // the last piece of K
      const int left = K - k;
#pragma unroll
      for (int r = 0; r < R; ++r) b[r] = skinny_nt_load(brow[r] + k, left);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (!TA) {
          a[m] = skinny_nt_load(arow[m] + k, left);
        } else {
          a[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
          if (left > 0) {
            float h[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              h[e] = A[(size_t)(e < left ? k + e : k + left - 1) * lda + am[m]];
#pragma unroll
            for (int e = 0; e < 4; ++e) a[m][e] = e < left ? h[e] : 0.0f;
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[m * R + r] = fmaf(a[m][e], b[r][e], acc[m * R + r]);
  }

  // the lanes' sums: after the halving lane l holds the wave's sum number
  // l >> (6 - log2 V) (the lanes of a group of 64 / V hold the same one)
  const int base = skinny_halve<V, 1>(acc, lane);
  if ((lane & ((64 >> LOGV) - 1)) == 0) red[wave * V + base] = acc[0];
  __syncthreads();
  const int t = threadIdx.x;
  if (t >= V) return;
  float s = red[t];
#pragma unroll
  for (int w = 1; w < SKINNY_NT_WAVES; ++w) s += red[w * V + t];
  const int m = t / R, r = t % R;
  if (m >= M || n0 + r >= N) return;
  float* c = g.C + (size_t)m * g.ldc + n0 + r;
  float o = g.alpha * s;
  if (g.beta != 0.0f) o = fmaf(g.beta, *c, o);
  *c = o;
}

// ---- small M, B stored K x N, in one pass -----------------------------------
//
// Row k of B is contiguous along N.  A workgroup of SKINNY_KN_WAVES waves
// takes SKINNY_KN_COLS columns of C over all of K: each lane takes 4 adjacent
// columns (16 bytes of a row, 8 lanes per 128-byte line) and, of every unit
// of 32 rows, the 4 consecutive rows 4g .. 4g+3 of its row group g (8 row
// groups per wave), so that its 4 k also form one 16-byte piece of each row
// of A.  The waves split K into contiguous runs of units; each lane keeps
// MT x 4 sums (its columns times the rows of A).  The 8 row groups' sums meet
// by recursive halving over the lane bits that select the row group, the
// waves' through LDS in wave order, and one thread per output applies alpha
// and beta: every sum is taken in a fixed order, no workspace.

constexpr int SKINNY_KN_WAVES = 16;
constexpr int SKINNY_KN_THREADS = 64 * SKINNY_KN_WAVES;
constexpr int SKINNY_KN_COLS = 32;              // columns of C per workgroup
constexpr int SKINNY_KN_LPR = SKINNY_KN_COLS / 4;  // lanes per row of B
constexpr int SKINNY_KN_RG = 64 / SKINNY_KN_LPR;   // row groups per wave
constexpr int SKINNY_KN_UNIT = 4 * SKINNY_KN_RG;   // rows of B per unit
static_assert(SKINNY_KN_RG == 8, "three halving bits");

// Grid: ceil(N / SKINNY_KN_COLS) workgroups.  MT >= M >= 1, N >= 1,
// K <= INT_MAX - SKINNY_KN_UNIT.  TA: A stored K x M.
template <int MT, bool TA>
__global__ void __launch_bounds__(SKINNY_KN_THREADS, 4) skinny_kn_kernel(GemmArgs g) {
  constexpr int V = MT * 4;                  // sums per lane: acc[m * 4 + column]
  constexpr int LOGV = V == 4 ? 2 : V == 8 ? 3 : V == 16 ? 4 : 5;
  static_assert(V == 4 || V == 8 || V == 16 || V == 32, "1, 2, 4 or 8 rows of A");
  constexpr int HALVE = LOGV < 3 ? LOGV : 3;  // halving exchanges of the three
  constexpr int CF = V >> HALVE;              // sums a lane holds after them
  // units in flight per wave: two with one row of A (registers allow)
  constexpr int BATCH = MT == 1 ? 2 : 1;
  __shared__ float red[SKINNY_KN_WAVES * SKINNY_KN_LPR * V];
  const int M = g.M, N = g.N, K = g.K;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * SKINNY_KN_COLS;
  const int cg = lane % SKINNY_KN_LPR, rg = lane / SKINNY_KN_LPR;
  const int n = n0 + 4 * cg;
  const int ncl = n < N ? n : N - 1;  // columns past N: clamped loads, never stored
  const int nleft = N - n;
  const float* __restrict__ A = g.A;
  const float* __restrict__ B = g.B;
  const int lda = g.lda, ldb = g.ldb;
  int am[MT];  // rows of A past M clamped to the last one
#pragma unroll
  for (int m = 0; m < MT; ++m) am[m] = m < M ? m : M - 1;
  const int nu = K / SKINNY_KN_UNIT + (K % SKINNY_KN_UNIT != 0);
  const int per = (nu + SKINNY_KN_WAVES - 1) / SKINNY_KN_WAVES;
  const int u0 = wave * per, u1 = u0 + per < nu ? u0 + per : nu;
  const bool cols_whole = n0 + SKINNY_KN_COLS <= N;

  float acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = 0.0f;
  for (int u = u0; u < u1; u += BATCH) {
    f32x4 b[BATCH][4], a[BATCH][MT];
    if (cols_whole && u + BATCH <= u1 && (u + BATCH) * SKINNY_KN_UNIT <= K) {
      // whole units inside N (wave-uniform): plain loads, all issued before
      // the first multiply-add
#pragma unroll
      for (int t = 0; t < BATCH; ++t) {
        const int k = (u + t) * SKINNY_KN_UNIT + 4 * rg;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4u v = *reinterpret_cast<const f32x4u*>(B + (size_t)(k + j) * ldb + n);
          b[t][j] = f32x4{v[0], v[1], v[2], v[3]};
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (!TA) {
            const f32x4u v = *reinterpret_cast<const f32x4u*>(A + (size_t)am[m] * lda + k);
            a[t][m] = f32x4{v[0], v[1], v[2], v[3]};
          } else {  // A(m, k) = A[k*lda + m]: one element per k
#pragma unroll
            for (int e = 0; e < 4; ++e) a[t][m][e] = A[(size_t)(k + e) * lda + am[m]];
          }
        }
      }
    } else {
      // the last units of K, or columns past N: rows past K are zero (not
      // loaded), partial rows and pieces of A load from clamped addresses
#pragma unroll
      for (int t = 0; t < BATCH; ++t) {
        const int k = (u + t) * SKINNY_KN_UNIT + 4 * rg;
        const int kleft = u + t < u1 ? K - k : 0;  // rows of B left from k
#pragma unroll
        for (int j = 0; j < 4; ++j)
          b[t][j] = j < kleft ? skinny_nt_load(B + (size_t)(k + j) * ldb + ncl, nleft)
                              : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (!TA) {
            a[t][m] = skinny_nt_load(A + (size_t)am[m] * lda + (kleft > 0 ? k : 0), kleft);
          } else {
            a[t][m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if (kleft > 0) {
              float h[4];
#pragma unroll
              for (int e = 0; e < 4; ++e)
                h[e] = A[(size_t)(e < kleft ? k + e : k + kleft - 1) * lda + am[m]];
#pragma unroll
              for (int e = 0; e < 4; ++e) a[t][m][e] = e < kleft ? h[e] : 0.0f;
            }
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < BATCH; ++t)
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[m * 4 + e] = fmaf(a[t][m][j], b[t][j][e], acc[m * 4 + e]);
  }

  // the row groups' sums: halving over the lane bits that select the row
  // group (offsets 32, 16, 8); afterwards a lane holds CF sums from `base`
  const int base = skinny_halve<V, SKINNY_KN_LPR>(acc, lane);
  // after whole-sum exchanges every lane of a pair holds the same sums: the
  // one whose exchanged row-group bits are zero writes them
  if ((rg & ((1 << (3 - HALVE)) - 1)) == 0) {
#pragma unroll
    for (int i = 0; i < CF; ++i) red[(wave * SKINNY_KN_LPR + cg) * V + base + i] = acc[i];
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (t >= SKINNY_KN_LPR * V) return;
  const int c = t / V, v = t % V;
  float s = red[c * V + v];
#pragma unroll
  for (int w = 1; w < SKINNY_KN_WAVES; ++w) s += red[(w * SKINNY_KN_LPR + c) * V + v];
  const int m = v / 4, col = n0 + 4 * c + v % 4;
  if (m >= M || col >= N) return;
  float* cp = g.C + (size_t)m * g.ldc + col;
  float o = g.alpha * s;
  if (g.beta != 0.0f) o = fmaf(g.beta, *cp, o);
  *cp = o;
}

// ---- small M on the matrix cores, K split ---------------------------------
//
// For a few rows of A (at most one tile row) against a wide B in either
// storage: workgroup b takes tile b % tiles (tn = tile % tiles_n, tm =
// tile / tiles_n) over the K range [s*kps, min((s+1)*kps, K)) of split
// s = b / tiles, kps a multiple of the tile's K step.  That range is the
// whole K of a sub-problem whose A and B start kps*s values of k in, so
// tile_accumulate runs on it unchanged (the last split takes the ragged end
// of K).  The partial sums, rows < M and columns < N, go to ws[s][m][n]
// (rows of skinny_ws_stride(N) floats); skinny_reduce_kernel adds the
// splits in split order and applies alpha and beta.
template <class T, int MODE, bool TA, bool TB>
__global__ void __launch_bounds__(T::THREADS, T::OCC)
    mfma_splitk_kernel(GemmArgs g, int tiles_m, int tiles_n, int kps,
                       float* __restrict__ ws) {
  __shared__ __attribute__((aligned(1024))) float lds[TileLds<T, MODE>::FLOATS];
  const int tiles = tiles_m * tiles_n;
  const int split = blockIdx.x / tiles, tile = blockIdx.x - split * tiles;
  const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
  const int k0 = split * kps;
  GemmArgs sub = g;
  sub.K = g.K - k0 < kps ? g.K - k0 : kps;
  sub.A = g.A + (TA ? (size_t)k0 * g.lda : (size_t)k0);
  sub.B = g.B + (TB ? (size_t)k0 : (size_t)k0 * g.ldb);
  f32x16 acc[T::FM][T::FN];
  zero_acc<T>(acc);
  tile_accumulate<T, MODE, TA, TB>(sub, lds, tm * T::BM, tn * T::BN, 0,
                                   tile_k_steps<T>(sub.K), acc, acc);
  const WaveCoords<T> w;
  if (w.kg != 0) return;  // the first K group holds the tile's sums
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
}

}  // namespace sgemm
