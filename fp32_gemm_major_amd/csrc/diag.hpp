// Diagnostic kernel: the sustained rate of v_mfma_f32_32x32x2_f32 on this
// device with no memory traffic.  Each wave keeps eight independent 32x32
// accumulators and issues `iters` rounds of eight MFMAs, so the matrix pipe
// always has independent work; the result is the ceiling a GEMM kernel can
// approach on the same clock.
#pragma once

#include <hip/hip_runtime.h>

namespace sgemm {

constexpr int kChainThreads = 256;  // 4 waves
constexpr int kChainAcc = 8;

__global__ void __launch_bounds__(kChainThreads)
    mfma_chain_kernel(float* __restrict__ out, int iters, float a0, float b0) {
  typedef float f32x16_t __attribute__((ext_vector_type(16)));
  f32x16_t acc[kChainAcc];
#pragma unroll
  for (int i = 0; i < kChainAcc; ++i) acc[i] = f32x16_t(0.0f);
  const float a = a0 + threadIdx.x * 1e-7f, b = b0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kChainAcc; ++i)
      acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[i], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kChainAcc; ++i) s += acc[i][threadIdx.x & 15];
  out[blockIdx.x * kChainThreads + threadIdx.x] = s;
}

}  // namespace sgemm
