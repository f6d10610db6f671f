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

// The same chain for 16-bit inputs: v_mfma_f32_32x32x16_bf16 (DT16 = 1) or
// v_mfma_f32_32x32x16_f16 (DT16 = 2), 32768 flops per MFMA per wave; and for
// 8-bit inputs, v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales on E4M3
// (DT16 = 3) or E5M2 (DT16 = 4), 131072 flops per MFMA per wave.
template <int DT16>
__global__ void __launch_bounds__(kChainThreads)
    mfma_chain16_kernel(float* __restrict__ out, int iters) {
  typedef float f32x16_t __attribute__((ext_vector_type(16)));
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
  typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
  typedef int i32x8_t __attribute__((ext_vector_type(8)));
  f32x16_t acc[kChainAcc];
#pragma unroll
  for (int i = 0; i < kChainAcc; ++i) acc[i] = f32x16_t(0.0f);
  // small finite values in both formats (0x3C00 + lane bits: about 1)
  const unsigned w = 0x3C003C00u | (threadIdx.x & 7u);
  const u32x4_t x = {w, w, w, w};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kChainAcc; ++i) {
      if constexpr (DT16 == 1) {
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, x), __builtin_bit_cast(bf16x8_t, x), acc[i], 0,
            0, 0);
      } else if constexpr (DT16 == 2) {
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
            __builtin_bit_cast(f16x8_t, x), __builtin_bit_cast(f16x8_t, x), acc[i], 0, 0,
            0);
      } else {
        // (the bytes 0x00 and 0x3C are finite in both 8-bit formats)
        const i32x8_t y = {(int)w, (int)w, (int)w, (int)w, (int)w, (int)w, (int)w, (int)w};
        acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            y, y, acc[i], DT16 == 3 ? 0 : 1, DT16 == 3 ? 0 : 1, 0, 127, 0, 127);
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kChainAcc; ++i) s += acc[i][threadIdx.x & 15];
  out[blockIdx.x * kChainThreads + threadIdx.x] = s;
}

}  // namespace sgemm
