// Measurement kernel: the sustained bf16 MFMA rate of the chip with no memory
// traffic, the practical ceiling against which the Newton-Schulz products are
// read (under sustained MFMA load the clock settles well below the one at
// which the dense peak is quoted).  Each of 8 waves per workgroup keeps eight
// independent 32x32 fp32 accumulators and issues the same
// v_mfma_f32_32x32x16_bf16 that the products use, 8 per iteration, on
// operands whose bits change every iteration (xorshift-seeded, exponents kept
// small so that every value stays finite), as real data does.  One float per
// wave (the sum of its accumulators) is stored, so that nothing is optimized
// away.
#pragma once

#include "common.hpp"

namespace mfsdp {

constexpr int kProbeThreads = 512;
constexpr int kProbeMfmaPerIter = 8;

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(float* __restrict__ out,
                                                                   int iters) {
  const int tid = threadIdx.x;
  f32x16_t acc[kProbeMfmaPerIter];
#pragma unroll
  for (int j = 0; j < kProbeMfmaPerIter; ++j) acc[j] = f32x16_t{};
  u32x4_t ai[4], bi[4];
  uint32_t x = 0x9E3779B9u * static_cast<uint32_t>(tid + 1) + blockIdx.x;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x ^= x << 13; x ^= x >> 17; x ^= x << 5;
      ai[j][k] = x & 0x3fff3fffu;   // bf16 pairs of magnitude < 2
      x ^= x << 13; x ^= x >> 17; x ^= x << 5;
      bi[j][k] = x & 0x3fff3fffu;
    }
  }
  for (int it = 0; it < iters; ++it) {
    // flips mantissa and low exponent bits (never bit 14, the top exponent
    // bit, nor the sign): every value stays positive and below 2
    const uint32_t flip = 0x00550055u * static_cast<uint32_t>(it & 7);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ai[j] ^= flip;
      bi[j] ^= flip << 1;
    }
#pragma unroll
    for (int j = 0; j < kProbeMfmaPerIter; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8_t, ai[j & 3]), __builtin_bit_cast(bf16x8_t, bi[(j >> 1) & 3]),
          acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kProbeMfmaPerIter; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  if ((tid & 63) == 0) out[static_cast<size_t>(blockIdx.x) * (kProbeThreads / 64) + (tid >> 6)] = s;
}

}  // namespace mfsdp
