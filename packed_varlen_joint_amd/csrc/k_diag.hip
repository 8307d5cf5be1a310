// Diagnostic: the sustained bf16 matrix-core throughput of the whole chip, as
// the ceiling the attention kernels are measured against beside the published
// dense peak.  Every SIMD runs waves that issue only independent
// v_mfma_f32_32x32x16_bf16 (four accumulator chains, no memory in the loop) on
// operands derived from a seed.

#include "pvj_device.h"
#include "pvj_launch.h"

namespace pvj {

constexpr int kDiagThreads = 256;

__global__ __launch_bounds__(kDiagThreads) void mfma_peak_kernel(int iters, uint32_t seed,
                                                                float* __restrict__ sink) {
  f32x16 acc[4] = {};
  bf16x8 a, b;
  uint32_t x = seed ^ (blockIdx.x * 747796405u + threadIdx.x * 2891336453u);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x = x * 1664525u + 1013904223u;
    a[i] = (bf16)((float)(x >> 8) * (1.0f / 16777216.0f) - 0.5f);
    x = x * 1664525u + 1013904223u;
    b[i] = (bf16)((float)(x >> 8) * (1.0f / 16777216.0f) - 0.5f);
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 4; ++k) mma16(acc[k], a, b);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[k][j];
  sink[(size_t)blockIdx.x * kDiagThreads + threadIdx.x] = s;
}

// blocks: 2 workgroups of 4 waves per CU on 256 CUs, `rounds` times over
hipError_t launch_mfma_peak(int rounds, int iters, float* sink, double* flop, hipStream_t st) {
  const int blocks = 256 * 2 * rounds;
  *flop = (double)blocks * (kDiagThreads / 64) * iters * 4 * 32.0 * 32.0 * 16.0 * 2.0;
  mfma_peak_kernel<<<blocks, kDiagThreads, 0, st>>>(iters, 0x9e3779b9u, sink);
  return hipGetLastError();
}

}  // namespace pvj
