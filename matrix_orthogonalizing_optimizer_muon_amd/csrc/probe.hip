// Matrix-core rate probe: bf16 MFMAs on register operands only, no memory
// traffic in the loop.  It measures the rate the chip sustains on its matrix
// cores at the clock it holds under that load, the reference point beside the
// 2.5 PFLOP/s dense bf16 figure of the specification.  Not part of the
// optimizer step.
#include "common.hpp"

namespace muon {

namespace {

constexpr int kProbeChains = 4;   // independent accumulators per wave

__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* sink) {
  // operands that depend on the lane, so nothing folds at compile time
  const float x = 1.0f + static_cast<float>(threadIdx.x) * (1.0f / 1024.0f);
  bf16x8_t a, b;
  static_for<8>([&](auto q) {
    constexpr int Q = decltype(q)::value;
    a[Q] = static_cast<__bf16>(x * (Q + 1) * 1e-3f);
    b[Q] = static_cast<__bf16>(x * (8 - Q) * 1e-3f);
  });
  f32x16_t acc[kProbeChains];
  static_for<kProbeChains>([&](auto c) { acc[decltype(c)::value] = f32x16_t{}; });
  for (int i = 0; i < iters; ++i) {
    static_for<kProbeChains>([&](auto c) {
      constexpr int C = decltype(c)::value;
      acc[C] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[C], 0, 0, 0);
    });
  }
  float s = 0.0f;
  static_for<kProbeChains>([&](auto c) {
    static_for<16>([&](auto e) { s += acc[decltype(c)::value][decltype(e)::value]; });
  });
  if (threadIdx.x == 0) sink[blockIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_probe(int blocks, int iters, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, s, iters, sink);
  return hipGetLastError();
}

}  // namespace muon
