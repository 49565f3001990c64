// Matrix-core rate probe: bf16 MFMAs on register operands only, no memory
// traffic in the loop.  It measures the rate the chip sustains on its matrix
// cores at the clock it holds under that load, the reference point beside the
// 2.5 PFLOP/s dense bf16 figure of the specification.  Not part of the
// optimizer step.
//
// The rate depends on the operand bits: the matrix cores draw more power on
// random operands than on smooth ones, and the chip then holds a lower clock.
// Two operand kinds are offered:
//   MUON_PROBE_RANDOM  pseudo-random bf16 of both signs (a xorshift32 stream per
//                      lane), like the Newton-Schulz iterates;
//   MUON_PROBE_SMOOTH  small positive values that vary slowly across lanes.
// Each wave keeps eight fragment pairs and eight accumulators (32 x 32 blocks)
// and cycles through them, so consecutive MFMAs see different operands and no
// MFMA waits on the previous result.
#include "common.hpp"

namespace muon {

namespace {

constexpr int kProbeAcc = 8;   // independent accumulators per wave

template <int KIND>
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* sink) {
  const int tid = threadIdx.x;
  bf16x8_t a[kProbeAcc], b[kProbeAcc];
  uint32_t h = 0x9e3779b9u * static_cast<uint32_t>(tid + 1) + 0x85ebca6bu * static_cast<uint32_t>(blockIdx.x + 7);
  const float x = 1.0f + static_cast<float>(tid) * (1.0f / 1024.0f);
  auto next = [&]() {
    h ^= h << 13;
    h ^= h >> 17;
    h ^= h << 5;
    return static_cast<float>(h >> 8) * (1.0f / 16777216.0f) * 2.0f - 1.0f;   // uniform in [-1, 1)
  };
  static_for<kProbeAcc>([&](auto s) {
    constexpr int S = decltype(s)::value;
    static_for<8>([&](auto q) {
      constexpr int Q = decltype(q)::value;
      if (KIND == MUON_PROBE_RANDOM) {
        a[S][Q] = static_cast<__bf16>(0.05f * next());
        b[S][Q] = static_cast<__bf16>(0.05f * next());
      } else {
        a[S][Q] = static_cast<__bf16>(x * (Q + (S & 3) + 1) * 1e-3f);
        b[S][Q] = static_cast<__bf16>(x * (8 - Q + (S >> 2)) * 1e-3f);
      }
    });
  });
  f32x16_t acc[kProbeAcc];
  static_for<kProbeAcc>([&](auto c) { acc[decltype(c)::value] = f32x16_t{}; });
  for (int i = 0; i < iters; ++i) {
    // 32 MFMAs: accumulator c takes fragment pair (c + r) mod 8 in round r
    static_for<4 * kProbeAcc>([&](auto k) {
      constexpr int K = decltype(k)::value;
      constexpr int C = K % kProbeAcc, P = (K % kProbeAcc + K / kProbeAcc) % kProbeAcc;
      acc[C] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[P], b[(P + 3) % kProbeAcc], acc[C], 0, 0, 0);
    });
  }
  float s = 0.0f;
  static_for<kProbeAcc>([&](auto c) {
    static_for<16>([&](auto e) { s += acc[decltype(c)::value][decltype(e)::value]; });
  });
  if (tid == 0) sink[blockIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_probe(int blocks, int iters, int operands, float* sink, hipStream_t s) {
  if (operands == MUON_PROBE_RANDOM)
    hipLaunchKernelGGL(mfma_probe_kernel<MUON_PROBE_RANDOM>, dim3(blocks), dim3(256), 0, s, iters, sink);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<MUON_PROBE_SMOOTH>, dim3(blocks), dim3(256), 0, s, iters, sink);
  return hipGetLastError();
}

}  // namespace muon
