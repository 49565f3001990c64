// Matrix-core rate probe: bf16 MFMAs on register operands only, no memory
// traffic in the loop (and, at the end of the file, an HBM stream probe).  It measures the rate the chip sustains on its matrix
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

// HBM stream probe: unit u of a launch reads R 16-byte chunks of src and
// writes W 16-byte chunks of dst, chunk i of every unit side by side
// (src[i * units + u]), so each load and store instruction of a wave covers
// 1 KB of consecutive bytes.  A thread takes U units 256 apart and issues
// all of their loads before any store (R * U loads in flight).  Loads and
// stores are nontemporal, as in the optimizer's passes.  Stored chunk k is
// the XOR of the unit's loads with k in its first word, so no load can be
// dropped.
template <int R, int W, int U>
__global__ __launch_bounds__(256) void hbm_probe_kernel(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                        int64_t units) {
  const int64_t u0 = static_cast<int64_t>(blockIdx.x) * (256 * U) + threadIdx.x;
  u32x4_t v[U][R];
  static_for<U>([&](auto j) {
    const int64_t u = min(u0 + 256 * decltype(j)::value, units - 1);   // the tail reloads the last unit
    static_for<R>([&](auto i) {
      v[decltype(j)::value][decltype(i)::value] = __builtin_nontemporal_load(src + decltype(i)::value * units + u);
    });
  });
  static_for<U>([&](auto j) {
    constexpr int J = decltype(j)::value;
    const int64_t u = u0 + 256 * J;
    if (u >= units) return;
    u32x4_t x = v[J][0];
    static_for<R - 1>([&](auto i) { x ^= v[J][decltype(i)::value + 1]; });
    static_for<W>([&](auto k) {
      u32x4_t y = x;
      y[0] ^= static_cast<uint32_t>(decltype(k)::value);
      __builtin_nontemporal_store(y, dst + decltype(k)::value * units + u);
    });
  });
}

}  // namespace

template <int R, int W>
hipError_t launch_hbm_mix(const u32x4_t* in, u32x4_t* out, int64_t units, int unroll, hipStream_t s) {
  const dim3 block(256);
  if (unroll == 1)
    hipLaunchKernelGGL((hbm_probe_kernel<R, W, 1>), dim3(static_cast<unsigned>((units + 255) / 256)), block, 0, s,
                       in, out, units);
  else
    hipLaunchKernelGGL((hbm_probe_kernel<R, W, 4>), dim3(static_cast<unsigned>((units + 1023) / 1024)), block, 0, s,
                       in, out, units);
  return hipGetLastError();
}

hipError_t launch_hbm_probe(const void* src, void* dst, int64_t units, int reads, int writes, int unroll,
                            hipStream_t s) {
  const u32x4_t* in = static_cast<const u32x4_t*>(src);
  u32x4_t* out = static_cast<u32x4_t*>(dst);
  if (reads == 1 && writes == 1) return launch_hbm_mix<1, 1>(in, out, units, unroll, s);
  if (reads == 3 && writes == 4) return launch_hbm_mix<3, 4>(in, out, units, unroll, s);
  if (reads == 2 && writes == 1) return launch_hbm_mix<2, 1>(in, out, units, unroll, s);
  return hipErrorInvalidValue;
}

hipError_t launch_mfma_probe(int blocks, int iters, int operands, float* sink, hipStream_t s) {
  if (operands == MUON_PROBE_RANDOM)
    hipLaunchKernelGGL(mfma_probe_kernel<MUON_PROBE_RANDOM>, dim3(blocks), dim3(256), 0, s, iters, sink);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<MUON_PROBE_SMOOTH>, dim3(blocks), dim3(256), 0, s, iters, sink);
  return hipGetLastError();
}

}  // namespace muon
