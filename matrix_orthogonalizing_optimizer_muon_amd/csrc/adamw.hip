// AdamW for the parameters Muon does not take (the MuonClip page routes
// embeddings, the output head and 1-D parameters to AdamW without writing it
// out, so this is the standard decoupled form):
//   m <- b1 m + (1 - b1) g,  v <- b2 v + (1 - b2) g^2,
//   p <- p (1 - lr wd) - lr (m c1) / (sqrt(v c2) + eps),  c = 1 / (1 - b^t).
// One HBM pass over many tensors per launch (a block finds its tensor in the
// block prefix table), 16 elements per thread, fp32 math, one rounding of p.
#include "common.hpp"

namespace muon {

namespace {

__device__ __forceinline__ void adamw_one(float& p, float g, float& m, float& v, const AdamWLaunch& A) {
  m = fmaf(A.beta1, m, (1.0f - A.beta1) * g);
  v = fmaf(A.beta2, v, (1.0f - A.beta2) * (g * g));
  const float denom = sqrtf(v * A.c2) + A.eps;
  p = fmaf(-A.lr, (m * A.c1) / denom, p * A.decay);
}

// One block = kSpan consecutive elements of one tensor; thread t takes the
// 4-element groups at t*4 + c*1024 (c = 0..3), so each load instruction of a
// wave covers one contiguous run (1 KB of m or v) and each thread has all 16
// of its loads in flight before any arithmetic.
constexpr int kChunks = 4;
constexpr int kSpan = 256 * 4 * kChunks;

// Every byte is read once and written once per step: nontemporal loads and
// stores (6.01-6.05 -> 6.36 TB/s on 235M bf16 parameters, A/B on one box;
// the coalesced layout alone gave 1%).
template <typename T>
__device__ __forceinline__ T ld(const T* p) {
  return __builtin_nontemporal_load(p);
}
template <typename T>
__device__ __forceinline__ void st(T* p, T v) {
  __builtin_nontemporal_store(v, p);
}

template <typename PT>
__global__ __launch_bounds__(256) void adamw_kernel(AdamWLaunch A) {
  const int b = blockIdx.x;
  int t = 0;
  while (t + 1 < A.ntensors && b >= A.blk_start[t + 1]) ++t;
  const AdamWTensor& T = A.t[t];
  const int64_t base = static_cast<int64_t>(b - A.blk_start[t]) * kSpan;
  PT* P = static_cast<PT*>(T.p);
  const PT* G = static_cast<const PT*>(T.g);
  const int tid = threadIdx.x;
  if (T.vec && base + kSpan <= T.n) {
    float p[kChunks][4], g[kChunks][4];
    f32x4_t m[kChunks], v[kChunks];
    static_for<kChunks>([&](auto c) {
      constexpr int C = decltype(c)::value;
      const int64_t e = base + C * 1024 + tid * 4;
      m[C] = ld(reinterpret_cast<const f32x4_t*>(T.m + e));
      v[C] = ld(reinterpret_cast<const f32x4_t*>(T.v + e));
      if constexpr (sizeof(PT) == 2) {
        const u32x2_t pw = ld(reinterpret_cast<const u32x2_t*>(P + e));
        const u32x2_t gw = ld(reinterpret_cast<const u32x2_t*>(G + e));
        p[C][0] = bf16_to_f32(pw[0] & 0xffff); p[C][1] = bf16_to_f32(pw[0] >> 16);
        p[C][2] = bf16_to_f32(pw[1] & 0xffff); p[C][3] = bf16_to_f32(pw[1] >> 16);
        g[C][0] = bf16_to_f32(gw[0] & 0xffff); g[C][1] = bf16_to_f32(gw[0] >> 16);
        g[C][2] = bf16_to_f32(gw[1] & 0xffff); g[C][3] = bf16_to_f32(gw[1] >> 16);
      } else {
        const f32x4_t pw = ld(reinterpret_cast<const f32x4_t*>(P + e));
        const f32x4_t gw = ld(reinterpret_cast<const f32x4_t*>(G + e));
        static_for<4>([&](auto q) {
          constexpr int Q = decltype(q)::value;
          p[C][Q] = pw[Q];
          g[C][Q] = gw[Q];
        });
      }
    });
    static_for<kChunks>([&](auto c) {
      constexpr int C = decltype(c)::value;
      const int64_t e = base + C * 1024 + tid * 4;
      float mm[4], vv[4];
      static_for<4>([&](auto q) {
        constexpr int Q = decltype(q)::value;
        mm[Q] = m[C][Q];
        vv[Q] = v[C][Q];
        adamw_one(p[C][Q], g[C][Q], mm[Q], vv[Q], A);
      });
      st(reinterpret_cast<f32x4_t*>(T.m + e), f32x4_t{mm[0], mm[1], mm[2], mm[3]});
      st(reinterpret_cast<f32x4_t*>(T.v + e), f32x4_t{vv[0], vv[1], vv[2], vv[3]});
      if constexpr (sizeof(PT) == 2) {
        st(reinterpret_cast<u32x2_t*>(P + e), u32x2_t{pack2_bf16(p[C][0], p[C][1]), pack2_bf16(p[C][2], p[C][3])});
      } else {
        st(reinterpret_cast<f32x4_t*>(P + e), f32x4_t{p[C][0], p[C][1], p[C][2], p[C][3]});
      }
    });
  } else {
    // the tensor's last, partial block (or unaligned tensors): one element at a time
    for (int c = 0; c < kChunks; ++c) {
      for (int q = 0; q < 4; ++q) {
        const int64_t e = base + c * 1024 + tid * 4 + q;
        if (e >= T.n) continue;
        float p, g;
        if constexpr (sizeof(PT) == 2) {
          p = bf16_to_f32(reinterpret_cast<const bf16_t*>(P)[e]);
          g = bf16_to_f32(reinterpret_cast<const bf16_t*>(G)[e]);
        } else {
          p = P[e];
          g = G[e];
        }
        float m = T.m[e], v = T.v[e];
        adamw_one(p, g, m, v, A);
        T.m[e] = m;
        T.v[e] = v;
        if constexpr (sizeof(PT) == 2) reinterpret_cast<bf16_t*>(P)[e] = f32_to_bf16(p);
        else P[e] = p;
      }
    }
  }
}

}  // namespace

hipError_t launch_adamw(const AdamWLaunch& A, int dtype, int blocks, hipStream_t s) {
  if (dtype == MUON_DTYPE_BF16)
    hipLaunchKernelGGL(adamw_kernel<bf16_t>, dim3(blocks), dim3(256), 0, s, A);
  else
    hipLaunchKernelGGL(adamw_kernel<float>, dim3(blocks), dim3(256), 0, s, A);
  return hipGetLastError();
}

}  // namespace muon
