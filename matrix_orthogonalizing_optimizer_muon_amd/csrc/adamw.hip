// AdamW for the parameters Muon does not take (the MuonClip page routes
// embeddings, the output head and 1-D parameters to AdamW without writing it
// out, so this is the standard decoupled form):
//   m <- b1 m + (1 - b1) g,  v <- b2 v + (1 - b2) g^2,
//   p <- p (1 - lr wd) - lr (m c1) / (sqrt(v c2) + eps),  c = 1 / (1 - b^t).
// One HBM pass over many tensors per launch (a block finds its tensor in the
// block prefix table), 8 elements per thread, fp32 math, one rounding of p.
#include "common.hpp"

namespace muon {

namespace {

__device__ __forceinline__ void adamw_one(float& p, float g, float& m, float& v, const AdamWLaunch& A) {
  m = fmaf(A.beta1, m, (1.0f - A.beta1) * g);
  v = fmaf(A.beta2, v, (1.0f - A.beta2) * (g * g));
  const float denom = sqrtf(v * A.c2) + A.eps;
  p = fmaf(-A.lr, (m * A.c1) / denom, p * A.decay);
}

template <typename PT>
__global__ __launch_bounds__(256) void adamw_kernel(AdamWLaunch A) {
  const int b = blockIdx.x;
  int t = 0;
  while (t + 1 < A.ntensors && b >= A.blk_start[t + 1]) ++t;
  const AdamWTensor& T = A.t[t];
  const int64_t e0 = (static_cast<int64_t>(b - A.blk_start[t]) * 256 + threadIdx.x) * 8;
  if (e0 >= T.n) return;
  PT* P = static_cast<PT*>(T.p);
  const PT* G = static_cast<const PT*>(T.g);
  if (T.vec && e0 + 7 < T.n) {
    float p[8], g[8], m[8], v[8];
    const f32x4_t* m4 = reinterpret_cast<const f32x4_t*>(T.m + e0);
    const f32x4_t* v4 = reinterpret_cast<const f32x4_t*>(T.v + e0);
    const f32x4_t ma = m4[0], mb = m4[1], va = v4[0], vb = v4[1];
    if constexpr (sizeof(PT) == 2) {
      const u32x4_t pw = *reinterpret_cast<const u32x4_t*>(P + e0);
      const u32x4_t gw = *reinterpret_cast<const u32x4_t*>(G + e0);
      static_for<4>([&](auto q) {
        constexpr int Q = decltype(q)::value;
        p[2 * Q] = bf16_to_f32(pw[Q] & 0xffff);
        p[2 * Q + 1] = bf16_to_f32(pw[Q] >> 16);
        g[2 * Q] = bf16_to_f32(gw[Q] & 0xffff);
        g[2 * Q + 1] = bf16_to_f32(gw[Q] >> 16);
      });
    } else {
      const f32x4_t* p4 = reinterpret_cast<const f32x4_t*>(P + e0);
      const f32x4_t* g4 = reinterpret_cast<const f32x4_t*>(G + e0);
      const f32x4_t pa = p4[0], pb = p4[1], ga = g4[0], gb = g4[1];
      static_for<4>([&](auto q) {
        constexpr int Q = decltype(q)::value;
        p[Q] = pa[Q]; p[Q + 4] = pb[Q];
        g[Q] = ga[Q]; g[Q + 4] = gb[Q];
      });
    }
    static_for<4>([&](auto q) {
      constexpr int Q = decltype(q)::value;
      m[Q] = ma[Q]; m[Q + 4] = mb[Q];
      v[Q] = va[Q]; v[Q + 4] = vb[Q];
    });
    static_for<8>([&](auto q) {
      constexpr int Q = decltype(q)::value;
      adamw_one(p[Q], g[Q], m[Q], v[Q], A);
    });
    f32x4_t* mo = reinterpret_cast<f32x4_t*>(T.m + e0);
    f32x4_t* vo = reinterpret_cast<f32x4_t*>(T.v + e0);
    mo[0] = f32x4_t{m[0], m[1], m[2], m[3]};
    mo[1] = f32x4_t{m[4], m[5], m[6], m[7]};
    vo[0] = f32x4_t{v[0], v[1], v[2], v[3]};
    vo[1] = f32x4_t{v[4], v[5], v[6], v[7]};
    if constexpr (sizeof(PT) == 2) {
      u32x4_t pw;
      static_for<4>([&](auto q) {
        constexpr int Q = decltype(q)::value;
        pw[Q] = pack2_bf16(p[2 * Q], p[2 * Q + 1]);
      });
      *reinterpret_cast<u32x4_t*>(P + e0) = pw;
    } else {
      f32x4_t* p4 = reinterpret_cast<f32x4_t*>(P + e0);
      p4[0] = f32x4_t{p[0], p[1], p[2], p[3]};
      p4[1] = f32x4_t{p[4], p[5], p[6], p[7]};
    }
  } else {
    for (int q = 0; q < 8 && e0 + q < T.n; ++q) {
      const int64_t e = e0 + q;
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

}  // namespace

hipError_t launch_adamw(const AdamWLaunch& A, int dtype, int blocks, hipStream_t s) {
  if (dtype == MUON_DTYPE_BF16)
    hipLaunchKernelGGL(adamw_kernel<bf16_t>, dim3(blocks), dim3(256), 0, s, A);
  else
    hipLaunchKernelGGL(adamw_kernel<float>, dim3(blocks), dim3(256), 0, s, A);
  return hipGetLastError();
}

}  // namespace muon
