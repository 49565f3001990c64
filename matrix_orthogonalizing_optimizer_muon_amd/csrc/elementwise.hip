// HBM-bound passes of the Muon step: the momentum/Nesterov/Frobenius pass,
// the per-matrix norm finalisation and the scaled, decayed parameter write.
//
// Momentum and lookahead follow "MuonClip", section 02 (M_t = mu M_{t-1} +
// G_t, with the Nesterov lookahead U = G_t + mu M_t); the Frobenius
// normalisation follows "Muon and MuonClip: orthogonalised updates for LLM
// training", Newton-Schulz subsection (X_0 = G / ||G||_F); the parameter write
// follows "MuonClip", section 03 (W_t = W_{t-1} - lr (scale O_t + wd W_{t-1})).
#include <utility>

#include "common.hpp"

namespace muon {

namespace {

constexpr int kTile = 64;      // momentum tile edge (original layout)
constexpr int kTrPitch = 66;   // LDS pitch of the transposed tile, bf16 units

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// One block = two horizontally adjacent 64 x 64 tiles of one matrix in its
// original layout (one at the end of an odd row of tiles), covering the
// zero-padded extent so that every byte of the padded Newton-Schulz inputs is
// written.  Writes M (in place), U rounded to bf16 in its own layout (D1) and
// transposed (D2), and each tile's sum of u^2.  When both tiles lie inside
// the matrix, all of their loads are issued first: each row of the pair is
// one contiguous 256-byte (G) and 512-byte (M) run.  Against one 64 x 64 tile
// per block: 5.51-5.57 -> 6.04-6.06 TB/s for the pass on the MuonClip layer
// (A/B on one box).
template <typename GT>
__global__ __launch_bounds__(256) void momentum_norm_kernel(MomentumLaunch L) {
  __shared__ __attribute__((aligned(16))) bf16_t tr[2][kTile * kTrPitch];
  __shared__ double wsum[2][4];

  int blk = blockIdx.x;
  int gi = 0;
  while (gi + 1 < L.ngroups && blk >= L.prefix[gi + 1]) ++gi;
  const MomentumGroup& g = L.g[gi];
  const int local = blk - L.prefix[gi];
  const int per_mat = g.tiles_r * g.pairs_c;
  const int mat = local / per_mat;
  const int t = local - mat * per_mat;
  const int tr_row = t / g.pairs_c, tc0 = 2 * (t - tr_row * g.pairs_c);
  const int ntile = min(2, g.tiles_c - tc0);
  const int i0 = tr_row * kTile;

  const GT* G = static_cast<const GT*>(g.G) + mat * g.bstride;
  float* M = g.M ? g.M + mat * g.bstride : nullptr;
  bf16_t* D1 = g.D1 + mat * g.d_stride;
  bf16_t* D2 = g.D2 + mat * g.d_stride;

  const int tid = threadIdx.x;
  const int c0 = (tid & 15) * 4;
  const int rsub = tid >> 4;
  const float mu = L.mu;
  double ss[2] = {0.0, 0.0};

  // stores U of one 4-element row segment of tile h (own layout + the LDS
  // tile for the transposed copy) and accumulates its squares.  The
  // own-layout copy is stored nontemporally: 5.42 -> 5.58 TB/s for the pass
  // on the MuonClip layer (three tall matrices, one wide); nontemporal stores
  // of the transposed copy (its 16-byte rows written from LDS) cost 10%.
  auto emit = [&](int h, int r, const float (&u)[4]) {
    const int j0 = (tc0 + h) * kTile;
    bf16_t ub[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ss[h] += static_cast<double>(u[q]) * static_cast<double>(u[q]);
      ub[q] = f32_to_bf16(u[q]);
      tr[h][(c0 + q) * kTrPitch + r] = ub[q];
    }
    uint2 packed;
    packed.x = static_cast<uint32_t>(ub[0]) | (static_cast<uint32_t>(ub[1]) << 16);
    packed.y = static_cast<uint32_t>(ub[2]) | (static_cast<uint32_t>(ub[3]) << 16);
    __builtin_nontemporal_store(u32x2_t{packed.x, packed.y}, reinterpret_cast<u32x2_t*>(D1 + static_cast<int64_t>(i0 + r) * g.cp + j0 + c0));
  };
  auto inside = [&](int h) {
    return h < ntile && g.vec && (i0 + kTile <= g.rows) && ((tc0 + h + 1) * kTile <= g.cols);
  };
  // Tiles wholly inside the matrix: every load first (16 per tile and thread
  // in flight), then compute and store.  G and M are read once per step:
  // nontemporal loads (M is also written back nontemporally) measured 5.1 ->
  // 5.4 TB/s for this pass.
  // (HM: momentum present; a compile-time choice, so that no branch separates
  // the loads and each wave has all of them in flight)
  auto interior = [&](auto nt, int h0, auto hm) {
    constexpr int NT = decltype(nt)::value;   // tiles handled together, from tile h0
    constexpr bool HM = decltype(hm)::value;
    float gv[NT][4][4], mv[NT][4][4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
#pragma unroll
      for (int hh = 0; hh < NT; ++hh) {
        const int64_t e = static_cast<int64_t>(i0 + rsub + 16 * p) * g.cols + (tc0 + h0 + hh) * kTile + c0;
        if constexpr (sizeof(GT) == 2) {
          const u32x2_t rawv = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(G + e));
          gv[hh][p][0] = bf16_to_f32(rawv[0] & 0xffff);
          gv[hh][p][1] = bf16_to_f32(rawv[0] >> 16);
          gv[hh][p][2] = bf16_to_f32(rawv[1] & 0xffff);
          gv[hh][p][3] = bf16_to_f32(rawv[1] >> 16);
        } else {
          const float4 raw = *reinterpret_cast<const float4*>(G + e);
          gv[hh][p][0] = raw.x; gv[hh][p][1] = raw.y; gv[hh][p][2] = raw.z; gv[hh][p][3] = raw.w;
        }
        if constexpr (HM) {
          const f32x4_t m4v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(M + e));
          mv[hh][p][0] = m4v[0]; mv[hh][p][1] = m4v[1]; mv[hh][p][2] = m4v[2]; mv[hh][p][3] = m4v[3];
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < NT; ++hh) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int r = rsub + 16 * p;
        float u[4];
        if constexpr (HM) {
          float mn[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            mn[q] = fmaf(mu, mv[hh][p][q], gv[hh][p][q]);
            u[q] = L.nesterov ? fmaf(mu, mn[q], gv[hh][p][q]) : mn[q];
          }
          const int64_t e = static_cast<int64_t>(i0 + r) * g.cols + (tc0 + h0 + hh) * kTile + c0;
          f32x4_t mo = {mn[0], mn[1], mn[2], mn[3]};
          __builtin_nontemporal_store(mo, reinterpret_cast<f32x4_t*>(M + e));
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) u[q] = gv[hh][p][q];
        }
        emit(h0 + hh, r, u);
      }
    }
  };
  // a tile crossing the matrix edge (zero beyond it), one element at a time
  auto edge = [&](int h) {
    const int j0 = (tc0 + h) * kTile;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = rsub + 16 * p;
      const int i = i0 + r;
      float u[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = j0 + c0 + q;
        u[q] = 0.0f;
        if (i < g.rows && j < g.cols) {
          const int64_t e = static_cast<int64_t>(i) * g.cols + j;
          float gvs;
          if constexpr (sizeof(GT) == 2) gvs = bf16_to_f32(reinterpret_cast<const bf16_t*>(G)[e]);
          else gvs = static_cast<float>(G[e]);
          if (M) {
            const float mn = fmaf(mu, M[e], gvs);
            M[e] = mn;
            u[q] = L.nesterov ? fmaf(mu, mn, gvs) : mn;
          } else {
            u[q] = gvs;
          }
        }
      }
      emit(h, r, u);
    }
  };
  using Pair = std::integral_constant<int, 2>;
  using Single = std::integral_constant<int, 1>;
  if (inside(0) && inside(1)) {
    if (M) interior(Pair{}, 0, std::true_type{});
    else interior(Pair{}, 0, std::false_type{});
  } else {
    for (int h = 0; h < ntile; ++h) {
      if (!inside(h)) edge(h);
      else if (M) interior(Single{}, h, std::true_type{});
      else interior(Single{}, h, std::false_type{});
    }
  }

  for (int h = 0; h < 2; ++h) {
    const double w = wave_sum(ss[h]);
    if ((tid & 63) == 0) wsum[h][tid >> 6] = w;
  }
  __syncthreads();

  // Transposed tiles: row jj of D2 (original column j0 + jj), 16 consecutive
  // original rows per thread.
  for (int h = 0; h < ntile; ++h) {
    const int jj = tid >> 2;
    const int ii = (tid & 3) * 16;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(tr[h] + jj * kTrPitch + ii);
    uint32_t w[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) w[q] = src[q];
    bf16_t* dst = D2 + static_cast<int64_t>((tc0 + h) * kTile + jj) * g.rp + i0 + ii;
    reinterpret_cast<uint4*>(dst)[0] = make_uint4(w[0], w[1], w[2], w[3]);
    reinterpret_cast<uint4*>(dst)[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
  if (tid < ntile) {
    g.partials[static_cast<int64_t>(mat) * g.tiles_per_mat + tr_row * g.tiles_c + tc0 + tid] =
        ((wsum[tid][0] + wsum[tid][1]) + wsum[tid][2]) + wsum[tid][3];
  }
}

// One block per matrix: fixed-order sum of the tile partials (each thread a
// strided slice, four independent accumulators so the loads overlap, then a
// fixed tree over threads), then 1 / (sqrt(sum) + eps).
__global__ __launch_bounds__(256) void norm_finalize_kernel(FinalizeLaunch L) {
  __shared__ double red[4];
  const int blk = blockIdx.x;
  int gi = 0;
  while (gi + 1 < L.ngroups && blk >= L.prefix[gi + 1]) ++gi;
  const int mat = blk - L.prefix[gi];
  const int n = L.tiles_per_mat[gi];
  const double* p = L.partials[gi] + static_cast<int64_t>(mat) * n;
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
  int k = threadIdx.x;
  for (; k + 768 < n; k += 1024) {
    s0 += p[k];
    s1 += p[k + 256];
    s2 += p[k + 512];
    s3 += p[k + 768];
  }
  for (; k < n; k += 256) s0 += p[k];
  double s = wave_sum((s0 + s1) + (s2 + s3));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double tot = (red[0] + red[1]) + (red[2] + red[3]);
    L.inv_norm[gi][mat] = static_cast<float>(1.0 / (sqrt(tot) + static_cast<double>(L.eps)));
  }
}

// W <- decay * W - step * O over one group; 8 elements per thread.
template <typename WT>
__global__ __launch_bounds__(256) void param_update_kernel(UpdateLaunch L) {
  const int64_t blk = blockIdx.x;
  int gi = 0;
  while (gi + 1 < L.ngroups && blk >= L.prefix[gi + 1]) ++gi;
  const UpdateGroup& g = L.g[gi];
  const int64_t local = blk - L.prefix[gi];
  const int64_t per_mat = g.blocks / g.batch;
  const int mat = static_cast<int>(local / per_mat);
  const int64_t e0 = (local - mat * per_mat) * 2048 + threadIdx.x * 8;
  const int64_t n = static_cast<int64_t>(g.rows) * g.cols;
  if (e0 >= n) return;
  WT* W = static_cast<WT*>(g.W) + mat * g.bstride;
  const bf16_t* O = g.O + mat * g.o_bstride;
  const float decay = g.decay, step = g.step;
  if (g.vec && e0 + 7 < n) {
    // O and W are read once: nontemporal loads (6.2 -> 6.7 TB/s, bf16 W)
    const int i = static_cast<int>(e0 / g.cols), j = static_cast<int>(e0 - static_cast<int64_t>(i) * g.cols);
    const u32x4_t ovv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(O + static_cast<int64_t>(i) * g.o_ld + j));
    const uint4 ov = make_uint4(ovv[0], ovv[1], ovv[2], ovv[3]);
    float o[8];
    o[0] = bf16_to_f32(ov.x & 0xffff); o[1] = bf16_to_f32(ov.x >> 16);
    o[2] = bf16_to_f32(ov.y & 0xffff); o[3] = bf16_to_f32(ov.y >> 16);
    o[4] = bf16_to_f32(ov.z & 0xffff); o[5] = bf16_to_f32(ov.z >> 16);
    o[6] = bf16_to_f32(ov.w & 0xffff); o[7] = bf16_to_f32(ov.w >> 16);
    if constexpr (sizeof(WT) == 2) {
      const u32x4_t wvv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(W + e0));
      uint4 wv = make_uint4(wvv[0], wvv[1], wvv[2], wvv[3]);
      uint32_t* wp = reinterpret_cast<uint32_t*>(&wv);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = fmaf(-step, o[2 * q], decay * bf16_to_f32(wp[q] & 0xffff));
        const float hi = fmaf(-step, o[2 * q + 1], decay * bf16_to_f32(wp[q] >> 16));
        wp[q] = pack2_bf16(lo, hi);
      }
      *reinterpret_cast<uint4*>(W + e0) = wv;
    } else {
      float4* wp = reinterpret_cast<float4*>(W + e0);
      float4 a = wp[0], b = wp[1];
      a.x = fmaf(-step, o[0], decay * a.x); a.y = fmaf(-step, o[1], decay * a.y);
      a.z = fmaf(-step, o[2], decay * a.z); a.w = fmaf(-step, o[3], decay * a.w);
      b.x = fmaf(-step, o[4], decay * b.x); b.y = fmaf(-step, o[5], decay * b.y);
      b.z = fmaf(-step, o[6], decay * b.z); b.w = fmaf(-step, o[7], decay * b.w);
      wp[0] = a; wp[1] = b;
    }
  } else {
    for (int q = 0; q < 8; ++q) {
      const int64_t e = e0 + q;
      if (e >= n) break;
      const int i = static_cast<int>(e / g.cols), j = static_cast<int>(e - static_cast<int64_t>(i) * g.cols);
      const float o = bf16_to_f32(O[static_cast<int64_t>(i) * g.o_ld + j]);
      if constexpr (sizeof(WT) == 2) {
        bf16_t* w = reinterpret_cast<bf16_t*>(W) + e;
        *w = f32_to_bf16(fmaf(-step, o, decay * bf16_to_f32(*w)));
      } else {
        W[e] = fmaf(-step, o, decay * W[e]);
      }
    }
  }
}

}  // namespace

hipError_t launch_momentum_norm(const MomentumLaunch& L, int grad_dtype, int nblocks, hipStream_t s) {
  if (grad_dtype == MUON_DTYPE_BF16)
    hipLaunchKernelGGL(momentum_norm_kernel<bf16_t>, dim3(nblocks), dim3(256), 0, s, L);
  else
    hipLaunchKernelGGL(momentum_norm_kernel<float>, dim3(nblocks), dim3(256), 0, s, L);
  return hipGetLastError();
}

hipError_t launch_norm_finalize(const FinalizeLaunch& L, int nmats, hipStream_t s) {
  hipLaunchKernelGGL(norm_finalize_kernel, dim3(nmats), dim3(256), 0, s, L);
  return hipGetLastError();
}

hipError_t launch_param_update(const UpdateLaunch& L, int param_dtype, int64_t nblocks, hipStream_t s) {
  if (param_dtype == MUON_DTYPE_BF16)
    hipLaunchKernelGGL(param_update_kernel<bf16_t>, dim3(static_cast<unsigned>(nblocks)), dim3(256), 0, s, L);
  else
    hipLaunchKernelGGL(param_update_kernel<float>, dim3(static_cast<unsigned>(nblocks)), dim3(256), 0, s, L);
  return hipGetLastError();
}

}  // namespace muon
