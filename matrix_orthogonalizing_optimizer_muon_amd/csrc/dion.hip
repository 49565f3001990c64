// Dion's rank-r step ("About Muon: Muon At Scale", section "What Breaks at
// Scale", subsection "The Matrix Does Not Fit"), per matrix:
//   B = M + G;  P = orth(B Q);  R = B^T P;
//   M <- B - (1 - mu) P R^T;  Q <- ColNorm(R);  W <- W - lr P Q^T
// orth is Cholesky-QR applied twice: the Gram matrix P^T P is summed in fp64
// over row chunks, factored and inverted in fp64 inside one workgroup's LDS,
// and P <- P L^-T runs as an fp32 product; the second pass restores the
// orthogonality the first loses to fp32 rounding (about cond(B Q) x 1e-7).
//
// Every product is an fp32 MFMA GEMM (v_mfma_f32_32x32x2_f32) on 64 x 64
// output tiles, 4 waves of 32 x 32, K staged 32 at a time through LDS (k-major,
// so a wave's fragment reads are consecutive floats), the next chunk's global
// loads in flight during the current chunk's MFMAs.  B = M + G is formed while
// staging, never stored.  The modes differ only in how operands are fetched:
//   BQ   P0 = B Q        A = B rows (k = columns of B), B op = Q rows
//   PL   P  = P0 L^-T    A = P0 rows, B op = rows of L^-T
//   BTP  R  = B^T P      A = columns of B (k = rows of B), B op = P rows
//   UPD  M <- B - (1-mu) P R^T and W <- W - lr P diag(1/|R_c|) R^T: A = P rows
//        (and P scaled by the column norms), B op = R rows (k = rank index)
#include "common.hpp"

namespace muon {

namespace {

constexpr int kDT = 64;        // output tile edge
constexpr int kDK = 32;        // k chunk
constexpr int kDP = kDT + 4;   // LDS row pitch (floats)
constexpr int kGramRows = 128; // rows of P per Gram partial
constexpr int kMaxRank = 128;

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(w[q] << 16);
      v[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
    }
  } else {
    const f32x4_t a = reinterpret_cast<const f32x4_t*>(p)[0];
    const f32x4_t b = reinterpret_cast<const f32x4_t*>(p)[1];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[q] = a[q];
      v[4 + q] = b[q];
    }
  }
}

__device__ __forceinline__ void zero8(float (&v)[8]) {
#pragma unroll
  for (int q = 0; q < 8; ++q) v[q] = 0.0f;
}

template <typename T, int MODE>
__global__ __launch_bounds__(256) void dion_gemm_kernel(DionArgs a) {
  __shared__ __attribute__((aligned(16))) float As[kDK * kDP];
  __shared__ __attribute__((aligned(16))) float As2[(MODE == DION_UPD ? kDK : 1) * kDP];
  __shared__ __attribute__((aligned(16))) float Bs[kDK * kDP];

  const int mat = blockIdx.z;
  const int row0 = blockIdx.y * kDT, col0 = blockIdx.x * kDT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int m = a.m, n = a.n, rp = a.rp;
  const int K = (MODE == DION_BQ) ? n : (MODE == DION_BTP ? m : rp);

  const float* M = a.M + mat * a.bstride;
  const T* G = static_cast<const T*>(a.G) + mat * a.bstride;
  const float* Q = a.Q + mat * a.q_stride;
  const float* Asrc = a.src + mat * a.src_stride;
  const float* Bsrc = a.bsrc + mat * a.bsrc_stride;
  const float* inv = a.inv + mat * rp;

  // staging maps.  Row-major A (k contiguous): thread -> row t/4, k 8 (t%4).
  // k-major operands (index contiguous): thread -> k t/8, index 8 (t%8).
  const int ar = tid >> 2, ak = (tid & 3) * 8;
  const int bk = tid >> 3, bc = (tid & 7) * 8;
  float va[8], vb[8];
  auto load = [&](int k0) {
    if constexpr (MODE == DION_BQ) {
      const int i = row0 + ar, k = k0 + ak;
      if (i < m && k < n) {
        const int64_t e = static_cast<int64_t>(i) * n + k;
        float g[8];
        load8(M + e, va);
        load8(G + e, g);
#pragma unroll
        for (int q = 0; q < 8; ++q) va[q] += g[q];
      } else {
        zero8(va);
      }
      const int kb = k0 + bk, c = col0 + bc;
      if (kb < n && c < a.r) load8(Q + static_cast<int64_t>(kb) * a.r + c, vb);
      else zero8(vb);
    } else if constexpr (MODE == DION_PL) {
      const int i = row0 + ar;
      if (i < m) load8(Asrc + static_cast<int64_t>(i) * rp + k0 + ak, va);
      else zero8(va);
      const int c = col0 + bc;
      if (c < rp) load8(Bsrc + static_cast<int64_t>(k0 + bk) * rp + c, vb);
      else zero8(vb);
    } else if constexpr (MODE == DION_BTP) {
      // A[j][k] = B[k][j]: rows k of B, 8 consecutive j
      const int k = k0 + bk, j = row0 + bc;
      if (k < m && j < n) {
        const int64_t e = static_cast<int64_t>(k) * n + j;
        float g[8];
        load8(M + e, va);
        load8(G + e, g);
#pragma unroll
        for (int q = 0; q < 8; ++q) va[q] += g[q];
      } else {
        zero8(va);
      }
      const int c = col0 + bc;
      if (k < m && c < rp) load8(Bsrc + static_cast<int64_t>(k) * rp + c, vb);
      else zero8(vb);
    } else {  // DION_UPD
      const int i = row0 + ar;
      if (i < m) load8(Asrc + static_cast<int64_t>(i) * rp + k0 + ak, va);
      else zero8(va);
      const int j = col0 + ar;   // R rows j, k = rank index contiguous
      if (j < n) load8(Bsrc + static_cast<int64_t>(j) * rp + k0 + ak, vb);
      else zero8(vb);
    }
  };
  auto store = [&](int k0) {
    if constexpr (MODE == DION_BTP) {
#pragma unroll
      for (int q = 0; q < 8; ++q) As[bk * kDP + bc + q] = va[q];
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) As[(ak + q) * kDP + ar] = va[q];
      if constexpr (MODE == DION_UPD) {
#pragma unroll
        for (int q = 0; q < 8; ++q) As2[(ak + q) * kDP + ar] = va[q] * inv[k0 + ak + q];
      }
    }
    if constexpr (MODE == DION_UPD) {
#pragma unroll
      for (int q = 0; q < 8; ++q) Bs[(ak + q) * kDP + ar] = vb[q];
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) Bs[bk * kDP + bc + q] = vb[q];
    }
  };

  f32x16_t acc = f32x16_t{}, acc2 = f32x16_t{};
  const int nk = (K + kDK - 1) / kDK;
  const int fr = lane & 31, fk = lane >> 5;
  load(0);
  for (int kc = 0; kc < nk; ++kc) {
    lds_barrier();                 // every wave is done with the previous chunk
    store(kc * kDK);
    lds_barrier();
    if (kc + 1 < nk) load((kc + 1) * kDK);
#pragma unroll
    for (int s = 0; s < kDK / 2; ++s) {
      const int kr = 2 * s + fk;
      const float bv = Bs[kr * kDP + wc * 32 + fr];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(As[kr * kDP + wr * 32 + fr], bv, acc, 0, 0, 0);
      if constexpr (MODE == DION_UPD)
        acc2 = __builtin_amdgcn_mfma_f32_32x32x2f32(As2[kr * kDP + wr * 32 + fr], bv, acc2, 0, 0, 0);
    }
  }

  // epilogue: acc[e] is element (wr 32 + 8 (e/4) + 4 (lane/32) + e%4, wc 32 + lane%32)
  const int erow = row0 + wr * 32 + 4 * fk, ecol = col0 + wc * 32 + fr;
  if constexpr (MODE == DION_UPD) {
    if (ecol < n) {
      T* W = static_cast<T*>(a.W) + mat * a.bstride;
      float* Mw = a.M + mat * a.bstride;
      const float keep = 1.0f - a.mu;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int i = erow + 8 * (e >> 2) + (e & 3);
        if (i < m) {
          const int64_t idx = static_cast<int64_t>(i) * n + ecol;
          float g;
          if constexpr (sizeof(T) == 2) g = bf16_to_f32(G[idx]);
          else g = G[idx];
          const float b = Mw[idx] + g;
          Mw[idx] = fmaf(-keep, acc[e], b);
          if constexpr (sizeof(T) == 2) W[idx] = f32_to_bf16(fmaf(-a.lr, acc2[e], bf16_to_f32(W[idx])));
          else W[idx] = fmaf(-a.lr, acc2[e], W[idx]);
        }
      }
    }
  } else {
    const int nrows = (MODE == DION_BTP) ? n : m;
    float* D = a.dst + mat * a.dst_stride;
    if (ecol < rp) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int i = erow + 8 * (e >> 2) + (e & 3);
        if (i < nrows) D[static_cast<int64_t>(i) * rp + ecol] = acc[e];
      }
    }
  }
}

// Partial Gram matrix of rows [128 s, 128 s + 128) of P (fp32 [m][rp]) in
// fp64 (products of two fp32 values are exact in fp64): grid (nsplit, batch).
// Thread t owns the 8 x 8 block (x0, y0) = 8 (t / 16, t % 16) of the rp x rp
// result (blocks beyond rp idle), so each row of P gives 64 FMAs per 16 reads.
__global__ __launch_bounds__(256) void dion_gram_kernel(DionArgs a) {
  __shared__ __attribute__((aligned(16))) float Ps[kGramRows * kMaxRank];
  const int s = blockIdx.x, mat = blockIdx.y, tid = threadIdx.x;
  const int rp = a.rp, m = a.m;
  const float* P = a.src + mat * a.src_stride;
  const int i0 = s * kGramRows;
  for (int e = tid; e < kGramRows * rp; e += 256) {
    const int i = e / rp;
    Ps[e] = (i0 + i < m) ? P[static_cast<int64_t>(i0) * rp + e] : 0.0f;
  }
  __syncthreads();
  const int x0 = 8 * (tid >> 4), y0 = 8 * (tid & 15);
  if (x0 >= rp || y0 >= rp) return;
  double acc[8][8];
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int v = 0; v < 8; ++v) acc[u][v] = 0.0;
  for (int i = 0; i < kGramRows; ++i) {
    const float* row = Ps + i * rp;
    const f32x4_t xa = *reinterpret_cast<const f32x4_t*>(row + x0);
    const f32x4_t xb = *reinterpret_cast<const f32x4_t*>(row + x0 + 4);
    const f32x4_t ya = *reinterpret_cast<const f32x4_t*>(row + y0);
    const f32x4_t yb = *reinterpret_cast<const f32x4_t*>(row + y0 + 4);
    double xv[8], yv[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      xv[q] = xa[q];
      xv[4 + q] = xb[q];
      yv[q] = ya[q];
      yv[4 + q] = yb[q];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int v = 0; v < 8; ++v) acc[u][v] = fma(xv[u], yv[v], acc[u][v]);
  }
  double* out = a.gram + mat * a.gram_stride + static_cast<int64_t>(s) * rp * rp;
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int v = 0; v < 8; ++v) out[(x0 + u) * rp + y0 + v] = acc[u][v];
}

// S = the sum of a matrix's Gram partials in a fixed order, one entry per
// thread: grid (ceil(rp^2 / 256), batch).  Written to partial 0.
__global__ __launch_bounds__(256) void dion_gram_reduce_kernel(DionArgs a) {
  const int mat = blockIdx.y, ne = a.rp * a.rp;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= ne) return;
  double* part = a.gram + mat * a.gram_stride;
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
  int p = 0;
  for (; p + 3 < a.nsplit; p += 4) {
    s0 += part[static_cast<int64_t>(p) * ne + e];
    s1 += part[static_cast<int64_t>(p + 1) * ne + e];
    s2 += part[static_cast<int64_t>(p + 2) * ne + e];
    s3 += part[static_cast<int64_t>(p + 3) * ne + e];
  }
  for (; p < a.nsplit; ++p) s0 += part[static_cast<int64_t>(p) * ne + e];
  part[e] = (s0 + s1) + (s2 + s3);
}

// One workgroup per matrix: S (the reduced Gram matrix) = L L^T (right-looking,
// fp64, in LDS), L^-1 by columns into the upper triangle, then L^-T written as
// fp32 [rp][rp] for the product P L^-T.
// A pivot <= 1e-10 x the largest diagonal entry marks a direction the columns
// do not add: its column of L becomes the unit vector and its row of L^-1 zero,
// so P gets a zero column there.  Padding columns (index >= rank) are zero in
// P, get a unit pivot and an identity block in L^-T.
__global__ __launch_bounds__(256) void dion_chol_kernel(DionArgs a) {
  constexpr int SP = kMaxRank + 1;    // LDS pitch (doubles)
  __shared__ double S[kMaxRank * SP];
  __shared__ double ldiag[kMaxRank];
  __shared__ int dead[kMaxRank];
  __shared__ double dmax;
  const int mat = blockIdx.x, tid = threadIdx.x;
  const int rp = a.rp, r = a.r, ne = rp * rp;
  const double* Sg = a.gram + mat * a.gram_stride;   // the reduced Gram matrix
  {
    // rows of 256 / rp per pass (threads past the last whole row idle),
    // eight passes' loads in flight before their stores
    const int rpp = 256 / rp, lr = tid / rp, lc = tid - lr * rp;
    if (lr < rpp) {
      for (int i0 = 0; i0 < rp; i0 += 8 * rpp) {
        double v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u * rpp + lr;
          v[u] = (i < rp) ? Sg[i * rp + lc] : 0.0;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u * rpp + lr;
          if (i < rp) S[i * SP + lc] = v[u];
        }
      }
    }
  }
  __syncthreads();
  for (int c = r + tid; c < rp; c += 256) S[c * SP + c] = 1.0;
  if (tid == 0) {
    double d = 0.0;
    for (int c = 0; c < r; ++c) d = fmax(d, S[c * SP + c]);
    dmax = d;
  }
  __syncthreads();
  const double thr = 1e-10 * dmax;
  for (int c = 0; c < rp; ++c) {
    const double d = S[c * SP + c];
    const bool isdead = d <= thr;          // NaN stays live and propagates
    const double lcc = isdead ? 1.0 : sqrt(d);
    if (tid == 0) {
      ldiag[c] = lcc;
      dead[c] = isdead ? 1 : 0;
    }
    for (int i = c + 1 + tid; i < rp; i += 256) S[i * SP + c] = isdead ? 0.0 : S[i * SP + c] / lcc;
    __syncthreads();
    // trailing update of the lower triangle, threads as a 16 x 16 grid
    for (int i = c + 1 + (tid >> 4); i < rp; i += 16)
      for (int j = c + 1 + (tid & 15); j <= i; j += 16)
        S[i * SP + j] = fma(-S[i * SP + c], S[j * SP + c], S[i * SP + j]);
    __syncthreads();
  }
  // L^-1 by columns, thread j owning column j: for i > j,
  //   L^-1[i][j] = -(sum_{k=j}^{i-1} L[i][k] L^-1[k][j]) / L[i][i],
  // kept transposed in row j of the strict upper triangle (unused by L), so
  // no thread reads another's results and no barrier is needed
  if (tid < rp) {
    const int j = tid;
    const double djj = 1.0 / ldiag[j];
    for (int i = j + 1; i < rp; ++i) {
      double y = S[i * SP + j] * djj;
      for (int k = j + 1; k < i; ++k) y = fma(S[i * SP + k], S[j * SP + k], y);
      S[j * SP + i] = -y / ldiag[i];
    }
  }
  __syncthreads();
  // L^-T: the strict upper triangle as computed, 1 / L[c][c] on the diagonal,
  // zero below and in the columns of dropped directions
  float* Lt = a.Lt + mat * a.lt_stride;
  for (int e = tid; e < ne; e += 256) {
    const int k = e / rp, c = e - k * rp;
    double v = 0.0;
    if (!dead[c]) v = (k < c) ? S[k * SP + c] : (k == c ? 1.0 / ldiag[c] : 0.0);
    Lt[e] = static_cast<float>(v);
  }
}

// Column sums of squares of R (fp32 [n][rp]) over row chunks of 64, in fp64:
// grid (ceil(n / 64), batch), thread -> column t % rp, rows t / rp + k (256 / rp)
// (threads past the last whole group idle).  Written to the Gram workspace
// (free by now, sized for it) as [ceil(n/64)][rp].
__global__ __launch_bounds__(256) void dion_colsq_kernel(DionArgs a) {
  __shared__ double red[256];
  const int chunk = blockIdx.x, mat = blockIdx.y, tid = threadIdx.x;
  const int n = a.n, rp = a.rp;
  const float* R = a.R + mat * a.r_stride;
  const int per = 256 / rp;                    // threads per column (the rest idle)
  const int c = tid % rp, r0 = tid / rp;
  double s = 0.0;
  if (r0 < per) {
    for (int j = chunk * 64 + r0; j < min(n, chunk * 64 + 64); j += per) {
      const double v = R[static_cast<int64_t>(j) * rp + c];
      s = fma(v, v, s);
    }
  }
  red[tid] = s;
  __syncthreads();
  if (tid < rp) {
    double t = 0.0;
    for (int q = 0; q < per; ++q) t += red[q * rp + tid];
    a.gram[mat * a.gram_stride + static_cast<int64_t>(chunk) * rp + tid] = t;
  }
}

// 1/norm per column (sum of the chunk partials, fixed order; a zero column
// gives 0) and Q = R / norm over 64 rows: grid (ceil(n / 64), batch).
// Block 0 of a matrix also stores 1/norm for the update.
__global__ __launch_bounds__(256) void dion_qnorm_kernel(DionArgs a) {
  __shared__ float invs[kMaxRank];
  const int chunk = blockIdx.x, mat = blockIdx.y, tid = threadIdx.x;
  const int n = a.n, rp = a.rp, r = a.r, nch = (n + 63) / 64;
  const double* part = a.gram + mat * a.gram_stride;
  if (tid < rp) {
    double t = 0.0;
    for (int q = 0; q < nch; ++q) t += part[static_cast<int64_t>(q) * rp + tid];
    const float inv = (t == 0.0) ? 0.0f : static_cast<float>(1.0 / sqrt(t));
    invs[tid] = inv;
    if (chunk == 0) a.inv[mat * rp + tid] = inv;
  }
  __syncthreads();
  const float* R = a.R + mat * a.r_stride;
  float* Q = a.Q + mat * a.q_stride;
  for (int e = tid; e < 64 * r; e += 256) {
    const int j = chunk * 64 + e / r, c = e % r;
    if (j < n) Q[static_cast<int64_t>(j) * r + c] = R[static_cast<int64_t>(j) * rp + c] * invs[c];
  }
}

}  // namespace

hipError_t launch_dion_gemm(const DionArgs& A, int mode, int dtype, int batch, hipStream_t s) {
  const int rows = (mode == DION_BTP) ? A.n : A.m;
  const int cols = (mode == DION_UPD) ? A.n : A.rp;
  const dim3 grid((cols + kDT - 1) / kDT, (rows + kDT - 1) / kDT, batch), block(256);
  const bool bf = dtype == MUON_DTYPE_BF16;
  switch (mode) {
    case DION_BQ:
      if (bf) hipLaunchKernelGGL((dion_gemm_kernel<bf16_t, DION_BQ>), grid, block, 0, s, A);
      else hipLaunchKernelGGL((dion_gemm_kernel<float, DION_BQ>), grid, block, 0, s, A);
      break;
    case DION_PL: hipLaunchKernelGGL((dion_gemm_kernel<float, DION_PL>), grid, block, 0, s, A); break;
    case DION_BTP:
      if (bf) hipLaunchKernelGGL((dion_gemm_kernel<bf16_t, DION_BTP>), grid, block, 0, s, A);
      else hipLaunchKernelGGL((dion_gemm_kernel<float, DION_BTP>), grid, block, 0, s, A);
      break;
    default:
      if (bf) hipLaunchKernelGGL((dion_gemm_kernel<bf16_t, DION_UPD>), grid, block, 0, s, A);
      else hipLaunchKernelGGL((dion_gemm_kernel<float, DION_UPD>), grid, block, 0, s, A);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_dion_gram(const DionArgs& A, int batch, hipStream_t s) {
  hipLaunchKernelGGL(dion_gram_kernel, dim3(A.nsplit, batch), dim3(256), 0, s, A);
  return hipGetLastError();
}

hipError_t launch_dion_chol(const DionArgs& A, int batch, hipStream_t s) {
  hipLaunchKernelGGL(dion_chol_kernel, dim3(batch), dim3(256), 0, s, A);
  return hipGetLastError();
}

hipError_t launch_dion_gram_reduce(const DionArgs& A, int batch, hipStream_t s) {
  hipLaunchKernelGGL(dion_gram_reduce_kernel, dim3((A.rp * A.rp + 255) / 256, batch), dim3(256), 0, s, A);
  return hipGetLastError();
}

hipError_t launch_dion_colnorm(const DionArgs& A, int batch, hipStream_t s) {
  const dim3 grid((A.n + 63) / 64, batch);
  hipLaunchKernelGGL(dion_colsq_kernel, grid, dim3(256), 0, s, A);
  hipLaunchKernelGGL(dion_qnorm_kernel, grid, dim3(256), 0, s, A);
  return hipGetLastError();
}

}  // namespace muon
