// Newton-Schulz for thin matrices: wide view m x n with m <= kThinMaxM (96)
// and n too long for the single-workgroup step ("Muon and MuonClip:
// orthogonalised updates for LLM training", Newton-Schulz subsection:
// A = X X^T, B = b A + c A A, X <- a X + B X).
//
// With so few rows the m x m matrices A and B have no averaging over
// directions: a bf16 rounding of B moves every singular value the same way,
// and its error survives the five steps almost whole.  Here A and B are kept
// in fp32; only X is stored in bf16 between steps.  The products still run on
// bf16 MFMA: a fp32 operand is split into hi = bf16(v) and lo = bf16(v - hi),
// which together hold v to about 2^-17, and
//   A A ~ Ahi Ahi^T + Ahi Alo^T + Alo Ahi^T,   B X ~ Bhi X + Blo X
// (the dropped lo x lo term is 2^-18 of the product).  X X^T needs no split:
// bf16 x bf16 products are exact in the fp32 accumulators.
//
// One iteration is three launches, each batched over every thin matrix of
// the call:
//   thin_gram: one wave per (matrix, column chunk) sums X_c X_c^T over its
//              chunk into an fp32 partial;
//   thin_poly: one block per matrix adds the partials in chunk order (times
//              s^2 on the first step, s = 1 / (||U||_F + eps)), then forms
//              B = b A + c A A in fp32;
//   thin_bx:   one block per 128 columns computes X' = s (a X + B X) and
//              writes it (bf16) to the next iterate, or on the last step to
//              the output in the matrix's own layout.
#include "common.hpp"

namespace muon {

namespace {

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int thin_group(const ThinLaunch& L, int blk) {
  int gi = 0;
  while (gi + 1 < L.ngroups && blk >= L.prefix[gi + 1]) ++gi;
  return gi;
}

// ---------------------------------------------------------------- X X^T
// One wave per (matrix, chunk): the upper 32 x 32 blocks (r1 <= r2) of the
// chunk's Gram matrix, both written (in place and mirrored) to the fp32
// partial [mq][mq].  Fragments come straight from global memory: a lane
// reads 16 bytes of row 32 r + lane % 32 per k16 step, four steps at a time.
template <int MB>
__device__ __forceinline__ void thin_gram_body(const ThinGroup& g, int mat, int chunk) {
  constexpr int mq = 32 * MB;
  constexpr int NP = MB * (MB + 1) / 2;
  const int lane = threadIdx.x;
  const int frow = lane & 31, fk = (lane >> 5) * 8;
  const bf16_t* X = g.X + mat * g.x_stride;
  const int c0 = chunk * g.chunk;
  const int c1 = min(c0 + g.chunk, g.np);   // both multiples of 128
  f32x16_t acc[NP];
  static_for<NP>([&](auto p) { acc[decltype(p)::value] = f32x16_t{}; });
  const bf16_t* rowp[MB];
  static_for<MB>([&](auto r) {
    constexpr int R = decltype(r)::value;
    rowp[R] = X + static_cast<int64_t>(32 * R + frow) * g.np + fk;
  });
  for (int k0 = c0; k0 < c1; k0 += 64) {
    bf16x8_t f[4][MB];
    static_for<4 * MB>([&](auto x) {
      constexpr int S = decltype(x)::value / MB, R = decltype(x)::value % MB;
      f[S][R] = *reinterpret_cast<const bf16x8_t*>(rowp[R] + k0 + 16 * S);
    });
    static_for<4>([&](auto s) {
      constexpr int S = decltype(s)::value;
      static_for<MB>([&](auto r1) {
        constexpr int R1 = decltype(r1)::value;
        static_for<MB - R1>([&](auto d) {
          constexpr int R2 = R1 + decltype(d)::value;
          constexpr int P = R1 * MB - R1 * (R1 - 1) / 2 + (R2 - R1);
          acc[P] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[S][R1], f[S][R2], acc[P], 0, 0, 0);
        });
      });
    });
  }
  float* P = g.part + (static_cast<int64_t>(mat) * g.nchunk + chunk) * mq * mq;
  const int er = 4 * (lane >> 5);
  static_for<MB>([&](auto r1) {
    constexpr int R1 = decltype(r1)::value;
    static_for<MB - R1>([&](auto d) {
      constexpr int R2 = R1 + decltype(d)::value;
      constexpr int PI = R1 * MB - R1 * (R1 - 1) / 2 + (R2 - R1);
      static_for<16>([&](auto e) {
        constexpr int E = decltype(e)::value;
        const int i = 32 * R1 + 8 * (E / 4) + er + (E % 4);
        const int j = 32 * R2 + frow;
        P[i * mq + j] = acc[PI][E];
        if constexpr (R1 != R2) P[j * mq + i] = acc[PI][E];
      });
    });
  });
}

__global__ __launch_bounds__(64) void thin_gram_kernel(ThinLaunch L) {
  const int gi = thin_group(L, blockIdx.x);
  const ThinGroup& g = L.g[gi];
  const int local = blockIdx.x - L.prefix[gi];
  const int mat = local / g.nchunk, chunk = local - mat * g.nchunk;
  switch (g.mb) {
    case 1: thin_gram_body<1>(g, mat, chunk); break;
    case 2: thin_gram_body<2>(g, mat, chunk); break;
    default: thin_gram_body<3>(g, mat, chunk); break;
  }
}

// ------------------------------------------------------- B = b A + c A A
constexpr int kPolyNT = 256;
constexpr int kMq = 32 * kThinMaxMB;        // largest mq
constexpr int kPh = kMq + 8;                // bf16 plane pitch: 16-byte rows, conflict-free fragment reads

template <int MB>
__device__ __forceinline__ void thin_poly_body(const ThinLaunch& L, const ThinGroup& g, int mat, float* sAf,
                                               bf16_t* sAh, bf16_t* sAl) {
  constexpr int mq = 32 * MB;
  constexpr int pf = mq + 1;                 // fp32 plane pitch
  const int tid = threadIdx.x;
  const float s = (g.inv && L.first) ? g.inv[mat] : 1.0f;
  const float s2 = s * s;
  const float* P = g.part + static_cast<int64_t>(mat) * g.nchunk * mq * mq;
  for (int e = tid; e < mq * mq; e += kPolyNT) {
    float v = 0.0f;
    for (int c = 0; c < g.nchunk; ++c) v += P[static_cast<int64_t>(c) * mq * mq + e];
    v *= s2;
    const int i = e / mq, j = e - i * mq;
    sAf[i * pf + j] = v;
    const bf16_t hi = f32_to_bf16(v);
    sAh[i * kPh + j] = hi;
    sAl[i * kPh + j] = f32_to_bf16(v - bf16_to_f32(hi));
  }
  lds_barrier();
  float* Bm = g.Bm + static_cast<int64_t>(mat) * mq * mq;
  if (L.c == 0.0f) {
    // a cubic polynomial: B = b A
    for (int e = tid; e < mq * mq; e += kPolyNT) {
      const int i = e / mq, j = e - i * mq;
      Bm[e] = L.b * sAf[i * pf + j];
    }
    return;
  }
  const int lane = tid & 63, wave = tid >> 6;
  const int frow = lane & 31, fk = (lane >> 5) * 8, er = 4 * (lane >> 5);
  for (int blk = wave; blk < MB * MB; blk += kPolyNT / 64) {
    const int r1 = blk / MB, r2 = blk - r1 * MB;
    const bf16_t* ah = sAh + (32 * r1 + frow) * kPh + fk;
    const bf16_t* al = sAl + (32 * r1 + frow) * kPh + fk;
    const bf16_t* bh = sAh + (32 * r2 + frow) * kPh + fk;
    const bf16_t* bl = sAl + (32 * r2 + frow) * kPh + fk;
    f32x16_t acc{};
    static_for<mq / 16>([&](auto k) {
      constexpr int K0 = 16 * decltype(k)::value;
      const bf16x8_t fah = *reinterpret_cast<const bf16x8_t*>(ah + K0);
      const bf16x8_t fal = *reinterpret_cast<const bf16x8_t*>(al + K0);
      const bf16x8_t fbh = *reinterpret_cast<const bf16x8_t*>(bh + K0);
      const bf16x8_t fbl = *reinterpret_cast<const bf16x8_t*>(bl + K0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fah, fbh, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fah, fbl, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fal, fbh, acc, 0, 0, 0);
    });
    static_for<16>([&](auto e) {
      constexpr int E = decltype(e)::value;
      const int i = 32 * r1 + 8 * (E / 4) + er + (E % 4);
      const int j = 32 * r2 + frow;
      Bm[i * mq + j] = fmaf(L.b, sAf[i * pf + j], L.c * acc[E]);
    });
  }
}

__global__ __launch_bounds__(kPolyNT) void thin_poly_kernel(ThinLaunch L) {
  __shared__ float sAf[kMq * (kMq + 1)];
  __shared__ __attribute__((aligned(16))) bf16_t sAh[kMq * kPh];
  __shared__ __attribute__((aligned(16))) bf16_t sAl[kMq * kPh];
  const int gi = thin_group(L, blockIdx.x);
  const ThinGroup& g = L.g[gi];
  const int mat = blockIdx.x - L.prefix[gi];
  switch (g.mb) {
    case 1: thin_poly_body<1>(L, g, mat, sAf, sAh, sAl); break;
    case 2: thin_poly_body<2>(L, g, mat, sAf, sAh, sAl); break;
    default: thin_poly_body<3>(L, g, mat, sAf, sAh, sAl); break;
  }
}

// ------------------------------------------------- X' = s (a X + B X)
constexpr int kBxNT = 256;
constexpr int kBxCols = 128;                // columns of X per block
constexpr int kPx = kBxCols + 8;            // LDS pitch of the X tile (bf16)
constexpr int kStage = (kBxCols * kPh > kMq * kPx) ? kBxCols * kPh : kMq * kPx;

template <int MB>
__device__ __forceinline__ void thin_bx_body(const ThinLaunch& L, const ThinGroup& g, int mat, int cb,
                                             bf16_t* sBh, bf16_t* sBl, bf16_t* sX) {
  constexpr int mq = 32 * MB;
  const int tid = threadIdx.x;
  const int c0 = cb * kBxCols;
  // B as hi / lo bf16 planes
  const float* Bm = g.Bm + static_cast<int64_t>(mat) * mq * mq;
  for (int e = tid; e < mq * mq; e += kBxNT) {
    const int i = e / mq, j = e - i * mq;
    const float v = Bm[e];
    const bf16_t hi = f32_to_bf16(v);
    sBh[i * kPh + j] = hi;
    sBl[i * kPh + j] = f32_to_bf16(v - bf16_to_f32(hi));
  }
  // the X tile: rows 0..mq-1, columns c0..c0+127, 16-byte chunks
  const bf16_t* X = g.X + mat * g.x_stride;
  for (int q = tid; q < mq * (kBxCols / 8); q += kBxNT) {
    const int r = q / (kBxCols / 8), cc = (q % (kBxCols / 8)) * 8;
    *reinterpret_cast<u32x4_t*>(sX + r * kPx + cc) =
        *reinterpret_cast<const u32x4_t*>(X + static_cast<int64_t>(r) * g.np + c0 + cc);
  }
  lds_barrier();

  // D = X^T B^T: wave w owns columns 32 w .. 32 w + 31 of the tile (rows of
  // D) against all MB row blocks of B.  Accumulator element e of block R is
  // X'[32 R + lane % 32][32 w + 8 (e / 4) + 4 (lane / 32) + e % 4].
  const int lane = tid & 63, wave = tid >> 6;
  const int frow = lane & 31, fk = (lane >> 5) * 8, er = 4 * (lane >> 5);
  f32x16_t acc[MB];
  static_for<MB>([&](auto r) { acc[decltype(r)::value] = f32x16_t{}; });
  const bf16_t* xcol = sX + fk * kPx + 32 * wave + frow;
  static_for<mq / 16>([&](auto k) {
    constexpr int K0 = 16 * decltype(k)::value;
    u16x8_t w;
    static_for<8>([&](auto q) {
      constexpr int Q = decltype(q)::value;
      w[Q] = xcol[(K0 + Q) * kPx];
    });
    const bf16x8_t fx = __builtin_bit_cast(bf16x8_t, w);
    static_for<MB>([&](auto r) {
      constexpr int R = decltype(r)::value;
      const bf16x8_t fh = *reinterpret_cast<const bf16x8_t*>(sBh + (32 * R + frow) * kPh + K0 + fk);
      const bf16x8_t fl = *reinterpret_cast<const bf16x8_t*>(sBl + (32 * R + frow) * kPh + K0 + fk);
      acc[R] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fx, fh, acc[R], 0, 0, 0);
      acc[R] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fx, fl, acc[R], 0, 0, 0);
    });
  });
  const float s = (g.inv && L.first) ? g.inv[mat] : 1.0f;
  const float ca = s, ce = L.a * s;
  u32x2_t out[MB][4];
  static_for<MB>([&](auto r) {
    constexpr int R = decltype(r)::value;
    static_for<4>([&](auto q) {
      constexpr int Q = decltype(q)::value;
      const int i = 32 * R + frow, j = 32 * wave + 8 * Q + er;
      const u32x2_t xv = *reinterpret_cast<const u32x2_t*>(sX + i * kPx + j);
      f32x4_t v;
      v[0] = fmaf(ce, __uint_as_float(xv[0] << 16), ca * acc[R][4 * Q + 0]);
      v[1] = fmaf(ce, __uint_as_float(xv[0] & 0xffff0000u), ca * acc[R][4 * Q + 1]);
      v[2] = fmaf(ce, __uint_as_float(xv[1] << 16), ca * acc[R][4 * Q + 2]);
      v[3] = fmaf(ce, __uint_as_float(xv[1] & 0xffff0000u), ca * acc[R][4 * Q + 3]);
      out[R][Q] = __builtin_bit_cast(u32x2_t, __builtin_convertvector(v, bf16x4_t));
    });
  });
  lds_barrier();                 // every wave is done reading the X tile

  bf16_t* D = g.D + mat * g.d_stride;
  if (!g.d_trans) {
    // row-major [i][j]: staged into the X tile's place, then whole rows out
    static_for<MB>([&](auto r) {
      constexpr int R = decltype(r)::value;
      static_for<4>([&](auto q) {
        constexpr int Q = decltype(q)::value;
        *reinterpret_cast<u32x2_t*>(sX + (32 * R + frow) * kPx + 32 * wave + 8 * Q + er) = out[R][Q];
      });
    });
    lds_barrier();
    for (int q = tid; q < mq * (kBxCols / 8); q += kBxNT) {
      const int r = q / (kBxCols / 8), cc = (q % (kBxCols / 8)) * 8;
      const int gc = c0 + cc;
      if (r >= g.d_rvalid || gc >= g.d_cvalid) continue;
      const u32x4_t w = *reinterpret_cast<const u32x4_t*>(sX + r * kPx + cc);
      bf16_t* d = D + static_cast<int64_t>(r) * g.d_ld + gc;
      if (g.d_vec && gc + 7 < g.d_cvalid) {
        *reinterpret_cast<u32x4_t*>(d) = w;
      } else {
        for (int e = 0; e < 8 && gc + e < g.d_cvalid; ++e) d[e] = static_cast<bf16_t>((w[e >> 1] >> (16 * (e & 1))) & 0xffff);
      }
    }
  } else {
    // transposed [j][i] (a tall matrix's own layout), staged with pitch kPh
    static_for<MB>([&](auto r) {
      constexpr int R = decltype(r)::value;
      static_for<4>([&](auto q) {
        constexpr int Q = decltype(q)::value;
        const int i = 32 * R + frow, j = 32 * wave + 8 * Q + er;
        sX[(j + 0) * kPh + i] = static_cast<bf16_t>(out[R][Q][0] & 0xffff);
        sX[(j + 1) * kPh + i] = static_cast<bf16_t>(out[R][Q][0] >> 16);
        sX[(j + 2) * kPh + i] = static_cast<bf16_t>(out[R][Q][1] & 0xffff);
        sX[(j + 3) * kPh + i] = static_cast<bf16_t>(out[R][Q][1] >> 16);
      });
    });
    lds_barrier();
    for (int q = tid; q < kBxCols * (mq / 8); q += kBxNT) {
      const int jj = q / (mq / 8), ic = (q % (mq / 8)) * 8;
      const int gr = c0 + jj;
      if (gr >= g.d_rvalid || ic >= g.d_cvalid) continue;
      const u32x4_t w = *reinterpret_cast<const u32x4_t*>(sX + jj * kPh + ic);
      bf16_t* d = D + static_cast<int64_t>(gr) * g.d_ld + ic;
      if (g.d_vec && ic + 7 < g.d_cvalid) {
        *reinterpret_cast<u32x4_t*>(d) = w;
      } else {
        for (int e = 0; e < 8 && ic + e < g.d_cvalid; ++e) d[e] = static_cast<bf16_t>((w[e >> 1] >> (16 * (e & 1))) & 0xffff);
      }
    }
  }
}

__global__ __launch_bounds__(kBxNT) void thin_bx_kernel(ThinLaunch L) {
  __shared__ __attribute__((aligned(16))) bf16_t sBh[kMq * kPh];
  __shared__ __attribute__((aligned(16))) bf16_t sBl[kMq * kPh];
  __shared__ __attribute__((aligned(16))) bf16_t sX[kStage];
  const int gi = thin_group(L, blockIdx.x);
  const ThinGroup& g = L.g[gi];
  const int local = blockIdx.x - L.prefix[gi];
  const int nb = g.np / kBxCols;
  const int mat = local / nb, cb = local - mat * nb;
  switch (g.mb) {
    case 1: thin_bx_body<1>(L, g, mat, cb, sBh, sBl, sX); break;
    case 2: thin_bx_body<2>(L, g, mat, cb, sBh, sBl, sX); break;
    default: thin_bx_body<3>(L, g, mat, cb, sBh, sBl, sX); break;
  }
}

}  // namespace

hipError_t launch_thin(const ThinLaunch& L, int stage, int nblocks, hipStream_t s) {
  if (stage == 0) hipLaunchKernelGGL(thin_gram_kernel, dim3(nblocks), dim3(64), 0, s, L);
  else if (stage == 1) hipLaunchKernelGGL(thin_poly_kernel, dim3(nblocks), dim3(kPolyNT), 0, s, L);
  else hipLaunchKernelGGL(thin_bx_kernel, dim3(nblocks), dim3(kBxNT), 0, s, L);
  return hipGetLastError();
}

}  // namespace muon
