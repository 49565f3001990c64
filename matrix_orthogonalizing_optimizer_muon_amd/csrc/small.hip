// The whole Muon step for small matrices, one 512-thread workgroup per
// matrix and a single launch for every small matrix of a call.
//
// Per matrix, in the order of "MuonClip", section 07 (momentum, then
// Newton-Schulz, then the scaled and decayed write):
//   M <- mu M + G, U = G + mu M (lookahead) or M        ("MuonClip", section 02)
//   X0 = bf16(U) on the wide view (m <= n), s = 1 / (||U||_F + eps)
//   repeat: A = X X^T, B = b A + c A A, X <- a X + B X  ("Muon and MuonClip:
//           orthogonalised updates for LLM training", Newton-Schulz subsection;
//           the first iteration works on s X0, folded into its products)
//   W <- (1 - lr wd) W - lr scale O                     ("MuonClip", section 03)
// with the rounding points of the tiled path: bf16 operands, fp32
// accumulation, A, B and X rounded to bf16 once per product.  Matrices with
// at most kThinMaxM rows in the wide view keep A and B to about 2^-17
// instead, as a bf16 pair hi + lo (hi = bf16(v), lo = bf16(v - hi)), the way
// the thin tiled path does: with so few rows, a bf16 rounding of B moves
// every singular value the same way and is not averaged out.  Their products
// add the cross terms, A A ~ Ahi Ahi^T + Ahi Alo^T + Alo Ahi^T and
// B X ~ Bhi X + Blo X.
//
// X (at most 128 x 256) and A / B (at most 128 x 128) stay in LDS for the
// whole iteration, so a small matrix costs one launch instead of the
// 3 + 3 x steps launches of the tiled path, whose per-launch cost dominates
// at this size.  Products use v_mfma_f32_32x32x16_bf16 on 32 x 32 blocks,
// fragments double-buffered in registers; the memory phases move whole
// 16-byte chunks, every load of a round issued before its first use, and
// the parameters are fetched before the iteration so their latency hides
// behind it.  Barriers order LDS only (global stores are never waited for).
#include "common.hpp"

namespace muon {

namespace {

constexpr int kNT = 512;                    // 8 waves
constexpr int kPX = kSmallMaxN + 8;         // largest LDS row pitch of X (bf16)
constexpr int kPA = kSmallMaxM + 8;         // largest LDS row pitch of A / B

typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <typename T>
__device__ __forceinline__ float load_f32(const T* p, int e) {
  if constexpr (sizeof(T) == 2) return bf16_to_f32(p[e]);
  else return p[e];
}

template <typename T>
__device__ __forceinline__ void store_f32(T* p, int e, float v) {
  if constexpr (sizeof(T) == 2) p[e] = f32_to_bf16(v);
  else p[e] = v;
}

// Item c = k * kNT + tid of a grid with `cols` columns, k = 0, 1, ...: the
// row and column advance by fixed steps, so no division per item.
struct GridWalk {
  int i, j, di, dj, cols;
  __device__ GridWalk(int tid, int cols_) : cols(cols_) {
    i = tid / cols;
    j = tid - i * cols;
    di = kNT / cols;
    dj = kNT - di * cols;
  }
  __device__ __forceinline__ void next() {
    i += di;
    j += dj;
    if (j >= cols) {
      j -= cols;
      ++i;
    }
  }
};

// Eight consecutive elements as fp32 (p 16-byte aligned), and back.
template <typename T>
__device__ __forceinline__ f32x8_t load8(const T* p) {
  if constexpr (sizeof(T) == 2) {
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(p);
    f32x8_t v;
    static_for<4>([&](auto q) {
      constexpr int Q = decltype(q)::value;
      v[2 * Q] = __uint_as_float(w[Q] << 16);
      v[2 * Q + 1] = __uint_as_float(w[Q] & 0xffff0000u);
    });
    return v;
  } else {
    const f32x4_t a = reinterpret_cast<const f32x4_t*>(p)[0];
    const f32x4_t b = reinterpret_cast<const f32x4_t*>(p)[1];
    return f32x8_t{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
}

// bf16 rounding (nearest-even) of 8 / 4 values, packed two per dword
__device__ __forceinline__ u32x4_t pack8(const f32x8_t& v) {
  return __builtin_bit_cast(u32x4_t, __builtin_convertvector(v, bf16x8_t));
}
__device__ __forceinline__ u32x2_t pack4(const f32x4_t& v) {
  return __builtin_bit_cast(u32x2_t, __builtin_convertvector(v, bf16x4_t));
}
__device__ __forceinline__ f32x4_t unpack4(const u32x2_t& w) {
  return f32x4_t{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u), __uint_as_float(w[1] << 16),
                 __uint_as_float(w[1] & 0xffff0000u)};
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const f32x8_t& v) {
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<u32x4_t*>(p) = pack8(v);
  } else {
    reinterpret_cast<f32x4_t*>(p)[0] = f32x4_t{v[0], v[1], v[2], v[3]};
    reinterpret_cast<f32x4_t*>(p)[1] = f32x4_t{v[4], v[5], v[6], v[7]};
  }
}

// The step for one matrix whose wide view has MB blocks of 32 rows.
//
// LDS traffic is what bounds this size, so every epilogue access is 8 or 16
// bytes: an MFMA accumulator holds 4 consecutive rows of one output column,
// which is 4 consecutive elements of a row of the transposed output.  Hence
//   A = X X^T, B = b A + c A A^T: all MB x MB blocks are computed (the wave
//     with the most blocks has two either way) and each is stored transposed,
//     into the mirror block;
//   X' = B X is computed as its transpose D = X^T B^T (the operands swap
//     roles), whose accumulators are 4 consecutive columns of a row of X'.
template <typename T, int MB>
__device__ __forceinline__ void small_body(const SmallLaunch& L, const SmallGroup& g, int mat, bf16_t* sX,
                                           bf16_t* sA, bf16_t* sAl, double* red) {
  constexpr int mp = 32 * MB;
  constexpr bool SPLIT = MB <= kThinMaxMB;   // A and B as bf16 pairs (sA hi, sAl lo)
  constexpr int pa = mp + 8;                 // A / B row pitch: 16-byte rows, conflict-free fragment reads
  constexpr int nkm = mp / 16;               // k steps of the m x m contractions
  constexpr int NBLK = MB * MB;              // 32 x 32 blocks of an m x m product
  constexpr int CV = 8;                      // 8-element chunks per thread per round
  constexpr int CS = 16;                     // elements per thread per round (unaligned shapes)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = g.m, n = g.n;
  const int np = (n + 31) & ~31;
  const int px = np + 8;                     // X row pitch
  const int nb = np / 32;
  const int rows = g.rows, cols = g.cols, total = rows * cols;
  const bool tall = g.tall != 0;
  const bool vec = g.vec != 0;
  // wide-view position of original element (i, j)
  auto xat = [&](int i, int j) { return tall ? j * px + i : i * px + j; };

  for (int e = tid; e < mp * px / 2; e += kNT) reinterpret_cast<uint32_t*>(sX)[e] = 0u;
  lds_barrier();

  // ---- momentum, lookahead, bf16(U) on the wide view, sum of squares.
  // Each round issues all of its loads before any arithmetic or store.
  const T* G = static_cast<const T*>(g.G) + mat * g.bstride;
  float* M = g.M ? g.M + mat * g.bstride : nullptr;
  double ss = 0.0;
  if (vec) {
    // chunks of 8 consecutive row elements; for a tall matrix consecutive
    // threads take consecutive rows, so the transposed LDS writes of a wave
    // land in consecutive addresses
    const int c8 = cols / 8, nch = rows * c8;
    GridWalk w(tid, tall ? rows : c8);
    for (int base = 0; base < nch; base += CV * kNT) {
      f32x8_t gv[CV], mv[CV];
      int ci[CV], cj[CV];
      static_for<CV>([&](auto q) {
        constexpr int Q = decltype(q)::value;
        const bool ok = base + Q * kNT + tid < nch;
        ci[Q] = ok ? (tall ? w.j : w.i) : 0;
        cj[Q] = ok ? 8 * (tall ? w.i : w.j) : 0;
        if (!ok) ci[Q] = -1;
        const int e = (ok ? ci[Q] : 0) * cols + cj[Q];
        gv[Q] = load8(G + e);
        mv[Q] = M ? load8(M + e) : f32x8_t{};
        w.next();
      });
      static_for<CV>([&](auto q) {
        constexpr int Q = decltype(q)::value;
        f32x8_t u = gv[Q];
        if (M) {
          const f32x8_t mn = __builtin_elementwise_fma(f32x8_t(L.mu), mv[Q], gv[Q]);
          u = L.nesterov ? __builtin_elementwise_fma(f32x8_t(L.mu), mn, gv[Q]) : mn;
          mv[Q] = mn;
        }
        if (ci[Q] >= 0) {
          const int e = ci[Q] * cols + cj[Q];
          if (M) store8(M + e, mv[Q]);
          static_for<8>([&](auto r) {
            constexpr int R = decltype(r)::value;
            ss += static_cast<double>(u[R]) * static_cast<double>(u[R]);
          });
          const u32x4_t b = pack8(u);
          if (!tall) {
            *reinterpret_cast<u32x4_t*>(sX + ci[Q] * px + cj[Q]) = b;
          } else {
            static_for<8>([&](auto r) {
              constexpr int R = decltype(r)::value;
              sX[(cj[Q] + R) * px + ci[Q]] = static_cast<bf16_t>((b[R / 2] >> (16 * (R % 2))) & 0xffff);
            });
          }
        }
      });
    }
  } else {
    GridWalk w(tid, cols);
    for (int base = 0; base < total; base += CS * kNT) {
      float gv[CS], mv[CS];
      int ci[CS], cj[CS];
      static_for<CS>([&](auto q) {
        constexpr int Q = decltype(q)::value;
        const bool ok = base + Q * kNT + tid < total;
        ci[Q] = ok ? w.i : -1;
        cj[Q] = ok ? w.j : 0;
        const int e = ok ? w.i * cols + w.j : 0;
        gv[Q] = load_f32(G, e);
        mv[Q] = M ? M[e] : 0.0f;
        w.next();
      });
      static_for<CS>([&](auto q) {
        constexpr int Q = decltype(q)::value;
        float u = gv[Q];
        if (M) {
          const float mn = fmaf(L.mu, mv[Q], gv[Q]);
          u = L.nesterov ? fmaf(L.mu, mn, gv[Q]) : mn;
          mv[Q] = mn;
        }
        if (ci[Q] >= 0) {
          if (M) M[ci[Q] * cols + cj[Q]] = mv[Q];
          ss += static_cast<double>(u) * static_cast<double>(u);
          sX[xat(ci[Q], cj[Q])] = f32_to_bf16(u);
        }
      });
    }
  }

  // the parameters (vector path), fetched now and used after the iteration,
  // so their latency hides behind the Newton-Schulz products
  T* W = g.W ? static_cast<T*>(g.W) + mat * g.bstride : nullptr;
  const bool wpre = W && vec && rows * cols <= CV * 8 * kNT;
  f32x8_t wv[CV];
  if (wpre) {
    const int c8 = cols / 8, nch = rows * c8;
    GridWalk w(tid, tall ? rows : c8);
    static_for<CV>([&](auto q) {
      constexpr int Q = decltype(q)::value;
      const bool ok = Q * kNT + tid < nch;
      const int i = ok ? (tall ? w.j : w.i) : 0, j = ok ? 8 * (tall ? w.i : w.j) : 0;
      wv[Q] = load8(W + i * cols + j);
      w.next();
    });
  }

  ss = wave_sum_d(ss);
  if (lane == 0) red[wave] = ss;
  lds_barrier();
  double tot = 0.0;
#pragma unroll
  for (int w = 0; w < kNT / 64; ++w) tot += red[w];
  const float inv = static_cast<float>(1.0 / (sqrt(tot) + static_cast<double>(L.eps)));
  if (tid == 0 && g.inv) g.inv[mat] = inv;
  if (g.X0) {
    // X0 on the wide view, whole 16-byte row chunks where n allows
    bf16_t* X0 = g.X0 + mat * g.x0_stride;
    if (n % 8 == 0) {
      GridWalk w(tid, n / 8);
      for (int c = tid; c < m * (n / 8); c += kNT, w.next())
        *reinterpret_cast<u32x4_t*>(X0 + static_cast<int64_t>(w.i) * g.x0_ld + 8 * w.j) =
            *reinterpret_cast<const u32x4_t*>(sX + w.i * px + 8 * w.j);
    } else {
      GridWalk w(tid, n);
      for (int e = tid; e < m * n; e += kNT, w.next()) X0[static_cast<int64_t>(w.i) * g.x0_ld + w.j] = sX[w.i * px + w.j];
    }
  }

  const int frow = lane & 31;                // fragment row (A operand) / column (B operand)
  const int fk = (lane >> 5) * 8;            // fragment k offset
  const int er = 4 * (lane >> 5);            // first accumulator row of this lane
  const bool cubic = (L.c == 0.0f);

  // this wave's blocks of S S^T (S = sX or sA): k = wave and wave + 8
  int bi[2] = {0, 0}, bj[2] = {0, 0};
  const int mine = (wave + 8 < NBLK) ? 2 : (wave < NBLK ? 1 : 0);
  bi[0] = wave / MB;
  bj[0] = wave % MB;
  bi[1] = (wave + 8) / MB;
  bj[1] = (wave + 8) % MB;

  // acc[r] = block r of S S^T over nk k steps, fragments double-buffered in
  // registers (the next step's reads are in flight during this step's MFMA)
  auto sym_product = [&](const bf16_t* S, int ps, int nk, f32x16_t (&acc)[2]) {
    acc[0] = f32x16_t{};
    acc[1] = f32x16_t{};
    // two blocks in one block column: the column operand is read once
    auto run_shared = [&]() {
      const bf16_t* pa0 = S + (bi[0] * 32 + frow) * ps + fk;
      const bf16_t* pa1 = S + (bi[1] * 32 + frow) * ps + fk;
      const bf16_t* pb = S + (bj[0] * 32 + frow) * ps + fk;
      bf16x8_t fa[2][2], fb[2];
      auto ld = [&](auto slot, int k0) {
        constexpr int SL = decltype(slot)::value;
        fa[SL][0] = *reinterpret_cast<const bf16x8_t*>(pa0 + k0);
        fa[SL][1] = *reinterpret_cast<const bf16x8_t*>(pa1 + k0);
        fb[SL] = *reinterpret_cast<const bf16x8_t*>(pb + k0);
      };
      auto mm = [&](auto slot) {
        constexpr int SL = decltype(slot)::value;
        acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[SL][0], fb[SL], acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[SL][1], fb[SL], acc[1], 0, 0, 0);
      };
      ld(std::integral_constant<int, 0>{}, 0);
      for (int kk = 0; kk < nk; kk += 2) {
        ld(std::integral_constant<int, 1>{}, 16 * (kk + 1));
        mm(std::integral_constant<int, 0>{});
        if (kk + 2 < nk) ld(std::integral_constant<int, 0>{}, 16 * (kk + 2));
        mm(std::integral_constant<int, 1>{});
      }
    };
    auto run = [&](auto nacc) {
      constexpr int NA = decltype(nacc)::value;
      const bf16_t* pa_[NA];
      const bf16_t* pb_[NA];
      static_for<NA>([&](auto r) {
        constexpr int R = decltype(r)::value;
        pa_[R] = S + (bi[R] * 32 + frow) * ps + fk;
        pb_[R] = S + (bj[R] * 32 + frow) * ps + fk;
      });
      bf16x8_t fa[2][NA], fb[2][NA];
      auto ld = [&](auto slot, int k0) {
        constexpr int SL = decltype(slot)::value;
        static_for<NA>([&](auto r) {
          constexpr int R = decltype(r)::value;
          fa[SL][R] = *reinterpret_cast<const bf16x8_t*>(pa_[R] + k0);
          fb[SL][R] = *reinterpret_cast<const bf16x8_t*>(pb_[R] + k0);
        });
      };
      auto mm = [&](auto slot) {
        constexpr int SL = decltype(slot)::value;
        static_for<NA>([&](auto r) {
          constexpr int R = decltype(r)::value;
          acc[R] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[SL][R], fb[SL][R], acc[R], 0, 0, 0);
        });
      };
      ld(std::integral_constant<int, 0>{}, 0);
      for (int kk = 0; kk < nk; kk += 2) {   // nk is even
        ld(std::integral_constant<int, 1>{}, 16 * (kk + 1));
        mm(std::integral_constant<int, 0>{});
        if (kk + 2 < nk) ld(std::integral_constant<int, 0>{}, 16 * (kk + 2));
        mm(std::integral_constant<int, 1>{});
      }
    };
    if (mine == 2 && bj[0] == bj[1]) run_shared();
    else if (mine == 2) run(std::integral_constant<int, 2>{});
    else if (mine == 1) run(std::integral_constant<int, 1>{});
  };
  // LDS offset, in sA, of group q (4 consecutive accumulator rows) of block r
  // stored transposed: row bj * 32 + frow, columns bi * 32 + er + 8 q + (0..3)
  auto tpos = [&](int r, int q) { return (bj[r] * 32 + frow) * pa + bi[r] * 32 + er + 8 * q; };
  auto sym_store = [&](const f32x16_t (&acc)[2]) {
    static_for<2>([&](auto r) {
      constexpr int R = decltype(r)::value;
      if (R < mine) {
        static_for<4>([&](auto q) {
          constexpr int Q = decltype(q)::value;
          const f32x4_t v{acc[R][4 * Q], acc[R][4 * Q + 1], acc[R][4 * Q + 2], acc[R][4 * Q + 3]};
          const u32x2_t hi = pack4(v);
          *reinterpret_cast<u32x2_t*>(sA + tpos(R, Q)) = hi;
          if constexpr (SPLIT) *reinterpret_cast<u32x2_t*>(sAl + tpos(R, Q)) = pack4(v - unpack4(hi));
        });
      }
    });
  };
  // A A^T from the pair planes: Ahi Ahi^T + Ahi Alo^T + Alo Ahi^T
  auto sym_product_split = [&](f32x16_t (&acc)[2]) {
    static_for<2>([&](auto r) {
      constexpr int R = decltype(r)::value;
      acc[R] = f32x16_t{};
      if (R < mine) {
        const int oa = (bi[R] * 32 + frow) * pa + fk, ob = (bj[R] * 32 + frow) * pa + fk;
        for (int kk = 0; kk < nkm; ++kk) {
          const bf16x8_t fah = *reinterpret_cast<const bf16x8_t*>(sA + oa + 16 * kk);
          const bf16x8_t fal = *reinterpret_cast<const bf16x8_t*>(sAl + oa + 16 * kk);
          const bf16x8_t fbh = *reinterpret_cast<const bf16x8_t*>(sA + ob + 16 * kk);
          const bf16x8_t fbl = *reinterpret_cast<const bf16x8_t*>(sAl + ob + 16 * kk);
          acc[R] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fah, fbh, acc[R], 0, 0, 0);
          acc[R] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fah, fbl, acc[R], 0, 0, 0);
          acc[R] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fal, fbh, acc[R], 0, 0, 0);
        }
      }
    });
  };

  f32x16_t acc[2];
  for (int t = 0; t < L.steps; ++t) {
    const float s1 = (t == 0) ? inv : 1.0f;   // the normalisation, folded into the first iteration

    // A = s1^2 X X^T
    sym_product(sX, px, np / 16, acc);
    static_for<2>([&](auto r) { acc[decltype(r)::value] *= s1 * s1; });
    sym_store(acc);
    lds_barrier();

    // B = c A A^T + b A, over A in place once every wave has read it.  The
    // element stored at (j, i) is c (A A^T)_ij + b A_ji, read from that place.
    if (!cubic) {
      if constexpr (SPLIT) sym_product_split(acc);
      else sym_product(sA, pa, nkm, acc);
      static_for<2>([&](auto r) {
        constexpr int R = decltype(r)::value;
        if (R < mine) {
          static_for<4>([&](auto q) {
            constexpr int Q = decltype(q)::value;
            f32x4_t a = unpack4(*reinterpret_cast<const u32x2_t*>(sA + tpos(R, Q)));
            if constexpr (SPLIT) a += unpack4(*reinterpret_cast<const u32x2_t*>(sAl + tpos(R, Q)));
            static_for<4>([&](auto x) {
              constexpr int E = decltype(x)::value;
              acc[R][4 * Q + E] = fmaf(L.b, a[E], L.c * acc[R][4 * Q + E]);
            });
          });
        }
      });
      lds_barrier();
      sym_store(acc);
      lds_barrier();
    }

    // X <- ca (P X) + a s1 X with P = B (or A and ca = b s1 for a cubic),
    // as D = X^T P^T: wave w owns the 32 columns jb = w of X' (the rows of D)
    // and all MB row blocks of X'.  Lane: X'[R 32 + frow][jb 32 + er + 8 q + (0..3)].
    const float ca = (cubic ? L.b : 1.0f) * s1, ce = L.a * s1;
    const int jb = wave;
    f32x16_t xa[MB];
    static_for<MB>([&](auto r) { xa[decltype(r)::value] = f32x16_t{}; });
    auto xpos = [&](int r, int q) { return (r * 32 + frow) * px + jb * 32 + er + 8 * q; };
    if (jb < nb) {
      const bf16_t* xcol = sX + fk * px + jb * 32 + frow;   // X[k][jb 32 + frow], k = fk + ..
      const bf16_t* prow = sA + frow * pa + fk;             // P[r 32 + frow][k], k = fk + ..
      const bf16_t* prowl = sAl + frow * pa + fk;           // its lo plane (SPLIT)
      bf16x8_t fx[2], fp[2][MB], fl[2][MB];
      auto ld = [&](auto slot, auto kstep) {
        constexpr int SL = decltype(slot)::value, K0 = 16 * decltype(kstep)::value;
        u16x8_t w;
        static_for<8>([&](auto q) {
          constexpr int Q = decltype(q)::value;
          w[Q] = xcol[(K0 + Q) * px];
        });
        fx[SL] = __builtin_bit_cast(bf16x8_t, w);
        static_for<MB>([&](auto r) {
          constexpr int R = decltype(r)::value;
          fp[SL][R] = *reinterpret_cast<const bf16x8_t*>(prow + R * 32 * pa + K0);
          if constexpr (SPLIT) fl[SL][R] = *reinterpret_cast<const bf16x8_t*>(prowl + R * 32 * pa + K0);
        });
      };
      ld(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
      static_for<nkm>([&](auto k) {
        constexpr int KS = decltype(k)::value;
        if constexpr (KS + 1 < nkm) ld(std::integral_constant<int, (KS + 1) & 1>{}, std::integral_constant<int, KS + 1>{});
        static_for<MB>([&](auto r) {
          constexpr int R = decltype(r)::value;
          xa[R] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fx[KS & 1], fp[KS & 1][R], xa[R], 0, 0, 0);
          if constexpr (SPLIT) xa[R] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fx[KS & 1], fl[KS & 1][R], xa[R], 0, 0, 0);
        });
      });
      static_for<MB>([&](auto r) {
        constexpr int R = decltype(r)::value;
        static_for<4>([&](auto q) {
          constexpr int Q = decltype(q)::value;
          const f32x4_t x = unpack4(*reinterpret_cast<const u32x2_t*>(sX + xpos(R, Q)));
          static_for<4>([&](auto e) {
            constexpr int E = decltype(e)::value;
            xa[R][4 * Q + E] = fmaf(ce, x[E], ca * xa[R][4 * Q + E]);
          });
        });
      });
    }
    lds_barrier();                          // every wave is done reading X
    if (jb < nb) {
      static_for<MB>([&](auto r) {
        constexpr int R = decltype(r)::value;
        static_for<4>([&](auto q) {
          constexpr int Q = decltype(q)::value;
          const f32x4_t v{xa[R][4 * Q], xa[R][4 * Q + 1], xa[R][4 * Q + 2], xa[R][4 * Q + 3]};
          *reinterpret_cast<u32x2_t*>(sX + xpos(R, Q)) = pack4(v);
        });
      });
    }
    lds_barrier();
  }

  // ---- the result in the original layout, then the parameter write
  // 8 consecutive elements of original row i from column j (bf16 bits)
  auto orow8 = [&](int i, int j) {
    if (!tall) return *reinterpret_cast<const u32x4_t*>(sX + i * px + j);
    u16x8_t h;
    static_for<8>([&](auto r) {
      constexpr int R = decltype(r)::value;
      h[R] = sX[(j + R) * px + i];
    });
    return __builtin_bit_cast(u32x4_t, h);
  };
  if (g.O) {
    bf16_t* O = g.O + mat * g.o_stride;
    if (g.ovec) {
      const int c8 = cols / 8, nch = rows * c8;
      GridWalk w(tid, tall ? rows : c8);
      for (int c = tid; c < nch; c += kNT, w.next()) {
        const int i = tall ? w.j : w.i, j = 8 * (tall ? w.i : w.j);
        *reinterpret_cast<u32x4_t*>(O + static_cast<int64_t>(i) * g.o_ld + j) = orow8(i, j);
      }
    } else {
      GridWalk w(tid, cols);
      for (int e = tid; e < total; e += kNT, w.next()) O[static_cast<int64_t>(w.i) * g.o_ld + w.j] = sX[xat(w.i, w.j)];
    }
  }
  if (W) {
    if (vec) {
      const int c8 = cols / 8, nch = rows * c8;
      GridWalk w(tid, tall ? rows : c8);
      for (int base = 0; base < nch; base += CV * kNT) {
        int ci[CV], cj[CV];
        static_for<CV>([&](auto q) {
          constexpr int Q = decltype(q)::value;
          const bool ok = base + Q * kNT + tid < nch;
          ci[Q] = ok ? (tall ? w.j : w.i) : -1;
          cj[Q] = ok ? 8 * (tall ? w.i : w.j) : 0;
          if (!wpre) wv[Q] = load8(W + (ok ? ci[Q] : 0) * cols + cj[Q]);
          w.next();
        });
        static_for<CV>([&](auto q) {
          constexpr int Q = decltype(q)::value;
          if (ci[Q] >= 0) {
            const u32x4_t ob = orow8(ci[Q], cj[Q]);
            f32x8_t o;
            static_for<4>([&](auto r) {
              constexpr int R = decltype(r)::value;
              o[2 * R] = __uint_as_float(ob[R] << 16);
              o[2 * R + 1] = __uint_as_float(ob[R] & 0xffff0000u);
            });
            const f32x8_t nw = __builtin_elementwise_fma(f32x8_t(-g.step), o, f32x8_t(g.decay) * wv[Q]);
            store8(W + ci[Q] * cols + cj[Q], nw);
          }
        });
      }
    } else {
      GridWalk w(tid, cols);
      for (int base = 0; base < total; base += CS * kNT) {
        float wv[CS];
        int ci[CS], cj[CS];
        static_for<CS>([&](auto q) {
          constexpr int Q = decltype(q)::value;
          const bool ok = base + Q * kNT + tid < total;
          ci[Q] = ok ? w.i : -1;
          cj[Q] = ok ? w.j : 0;
          wv[Q] = load_f32(W, ok ? w.i * cols + w.j : 0);
          w.next();
        });
        static_for<CS>([&](auto q) {
          constexpr int Q = decltype(q)::value;
          if (ci[Q] >= 0) {
            const float o = bf16_to_f32(sX[xat(ci[Q], cj[Q])]);
            store_f32(W, ci[Q] * cols + cj[Q], fmaf(-g.step, o, g.decay * wv[Q]));
          }
        });
      }
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kNT) void small_step_kernel(SmallLaunch L) {
  __shared__ __attribute__((aligned(16))) bf16_t sX[kSmallMaxM * kPX];
  __shared__ __attribute__((aligned(16))) bf16_t sA[kSmallMaxM * kPA];
  __shared__ __attribute__((aligned(16))) bf16_t sAl[kThinMaxM * (kThinMaxM + 8)];
  __shared__ double red[kNT / 64];

  int gi = 0;
  while (gi + 1 < L.ngroups && static_cast<int>(blockIdx.x) >= L.prefix[gi + 1]) ++gi;
  const SmallGroup& g = L.g[gi];
  const int mat = blockIdx.x - L.prefix[gi];
  switch ((g.m + 31) / 32) {
    case 1: small_body<T, 1>(L, g, mat, sX, sA, sAl, red); break;
    case 2: small_body<T, 2>(L, g, mat, sX, sA, sAl, red); break;
    case 3: small_body<T, 3>(L, g, mat, sX, sA, sAl, red); break;
    default: small_body<T, 4>(L, g, mat, sX, sA, sAl, red); break;
  }
}

}  // namespace

hipError_t launch_small_step(const SmallLaunch& L, int dtype, int nmats, hipStream_t s) {
  if (dtype == MUON_DTYPE_BF16)
    hipLaunchKernelGGL(small_step_kernel<bf16_t>, dim3(nmats), dim3(kNT), 0, s, L);
  else
    hipLaunchKernelGGL(small_step_kernel<float>, dim3(nmats), dim3(kNT), 0, s, L);
  return hipGetLastError();
}

}  // namespace muon
