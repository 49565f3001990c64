// Newton-Schulz matrix products on CDNA4 bf16 MFMA ("Muon and MuonClip:
// orthogonalised updates for LLM training", section 2, Newton-Schulz
// subsection: A = X X^T, B = b A + c A A, X <- a X + B X; "MuonClip",
// section 02, quintic step on the cheaper orientation).
//
// Every product of the iteration is an "NT" contraction whose two operands
// are row-major with the contraction index contiguous:
//   A = X X^T                P = Q = X  (m x n),  K = n, symmetric output
//   B = b A + c A A^T        P = Q = A  (m x m),  K = m, symmetric output (A = A^T)
//   X' = a X + B X           P = B,  Q = X^T (n x m), K = m
// so both MFMA operands are 16-byte row segments, staged through LDS.  The
// b A and a X terms are added in fp32 in the epilogue, from the stored bf16
// A and X (folding a I into B would round a + B_ii to bf16).  The
// symmetric products compute only tiles ti <= tj and write each off-diagonal
// tile twice (in place and mirrored).  X is kept in both layouts (X and X^T):
// the epilogue of X' writes both, so no transpose pass is ever needed.
//
// Tiling: TILE x TILE output per 512-thread block, 2 x 4 waves, each wave a
// (TILE/2) x (TILE/4) sub-tile of 32 x 32 MFMA blocks (v_mfma_f32_32x32x16_bf16),
// K staged 64 at a time in double-buffered, padded LDS.  When a symmetric
// product's tile count leaves a partial last wave on the chip, those last
// tiles run instead as 256 x 128 column halves (4 x 2 waves of 64 x 64) in a
// second launch: twice the blocks at half the work each, with every output
// element accumulated over K in the same order as in a whole tile.
#include <utility>

#include "common.hpp"

namespace muon {

namespace {

constexpr int kBK = 64;
constexpr int kPitch = kBK + 8;  // padded LDS row (bf16): 144 bytes, conflict-free b128 reads

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

// Output values of one lane for MFMA block (A, B), row group Qd: four
// consecutive rows i0 + 32 A + 8 Qd + (0..3) of column j0 + 32 B, as fp32
//   v = ca * acc + ce * Et[j][i]
// rounded once to bf16 (v_cvt_pk_bf16_f32, nearest-even), two per dword.
struct EpiArgs {
  float ca, ce;
  const bf16_t* Et;   // staged Et tile in LDS (row pitch lde), or null
  int lde;
  int li0, lj0;       // this lane's first row / column inside the tile (block (0, 0))
  int ljE;            // this lane's first row of the staged E tile (Et)
};

template <int A, int B, int Qd>
__device__ __forceinline__ u32x2_t epi_quad(const f32x16_t& acc, const EpiArgs& e) {
  f32x4_t v;
  static_for<4>([&](auto r) {
    constexpr int R = decltype(r)::value;
    v[R] = e.ca * acc[4 * Qd + R];
  });
  if (e.Et) {
    // the Et tile staged in LDS, layout [j][i]
    const u32x2_t ev = *reinterpret_cast<const u32x2_t*>(e.Et + (e.ljE + 32 * B) * e.lde + e.li0 + 32 * A + 8 * Qd);
    v[0] = fmaf(e.ce, bf16_to_f32(ev[0] & 0xffff), v[0]);
    v[1] = fmaf(e.ce, bf16_to_f32(ev[0] >> 16), v[1]);
    v[2] = fmaf(e.ce, bf16_to_f32(ev[1] & 0xffff), v[2]);
    v[3] = fmaf(e.ce, bf16_to_f32(ev[1] >> 16), v[3]);
  }
  return __builtin_bit_cast(u32x2_t, __builtin_convertvector(v, bf16x4_t));
}

// Stage the ROWS x COLS block src[r0 + r][c0 + c] (leading dimension ld) in
// LDS with row pitch EP.  The caller guarantees the whole block lies inside
// src (the epilogue's E operand is always a padded workspace matrix).
template <int ROWS, int COLS, int EP, int NT>
__device__ __forceinline__ void copy_in(bf16_t* st, const bf16_t* src, int ld, int r0, int c0, int tid) {
  constexpr int CPRW = COLS / 8;
  constexpr int N = ROWS * CPRW / NT;
  static_assert(ROWS * CPRW % NT == 0, "copy map must cover the block exactly");
  static_for<N>([&](auto k) {
    const int c = tid + NT * decltype(k)::value;
    const int row = c / CPRW, cc = (c % CPRW) * 8;
    *reinterpret_cast<u32x4_t*>(st + row * EP + cc) =
        *reinterpret_cast<const u32x4_t*>(src + static_cast<int64_t>(r0 + row) * ld + c0 + cc);
  });
}

// Copy a ROWS x COLS bf16 block staged in LDS (row pitch EP elements) to
// dst[r][c] (leading dimension ld), rows < rvalid - r0, cols < cvalid - c0,
// 16 bytes per store where the chunk is whole and aligned.
template <int ROWS, int COLS, int EP, int NT>
__device__ __forceinline__ void copy_out(const bf16_t* st, bf16_t* dst, int ld, int r0, int c0, int rvalid,
                                         int cvalid, bool vec16, int tid) {
  constexpr int CPRW = COLS / 8;
  constexpr int N = ROWS * CPRW / NT;
  static_assert(ROWS * CPRW % NT == 0, "copy map must cover the block exactly");
#pragma unroll 4
  for (int k = 0; k < N; ++k) {
    const int c = tid + NT * k;
    const int row = c / CPRW, cc = (c % CPRW) * 8;
    const int gr = r0 + row, gc = c0 + cc;
    if (gr >= rvalid || gc >= cvalid) continue;
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(st + row * EP + cc);
    bf16_t* d = dst + static_cast<int64_t>(gr) * ld + gc;
    if (vec16 && gc + 7 < cvalid) {
      *reinterpret_cast<u32x4_t*>(d) = w;
    } else {
      for (int q = 0; q < 8 && gc + q < cvalid; ++q)
        d[q] = static_cast<bf16_t>((w[q >> 1] >> (16 * (q & 1))) & 0xffff);
    }
  }
}

// One block computes a TM x TN output tile of a product whose tiles are
// TM x TM (TN = TM), or one of the TM / TN column slices of such a tile
// (TN < TM: the slices of the last, partial wave of a launch).  Eight waves in
// a WR x WC grid.
template <int TM, int TN, int STAGE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ns_gemm_kernel(GemmLaunch L) {
  constexpr int NT = 512;
  constexpr int WC = (TN == TM) ? 4 : 2;   // waves along the tile's columns
  constexpr int WR = 8 / WC;               // and rows
  constexpr int WT = TM / WR;              // wave sub-tile rows
  constexpr int WN = TN / WC;              // wave sub-tile cols
  constexpr int F = WT / 32;               // 32x32 MFMA blocks along rows
  constexpr int G = WN / 32;               // along cols
  constexpr int NSLICE = TM / TN;          // column slices per tile
  constexpr int CPR = kBK / 8;             // 16-byte chunks per tile row of a K slice
  constexpr int RPP = NT / CPR;            // tile rows covered by one pass of the block
  constexpr int NCP = TM / RPP;            // passes (chunks per thread) for P
  constexpr int NCQ = TN / RPP;            // and for Q
  static_assert(TM % RPP == 0 && TN % RPP == 0, "staging map must cover the tile exactly");
  static_assert(F >= 1 && G >= 1 && TM % TN == 0, "wave grid must fit the tile");

  // two stages of the P and Q slices; the epilogue reuses the whole buffer
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * (TM + TN) * kPitch];
  auto sP = [&](int buf) { return smem + buf * (TM + TN) * kPitch; };   // a stage: P then Q slice
  auto sQ = [&](int buf) { return smem + buf * (TM + TN) * kPitch + TM * kPitch; };

  // ---- block -> (problem, matrix, tile, column slice)
  int vb, slice = 0;
  if (NSLICE == 1) {
    vb = blockIdx.x;
  } else {
    // the slices of one tile are adjacent in each XCD's contiguous range, so
    // they mostly share that XCD's cache for the common P panel
    const int r = xcd_remap(blockIdx.x, gridDim.x);
    vb = L.lin0 + r / NSLICE;
    slice = r % NSLICE;
  }
  int gi = 0;
  while (gi + 1 < L.nprob && vb >= L.prefix[gi + 1]) ++gi;
  const GemmProb& p = L.p[gi];
  // Each problem's index range is a multiple of 8 long, so index b runs on
  // XCD b % 8 whatever problem it falls in; inside a problem each XCD takes
  // one contiguous eighth of its tiles (column bands: see below).  Every XCD
  // thus gets the same share of each problem, whatever their contraction
  // lengths.
  const int lb = vb - L.prefix[gi];
  const int local = L.band ? lb : xcd_remap(lb, L.prefix[gi + 1] - L.prefix[gi]);
  if (local >= p.ntiles) return;   // padding of the problem's range
  int mat = local / p.tiles_per_mat;
  int t = local - mat * p.tiles_per_mat;
  int ti, tj;
  if (L.band) {
    // Column bands: block i runs on XCD x = i % 8, which owns columns
    // [x tn/8, (x+1) tn/8) of every matrix; every XCD walks the same 8-row
    // group at the same time (each problem's block range starts at a
    // multiple of 8), so the row panels they share come from the
    // memory-side cache rather than HBM.  Inside a group, column-major.
    const int x = local & 7, w = local >> 3;
    const int bw = p.tn / 8;
    const int per = p.tm * bw;
    mat = w / per;
    const int u = w - mat * per;
    const int g8 = u / (8 * bw);
    const int rows = min(8, p.tm - 8 * g8);
    const int v = u - g8 * 8 * bw;
    ti = 8 * g8 + v % rows;
    tj = x * bw + v / rows;
  } else if (p.sym) {
    {
      constexpr int SB = 8;
      // super-blocks of SB x SB tiles over the upper triangle, row-major over
      // super-blocks; inside a super-block column-major (upper part only on the
      // diagonal super-blocks)
      const int nsb = (p.tm + SB - 1) / SB;
      int bi = 0, bj = 0, found = 0;
      for (bi = 0; bi < nsb && !found; ++bi) {
        for (bj = bi; bj < nsb; ++bj) {
          const int r0 = bi * SB, c0 = bj * SB;
          const int rn = min(SB, p.tm - r0), cn = min(SB, p.tm - c0);
          int cnt = 0;
          if (bi == bj) cnt = rn * (rn + 1) / 2; else cnt = rn * cn;
          if (t < cnt) {
            if (bi == bj) {
              int cc = 0;
              while (t >= cc + 1) { t -= cc + 1; ++cc; }   // column cc holds rows 0..cc
              ti = r0 + t; tj = c0 + cc;
            } else {
              ti = r0 + t % rn; tj = c0 + t / rn;
            }
            found = 1;
            break;
          }
          t -= cnt;
        }
      }
    }
  } else {
    constexpr int GM = 8;
    const int gsz = GM * p.tn;
    const int grp = t / gsz;
    const int first = grp * GM;
    const int gm = min(p.tm - first, GM);
    const int r = t - grp * gsz;
    ti = first + r % gm;
    tj = r / gm;
  }
  const int row0 = ti * TM;                 // first output row of this block
  const int col0 = tj * TM + slice * TN;    // first output column

  const bf16_t* Pg = p.P + mat * p.sP + static_cast<int64_t>(row0) * p.ldp;
  const bf16_t* Qg = p.Q + mat * p.sQ + static_cast<int64_t>(col0) * p.ldq;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr0 = (wave / WC) * WT;  // wave row offset in the tile
  const int wc0 = (wave % WC) * WN;  // wave col offset in the tile

  // global -> register staging map: chunk c of this thread covers tile row
  // (tid / CPR + RPP * c), 8 bf16 at column 8 * (tid % CPR) of the K slice.
  const int lrow = tid / CPR;
  const int lkc = (tid % CPR) * 8;

  // global -> register staging through buffer loads: chunk c of this thread
  // is tile row lrow + RPP*c, 16 bytes at column lkc of the K slice
  const __amdgpu_buffer_rsrc_t rsP = __builtin_amdgcn_make_buffer_rsrc((void*)Pg, 0, 0x7fffffff, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsQ = __builtin_amdgcn_make_buffer_rsrc((void*)Qg, 0, 0x7fffffff, 0x00020000);
  const int vP = (lrow * p.ldp + lkc) * 2;
  const int vQ = (lrow * p.ldq + lkc) * 2;
  const int sstrP = RPP * p.ldp * 2, sstrQ = RPP * p.ldq * 2;
  const int sOff = (lrow * kPitch + lkc) * 2;   // bytes inside an LDS stage
  u32x4_t rP[NCP], rQ[NCQ];
  const int KT = p.K / kBK;
  auto gload = [&](int kslice) {
    const int kb = min(kslice, KT - 1) * kBK * 2;
    static_for<NCP>([&](auto c) { rP[c] = __builtin_amdgcn_raw_buffer_load_b128(rsP, vP, kb + c * sstrP, 0); });
    static_for<NCQ>([&](auto c) { rQ[c] = __builtin_amdgcn_raw_buffer_load_b128(rsQ, vQ, kb + c * sstrQ, 0); });
  };
  auto sstore = [&](int buf) {
    char* bP = reinterpret_cast<char*>(sP(buf)) + sOff;
    char* bQ = reinterpret_cast<char*>(sQ(buf)) + sOff;
    static_for<NCP>([&](auto c) { *reinterpret_cast<u32x4_t*>(bP + c * RPP * kPitch * 2) = rP[c]; });
    static_for<NCQ>([&](auto c) { *reinterpret_cast<u32x4_t*>(bQ + c * RPP * kPitch * 2) = rQ[c]; });
  };
  // LDS-only barrier: the prefetch loads stay in flight across it
  auto barrier = [&]() { lds_barrier(); };

  f32x16_t acc[F][G];
  static_for<F * G>([&](auto ab) { acc[ab / G][ab % G] = f32x16_t{}; });

  const int frow = lane & 31;
  const int fk = (lane >> 5) * 8;
  const int aoff = ((wr0 + frow) * kPitch + fk) * 2;
  const int boff = ((wc0 + frow) * kPitch + fk) * 2;
  bf16x8_t fa[2][F], fb[2][G];
  auto read_frags = [&](int buf, int s, auto slot) {
    const char* bP = reinterpret_cast<const char*>(sP(buf)) + aoff + s * 32;
    const char* bQ = reinterpret_cast<const char*>(sQ(buf)) + boff + s * 32;
    static_for<F>([&](auto a) { fa[slot][a] = *reinterpret_cast<const bf16x8_t*>(bP + a * 32 * kPitch * 2); });
    static_for<G>([&](auto b) { fb[slot][b] = *reinterpret_cast<const bf16x8_t*>(bQ + b * 32 * kPitch * 2); });
  };
  auto mfmas = [&](auto slot) {
    static_for<F * G>([&](auto ab) {
      constexpr int A = decltype(ab)::value / G, B = decltype(ab)::value % G;
      acc[A][B] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][A], fb[slot][B], acc[A][B], 0, 0, 0);
    });
  };
  // interleave: per MFMA one LDS read (first F+G MFMAs), optionally global loads
  auto pattern = [&](int nv, int nw) {
    for (int q = 0; q < F * G; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (q < F + G) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (q < nv) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      if (q < nw) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    }
  };
  constexpr int S = kBK / 16;   // 4 K-substeps per slice

  gload(0);
  sstore(0);
  gload(1);
  barrier();
  read_frags(0, 0, std::integral_constant<int, 0>{});
  // The E tile of whole 256-tiles (the epilogue's a X or b A term) rides in
  // the last two K slices' prefetch slots, which would otherwise repeat the
  // last slice: rows 128-255 during the second-to-last slice (then staged in
  // the spare LDS stage during the last), rows 0-127 during the last (staged
  // by the epilogue).  8 chunks per thread in the copy-in map per half.
  constexpr bool PRE = (TM == 256 && TN == 256);
  constexpr int EPT = TM + 8;                  // staged Ct / Et tile row pitch, TN rows
  static_assert(!PRE || (NCP + NCQ == 128 * (TM / 8) / NT && 128 * EPT <= (TM + TN) * kPitch),
                "an E half must fill the staging registers and fit one stage");
  const bool pre = PRE && p.Et != nullptr;
  const int er = tid / (TM / 8), ec = (tid % (TM / 8)) * 8;   // this thread's E chunk
  auto gload_e = [&](int half) {
    const bf16_t* E = p.Et + mat * p.sEt + static_cast<int64_t>(col0 + 128 * half) * p.lde + row0;
    const int r = er, cc = ec;
    static_for<NCP>([&](auto c) {
      rP[c] = *reinterpret_cast<const u32x4_t*>(E + static_cast<int64_t>(r + (NT / (TM / 8)) * c) * p.lde + cc);
    });
    static_for<NCQ>([&](auto c) {
      rQ[c] = *reinterpret_cast<const u32x4_t*>(E + static_cast<int64_t>(r + (NT / (TM / 8)) * (NCP + c)) * p.lde + cc);
    });
  };
  // an E half in the staging registers, to rows 0-127 of a stage-sized region
  auto sstore_e = [&](bf16_t* base) {
    static_for<NCP>([&](auto c) {
      *reinterpret_cast<u32x4_t*>(base + (er + (NT / (TM / 8)) * c) * EPT + ec) = rP[c];
    });
    static_for<NCQ>([&](auto c) {
      *reinterpret_cast<u32x4_t*>(base + (er + (NT / (TM / 8)) * (NCP + c)) * EPT + ec) = rQ[c];
    });
  };
  // one K slice: MODE 0 stages slice kt + 1 and prefetches kt + 2; MODE 1
  // (second-to-last) stages the last slice and fetches E rows 128-255;
  // MODE 2 (last) stages those E rows into the spare stage and fetches rows 0-127
  auto kslice = [&](int kt, auto mode) {
    constexpr int MODE = decltype(mode)::value;
    const int cur = kt & 1;
    static_for<S - 1>([&](auto s) {
      constexpr int SS = decltype(s)::value;
      read_frags(cur, SS + 1, std::integral_constant<int, (SS + 1) & 1>{});
      if constexpr (SS == S - 2 && MODE == 0) {
        // stage slice kt+1 (loaded one iteration ago), then prefetch kt+2
        sstore(cur ^ 1);
        gload(kt + 2);
      }
      if constexpr (SS == S - 2 && MODE == 1) {
        sstore(cur ^ 1);
        if (pre) gload_e(1);
      }
      if constexpr (SS == S - 2 && MODE == 2) {
        if (pre) {
          sstore_e(sP(cur ^ 1));
          gload_e(0);
        }
      }
      mfmas(std::integral_constant<int, SS & 1>{});
      pattern(SS == S - 2 && MODE == 0 ? NCP + NCQ : 0, SS == S - 2 && MODE == 0 ? NCP + NCQ : 0);
    });
    if constexpr (MODE != 2) {
      barrier();
      read_frags(cur ^ 1, 0, std::integral_constant<int, 0>{});
    }
    mfmas(std::integral_constant<int, (S - 1) & 1>{});
    pattern(0, 0);
  };
  for (int kt = 0; kt < KT - 2; ++kt) kslice(kt, std::integral_constant<int, 0>{});
  kslice(KT - 2, std::integral_constant<int, 1>{});
  kslice(KT - 1, std::integral_constant<int, 2>{});
  __builtin_amdgcn_s_waitcnt(0);

  // ---- epilogue.  Element e of acc[a][b] holds C[i][j] with
  //   i = row0 + wr0 + 32 a + 8 (e / 4) + 4 (lane / 32) + (e % 4),
  //   j = col0 + wc0 + 32 b + (lane % 32).
  // The rounded tile goes through LDS so both layouts leave in 16-byte
  // stores of whole rows (direct stores from this layout would be 2- or
  // 8-byte pieces of many cache lines).
  float sc = 1.0f;
  if (p.alpha_pow) {
    const float al = p.alpha[mat];
    sc = (p.alpha_pow == 2) ? al * al : al;
  }
  constexpr int EPC = TN + 8;                  // staged C tile row pitch (bf16), TM rows
  static_assert(TM * EPC <= 2 * (TM + TN) * kPitch && TN * EPT <= 2 * (TM + TN) * kPitch,
                "staged tile must fit the LDS buffer");
  EpiArgs e;
  e.ca = p.c_acc * sc;
  e.ce = p.c_e * sc;
  e.Et = nullptr;
  e.lde = EPT;
  e.li0 = wr0 + 4 * (lane >> 5);
  e.lj0 = wc0 + (lane & 31);
  e.ljE = e.lj0;
  bf16_t* C = p.C ? p.C + mat * p.sC : nullptr;
  bf16_t* Ct = (p.Ct && (!p.sym || ti != tj)) ? p.Ct + mat * p.sCt : nullptr;
  lds_barrier();                // every wave is done with the K slices
  if (pre) {
    // E rows 128-255 wait in the spare stage (KT & 1); rows 0-127, in the
    // registers, go to the stage the last K slice used
    sstore_e(sP((KT - 1) & 1));
    lds_barrier();
    const bool hi = wc0 >= 128;
    e.Et = sP(hi ? KT & 1 : (KT - 1) & 1);
    e.ljE = hi ? e.lj0 - 128 : e.lj0;
  } else if (p.Et) {
    // E[j][i] block (the transposed layout of this output block), coalesced into LDS
    copy_in<TN, TM, EPT, NT>(smem, p.Et + mat * p.sEt, p.lde, col0, row0, tid);
    lds_barrier();
    e.Et = smem;
  }
  u32x2_t quad[F][G][4];
  static_for<F * G * 4>([&](auto x) {
    constexpr int X = decltype(x)::value;
    constexpr int A = X / (4 * G), B = (X / 4) % G, Qd = X % 4;
    quad[A][B][Qd] = epi_quad<A, B, Qd>(acc[A][B], e);
  });
  const int li0 = e.li0;                       // local row of quad (0, 0, 0)
  const int lj0 = e.lj0;                       // local column of block (., 0)
  if (p.Et) {
    lds_barrier();              // the staged E tile is read; reuse the buffer
  }
  if (Ct) {
    // transposed layout [j][i]: each quad is 4 consecutive i of one j
    static_for<F * G * 4>([&](auto x) {
      constexpr int X = decltype(x)::value;
      constexpr int A = X / (4 * G), B = (X / 4) % G, Qd = X % 4;
      *reinterpret_cast<u32x2_t*>(smem + (lj0 + 32 * B) * EPT + li0 + 32 * A + 8 * Qd) = quad[A][B][Qd];
    });
    lds_barrier();
    copy_out<TN, TM, EPT, NT>(smem, Ct, p.ldct, col0, row0, p.nvalid, p.mvalid, p.ct16 != 0, tid);
    lds_barrier();
  }
  if (C) {
    // row-major layout [i][j]
    static_for<F * G * 4>([&](auto x) {
      constexpr int X = decltype(x)::value;
      constexpr int A = X / (4 * G), B = (X / 4) % G, Qd = X % 4;
      bf16_t* d = smem + (li0 + 32 * A + 8 * Qd) * EPC + lj0 + 32 * B;
      const u32x2_t w = quad[A][B][Qd];
      d[0] = static_cast<bf16_t>(w[0] & 0xffff);
      d[EPC] = static_cast<bf16_t>(w[0] >> 16);
      d[2 * EPC] = static_cast<bf16_t>(w[1] & 0xffff);
      d[3 * EPC] = static_cast<bf16_t>(w[1] >> 16);
    });
    lds_barrier();
    copy_out<TM, TN, EPC, NT>(smem, C, p.ldc, row0, col0, p.mvalid, p.nvalid, p.c16 != 0, tid);
  }
}

}  // namespace

hipError_t launch_ns_gemm(const GemmLaunch& L, int tile, int stage, int nblocks, hipStream_t s) {
  // one symbol per (tile, stage) so kernel traces attribute time per product
  const dim3 grid(nblocks), block(512);
  if (tile == 256) {
    if (stage == 0) hipLaunchKernelGGL((ns_gemm_kernel<256, 256, 0>), grid, block, 0, s, L);
    else if (stage == 1) hipLaunchKernelGGL((ns_gemm_kernel<256, 256, 1>), grid, block, 0, s, L);
    else hipLaunchKernelGGL((ns_gemm_kernel<256, 256, 2>), grid, block, 0, s, L);
  } else {
    if (stage == 0) hipLaunchKernelGGL((ns_gemm_kernel<128, 128, 0>), grid, block, 0, s, L);
    else if (stage == 1) hipLaunchKernelGGL((ns_gemm_kernel<128, 128, 1>), grid, block, 0, s, L);
    else hipLaunchKernelGGL((ns_gemm_kernel<128, 128, 2>), grid, block, 0, s, L);
  }
  return hipGetLastError();
}

hipError_t launch_ns_gemm_slices(const GemmLaunch& L, int stage, int nblocks, hipStream_t s) {
  // 256 x 128 column slices of 256-tiles: blocks 2u and 2u + 1 (after the XCD
  // remap) are the two halves of tile L.lin0 + u
  const dim3 grid(nblocks), block(512);
  if (stage == 0) hipLaunchKernelGGL((ns_gemm_kernel<256, 128, 0>), grid, block, 0, s, L);
  else if (stage == 1) hipLaunchKernelGGL((ns_gemm_kernel<256, 128, 1>), grid, block, 0, s, L);
  else hipLaunchKernelGGL((ns_gemm_kernel<256, 128, 2>), grid, block, 0, s, L);
  return hipGetLastError();
}

}  // namespace muon
