// Newton-Schulz matrix products on CDNA4 bf16 MFMA ("Muon and MuonClip:
// orthogonalised updates for LLM training", section 2, Newton-Schulz
// subsection: A = X X^T, B = b A + c A A, X <- a X + B X; "MuonClip",
// section 02, quintic step on the cheaper orientation).
//
// Every product of the iteration is an "NT" contraction whose two operands
// are row-major with the contraction index contiguous:
//   A = X X^T                P = Q = X  (m x n),  K = n, symmetric output
//   B = a I + b A + c A A^T  P = Q = A  (m x m),  K = m, symmetric output (A = A^T)
//   X' = B X                 P = B,  Q = X^T (n x m), K = m
// (a X + (b A + c A A) X is computed as (a I + b A + c A A) X: one rounding of
// the polynomial matrix, no a X term in the last product.)
// so both MFMA operands are 16-byte row segments, staged through LDS.  The
// symmetric products compute only tiles ti <= tj and write each off-diagonal
// tile twice (in place and mirrored).  X is kept in both layouts (X and X^T):
// the epilogue of X' writes both, so no transpose pass is ever needed.
//
// Tiling: TILE x TILE output per 256-thread block, 2 x 2 waves, each wave a
// (TILE/2) x (TILE/2) sub-tile of 32 x 32 MFMA blocks (v_mfma_f32_32x32x16_bf16),
// K staged 32 at a time in double-buffered, padded LDS.
#include <utility>

#include "common.hpp"

namespace muon {

namespace {

constexpr int kBK = 64;
constexpr int kPitch = kBK + 8;  // padded LDS row (bf16): 144 bytes, conflict-free b128 reads

struct EpiArgs {
  float ca, ce, cd;
  bf16_t* C;
  bf16_t* Ct;
  const bf16_t* Et;
  int ldc, ldct, lde, mvalid, nvalid, ct_vec;
  int i0, j0;  // this lane's first row and its column inside block (0, 0)
};

// Epilogue of one 32x32 MFMA block (a, b): four groups of four consecutive
// rows per lane.  Compile-time block indices keep the accumulators in
// registers.
template <int A, int B>
__device__ __forceinline__ void epilogue_block(const f32x16_t& acc, const EpiArgs& e) {
  const int j = e.j0 + 32 * B;
  if (j >= e.nvalid) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = e.i0 + 32 * A + 8 * q;
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = e.ca * acc[4 * q + r] + ((i + r == j) ? e.cd : 0.0f);
    if (e.Et) {
      const uint2 ev = *reinterpret_cast<const uint2*>(e.Et + static_cast<int64_t>(j) * e.lde + i);
      v[0] = fmaf(e.ce, bf16_to_f32(ev.x & 0xffff), v[0]);
      v[1] = fmaf(e.ce, bf16_to_f32(ev.x >> 16), v[1]);
      v[2] = fmaf(e.ce, bf16_to_f32(ev.y & 0xffff), v[2]);
      v[3] = fmaf(e.ce, bf16_to_f32(ev.y >> 16), v[3]);
    }
    bf16_t o[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = f32_to_bf16(v[r]);
    if (e.C) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (i + r < e.mvalid) e.C[static_cast<int64_t>(i + r) * e.ldc + j] = o[r];
    }
    if (e.Ct) {
      bf16_t* dst = e.Ct + static_cast<int64_t>(j) * e.ldct + i;
      if (e.ct_vec && i + 3 < e.mvalid) {
        uint2 pk;
        pk.x = static_cast<uint32_t>(o[0]) | (static_cast<uint32_t>(o[1]) << 16);
        pk.y = static_cast<uint32_t>(o[2]) | (static_cast<uint32_t>(o[3]) << 16);
        *reinterpret_cast<uint2*>(dst) = pk;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (i + r < e.mvalid) dst[r] = o[r];
      }
    }
  }
}

template <int F, int G, int... Is>
__device__ __forceinline__ void epilogue_all(const f32x16_t (&acc)[F][G], const EpiArgs& e,
                                             std::integer_sequence<int, Is...>) {
  (epilogue_block<Is / G, Is % G>(acc[Is / G][Is % G], e), ...);
}

template <int TILE, int STAGE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ns_gemm_kernel(GemmLaunch L) {
  constexpr int NT = 512;
  constexpr int WT = TILE / 2;       // wave sub-tile rows
  constexpr int WN = TILE / 4;       // wave sub-tile cols
  constexpr int F = WT / 32;         // 32x32 MFMA blocks along rows
  constexpr int G = WN / 32;         // along cols
  constexpr int CPR = kBK / 8;        // 16-byte chunks per tile row of a K slice
  constexpr int RPP = NT / CPR;       // tile rows covered by one pass of the block
  constexpr int NCH = TILE / RPP;     // passes (chunks per thread per operand)
  static_assert(TILE % RPP == 0, "staging map must cover the tile exactly");

  __shared__ __attribute__((aligned(16))) bf16_t sP[2][TILE * kPitch];
  __shared__ __attribute__((aligned(16))) bf16_t sQ[2][TILE * kPitch];

  // ---- block -> (problem, matrix, tile)
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  int gi = 0;
  while (gi + 1 < L.nprob && lin >= L.prefix[gi + 1]) ++gi;
  const GemmProb& p = L.p[gi];
  const int local = lin - L.prefix[gi];
  const int mat = local / p.tiles_per_mat;
  int t = local - mat * p.tiles_per_mat;
  int ti, tj;
  if (p.sym) {
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

  const bf16_t* Pg = p.P + mat * p.sP + static_cast<int64_t>(ti) * TILE * p.ldp;
  const bf16_t* Qg = p.Q + mat * p.sQ + static_cast<int64_t>(tj) * TILE * p.ldq;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr0 = (wave >> 2) * WT;  // wave row offset in the tile
  const int wc0 = (wave & 3) * WN;   // wave col offset in the tile

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
  u32x4_t rP[NCH], rQ[NCH];
  const int KT = p.K / kBK;
  auto gload = [&](int kslice) {
    const int kb = min(kslice, KT - 1) * kBK * 2;
    static_for<NCH>([&](auto c) {
      rP[c] = __builtin_amdgcn_raw_buffer_load_b128(rsP, vP, kb + c * sstrP, 0);
      rQ[c] = __builtin_amdgcn_raw_buffer_load_b128(rsQ, vQ, kb + c * sstrQ, 0);
    });
  };
  auto sstore = [&](int buf) {
    char* bP = reinterpret_cast<char*>(sP[buf]) + sOff;
    char* bQ = reinterpret_cast<char*>(sQ[buf]) + sOff;
    static_for<NCH>([&](auto c) {
      *reinterpret_cast<u32x4_t*>(bP + c * RPP * kPitch * 2) = rP[c];
      *reinterpret_cast<u32x4_t*>(bQ + c * RPP * kPitch * 2) = rQ[c];
    });
  };
  // barrier without the workgroup fence of __syncthreads (that fence would
  // drain the prefetch loads): this wave's LDS traffic done, then s_barrier
  auto barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
  };

  f32x16_t acc[F][G];
  static_for<F * G>([&](auto ab) { acc[ab / G][ab % G] = f32x16_t{}; });

  const int frow = lane & 31;
  const int fk = (lane >> 5) * 8;
  const int aoff = ((wr0 + frow) * kPitch + fk) * 2;
  const int boff = ((wc0 + frow) * kPitch + fk) * 2;
  bf16x8_t fa[2][F], fb[2][G];
  auto read_frags = [&](int buf, int s, auto slot) {
    const char* bP = reinterpret_cast<const char*>(sP[buf]) + aoff + s * 32;
    const char* bQ = reinterpret_cast<const char*>(sQ[buf]) + boff + s * 32;
    static_for<F>([&](auto a) { fa[slot][a] = *reinterpret_cast<const bf16x8_t*>(bP + a * 32 * kPitch * 2); });
    static_for<G>([&](auto b) { fb[slot][b] = *reinterpret_cast<const bf16x8_t*>(bQ + b * 32 * kPitch * 2); });
  };
  auto mfmas = [&](auto slot) {
    static_for<F * G>([&](auto ab) {
      constexpr int A = decltype(ab)::value / G, B = decltype(ab)::value % G;
      acc[A][B] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][A], fb[slot][B], acc[A][B], 0, 0, 0);
    });
  };
  // interleave: per MFMA one LDS read (first 2F MFMAs), optionally global loads
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
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    static_for<S - 1>([&](auto s) {
      constexpr int SS = decltype(s)::value;
      read_frags(cur, SS + 1, std::integral_constant<int, (SS + 1) & 1>{});
      if constexpr (SS == S - 2) {
        // stage slice kt+1 (loaded one iteration ago), then prefetch kt+2
        sstore(cur ^ 1);
        gload(kt + 2);
      }
      mfmas(std::integral_constant<int, SS & 1>{});
      pattern(SS == S - 2 ? 2 * NCH : 0, SS == S - 2 ? 2 * NCH : 0);
    });
    barrier();
    read_frags(cur ^ 1, 0, std::integral_constant<int, 0>{});
    mfmas(std::integral_constant<int, (S - 1) & 1>{});
    pattern(0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);

  // ---- epilogue.  Element e of acc[a][b] holds C[i][j] with
  //   i = tile_i0 + wr0 + 32 a + 8 (e / 4) + 4 (lane / 32) + (e % 4),
  //   j = tile_j0 + wc0 + 32 b + (lane % 32).
  float sc = 1.0f;
  if (p.alpha_pow) {
    const float al = p.alpha[mat];
    sc = (p.alpha_pow == 2) ? al * al : al;
  }
  EpiArgs e;
  e.ca = p.c_acc * sc;
  e.ce = p.c_e * sc;
  e.cd = p.c_diag * sc;
  e.C = p.C ? p.C + mat * p.sC : nullptr;
  e.Ct = (p.Ct && (!p.sym || ti != tj)) ? p.Ct + mat * p.sCt : nullptr;
  e.Et = p.Et ? p.Et + mat * p.sEt : nullptr;
  e.ldc = p.ldc; e.ldct = p.ldct; e.lde = p.lde;
  e.mvalid = p.mvalid; e.nvalid = p.nvalid; e.ct_vec = p.ct_vec;
  e.i0 = ti * TILE + wr0 + 4 * (lane >> 5);
  e.j0 = tj * TILE + wc0 + (lane & 31);
  epilogue_all<F, G>(acc, e, std::make_integer_sequence<int, F * G>{});
}

}  // namespace

hipError_t launch_ns_gemm(const GemmLaunch& L, int tile, int stage, int nblocks, hipStream_t s) {
  // one symbol per (tile, stage) so kernel traces attribute time per product
  const dim3 grid(nblocks), block(512);
  if (tile == 256) {
    if (stage == 0) hipLaunchKernelGGL((ns_gemm_kernel<256, 0>), grid, block, 0, s, L);
    else if (stage == 1) hipLaunchKernelGGL((ns_gemm_kernel<256, 1>), grid, block, 0, s, L);
    else hipLaunchKernelGGL((ns_gemm_kernel<256, 2>), grid, block, 0, s, L);
  } else {
    if (stage == 0) hipLaunchKernelGGL((ns_gemm_kernel<128, 0>), grid, block, 0, s, L);
    else if (stage == 1) hipLaunchKernelGGL((ns_gemm_kernel<128, 1>), grid, block, 0, s, L);
    else hipLaunchKernelGGL((ns_gemm_kernel<128, 2>), grid, block, 0, s, L);
  }
  return hipGetLastError();
}

}  // namespace muon
