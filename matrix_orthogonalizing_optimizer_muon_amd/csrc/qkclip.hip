// QK-Clip on CDNA4: the per-head maximum pre-softmax logit and the per-head
// W_q / W_k rescale.
//
// S_max^h = logit_scale * max over batch rows, i and j (j <= i when causal)
// of q_i^h . k_j^h ("Muon and MuonClip: orthogonalised updates for LLM
// training", "The exploding-logit problem"; "MuonClip", section 05 per-head
// signal).  gamma_h = min(1, tau / S_max^h); rows of head h in W_q scale by
// gamma^alpha and in W_k by gamma^(1 - alpha) ("MuonClip", section 05
// balanced rescale; "About Muon: Muon At Scale", "When Softmax Collapses").
//
// The statistic is a causal Q K^T contraction reduced by max, so it runs as
// a flash-style MFMA loop: one block per (batch row, head, 512 queries for
// d = 128, 256 otherwise), the queries' fragments held in registers, 64-key
// blocks (128 for d = 64) staged through LDS, the logits never stored.
// Maxima are reduced across the wavefront with cross-lane max, across the
// block through LDS, and across blocks by a second, fixed-order kernel (no
// atomics, no initialisation pass).  Blocks are numbered heaviest query block
// first: each XCD (block b runs on XCD b % 8) owns a contiguous range of
// (batch row, head) pairs and walks it in groups of 8, the group's query
// blocks heaviest first, so the long causal rows start first on every CU, the
// short ones fill the end, and the group's heads share the XCD's L2 for K.
// Head counts that do not split that way take the same order across all
// pairs.
#include <algorithm>
#include <mutex>

#include "common.hpp"

// Scratch of qkclip_rowmax_noalloc: the row-max pass's per-block partial
// maxima, for callers that cannot allocate.  Each GPU the library runs on
// holds its own copy until the process ends.  Host code never uses this name
// as an address (on the host it is a stand-in, not device memory): the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) float scratch[muon::kNoAllocPartials];

namespace muon {

hipError_t noalloc_partials(float** out) {
  static std::mutex mu;
  static float* ptrs[kMaxDevices] = {nullptr};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptrs[dev] = static_cast<float*>(p);
  }
  *out = ptrs[dev];
  return hipSuccess;
}

namespace {

constexpr int kQB = 256;   // queries per block (4 waves x 64)
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// d = 64 and 256: one block = 256 consecutive queries of one (batch row,
// head); 4 waves of 64 query rows, one per SIMD, and two blocks per CU: their
// barriers are independent, so one block's MFMAs run while the other stages
// keys or waits.  The queries' fragments stay in registers for
// the whole key sweep; KB keys at a time are staged through double-buffered
// LDS (registers one stage ahead, barrier without the workgroup fence so the
// prefetch stays in flight).  Logits are reduced by max in registers; only
// blocks on the causal diagonal (or the ragged tail) evaluate the mask.
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void qk_rowmax_kernel(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, int B,
                      int T, int H, int causal, float* __restrict__ partial, int nqb) {
  constexpr int KB = (D == 64) ? 128 : 64;    // keys per LDS stage
  constexpr int NB = KB / 32;                 // 32-key MFMA blocks per stage
  constexpr int PITCH = D + 8;                // padded LDS row, bf16 units
  constexpr int KS = D / 16;                  // MFMA K-substeps
  constexpr int CPR = D / 8;                  // 16-byte chunks per key row
  constexpr int RPP = kThreads / CPR;         // key rows per pass
  constexpr int NCH = KB / RPP;               // chunks per thread per stage
  static_assert(KB % RPP == 0, "staging map must cover the stage exactly");
  __shared__ __attribute__((aligned(16))) bf16_t sK[2][KB * PITCH];
  __shared__ float wmax[kWaves];
  __shared__ int wnan[kWaves];

  const int nbh = B * H;
  int bh, qb;
  if (!xcd_group_order(blockIdx.x, nbh, nqb, 8, &bh, &qb)) {
    bh = blockIdx.x % nbh;                 // heaviest query blocks of every pair first
    qb = nqb - 1 - blockIdx.x / nbh;
  }
  const int b = bh / H, h = bh - b * H;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row_stride = static_cast<int64_t>(H) * D;
  const bf16_t* Qb = Q + static_cast<int64_t>(b) * T * row_stride + static_cast<int64_t>(h) * D;
  const bf16_t* Kb = K + static_cast<int64_t>(b) * T * row_stride + static_cast<int64_t>(h) * D;

  const int r0 = qb * kQB + wave * 64;  // first query row of this wave
  const int frow = lane & 31, fk = (lane >> 5) * 8;

  // Rows past T load row T - 1 instead (every load unconditional, so the
  // compiler can count outstanding loads instead of draining them all before
  // each LDS store); their logits are masked out below.
  bf16x8_t qf[2][KS];
  static_for<2>([&](auto a) {
    const int row = min(r0 + a * 32 + frow, T - 1);
    static_for<KS>([&](auto s) {
      qf[a][s] = *reinterpret_cast<const bf16x8_t*>(Qb + row * row_stride + s * 16 + fk);
    });
  });

  const int kend = causal ? min(T, (qb + 1) * kQB) : T;
  const int nkb = (kend + KB - 1) / KB;

  const int lrow = tid / CPR, lcol = (tid % CPR) * 8;
  // NS register sets: key block kb + NS is loaded while kb computes; with two
  // sets, kb + 1 waits in the other one for the LDS buffer kb leaves (one set
  // for d = 256, whose query fragments take the registers)
  constexpr int NS = (D <= 128) ? 2 : 1;
  u32x4_t rk[NS][NCH];
  auto gload = [&](int kb, auto set) {
    constexpr int SET = decltype(set)::value;
    static_for<NCH>([&](auto c) {
      const int j = min(kb * KB + lrow + c * RPP, T - 1);
      rk[SET][c] = *reinterpret_cast<const u32x4_t*>(Kb + j * row_stride + lcol);
    });
  };
  auto sstore = [&](int buf, auto set) {
    constexpr int SET = decltype(set)::value;
    static_for<NCH>([&](auto c) {
      *reinterpret_cast<u32x4_t*>(&sK[buf][(lrow + c * RPP) * PITCH + lcol]) = rk[SET][c];
    });
  };
  // LDS-only barrier: the prefetch loads stay in flight across it
  auto barrier = [&]() { lds_barrier(); };

  float m = -INFINITY;

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // prefetches past the last key block reload the last block into a set
  // that is never stored, rather than branching around the loads
  gload(0, S0{});
  if constexpr (NS == 2) gload(min(1, nkb - 1), S1{});
  sstore(0, S0{});
  barrier();
  auto body = [&](int kb, auto par) {
    constexpr int P = decltype(par)::value;
    constexpr int LS = (NS == 2) ? P : 0;          // set receiving block kb + NS
    constexpr int SS = (NS == 2) ? (P ^ 1) : 0;    // set holding block kb + 1
    const int cur = kb & 1;
    const bool more = kb + 1 < nkb;
    gload(min(kb + NS, nkb - 1), std::integral_constant<int, LS>{});
    const int c0 = kb * KB;
    const bool any = (r0 < T) && (!causal || c0 <= r0 + 63);
    if (any) {
      f32x16_t acc[2][NB];
      static_for<2 * NB>([&](auto ab) { acc[ab / NB][ab % NB] = f32x16_t{}; });
      const bf16_t* sKc = sK[cur];
      // K fragments double-buffered: substep s + 1 is read while s multiplies
      bf16x8_t kf[2][NB];
      auto read_kf = [&](auto sub) {
        constexpr int SUB = decltype(sub)::value;
        static_for<NB>([&](auto n) {
          kf[SUB & 1][n] = *reinterpret_cast<const bf16x8_t*>(&sKc[(n * 32 + frow) * PITCH + SUB * 16 + fk]);
        });
      };
      read_kf(std::integral_constant<int, 0>{});
      static_for<KS>([&](auto s) {
        constexpr int SS = decltype(s)::value;
        if constexpr (SS + 1 < KS) read_kf(std::integral_constant<int, SS + 1>{});
        static_for<2 * NB>([&](auto ab) {
          constexpr int A = decltype(ab)::value / NB, N = decltype(ab)::value % NB;
          acc[A][N] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[A][SS], kf[SS & 1][N], acc[A][N], 0, 0, 0);
        });
      });
      const bool full = (!causal || c0 + KB - 1 <= r0) && (r0 + 63 < T) && (c0 + KB - 1 < T);
      // IEEE maximum propagates NaN (v_maximum3_f32: two logits per instruction)
      if (full) {
        static_for<2 * NB>([&](auto ab) {
          constexpr int A = decltype(ab)::value / NB, N = decltype(ab)::value % NB;
          static_for<8>([&](auto e) {
            constexpr int E = 2 * decltype(e)::value;
            m = __builtin_elementwise_maximum(m, __builtin_elementwise_maximum(acc[A][N][E], acc[A][N][E + 1]));
          });
        });
      } else {
        static_for<2 * NB>([&](auto ab) {
          constexpr int A = decltype(ab)::value / NB, N = decltype(ab)::value % NB;
          const int j = c0 + N * 32 + (lane & 31);
          static_for<16>([&](auto e) {
            constexpr int E = decltype(e)::value;
            const int i = r0 + A * 32 + 8 * (E / 4) + 4 * (lane >> 5) + (E % 4);
            const bool ok = i < T && j < T && (!causal || j <= i);
            m = __builtin_elementwise_maximum(m, ok ? acc[A][N][E] : -INFINITY);
          });
        });
      }
    }
    if (more) sstore(cur ^ 1, std::integral_constant<int, SS>{});
    barrier();
  };
  int kb = 0;
  for (; kb + 1 < nkb; kb += 2) {
    body(kb, S0{});
    body(kb + 1, S1{});
  }
  if (kb < nkb) body(kb, S0{});

  const int has_nan = __any(m != m) ? 1 : 0;
  m = wave_max(m);
  if (lane == 0) {
    wmax[wave] = m;
    wnan[wave] = has_nan;
  }
  __syncthreads();
  if (tid == 0) {
    float r = wmax[0];
    int nan = wnan[0];
    for (int w = 1; w < kWaves; ++w) {
      r = fmaxf(r, wmax[w]);
      nan |= wnan[w];
    }
    if (nan) r = __uint_as_float(0x7fc00000u);
    partial[(static_cast<int64_t>(b) * H + h) * nqb + qb] = r;
  }
}

// d = 128: one block per (batch row, head, 512 queries), 8 waves of 64
// query rows, two per SIMD.  Waves 0-3 (group 0) and 4-7 (group 1) sit one per
// SIMD each and take turns: while one group runs its 32 MFMAs of a 64-key
// stage on register fragments, the other reduces its previous stage's logits
// by max, reads the next stage's key fragments from LDS and stages its half
// of a later key block; a barrier separates the turns, so each SIMD always has
// a wave issuing MFMAs.  Group g stages rows 32g..32g+31 of each key block,
// two blocks ahead through registers; wave rows interleave between the groups
// (row offset (2 slot + g) 64) so both reach the causal diagonal together.
// One block per CU (the 256 registers of two waves per SIMD).  A turn takes
// about 1.25x its 32 MFMAs of matrix-pipe time; the 4-wave form below, two
// blocks per CU with independent barriers, leaves the pipes idle more often.
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void qk_rowmax_pp_kernel(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, int B, int T, int H,
                         int causal, float* __restrict__ partial, int nqb) {
  constexpr int D = 128, KB = 64, NB = 2, PITCH = D + 8, KS = D / 16, QB = 512;
  __shared__ __attribute__((aligned(16))) bf16_t sK[2][KB * PITCH];
  __shared__ float wmax[8];
  __shared__ int wnan[8];

  const int nbh = B * H;
  int bh, qb;
  if (!xcd_group_order(blockIdx.x, nbh, nqb, 8, &bh, &qb)) {
    bh = blockIdx.x % nbh;                 // heaviest query blocks of every pair first
    qb = nqb - 1 - blockIdx.x / nbh;
  }
  const int b = bh / H, h = bh - b * H;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, slot = wave & 3;
  const int64_t row_stride = static_cast<int64_t>(H) * D;
  const bf16_t* Qb = Q + static_cast<int64_t>(b) * T * row_stride + static_cast<int64_t>(h) * D;
  const bf16_t* Kb = K + static_cast<int64_t>(b) * T * row_stride + static_cast<int64_t>(h) * D;
  const int r0 = qb * QB + (2 * slot + grp) * 64;  // first query row of this wave
  const int frow = lane & 31, fk = (lane >> 5) * 8;

  bf16x8_t qf[2][KS];
  static_for<2>([&](auto a) {
    const int row = min(r0 + a * 32 + frow, T - 1);
    static_for<KS>([&](auto s) {
      qf[a][s] = *reinterpret_cast<const bf16x8_t*>(Qb + row * row_stride + s * 16 + fk);
    });
  });

  const int kend = causal ? min(T, (qb + 1) * QB) : T;
  const int nkb = (kend + KB - 1) / KB;

  // staging: group g copies rows 32 g + (gt / 16) + 16 c, 16-byte chunk gt % 16
  const int gt = tid & 255;
  const int srow = 32 * grp + (gt >> 4), scol = (gt & 15) * 8;
  u32x4_t rk[2][2];   // [register set][chunk]
  auto gload = [&](int kb, auto set) __attribute__((always_inline)) {
    constexpr int SET = decltype(set)::value;
    const int k0 = min(kb, nkb - 1) * KB;
    static_for<2>([&](auto c) {
      const int j = min(k0 + srow + 16 * c, T - 1);
      rk[SET][c] = *reinterpret_cast<const u32x4_t*>(Kb + j * row_stride + scol);
    });
  };
  auto sstore = [&](int buf, auto set) __attribute__((always_inline)) {
    constexpr int SET = decltype(set)::value;
    static_for<2>([&](auto c) {
      *reinterpret_cast<u32x4_t*>(&sK[buf][(srow + 16 * c) * PITCH + scol]) = rk[SET][c];
    });
  };
  auto turn = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  bf16x8_t kf[KS][NB];
  auto read_frags = [&](int buf) __attribute__((always_inline)) {
    static_for<KS>([&](auto s) {
      static_for<NB>([&](auto n) {
        kf[s][n] = *reinterpret_cast<const bf16x8_t*>(&sK[buf][(n * 32 + frow) * PITCH + s * 16 + fk]);
      });
    });
  };
  f32x16_t acc[2][NB];
  auto any_of = [&](int kb) __attribute__((always_inline)) { return (r0 < T) && (!causal || kb * KB <= r0 + 63); };
  auto compute = [&](int kb) __attribute__((always_inline)) {
    if (any_of(kb)) {
      static_for<2 * NB>([&](auto ab) { acc[ab / NB][ab % NB] = f32x16_t{}; });
      static_for<KS>([&](auto s) {
        static_for<2 * NB>([&](auto ab) {
          constexpr int A = decltype(ab)::value / NB, N = decltype(ab)::value % NB;
          acc[A][N] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[A][s], kf[s][N], acc[A][N], 0, 0, 0);
        });
      });
    }
  };
  float m = -INFINITY;
  auto reduce = [&](int kb) __attribute__((always_inline)) {
    if (!any_of(kb)) return;
    const int c0 = kb * KB;
    const bool full = (!causal || c0 + KB - 1 <= r0) && (r0 + 63 < T) && (c0 + KB - 1 < T);
    // IEEE maximum propagates NaN (v_maximum3_f32: two logits per instruction)
    if (full) {
      static_for<2 * NB>([&](auto ab) {
        constexpr int A = decltype(ab)::value / NB, N = decltype(ab)::value % NB;
        static_for<8>([&](auto e) {
          constexpr int E = 2 * decltype(e)::value;
          m = __builtin_elementwise_maximum(m, __builtin_elementwise_maximum(acc[A][N][E], acc[A][N][E + 1]));
        });
      });
    } else {
      static_for<2 * NB>([&](auto ab) {
        constexpr int A = decltype(ab)::value / NB, N = decltype(ab)::value % NB;
        const int j = c0 + N * 32 + (lane & 31);
        static_for<16>([&](auto e) {
          constexpr int E = decltype(e)::value;
          const int i = r0 + A * 32 + 8 * (E / 4) + 4 * (lane >> 5) + (E % 4);
          const bool ok = i < T && j < T && (!causal || j <= i);
          m = __builtin_elementwise_maximum(m, ok ? acc[A][N][E] : -INFINITY);
        });
      });
    }
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // prologue: key block 0 (both halves) and block 1's half of group 0 in LDS;
  // group 0 holds its halves of blocks 2 and 3 in registers, group 1 its
  // halves of blocks 1 and 2
  gload(0, S0{});
  sstore(0, S0{});
  if (grp == 0) {
    gload(1, S1{});
    sstore(1, S1{});
    gload(2, S0{});
    gload(3, S1{});
  } else {
    gload(1, S1{});
    gload(2, S0{});
  }
  turn();
  // Turn 2k: group 0 multiplies block k while group 1 reads its fragments;
  // turn 2k + 1: the reverse.  Block j's LDS stage (j & 1) is written by
  // group 0 in turn 2j - 3 and by group 1 in turn 2j - 2, after the last
  // reads of block j - 2 (turn 2j - 4) and before the first reads of block j
  // (turn 2j - 1).
  if (grp == 0) {
    read_frags(0);
    auto step = [&](int k, auto par) __attribute__((always_inline)) {
      constexpr int P = decltype(par)::value;   // k & 1: register set of blocks k + 2 and k + 4
      compute(k);
      turn();
      reduce(k);
      if (k + 1 < nkb) read_frags((k + 1) & 1);
      if (k + 2 < nkb) sstore(k & 1, std::integral_constant<int, P>{});
      gload(k + 4, std::integral_constant<int, P>{});
      turn();
    };
    int k = 0;
    for (; k + 1 < nkb; k += 2) {
      step(k, S0{});
      step(k + 1, S1{});
    }
    if (k < nkb) step(k, S0{});
  } else {
    auto step = [&](int k, auto par) __attribute__((always_inline)) {
      constexpr int P = decltype(par)::value;   // (k + 1) & 1: register set of blocks k + 1 and k + 3
      if (k >= 1) reduce(k - 1);
      read_frags(k & 1);
      if (k + 1 < nkb) sstore((k + 1) & 1, std::integral_constant<int, P>{});
      gload(k + 3, std::integral_constant<int, P>{});
      turn();
      compute(k);
      turn();
    };
    int k = 0;
    for (; k + 1 < nkb; k += 2) {
      step(k, S1{});
      step(k + 1, S0{});
    }
    if (k < nkb) step(k, S1{});
    reduce(nkb - 1);
  }

  const int has_nan = __any(m != m) ? 1 : 0;
  m = wave_max(m);
  if (lane == 0) {
    wmax[wave] = m;
    wnan[wave] = has_nan;
  }
  __syncthreads();
  if (tid == 0) {
    float r = wmax[0];
    int nan = wnan[0];
    for (int w = 1; w < 8; ++w) {
      r = fmaxf(r, wmax[w]);
      nan |= wnan[w];
    }
    if (nan) r = __uint_as_float(0x7fc00000u);
    partial[(static_cast<int64_t>(b) * H + h) * nqb + qb] = r;
  }
}

// s_max[h] = logit_scale * max over (b, query block) of the partial maxima,
// NaN if any partial is NaN.
__global__ __launch_bounds__(64) void qk_reduce_kernel(const float* __restrict__ partial, int B,
                                                       int H, int nqb, float logit_scale,
                                                       float* __restrict__ s_max) {
  const int h = blockIdx.x;
  float m = -INFINITY;
  int nan = 0;
  const int n = B * nqb;
  for (int k = threadIdx.x; k < n; k += 64) {
    const int b = k / nqb, q = k - b * nqb;
    const float v = partial[(static_cast<int64_t>(b) * H + h) * nqb + q];
    nan |= (v != v);
    m = fmaxf(m, v);
  }
  m = wave_max(m);
  nan = __any(nan);
  if (threadIdx.x == 0) s_max[h] = nan ? __uint_as_float(0x7fc00000u) : m * logit_scale;
}

// Rescale the rows of head h (blockIdx.y) in slice z (blockIdx.z) by
// gamma^expo, gamma = tau / S_max^h, when S_max^h is finite and > tau.
// The common exponents take exact paths (sqrt for 1/2, gamma itself for 1).
template <typename WT>
__global__ __launch_bounds__(256) void qk_rescale_kernel(RescaleLaunch L, const float* __restrict__ s_max,
                                                         float tau, int32_t* __restrict__ clipped) {
  const int h = blockIdx.y, z = blockIdx.z;
  const float s = s_max[h];
  const bool finite = (__float_as_uint(s) & 0x7f800000u) != 0x7f800000u;
  const bool clip = finite && (s > tau);
  if (clipped && blockIdx.x == 0 && z == 0 && threadIdx.x == 0) clipped[h] = finite ? (clip ? 1 : 0) : -1;
  if (!clip) return;
  const RescaleMat& R = L.m[z];
  const int64_t n = static_cast<int64_t>(R.rows_per_head) * R.cols;
  const int64_t e0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (e0 >= n) return;
  const float gamma = tau / s;
  const float ex = R.expo;
  float f;
  if (ex == 0.5f) f = sqrtf(gamma);
  else if (ex == 1.0f) f = gamma;
  else if (ex == 0.0f) f = 1.0f;
  else f = powf(gamma, ex);
  WT* W = static_cast<WT*>(R.W) + static_cast<int64_t>(h) * R.head_pitch * R.cols;
  if (R.vec && e0 + 7 < n) {
    if constexpr (sizeof(WT) == 2) {
      u32x4_t w = *reinterpret_cast<const u32x4_t*>(W + e0);
      static_for<4>([&](auto q) {
        constexpr int Qi = decltype(q)::value;
        const float lo = bf16_to_f32(w[Qi] & 0xffff) * f;
        const float hi = bf16_to_f32(w[Qi] >> 16) * f;
        w[Qi] = pack2_bf16(lo, hi);
      });
      *reinterpret_cast<u32x4_t*>(W + e0) = w;
    } else {
      f32x4_t* p = reinterpret_cast<f32x4_t*>(W + e0);
      p[0] = p[0] * f;
      p[1] = p[1] * f;
    }
  } else {
    for (int q = 0; q < 8 && e0 + q < n; ++q) {
      if constexpr (sizeof(WT) == 2) {
        bf16_t* w = reinterpret_cast<bf16_t*>(W) + e0 + q;
        *w = f32_to_bf16(bf16_to_f32(*w) * f);
      } else {
        W[e0 + q] *= f;
      }
    }
  }
}

}  // namespace

hipError_t launch_qk_rowmax(const bf16_t* Q, const bf16_t* K, int B, int T, int H, int d_head,
                            int causal, float* partial, int nqb, hipStream_t s) {
  const int nblocks = B * H * nqb;
  switch (d_head) {
    case 64:
      hipLaunchKernelGGL(qk_rowmax_kernel<64>, dim3(nblocks), dim3(kThreads), 0, s, Q, K, B, T, H, causal, partial, nqb);
      break;
    case 128:
      hipLaunchKernelGGL(qk_rowmax_pp_kernel, dim3(nblocks), dim3(512), 0, s, Q, K, B, T, H, causal, partial, nqb);
      break;
    case 256:
      hipLaunchKernelGGL(qk_rowmax_kernel<256>, dim3(nblocks), dim3(kThreads), 0, s, Q, K, B, T, H, causal, partial, nqb);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_qk_reduce(const float* partial, int B, int H, int nqb, float logit_scale,
                            float* s_max, hipStream_t s) {
  hipLaunchKernelGGL(qk_reduce_kernel, dim3(H), dim3(64), 0, s, partial, B, H, nqb, logit_scale, s_max);
  return hipGetLastError();
}

hipError_t launch_qk_rescale(const RescaleLaunch& L, int dtype, int H, const float* s_max, float tau,
                             int32_t* clipped, hipStream_t s) {
  int64_t nmax = 0;
  for (int z = 0; z < L.nmat; ++z) nmax = std::max<int64_t>(nmax, static_cast<int64_t>(L.m[z].rows_per_head) * L.m[z].cols);
  const int bx = static_cast<int>((nmax + 2047) / 2048);
  if (dtype == MUON_DTYPE_BF16)
    hipLaunchKernelGGL(qk_rescale_kernel<bf16_t>, dim3(bx, H, L.nmat), dim3(256), 0, s, L, s_max, tau, clipped);
  else
    hipLaunchKernelGGL(qk_rescale_kernel<float>, dim3(bx, H, L.nmat), dim3(256), 0, s, L, s_max, tau, clipped);
  return hipGetLastError();
}

}  // namespace muon
