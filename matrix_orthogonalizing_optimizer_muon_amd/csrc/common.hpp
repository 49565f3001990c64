// Shared device helpers and launch descriptors for libmuon (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "../../include/muon.h"

namespace muon {

typedef uint16_t bf16_t;  // bf16 bit pattern in memory
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// bf16 <-> fp32.  Widening is exact; narrowing rounds to nearest, ties to
// even, and keeps NaN quiet.
__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// Compile-time loop: f(std::integral_constant<int, i>{}) for i = 0..N-1.
// Register arrays indexed only through such constants are promoted to
// registers from the start (a runtime loop index, even one unrolled later,
// can leave them in scratch or LDS).
template <typename Fn, int... Is>
__device__ __forceinline__ void static_for_impl(Fn&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Workgroup barrier ordering LDS accesses only: release / acquire fences
// restricted to the local address space, so the wait before s_barrier
// covers LDS operations and not global loads in flight (prefetches) or
// global stores (which __syncthreads would wait for).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Blocks are dispatched round-robin over the 8 XCDs (block b -> XCD b % 8).
// This bijection hands each XCD one contiguous range of logical work items,
// so the blocks an XCD runs at the same time share operands in its L2.
__device__ __forceinline__ int xcd_remap(int b, int nblocks) {
  const int per = nblocks / 8, rem = nblocks % 8;
  const int x = b % 8, idx = b / 8;
  return (x < rem) ? x * (per + 1) + idx : rem * (per + 1) + (x - rem) * per + idx;
}

// Block order for causal grids of (head, query block) pairs, heaviest first
// inside small groups of heads: block b runs on XCD b % 8; when nbh heads
// split into 8 ranges of whole groups of gh, XCD x walks its range group by
// group, each group's query blocks heaviest first across its heads (qb
// counts down).  The heads of a group share the XCD's L2, and the light
// blocks of a group fill in behind its heavy ones.  Returns false (and sets
// nothing) when nbh does not split that way.
__device__ __forceinline__ bool xcd_group_order(int b, int nbh, int nqb, int gh, int* bh, int* qb) {
  if (nbh % (8 * gh) != 0) return false;
  const int x = b % 8, idx = b / 8;
  const int g = idx / (gh * nqb), r = idx - g * (gh * nqb);
  *qb = nqb - 1 - r / gh;
  *bh = x * (nbh / 8) + g * gh + r % gh;
  return true;
}

// Kernel kinds, used by the optional event profiler.
enum KernelKind {
  KIND_MOMENTUM_NORM = 0,
  KIND_NORM_FINALIZE = 1,
  KIND_NS_SYRK = 2,
  KIND_NS_POLY = 3,
  KIND_NS_BX = 4,
  KIND_PARAM_UPDATE = 5,
  KIND_QK_ROWMAX = 6,
  KIND_QK_REDUCE = 7,
  KIND_QK_RESCALE = 8,
  KIND_ADAMW = 9,
  KIND_ATTN_FWD = 10,
  KIND_NS_SYRK_SLICES = 11,
  KIND_NS_POLY_SLICES = 12,
  KIND_SMALL_STEP = 13,
  KIND_DION_BQ = 14,
  KIND_DION_GRAM = 15,
  KIND_DION_CHOL = 16,
  KIND_DION_PL = 17,
  KIND_DION_BTP = 18,
  KIND_DION_COLNORM = 19,
  KIND_DION_UPDATE = 20,
  KIND_THIN_GRAM = 21,
  KIND_THIN_POLY = 22,
  KIND_THIN_BX = 23,
  KIND_COUNT = 24
};

// ---------------------------------------------------------------------------
// Newton-Schulz GEMM launch: C[i][j] = sum_k P[i][k] * Q[j][k] over
// `batch` matrices of a problem, every problem of a launch sharing one tile
// size.  Epilogue: v = s * (c_acc * acc + c_e * E(i, j)), where s is 1,
// alpha[mat] or alpha[mat]^2, and E(i, j) is read as Et[j][i] (so that a
// lane's four consecutive rows are one 8-byte load).
// ---------------------------------------------------------------------------
constexpr int kMaxProbs = MUON_MAX_GROUPS;

struct GemmProb {
  const bf16_t* P;
  const bf16_t* Q;
  const bf16_t* Et;
  const float* alpha;
  bf16_t* C;   // row-major output C[i][j], or null
  bf16_t* Ct;  // transposed output Ct[j][i] (the mirror when sym), or null
  int64_t sP, sQ, sEt, sC, sCt;  // per-matrix strides, elements
  int ldp, ldq, lde, ldc, ldct;  // leading dimensions, elements
  int K;                         // contraction length, multiple of 32
  int tm, tn;                    // tiles along i and j
  int tiles_per_mat;
  int ntiles;       // batch * tiles_per_mat
  int sym;          // 1: only tiles ti <= tj, written at (ti,tj) and mirrored
  int alpha_pow;    // 0: s = 1, 1: s = alpha, 2: s = alpha^2
  int mvalid, nvalid;  // outputs are written only for i < mvalid, j < nvalid
  int c16, ct16;    // 1 if C / Ct rows allow aligned 16-byte stores
  float c_acc, c_e;
};

struct GemmLaunch {
  int nprob;
  int band;         // non-symmetric products with tn % 8 == 0: column bands per XCD
  int lin0;         // column-slice launches: first tile (in the launch's tile order) covered
  int prefix[kMaxProbs + 1];  // launch-index range of each problem: ntiles rounded up to a
                               // multiple of 8 (the padding blocks exit at once)
  GemmProb p[kMaxProbs];
};

// ---------------------------------------------------------------------------
// Elementwise launch descriptors.
// ---------------------------------------------------------------------------
struct MomentumGroup {
  const void* G;      // grad (param dtype), or the input of ns_orthogonalize
  float* M;           // momentum (null: no momentum, U = G)
  int64_t bstride;    // elements between matrices of G / M
  int rows, cols;     // original layout
  int rp, cp;         // padded original layout (multiples of 64)
  bf16_t* D1;         // U in its own layout, ld = cp, stride d_stride
  bf16_t* D2;         // U transposed, ld = rp, stride d_stride
  int64_t d_stride;   // rp * cp
  double* partials;   // [batch][tiles_per_mat]
  int tiles_r, tiles_c, tiles_per_mat;
  int pairs_c;        // blocks along a row of tiles: (tiles_c + 1) / 2
  int batch;
  int vec;            // cols % 4 == 0 and bstride % 4 == 0
};

struct MomentumLaunch {
  int ngroups;
  int prefix[kMaxProbs + 1];  // block prefix over groups
  MomentumGroup g[kMaxProbs];
  float mu;
  int nesterov;
};

struct FinalizeLaunch {
  int ngroups;
  int prefix[kMaxProbs + 1];  // matrix prefix over groups
  const double* partials[kMaxProbs];
  int tiles_per_mat[kMaxProbs];
  float* inv_norm[kMaxProbs];
  float eps;
};

struct UpdateGroup {
  void* W;            // param, [batch][rows][cols], stride bstride
  const bf16_t* O;    // orthogonalised direction in W's layout, ld = o_ld
  int64_t bstride, o_bstride;
  int o_ld;
  int rows, cols, batch;
  int vec;            // cols % 8 == 0, bstride % 8 == 0, o_ld % 8 == 0
  int64_t blocks;     // blocks for this group
  float decay;        // 1 - lr * wd
  float step;         // lr * scale
};

struct UpdateLaunch {
  int ngroups;
  int64_t prefix[kMaxProbs + 1];
  UpdateGroup g[kMaxProbs];
};

// Whole step for small matrices (wide view m <= 128, n <= 256), one
// workgroup per matrix: momentum and lookahead, Frobenius norm, the
// Newton-Schulz iteration with every operand in LDS, and the update.
constexpr int kSmallMaxM = 128;
constexpr int kSmallMaxN = 256;

struct SmallGroup {
  const void* G;      // grad (param dtype) or the input of ns_orthogonalize, [rows][cols]
  float* M;           // momentum (null: U = G)
  void* W;            // param (null: no update)
  int64_t bstride;    // elements between matrices of G / M / W
  int rows, cols;     // original layout
  int tall;           // rows > cols: the wide view is the transpose
  int m, n;           // wide view, m <= n
  bf16_t* X0;         // bf16(U), wide [m][n] with ld x0_ld, stride x0_stride (or null)
  int64_t x0_stride;
  int x0_ld;
  bf16_t* O;          // the result in the original layout [rows][cols], ld o_ld
  int64_t o_stride;
  int o_ld;
  float* inv;         // 1 / (||U||_F + eps) per matrix
  float decay, step;  // W <- decay W - step O
  int vec;            // cols % 8 == 0, bstride % 8 == 0, G / M / W 16-byte aligned
  int ovec;           // cols % 8 == 0, o_ld % 8 == 0, o_stride % 8 == 0, O 16-byte aligned
};

struct SmallLaunch {
  int ngroups;
  int prefix[kMaxProbs + 1];  // matrix prefix over groups
  SmallGroup g[kMaxProbs];
  float mu;
  int nesterov;
  float eps;
  int steps;
  float a, b, c;
};

// Newton-Schulz for thin matrices (wide view m <= kThinMaxM rows, too long
// for the single-workgroup step): A and B kept in fp32, X in bf16.
constexpr int kThinMaxM = 96;
constexpr int kThinMaxMB = kThinMaxM / 32;

struct ThinGroup {
  const bf16_t* X;    // current iterate, wide [mp][np] bf16, ld np, zero-padded
  int64_t x_stride;   // elements between matrices of X
  int np;             // padded n, a multiple of 128
  int mb;             // 32-row blocks: mq = 32 mb >= m
  int chunk, nchunk;  // Gram partials: columns per chunk (multiple of 128), chunks
  float* part;        // fp32 [batch][nchunk][mq][mq]
  float* Bm;          // fp32 [batch][mq][mq]
  const float* inv;   // 1 / (||U||_F + eps) per matrix (applied on the first step)
  bf16_t* D;          // destination of X' (row-major [i][j], or [j][i] if d_trans)
  int64_t d_stride;
  int d_ld;
  int d_trans;
  int d_rvalid, d_cvalid;  // rows / columns of D written (D's own layout)
  int d_vec;          // d_ld % 8 == 0, d_stride % 8 == 0, D 16-byte aligned
  int batch;
};

struct ThinLaunch {
  int ngroups;
  int prefix[kMaxProbs + 1];  // block prefix over groups (per launch)
  ThinGroup g[kMaxProbs];
  int first;                  // first Newton-Schulz step: scale by inv
  float a, b, c;
};

// Dion's rank-r step: one argument block for every launch of a step; the
// GEMM launches set src / bsrc / dst to their operands.
enum DionMode { DION_BQ = 0, DION_PL = 1, DION_BTP = 2, DION_UPD = 3 };

struct DionArgs {
  const void* G;       // grad (param dtype), [m][n] per matrix
  float* M;            // momentum fp32
  void* W;             // param
  float* Q;            // rank state fp32 [n][r] per matrix, dense
  int64_t bstride;     // elements between matrices of G / M / W
  int64_t q_stride;    // n * r
  int m, n, r, rp;     // rp = r rounded up to 32
  int nsplit;          // Gram partials per matrix (row chunks of 128)
  float mu, lr;
  const float* src;    // GEMM A operand (P0 / P), [m][rp]
  int64_t src_stride;
  const float* bsrc;   // GEMM B operand (L^-T [rp][rp], P [m][rp] or R [n][rp])
  int64_t bsrc_stride;
  float* dst;          // GEMM output [rows][rp]
  int64_t dst_stride;
  float* R;            // [n][rp]
  int64_t r_stride;
  float* Lt;           // [rp][rp]
  int64_t lt_stride;
  float* inv;          // [rp] per matrix: 1 / column norm of R
  double* gram;        // [nsplit][rp][rp] per matrix
  int64_t gram_stride;
};

// Launchers (defined next to their kernels).  Each returns hipGetLastError().
hipError_t launch_momentum_norm(const MomentumLaunch& L, int grad_dtype, int nblocks, hipStream_t s);
hipError_t launch_norm_finalize(const FinalizeLaunch& L, int nmats, hipStream_t s);
hipError_t launch_ns_gemm(const GemmLaunch& L, int tile, int stage, int nblocks, hipStream_t s);
hipError_t launch_ns_gemm_slices(const GemmLaunch& L, int stage, int nblocks, hipStream_t s);
hipError_t launch_param_update(const UpdateLaunch& L, int param_dtype, int64_t nblocks, hipStream_t s);
hipError_t launch_small_step(const SmallLaunch& L, int dtype, int nmats, hipStream_t s);
// stage 0: Gram partials (one wave per matrix and chunk), 1: B per matrix,
// 2: X' per 128 columns
hipError_t launch_thin(const ThinLaunch& L, int stage, int nblocks, hipStream_t s);
hipError_t launch_dion_gemm(const DionArgs& A, int mode, int dtype, int batch, hipStream_t s);
hipError_t launch_dion_gram(const DionArgs& A, int batch, hipStream_t s);
hipError_t launch_dion_gram_reduce(const DionArgs& A, int batch, hipStream_t s);
hipError_t launch_dion_chol(const DionArgs& A, int batch, hipStream_t s);
hipError_t launch_dion_colnorm(const DionArgs& A, int batch, hipStream_t s);
// Queries per block of the row-max kernel for a head dimension (the partial
// maxima it writes number B * H * ceil(T / that)).
inline int qk_rowmax_query_block(int d_head) { return d_head == 128 ? 512 : 256; }
hipError_t launch_qk_rowmax(const bf16_t* Q, const bf16_t* K, int B, int T, int H, int d_head,
                            int causal, float* partial, int nqb, hipStream_t s);
hipError_t launch_qk_reduce(const float* partial, int B, int H, int nqb, float logit_scale,
                            float* s_max, hipStream_t s);
// qkclip_rowmax_noalloc: its partial maxima live in a file-scope __device__
// array of kNoAllocPartials floats (qkclip.hip); noalloc_partials gives that
// array's address on the current device (looked up once per device).
constexpr int kNoAllocPartials = 1 << 18;   // 1 MiB
constexpr int kMaxDevices = 64;
hipError_t noalloc_partials(float** out);
// Per-head row rescale of up to kMaxRescaleSlices row slices: head h owns
// rows [h * head_pitch, h * head_pitch + rows_per_head) of m[z].W (cols
// elements per row), scaled by gamma^expo.
constexpr int kMaxRescaleSlices = 4;
struct RescaleMat {
  void* W;
  int64_t head_pitch;  // rows
  int rows_per_head;
  int cols;
  float expo;
  int vec;             // 16-byte aligned, cols a multiple of 8
};
struct RescaleLaunch {
  int nmat;
  RescaleMat m[kMaxRescaleSlices];
};
hipError_t launch_qk_rescale(const RescaleLaunch& L, int dtype, int H, const float* s_max, float tau,
                             int32_t* clipped, hipStream_t s);

// Causal softmax attention forward (head dimension 128) that also writes
// one maximum raw logit per (batch row, head, query block, wave) to partial.
struct AttnArgs {
  const bf16_t* Q;
  const bf16_t* K;
  const bf16_t* V;
  bf16_t* O;
  float* lse;       // optional [B][H][T]
  float* partial;   // [B][H][nqb][4]
  int B, T, H, nqb;
  float scale;      // logit scale (1/sqrt(d))
  float c2;         // scale * log2(e)
};
hipError_t launch_attn_fwd(const AttnArgs& A, int causal, hipStream_t s);

// Multi-tensor AdamW: block b of a launch works on tensor t with
// blk_start[t] <= b < blk_start[t + 1], elements (b - blk_start[t]) * 2048 ...
constexpr int kAdamWMaxTensors = 48;
struct AdamWTensor {
  void* p;
  const void* g;
  float* m;
  float* v;
  int64_t n;
  int vec;  // p, g, m, v all 16-byte aligned
};
struct AdamWLaunch {
  int ntensors;
  float lr, beta1, beta2, eps, decay;  // decay = 1 - lr * weight_decay
  float c1, c2;                        // 1 / (1 - beta^t) bias corrections
  int blk_start[kAdamWMaxTensors + 1];
  AdamWTensor t[kAdamWMaxTensors];
};
hipError_t launch_adamw(const AdamWLaunch& A, int dtype, int blocks, hipStream_t s);

// Register-only bf16 MFMA loop (probe.hip): 256-thread blocks, each wave
// issuing 4 x iters v_mfma_f32_32x32x16_bf16.
hipError_t launch_mfma_probe(int blocks, int iters, int operands, float* sink, hipStream_t s);
hipError_t launch_hbm_probe(const void* src, void* dst, int64_t units, int reads, int writes, int unroll,
                            hipStream_t s);

// Profiler hooks (api.hip).
void prof_begin(int kind, hipStream_t s);
void prof_end(int kind, hipStream_t s);

}  // namespace muon
