// Stand-ins for the HIP runtime calls and the kernel launchers of libmuon, so
// that the library's host code (argument checks, workspace plans, launch
// descriptors) runs on a machine without a GPU, under AddressSanitizer and
// UBSan.  Nothing here touches device memory: every launcher checks the
// descriptor it receives against the buffers the driver registered (each
// pointer with the extent a kernel of that shape reads or writes must lie in
// one registered region) and counts the launch.  A violation prints what it
// found and aborts.
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "../../matrix_orthogonalizing_optimizer_muon_amd/csrc/common.hpp"

namespace {
struct Region {
  uintptr_t lo, hi;
};
std::vector<Region> g_regions;
long g_launches = 0;
const char* g_case = "";

[[noreturn]] void fail(const char* what, long a = 0, long b = 0) {
  fprintf(stderr, "stub check failed [%s]: %s (%ld, %ld)\n", g_case, what, a, b);
  abort();
}

// [p, p + bytes) inside one registered region
void need(const void* p, uint64_t bytes, const char* what) {
  if (!p) fail(what);
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  for (const Region& r : g_regions)
    if (lo >= r.lo && lo + bytes <= r.hi && lo + bytes >= lo) return;
  fail(what, static_cast<long>(lo), static_cast<long>(bytes));
}

// [a, a + na) and [b, b + nb) do not overlap
void disjoint(const void* a, uint64_t na, const void* b, uint64_t nb, const char* what) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  if (x < y + nb && y < x + na) fail(what, static_cast<long>(x), static_cast<long>(y));
}

// extent in bytes of a strided batch: `batch` matrices `stride` elements
// apart, each `rows` x `cols` with leading dimension ld
uint64_t extent(int64_t batch, int64_t stride, int64_t rows, int64_t ld, int64_t cols, int esz) {
  if (batch < 1 || rows < 1 || cols < 1) return 0;
  if (ld < cols) fail("leading dimension below the row length", ld, cols);
  return static_cast<uint64_t>(((batch - 1) * stride + (rows - 1) * ld + cols) * esz);
}
}  // namespace

extern "C" {
void stub_register(const void* p, uint64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  g_regions.push_back({lo, lo + bytes});
}
void stub_reset(const char* name) {
  g_regions.clear();
  g_launches = 0;
  g_case = name;
}
long stub_launches() { return g_launches; }

// HIP runtime: one device of 256 compute units; events are counters
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) {
  *v = 256;
  return hipSuccess;
}
static long g_event_id = 0;
hipError_t hipEventCreate(hipEvent_t* e) {
  *e = reinterpret_cast<hipEvent_t>(++g_event_id);
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t e, hipStream_t) { return e ? hipSuccess : hipErrorInvalidValue; }
hipError_t hipEventSynchronize(hipEvent_t e) { return e ? hipSuccess : hipErrorInvalidValue; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) {
  *ms = 0.001f;
  return hipSuccess;
}
}

namespace muon {

hipError_t launch_momentum_norm(const MomentumLaunch& L, int grad_dtype, int nblocks, hipStream_t) {
  ++g_launches;
  const int esz = grad_dtype == MUON_DTYPE_BF16 ? 2 : 4;
  if (L.ngroups < 1 || L.ngroups > kMaxProbs || nblocks != L.prefix[L.ngroups] || L.prefix[0] != 0) fail("momentum prefix");
  for (int g = 0; g < L.ngroups; ++g) {
    const MomentumGroup& q = L.g[g];
    if (L.prefix[g + 1] - L.prefix[g] != q.batch * q.tiles_r * q.pairs_c) fail("momentum blocks", g);
    if (q.rp % 64 || q.cp % 64 || q.rp < q.rows || q.cp < q.cols) fail("momentum padding", q.rp, q.cp);
    if (q.tiles_r * 64 != q.rp || q.tiles_c * 64 != q.cp) fail("momentum tiles");
    need(q.G, extent(q.batch, q.bstride, q.rows, q.cols, q.cols, esz), "momentum G");
    if (q.M) need(q.M, extent(q.batch, q.bstride, q.rows, q.cols, q.cols, 4), "momentum M");
    const uint64_t d = extent(q.batch, q.d_stride, q.rp, q.cp, q.cp, 2);
    const uint64_t pb = static_cast<uint64_t>(q.batch) * q.tiles_per_mat * 8;
    need(q.D1, d, "momentum D1");
    need(q.D2, d, "momentum D2");
    need(q.partials, pb, "momentum partials");
    disjoint(q.D1, d, q.D2, d, "momentum D1 / D2");
    disjoint(q.D1, d, q.partials, pb, "momentum D1 / partials");
    disjoint(q.D2, d, q.partials, pb, "momentum D2 / partials");
  }
  return hipSuccess;
}

hipError_t launch_norm_finalize(const FinalizeLaunch& L, int nmats, hipStream_t) {
  ++g_launches;
  if (nmats != L.prefix[L.ngroups]) fail("finalize prefix");
  for (int g = 0; g < L.ngroups; ++g) {
    const int b = L.prefix[g + 1] - L.prefix[g];
    need(L.partials[g], static_cast<uint64_t>(b) * L.tiles_per_mat[g] * 8, "finalize partials");
    need(L.inv_norm[g], static_cast<uint64_t>(b) * 4, "finalize inv");
  }
  return hipSuccess;
}

static void check_gemm(const GemmLaunch& L, int tm_tile, int tn_tile, int nblocks) {
  if (L.nprob < 1 || L.nprob > kMaxProbs || L.prefix[0] != 0) fail("gemm problems", L.nprob);
  if (nblocks < 1 || nblocks > L.prefix[L.nprob] * (tm_tile / tn_tile)) fail("gemm grid", nblocks, L.prefix[L.nprob]);
  for (int k = 0; k < L.nprob; ++k) {
    const GemmProb& p = L.p[k];
    const int span = L.prefix[k + 1] - L.prefix[k];
    if (span % 8 || span < p.ntiles || span >= p.ntiles + 8) fail("gemm problem range", span, p.ntiles);
    if (p.K % 64) fail("gemm K not a multiple of the K slice", p.K);
    const int batch = p.ntiles / p.tiles_per_mat;
    if (batch * p.tiles_per_mat != p.ntiles) fail("gemm tiles per matrix");
    if (p.tiles_per_mat != (p.sym ? p.tm * (p.tm + 1) / 2 : p.tm * p.tn)) fail("gemm tile count");
    const int rows = p.tm * tm_tile, cols = (p.sym ? p.tm : p.tn) * tm_tile;
    const uint64_t eP = extent(batch, p.sP, rows, p.ldp, p.K, 2), eQ = extent(batch, p.sQ, cols, p.ldq, p.K, 2);
    need(p.P, eP, "gemm P");
    need(p.Q, eQ, "gemm Q");
    if (p.Et) need(p.Et, extent(batch, p.sEt, cols, p.lde, rows, 2), "gemm Et");
    const uint64_t eC = p.C ? extent(batch, p.sC, std::min(rows, p.mvalid), p.ldc, std::min(cols, p.nvalid), 2) : 0;
    const uint64_t eCt = p.Ct ? extent(batch, p.sCt, std::min(cols, p.nvalid), p.ldct, std::min(rows, p.mvalid), 2) : 0;
    if (p.C) need(p.C, eC, "gemm C");
    if (p.Ct) need(p.Ct, eCt, "gemm Ct");
    // outputs never alias the operands; C and C^T only as the same symmetric buffer
    if (p.C) disjoint(p.C, eC, p.P, eP, "gemm C / P"), disjoint(p.C, eC, p.Q, eQ, "gemm C / Q");
    if (p.Ct) disjoint(p.Ct, eCt, p.P, eP, "gemm Ct / P"), disjoint(p.Ct, eCt, p.Q, eQ, "gemm Ct / Q");
    if (p.C && p.Ct && p.C != p.Ct) disjoint(p.C, eC, p.Ct, eCt, "gemm C / Ct");
    if (p.sym && p.C && p.Ct && p.C != p.Ct) fail("symmetric product with two output buffers");
    if (p.alpha_pow) need(p.alpha, static_cast<uint64_t>(batch) * 4, "gemm alpha");
    if (!p.C && !p.Ct) fail("gemm without output");
  }
}

hipError_t launch_ns_gemm(const GemmLaunch& L, int tile, int stage, int nblocks, hipStream_t) {
  ++g_launches;
  if ((tile != 128 && tile != 256) || stage < 0 || stage > 2) fail("gemm tile / stage", tile, stage);
  check_gemm(L, tile, tile, nblocks);
  return hipSuccess;
}

hipError_t launch_ns_gemm_slices(const GemmLaunch& L, int stage, int nblocks, hipStream_t) {
  ++g_launches;
  if (stage < 0 || stage > 1 || nblocks % 2 || L.lin0 < 0) fail("slices stage / grid", stage, nblocks);
  if (L.lin0 + nblocks / 2 > L.prefix[L.nprob]) fail("slices past the last tile", L.lin0, nblocks);
  check_gemm(L, 256, 128, nblocks);
  return hipSuccess;
}

hipError_t launch_param_update(const UpdateLaunch& L, int param_dtype, int64_t nblocks, hipStream_t) {
  ++g_launches;
  const int esz = param_dtype == MUON_DTYPE_BF16 ? 2 : 4;
  if (nblocks != L.prefix[L.ngroups]) fail("update prefix");
  for (int g = 0; g < L.ngroups; ++g) {
    const UpdateGroup& u = L.g[g];
    if (L.prefix[g + 1] - L.prefix[g] != u.blocks) fail("update blocks");
    need(u.W, extent(u.batch, u.bstride, u.rows, u.cols, u.cols, esz), "update W");
    need(u.O, extent(u.batch, u.o_bstride, u.rows, u.o_ld, u.cols, 2), "update O");
  }
  return hipSuccess;
}

hipError_t launch_small_step(const SmallLaunch& L, int dtype, int nmats, hipStream_t) {
  ++g_launches;
  const int esz = dtype == MUON_DTYPE_BF16 ? 2 : 4;
  if (nmats != L.prefix[L.ngroups] || L.steps < 1) fail("small prefix");
  for (int g = 0; g < L.ngroups; ++g) {
    const SmallGroup& q = L.g[g];
    const int b = L.prefix[g + 1] - L.prefix[g];
    if (q.m > kSmallMaxM || q.n > kSmallMaxN || q.m > q.n) fail("small shape", q.m, q.n);
    need(q.G, extent(b, q.bstride, q.rows, q.cols, q.cols, esz), "small G");
    if (q.M) need(q.M, extent(b, q.bstride, q.rows, q.cols, q.cols, 4), "small M");
    if (q.W) need(q.W, extent(b, q.bstride, q.rows, q.cols, q.cols, esz), "small W");
    if (q.X0) need(q.X0, extent(b, q.x0_stride, q.m, q.x0_ld, q.n, 2), "small X0");
    need(q.O, extent(b, q.o_stride, q.rows, q.o_ld, q.cols, 2), "small O");
    if (q.inv) need(q.inv, static_cast<uint64_t>(b) * 4, "small inv");
  }
  return hipSuccess;
}

hipError_t launch_thin(const ThinLaunch& L, int stage, int nblocks, hipStream_t) {
  ++g_launches;
  if (nblocks != L.prefix[L.ngroups] || stage < 0 || stage > 2) fail("thin prefix / stage", nblocks, stage);
  for (int g = 0; g < L.ngroups; ++g) {
    const ThinGroup& q = L.g[g];
    const int mq = 32 * q.mb;
    const int per = stage == 0 ? q.nchunk : stage == 1 ? 1 : q.np / 128;
    if (L.prefix[g + 1] - L.prefix[g] != q.batch * per) fail("thin blocks", g, stage);
    if (q.mb < 1 || q.mb > kThinMaxMB || q.np % 128 || q.chunk % 128 || q.chunk < 128) fail("thin shape", q.mb, q.np);
    if (static_cast<int64_t>(q.nchunk) * q.chunk < q.np || (q.nchunk - 1) * q.chunk >= q.np) fail("thin chunks");
    const uint64_t eX = extent(q.batch, q.x_stride, mq, q.np, q.np, 2);
    const uint64_t eP = static_cast<uint64_t>(q.batch) * q.nchunk * mq * mq * 4;
    const uint64_t eB = static_cast<uint64_t>(q.batch) * mq * mq * 4;
    need(q.X, eX, "thin X");
    need(q.part, eP, "thin partials");
    need(q.Bm, eB, "thin B");
    disjoint(q.part, eP, q.Bm, eB, "thin partials / B");
    disjoint(q.part, eP, q.X, eX, "thin partials / X");
    disjoint(q.Bm, eB, q.X, eX, "thin B / X");
    if (L.first) need(q.inv, static_cast<uint64_t>(q.batch) * 4, "thin inv");
    if (stage == 2) {
      const int64_t r = q.d_trans ? std::min<int64_t>(q.np, q.d_rvalid) : std::min<int64_t>(mq, q.d_rvalid);
      const int64_t c = q.d_trans ? std::min<int64_t>(mq, q.d_cvalid) : std::min<int64_t>(q.np, q.d_cvalid);
      const uint64_t eD = extent(q.batch, q.d_stride, r, q.d_ld, c, 2);
      need(q.D, eD, "thin D");
      disjoint(q.D, eD, q.X, eX, "thin D / X");
      disjoint(q.D, eD, q.Bm, eB, "thin D / B");
    }
  }
  return hipSuccess;
}

hipError_t launch_qk_rowmax(const bf16_t* Q, const bf16_t* K, int B, int T, int H, int d_head, int, float* partial,
                            int nqb, hipStream_t) {
  ++g_launches;
  const uint64_t qk = static_cast<uint64_t>(B) * T * H * d_head * 2;
  need(Q, qk, "rowmax Q");
  need(K, qk, "rowmax K");
  need(partial, static_cast<uint64_t>(B) * H * nqb * 4, "rowmax partials");
  const int q = qk_rowmax_query_block(d_head);
  if (nqb != (T + q - 1) / q) fail("rowmax query block count");
  return hipSuccess;
}

hipError_t launch_qk_reduce(const float* partial, int B, int H, int nqb, float, float* s_max, hipStream_t) {
  ++g_launches;
  need(partial, static_cast<uint64_t>(B) * H * nqb * 4, "reduce partials");
  need(s_max, static_cast<uint64_t>(H) * 4, "reduce s_max");
  return hipSuccess;
}

hipError_t launch_qk_rescale(const RescaleLaunch& L, int dtype, int H, const float* s_max, float, int32_t* clipped,
                             hipStream_t) {
  ++g_launches;
  const int esz = dtype == MUON_DTYPE_BF16 ? 2 : 4;
  need(s_max, static_cast<uint64_t>(H) * 4, "rescale s_max");
  if (clipped) need(clipped, static_cast<uint64_t>(H) * 4, "rescale flags");
  for (int z = 0; z < L.nmat; ++z) {
    const RescaleMat& R = L.m[z];
    need(R.W, extent(H, R.head_pitch * R.cols, R.rows_per_head, R.cols, R.cols, esz), "rescale W");
  }
  return hipSuccess;
}

hipError_t launch_attn_fwd(const AttnArgs& A, int, hipStream_t) {
  ++g_launches;
  const uint64_t qkv = static_cast<uint64_t>(A.B) * A.T * A.H * 128 * 2;
  need(A.Q, qkv, "attn Q");
  need(A.K, qkv, "attn K");
  need(A.V, qkv, "attn V");
  need(A.O, qkv, "attn O");
  if (A.lse) need(A.lse, static_cast<uint64_t>(A.B) * A.H * A.T * 4, "attn lse");
  need(A.partial, static_cast<uint64_t>(A.B) * A.H * A.nqb * 4 * 4, "attn partials");
  return hipSuccess;
}

hipError_t launch_adamw(const AdamWLaunch& A, int dtype, int blocks, hipStream_t) {
  ++g_launches;
  const int esz = dtype == MUON_DTYPE_BF16 ? 2 : 4;
  if (A.ntensors < 1 || A.ntensors > kAdamWMaxTensors || blocks != A.blk_start[A.ntensors]) fail("adamw prefix");
  for (int t = 0; t < A.ntensors; ++t) {
    const AdamWTensor& T = A.t[t];
    if (A.blk_start[t + 1] - A.blk_start[t] != (T.n + 4095) / 4096) fail("adamw blocks", t);
    need(T.p, T.n * esz, "adamw p");
    need(T.g, T.n * esz, "adamw g");
    need(T.m, T.n * 4, "adamw m");
    need(T.v, T.n * 4, "adamw v");
  }
  return hipSuccess;
}

// dtype < 0: the launch does not say (its kernels do not read G or W), so
// their extents are checked at the smaller element size
static void check_dion(const DionArgs& A, int dtype, int batch) {
  const int esz = dtype == MUON_DTYPE_F32 ? 4 : 2;
  need(A.G, extent(batch, A.bstride, A.m, A.n, A.n, esz), "dion G");
  need(A.M, extent(batch, A.bstride, A.m, A.n, A.n, 4), "dion M");
  need(A.W, extent(batch, A.bstride, A.m, A.n, A.n, esz), "dion W");
  need(A.Q, extent(batch, A.q_stride, A.n, A.r, A.r, 4), "dion Q");
  need(A.R, extent(batch, A.r_stride, A.n, A.rp, A.rp, 4), "dion R");
  need(A.Lt, extent(batch, A.lt_stride, A.rp, A.rp, A.rp, 4), "dion Lt");
  need(A.inv, static_cast<uint64_t>(batch) * A.rp * 4, "dion inv");
  need(A.gram, static_cast<uint64_t>(batch) * A.gram_stride * 8, "dion gram");
  if (A.rp % 32 || A.rp < A.r) fail("dion padded rank", A.rp, A.r);
}

hipError_t launch_dion_gemm(const DionArgs& A, int mode, int dtype, int batch, hipStream_t) {
  ++g_launches;
  check_dion(A, dtype, batch);
  if (mode == DION_PL || mode == DION_UPD) need(A.src, extent(batch, A.src_stride, A.m, A.rp, A.rp, 4), "dion src");
  if (mode != DION_BQ) need(A.bsrc, 4, "dion bsrc");
  if (mode != DION_UPD) need(A.dst, 4, "dion dst");
  return hipSuccess;
}
hipError_t launch_dion_gram(const DionArgs& A, int batch, hipStream_t) {
  ++g_launches;
  check_dion(A, -1, batch);
  need(A.src, extent(batch, A.src_stride, A.m, A.rp, A.rp, 4), "dion gram src");
  return hipSuccess;
}
hipError_t launch_dion_gram_reduce(const DionArgs& A, int batch, hipStream_t) {
  ++g_launches;
  check_dion(A, -1, batch);
  return hipSuccess;
}
hipError_t launch_dion_chol(const DionArgs& A, int batch, hipStream_t) {
  ++g_launches;
  check_dion(A, -1, batch);
  return hipSuccess;
}
hipError_t launch_dion_colnorm(const DionArgs& A, int batch, hipStream_t) {
  ++g_launches;
  check_dion(A, -1, batch);
  return hipSuccess;
}

// the no-allocation row-max's scratch: a fixed address range, registered on
// each lookup (the real one is a __device__ array found by symbol)
hipError_t noalloc_partials(float** out) {
  const uintptr_t base = uintptr_t(0x7000) << 32;
  stub_register(reinterpret_cast<void*>(base), uint64_t(kNoAllocPartials) * 4);
  *out = reinterpret_cast<float*>(base);
  return hipSuccess;
}

hipError_t launch_mfma_probe(int blocks, int iters, int operands, float* sink, hipStream_t) {
  ++g_launches;
  if (blocks < 1 || iters < 1 || (operands != MUON_PROBE_RANDOM && operands != MUON_PROBE_SMOOTH)) fail("probe args");
  need(sink, static_cast<uint64_t>(blocks) * 4, "probe sink");
  return hipSuccess;
}

hipError_t launch_hbm_probe(const void* src, void* dst, int64_t units, int reads, int writes, int unroll,
                            hipStream_t) {
  ++g_launches;
  const bool mix = (reads == 1 && writes == 1) || (reads == 3 && writes == 4) || (reads == 2 && writes == 1);
  if (units < 1 || !mix || (unroll != 1 && unroll != 4)) fail("hbm probe args");
  need(src, static_cast<uint64_t>(units) * 16 * reads, "hbm probe src");
  need(dst, static_cast<uint64_t>(units) * 16 * writes, "hbm probe dst");
  return hipSuccess;
}

}  // namespace muon

// roctx ranges: the host build links no profiler library
extern "C" int roctxRangePushA(const char* message) { return message ? 0 : -1; }
extern "C" int roctxRangePop() { return 0; }
