// libmuon C ABI: argument checks, workspace layout and launch sequencing for
// the Muon step ("MuonClip", section 07 step order: momentum -> Newton-Schulz
// -> scaled, decayed update), Newton-Schulz alone, and QK-Clip.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <vector>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "common.hpp"

namespace muon {

// Named host ranges (roctx) around each entry point and the Muon step's
// stages, for `rocprofv3 --marker-trace`; near free when no tool is attached.
namespace {
struct Range {
  explicit Range(const char* name) { roctxRangePushA(name); }
  ~Range() { roctxRangePop(); }
  Range(const Range&) = delete;
  Range& operator=(const Range&) = delete;
};
}  // namespace

// ----------------------------------------------------------------------------
// optional event profiler
// ----------------------------------------------------------------------------
namespace {
struct ProfRec {
  int kind;
  hipEvent_t a, b;
};
bool g_prof_on = false;
std::vector<ProfRec> g_prof;
std::vector<hipEvent_t> g_event_pool;
int g_open_kind = -1;
hipEvent_t g_open_start = nullptr;

hipEvent_t pool_get() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

void prof_begin(int kind, hipStream_t s) {
  if (!g_prof_on) return;
  g_open_kind = kind;
  g_open_start = pool_get();
  if (g_open_start) (void)hipEventRecord(g_open_start, s);
}

void prof_end(int kind, hipStream_t s) {
  if (!g_prof_on || !g_open_start || g_open_kind != kind) return;
  hipEvent_t e = pool_get();
  if (!e) return;
  (void)hipEventRecord(e, s);
  g_prof.push_back({kind, g_open_start, e});
  g_open_start = nullptr;
  g_open_kind = -1;
}

// ----------------------------------------------------------------------------
// workspace plan
// ----------------------------------------------------------------------------
namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int round_up(int x, int m) { return (x + m - 1) / m * m; }

struct Plan {
  int batch, rows, cols;
  int64_t bstride;
  bool tall;
  int m, n;       // wide view, m <= n
  int tile;       // Newton-Schulz GEMM tile edge
  int mp, np;     // padded wide view (multiples of tile)
  int rp, cp;     // padded original layout
  int tiles_r, tiles_c, mom_tiles;
  bool thin;      // m <= kThinMaxM and too long for the single-workgroup step
  int mq, chunk, nchunk;   // thin: rows in 32-blocks, Gram partial chunking
  size_t off_X[2], off_Xt[2], off_A, off_B, off_part, off_inv, off_thin_part, off_thin_B;
};

// Groups whose wide view fits the single-workgroup step (X and A in LDS).
bool small_ok(int rows, int cols) {
  return std::min(rows, cols) <= kSmallMaxM && std::max(rows, cols) <= kSmallMaxN;
}

Plan make_plan(int batch, int rows, int cols, int64_t bstride, size_t& cursor) {
  Plan p{};
  p.batch = batch;
  p.rows = rows;
  p.cols = cols;
  p.bstride = bstride;
  p.tall = rows > cols;
  p.m = std::min(rows, cols);
  p.n = std::max(rows, cols);
  p.tile = (p.m >= 512) ? 256 : 128;
  p.mp = round_up(p.m, p.tile);
  p.np = round_up(p.n, p.tile);
  p.rp = p.tall ? p.np : p.mp;
  p.cp = p.tall ? p.mp : p.np;
  p.tiles_r = p.rp / 64;
  p.tiles_c = p.cp / 64;
  p.mom_tiles = p.tiles_r * p.tiles_c;
  p.thin = p.m <= kThinMaxM && !small_ok(rows, cols);
  const size_t xb = static_cast<size_t>(batch) * p.mp * p.np * sizeof(bf16_t);
  const size_t ab = p.thin ? 0 : static_cast<size_t>(batch) * p.mp * p.mp * sizeof(bf16_t);
  for (int k = 0; k < 2; ++k) {
    p.off_X[k] = cursor;
    cursor = align_up(cursor + xb);
    p.off_Xt[k] = cursor;
    cursor = align_up(cursor + xb);
  }
  p.off_A = cursor;
  cursor = align_up(cursor + ab);
  p.off_B = cursor;
  cursor = align_up(cursor + ab);
  p.off_part = cursor;
  cursor = align_up(cursor + static_cast<size_t>(batch) * p.mom_tiles * sizeof(double));
  p.off_inv = cursor;
  cursor = align_up(cursor + static_cast<size_t>(batch) * sizeof(float));
  if (p.thin) {
    // Gram partials over column chunks of 512 columns or more, at most 64
    // chunks per matrix; then B, both fp32
    p.mq = round_up(p.m, 32);
    p.chunk = 512 * ((p.np + 512 * 64 - 1) / (512 * 64));
    p.nchunk = (p.np + p.chunk - 1) / p.chunk;
    const size_t sq = static_cast<size_t>(p.mq) * p.mq * sizeof(float);
    p.off_thin_part = cursor;
    cursor = align_up(cursor + static_cast<size_t>(batch) * p.nchunk * sq);
    p.off_thin_B = cursor;
    cursor = align_up(cursor + static_cast<size_t>(batch) * sq);
  }
  return p;
}

bool dims_ok(int batch, int rows, int cols) {
  if (batch < 1 || rows < 1 || cols < 1) return false;
  // padded extents and per-matrix element counts stay inside int / the
  // grid limits used by the kernels
  if (rows > (1 << 20) || cols > (1 << 20)) return false;
  const int64_t mx = std::max(rows, cols) + 256, mn = std::min(rows, cols) + 256;
  if (mx * mn > (int64_t(1) << 31)) return false;
  return true;
}

int check_groups(const muon_group_t* groups, int n_groups) {
  if (!groups || n_groups < 1 || n_groups > MUON_MAX_GROUPS) return MUON_ERR_INVALID_ARG;
  for (int g = 0; g < n_groups; ++g) {
    const muon_group_t& G = groups[g];
    if (!dims_ok(G.batch, G.rows, G.cols) || G.reserved != 0) return MUON_ERR_INVALID_ARG;
    if (G.batch_stride < static_cast<int64_t>(G.rows) * G.cols) return MUON_ERR_INVALID_ARG;
  }
  return MUON_OK;
}

std::vector<Plan> plans_for(const muon_group_t* groups, int n_groups, size_t& total) {
  std::vector<Plan> v;
  size_t cursor = 0;
  for (int g = 0; g < n_groups; ++g)
    v.push_back(make_plan(groups[g].batch, groups[g].rows, groups[g].cols, groups[g].batch_stride, cursor));
  total = cursor;
  return v;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

#define MUON_LAUNCH(kind, stream, expr)            \
  do {                                             \
    prof_begin(kind, stream);                      \
    hipError_t e_ = (expr);                        \
    prof_end(kind, stream);                        \
    if (e_ != hipSuccess) return MUON_ERR_HIP;     \
  } while (0)

// Input of one group to the fused momentum / normalisation pass.
struct PrepIn {
  const void* G;
  float* M;
};

int launch_prep(const std::vector<Plan>& plans, const std::vector<PrepIn>& ins, int dtype, float mu,
                int nesterov, void* ws, hipStream_t s) {
  MomentumLaunch L{};
  L.ngroups = static_cast<int>(plans.size());
  L.mu = mu;
  L.nesterov = nesterov;
  int blocks = 0;
  const size_t esz = dtype == MUON_DTYPE_BF16 ? 2 : 4;
  for (size_t g = 0; g < plans.size(); ++g) {
    const Plan& p = plans[g];
    MomentumGroup& q = L.g[g];
    q.G = ins[g].G;
    q.M = ins[g].M;
    q.bstride = p.bstride;
    q.rows = p.rows;
    q.cols = p.cols;
    q.rp = p.rp;
    q.cp = p.cp;
    bf16_t* X0 = at<bf16_t>(ws, p.off_X[0]);
    bf16_t* X0t = at<bf16_t>(ws, p.off_Xt[0]);
    q.D1 = p.tall ? X0t : X0;
    q.D2 = p.tall ? X0 : X0t;
    q.d_stride = static_cast<int64_t>(p.rp) * p.cp;
    q.partials = at<double>(ws, p.off_part);
    q.tiles_r = p.tiles_r;
    q.tiles_c = p.tiles_c;
    q.tiles_per_mat = p.mom_tiles;
    q.pairs_c = (p.tiles_c + 1) / 2;
    q.batch = p.batch;
    q.vec = (p.cols % 4 == 0) && (p.bstride % 4 == 0) && aligned(q.G, 4 * esz) &&
            (q.M == nullptr || aligned(q.M, 16));
    L.prefix[g] = blocks;
    blocks += p.batch * p.tiles_r * q.pairs_c;
  }
  L.prefix[plans.size()] = blocks;
  MUON_LAUNCH(KIND_MOMENTUM_NORM, s, launch_momentum_norm(L, dtype, blocks, s));
  return MUON_OK;
}

int launch_finalize(const std::vector<Plan>& plans, float eps, void* ws, hipStream_t s) {
  FinalizeLaunch F{};
  F.ngroups = static_cast<int>(plans.size());
  F.eps = eps;
  int mats = 0;
  for (size_t g = 0; g < plans.size(); ++g) {
    F.prefix[g] = mats;
    F.partials[g] = at<double>(ws, plans[g].off_part);
    F.tiles_per_mat[g] = plans[g].mom_tiles;
    F.inv_norm[g] = at<float>(ws, plans[g].off_inv);
    mats += plans[g].batch;
  }
  F.prefix[plans.size()] = mats;
  MUON_LAUNCH(KIND_NORM_FINALIZE, s, launch_norm_finalize(F, mats, s));
  return MUON_OK;
}

// Final-step destination of a group: where the last X' is written.
struct FinalOut {
  bf16_t* ptr;      // null: keep in the workspace
  int64_t stride;   // elements between matrices
  int ld;           // leading dimension
};

enum Stage { STAGE_SYRK = 0, STAGE_POLY = 1, STAGE_BX = 2 };

// Compute units of the current device (one GEMM block runs per CU at a time);
// 0 if the query fails, which turns the last-wave split off.
int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cached[dev] = n;
  return n;
}

GemmProb make_prob(const Plan& p, int stage, int t, int steps, float a, float b, float c, void* ws,
                   const FinalOut* fin) {
  GemmProb q{};
  const int cur = t & 1, nxt = cur ^ 1;
  bf16_t* X = at<bf16_t>(ws, p.off_X[cur]);
  bf16_t* Xt = at<bf16_t>(ws, p.off_Xt[cur]);
  bf16_t* Xn = at<bf16_t>(ws, p.off_X[nxt]);
  bf16_t* Xtn = at<bf16_t>(ws, p.off_Xt[nxt]);
  bf16_t* A = at<bf16_t>(ws, p.off_A);
  bf16_t* B = at<bf16_t>(ws, p.off_B);
  const int64_t sx = static_cast<int64_t>(p.mp) * p.np, sa = static_cast<int64_t>(p.mp) * p.mp;
  const int T = p.mp / p.tile;
  q.alpha = at<float>(ws, p.off_inv);
  q.c16 = 1;
  q.ct16 = 1;
  if (stage == STAGE_SYRK) {
    q.P = X; q.Q = X; q.sP = sx; q.sQ = sx; q.ldp = p.np; q.ldq = p.np; q.K = p.np;
    q.C = A; q.Ct = A; q.sC = sa; q.sCt = sa; q.ldc = p.mp; q.ldct = p.mp;
    q.tm = T; q.tn = T; q.sym = 1; q.tiles_per_mat = T * (T + 1) / 2;
    q.alpha_pow = (t == 0) ? 2 : 0;
    q.c_acc = 1.0f; q.c_e = 0.0f;
    q.mvalid = p.mp; q.nvalid = p.mp;
  } else if (stage == STAGE_POLY) {
    q.P = A; q.Q = A; q.sP = sa; q.sQ = sa; q.ldp = p.mp; q.ldq = p.mp; q.K = p.mp;
    q.C = B; q.Ct = B; q.sC = sa; q.sCt = sa; q.ldc = p.mp; q.ldct = p.mp;
    q.Et = A; q.sEt = sa; q.lde = p.mp;
    q.tm = T; q.tn = T; q.sym = 1; q.tiles_per_mat = T * (T + 1) / 2;
    q.alpha_pow = 0;
    q.c_acc = c; q.c_e = b;
    q.mvalid = p.mp; q.nvalid = p.mp;
  } else {
    const int TN = p.np / p.tile;
    // c == 0 (a cubic polynomial): B = bA, so the product takes A and folds b
    // into the accumulator scale instead of forming B.
    const bool cubic = (c == 0.0f);
    q.P = cubic ? A : B; q.Q = Xt; q.sP = sa; q.sQ = sx; q.ldp = p.mp; q.ldq = p.mp; q.K = p.mp;
    q.Et = Xt; q.sEt = sx; q.lde = p.mp;
    q.tm = T; q.tn = TN; q.sym = 0; q.tiles_per_mat = T * TN;
    q.alpha_pow = (t == 0) ? 1 : 0;
    q.c_acc = cubic ? b : 1.0f; q.c_e = a;
    const bool last = (t == steps - 1);
    if (!last) {
      q.C = Xn; q.sC = sx; q.ldc = p.np;
      q.Ct = Xtn; q.sCt = sx; q.ldct = p.mp;
      q.mvalid = p.mp; q.nvalid = p.np;
    } else if (fin && fin->ptr) {
      // write the result straight into the caller's dense output
      q.mvalid = p.m; q.nvalid = p.n;
      const int v16 = (fin->ld % 8 == 0) && aligned(fin->ptr, 16) && (fin->stride % 8 == 0);
      if (!p.tall) { q.C = fin->ptr; q.sC = fin->stride; q.ldc = fin->ld; q.c16 = v16; }
      else { q.Ct = fin->ptr; q.sCt = fin->stride; q.ldct = fin->ld; q.ct16 = v16; }
    } else {
      q.mvalid = p.mp; q.nvalid = p.np;
      if (!p.tall) { q.C = Xn; q.sC = sx; q.ldc = p.np; }
      else { q.Ct = Xtn; q.sCt = sx; q.ldct = p.mp; }
    }
  }
  return q;
}

// One Newton-Schulz step t of every thin group: Gram partials, B, X'.
int run_thin(const std::vector<Plan>& plans, int t, int steps, float a, float b, float c, void* ws,
             const std::vector<FinalOut>* fins, hipStream_t s) {
  ThinLaunch L{};
  L.first = (t == 0) ? 1 : 0;
  L.a = a;
  L.b = b;
  L.c = c;
  std::vector<int> ids;
  for (size_t g = 0; g < plans.size(); ++g)
    if (plans[g].thin) ids.push_back(static_cast<int>(g));
  if (ids.empty()) return MUON_OK;
  const int cur = t & 1, nxt = cur ^ 1;
  const bool last = (t == steps - 1);
  L.ngroups = static_cast<int>(ids.size());
  for (size_t k = 0; k < ids.size(); ++k) {
    const Plan& p = plans[ids[k]];
    ThinGroup& q = L.g[k];
    q.X = at<bf16_t>(ws, p.off_X[cur]);
    q.x_stride = static_cast<int64_t>(p.mp) * p.np;
    q.np = p.np;
    q.mb = p.mq / 32;
    q.chunk = p.chunk;
    q.nchunk = p.nchunk;
    q.part = at<float>(ws, p.off_thin_part);
    q.Bm = at<float>(ws, p.off_thin_B);
    q.inv = at<float>(ws, p.off_inv);
    q.batch = p.batch;
    const FinalOut* fin = fins ? &(*fins)[ids[k]] : nullptr;
    if (!last) {
      q.D = at<bf16_t>(ws, p.off_X[nxt]);
      q.d_stride = q.x_stride;
      q.d_ld = p.np;
      q.d_trans = 0;
      q.d_rvalid = p.mq;
      q.d_cvalid = p.np;
      q.d_vec = 1;
    } else if (fin && fin->ptr) {
      // straight into the caller's dense output, in the matrix's own layout
      q.D = fin->ptr;
      q.d_stride = fin->stride;
      q.d_ld = fin->ld;
      q.d_trans = p.tall ? 1 : 0;
      q.d_rvalid = p.tall ? p.n : p.m;
      q.d_cvalid = p.tall ? p.m : p.n;
      q.d_vec = (fin->ld % 8 == 0) && aligned(fin->ptr, 16) && (fin->stride % 8 == 0);
    } else if (!p.tall) {
      q.D = at<bf16_t>(ws, p.off_X[nxt]);
      q.d_stride = q.x_stride;
      q.d_ld = p.np;
      q.d_trans = 0;
      q.d_rvalid = p.mq;
      q.d_cvalid = p.np;
      q.d_vec = 1;
    } else {
      // the workspace's transposed buffer [np][mp], the tall matrix's layout
      q.D = at<bf16_t>(ws, p.off_Xt[nxt]);
      q.d_stride = q.x_stride;
      q.d_ld = p.mp;
      q.d_trans = 1;
      q.d_rvalid = p.np;
      q.d_cvalid = p.mq;
      q.d_vec = 1;
    }
  }
  static const int kinds[3] = {KIND_THIN_GRAM, KIND_THIN_POLY, KIND_THIN_BX};
  for (int stage = 0; stage < 3; ++stage) {
    int blocks = 0;
    for (size_t k = 0; k < ids.size(); ++k) {
      const Plan& p = plans[ids[k]];
      L.prefix[k] = blocks;
      blocks += p.batch * (stage == 0 ? p.nchunk : stage == 1 ? 1 : p.np / 128);
    }
    L.prefix[ids.size()] = blocks;
    MUON_LAUNCH(kinds[stage], s, launch_thin(L, stage, blocks, s));
  }
  return MUON_OK;
}

int run_ns(const std::vector<Plan>& plans, int steps, float a, float b, float c, void* ws,
           const std::vector<FinalOut>* fins, hipStream_t s) {
  static const int kinds[3] = {KIND_NS_SYRK, KIND_NS_POLY, KIND_NS_BX};
  static const int slice_kinds[3] = {KIND_NS_SYRK_SLICES, KIND_NS_POLY_SLICES, KIND_NS_BX};
  for (int t = 0; t < steps; ++t) {
    int st = run_thin(plans, t, steps, a, b, c, ws, fins, s);
    if (st != MUON_OK) return st;
    for (int stage = 0; stage < 3; ++stage) {
      if (stage == STAGE_POLY && c == 0.0f) continue;
      for (int tile : {256, 128}) {
        GemmLaunch L{};
        int tiles = 0;
        // problems by decreasing contraction length, so that the blocks
        // dispatched last, which set the launch's tail, are the shortest
        std::vector<int> order;
        for (size_t g = 0; g < plans.size(); ++g)
          if (plans[g].tile == tile && !plans[g].thin) order.push_back(static_cast<int>(g));
        auto klen = [&](int g) { return stage == STAGE_SYRK ? plans[g].np : plans[g].mp; };
        std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return klen(x) > klen(y); });
        for (int g : order) {
          GemmProb q = make_prob(plans[g], stage, t, steps, a, b, c, ws, fins ? &(*fins)[g] : nullptr);
          q.ntiles = plans[g].batch * q.tiles_per_mat;
          L.prefix[L.nprob] = tiles;
          L.p[L.nprob] = q;
          tiles += (q.ntiles + 7) / 8 * 8;
          ++L.nprob;
        }
        if (L.nprob == 0) continue;
        L.prefix[L.nprob] = tiles;
        // column bands per XCD when every problem of a B X launch allows them
        L.band = (stage == STAGE_BX) ? 1 : 0;
        for (int k = 0; k < L.nprob; ++k)
          if (L.p[k].tn % 8 != 0) L.band = 0;
        // A symmetric 256-tile product whose tiles leave a last wave at most
        // half full runs those last tiles as column halves in a second launch:
        // the last wave then takes about half as long.
        const int ncu = cu_count();
        const int tail = (ncu > 0 && tiles > ncu) ? tiles % ncu : 0;
        const bool split = (stage != STAGE_BX) && tile == 256 && tail > 0 && 2 * tail <= ncu;
        MUON_LAUNCH(kinds[stage], s, launch_ns_gemm(L, tile, stage, split ? tiles - tail : tiles, s));
        if (split) {
          L.lin0 = tiles - tail;
          MUON_LAUNCH(slice_kinds[stage], s, launch_ns_gemm_slices(L, stage, 2 * tail, s));
        }
      }
    }
  }
  return MUON_OK;
}

float update_scale(int mode, int rows, int cols, float rms) {
  if (mode == MUON_SCALE_MOONLIGHT) return static_cast<float>(rms * sqrt(static_cast<double>(std::max(rows, cols))));
  if (mode == MUON_SCALE_SPECTRAL) return static_cast<float>(sqrt(static_cast<double>(rows) / cols));
  return 1.0f;
}

}  // namespace
}  // namespace muon

using namespace muon;

extern "C" {

const char* muon_status_string(int status) {
  switch (status) {
    case MUON_OK: return "ok";
    case MUON_ERR_INVALID_ARG: return "invalid argument";
    case MUON_ERR_UNSUPPORTED: return "unsupported configuration";
    case MUON_ERR_WORKSPACE: return "workspace missing or too small";
    case MUON_ERR_HIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

size_t muon_step_workspace_size(const muon_group_t* groups, int n_groups) {
  if (check_groups(groups, n_groups) != MUON_OK) return 0;
  size_t total = 0;
  plans_for(groups, n_groups, total);
  return total;
}

int muon_step_workspace_layout(const muon_group_t* groups, int n_groups, int g, int ns_steps,
                               muon_ws_layout_t* out) {
  int st = check_groups(groups, n_groups);
  if (st != MUON_OK) return st;
  if (!out || g < 0 || g >= n_groups || ns_steps < 1 || ns_steps > 64) return MUON_ERR_INVALID_ARG;
  size_t total = 0;
  std::vector<Plan> plans = plans_for(groups, n_groups, total);
  const Plan& p = plans[g];
  const int fin = ns_steps & 1;
  out->o_offset = p.tall ? p.off_Xt[fin] : p.off_X[fin];
  out->o_batch_stride = static_cast<int64_t>(p.mp) * p.np;
  out->o_ld = p.tall ? p.mp : p.np;
  out->inv_norm_offset = p.off_inv;
  out->x0_offset = p.off_X[0];
  out->x0_batch_stride = static_cast<int64_t>(p.mp) * p.np;
  out->x0_ld = p.np;
  return MUON_OK;
}

int muon_step(const muon_group_t* groups, int n_groups, int param_dtype, const muon_hparams_t* hp,
              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_groups(groups, n_groups);
  if (st != MUON_OK) return st;
  if (!hp || (param_dtype != MUON_DTYPE_F32 && param_dtype != MUON_DTYPE_BF16)) return MUON_ERR_INVALID_ARG;
  if (hp->ns_steps < 1 || hp->ns_steps > 64) return MUON_ERR_INVALID_ARG;
  if (hp->scale_mode < MUON_SCALE_MOONLIGHT || hp->scale_mode > MUON_SCALE_NONE) return MUON_ERR_INVALID_ARG;
  if (!(hp->ns_eps >= 0.0f) || !isfinite(hp->lr) || !isfinite(hp->momentum) || !isfinite(hp->weight_decay))
    return MUON_ERR_INVALID_ARG;
  for (int g = 0; g < n_groups; ++g)
    if (!groups[g].param || !groups[g].grad || !groups[g].momentum) return MUON_ERR_INVALID_ARG;
  size_t need = 0;
  std::vector<Plan> plans = plans_for(groups, n_groups, need);
  if (!workspace || workspace_bytes < need || !aligned(workspace, kAlign)) return MUON_ERR_WORKSPACE;
  Range range("muon_step");

  const int fin = hp->ns_steps & 1;
  // small groups: the whole step in one launch, one workgroup per matrix,
  // with X0, 1/||U|| and O left in the same workspace places as below
  SmallLaunch S{};
  int small_mats = 0;
  std::vector<int> big;
  for (int g = 0; g < n_groups; ++g) {
    const Plan& p = plans[g];
    if (!small_ok(p.rows, p.cols)) {
      big.push_back(g);
      continue;
    }
    SmallGroup& q = S.g[S.ngroups];
    q.G = groups[g].grad;
    q.M = groups[g].momentum;
    q.W = groups[g].param;
    q.bstride = p.bstride;
    q.rows = p.rows;
    q.cols = p.cols;
    q.tall = p.tall ? 1 : 0;
    q.m = p.m;
    q.n = p.n;
    q.X0 = at<bf16_t>(workspace, p.off_X[0]);
    q.x0_stride = static_cast<int64_t>(p.mp) * p.np;
    q.x0_ld = p.np;
    q.O = at<bf16_t>(workspace, p.tall ? p.off_Xt[fin] : p.off_X[fin]);
    q.o_stride = static_cast<int64_t>(p.mp) * p.np;
    q.o_ld = p.tall ? p.mp : p.np;
    q.inv = at<float>(workspace, p.off_inv);
    const float scale = update_scale(hp->scale_mode, p.rows, p.cols, hp->rms_target);
    q.decay = static_cast<float>(1.0 - static_cast<double>(hp->lr) * hp->weight_decay);
    q.step = static_cast<float>(static_cast<double>(hp->lr) * scale);
    q.vec = (p.cols % 8 == 0) && (p.bstride % 8 == 0) && aligned(q.G, 16) && aligned(q.M, 16) && aligned(q.W, 16);
    q.ovec = (p.cols % 8 == 0) && aligned(q.O, 16);
    S.prefix[S.ngroups] = small_mats;
    small_mats += p.batch;
    ++S.ngroups;
  }
  S.prefix[S.ngroups] = small_mats;
  if (S.ngroups > 0) {
    S.mu = hp->momentum;
    S.nesterov = hp->nesterov ? 1 : 0;
    S.eps = hp->ns_eps;
    S.steps = hp->ns_steps;
    S.a = hp->ns_a;
    S.b = hp->ns_b;
    S.c = hp->ns_c;
    MUON_LAUNCH(KIND_SMALL_STEP, stream, launch_small_step(S, param_dtype, small_mats, stream));
  }
  if (big.empty()) return MUON_OK;

  std::vector<Plan> bp;
  std::vector<PrepIn> ins;
  for (int g : big) {
    bp.push_back(plans[g]);
    ins.push_back({groups[g].grad, groups[g].momentum});
  }
  {
    Range stage("muon_step: momentum and normalisation");
    st = launch_prep(bp, ins, param_dtype, hp->momentum, hp->nesterov ? 1 : 0, workspace, stream);
    if (st != MUON_OK) return st;
    st = launch_finalize(bp, hp->ns_eps, workspace, stream);
    if (st != MUON_OK) return st;
  }
  {
    Range stage("muon_step: Newton-Schulz");
    st = run_ns(bp, hp->ns_steps, hp->ns_a, hp->ns_b, hp->ns_c, workspace, nullptr, stream);
    if (st != MUON_OK) return st;
  }
  Range stage("muon_step: update");

  UpdateLaunch U{};
  U.ngroups = static_cast<int>(big.size());
  int64_t blocks = 0;
  const size_t esz = param_dtype == MUON_DTYPE_BF16 ? 2 : 4;
  for (int k = 0; k < U.ngroups; ++k) {
    const int g = big[k];
    const Plan& p = bp[k];
    UpdateGroup& u = U.g[k];
    u.W = groups[g].param;
    u.O = at<bf16_t>(workspace, p.tall ? p.off_Xt[fin] : p.off_X[fin]);
    u.bstride = p.bstride;
    u.o_bstride = static_cast<int64_t>(p.mp) * p.np;
    u.o_ld = p.tall ? p.mp : p.np;
    u.rows = p.rows;
    u.cols = p.cols;
    u.batch = p.batch;
    u.vec = (p.cols % 8 == 0) && (p.bstride % 8 == 0) && aligned(u.W, 8 * esz);
    const int64_t per = (static_cast<int64_t>(p.rows) * p.cols + 2047) / 2048;
    u.blocks = per * p.batch;
    const float scale = update_scale(hp->scale_mode, p.rows, p.cols, hp->rms_target);
    u.decay = static_cast<float>(1.0 - static_cast<double>(hp->lr) * hp->weight_decay);
    u.step = static_cast<float>(static_cast<double>(hp->lr) * scale);
    U.prefix[k] = blocks;
    blocks += u.blocks;
  }
  U.prefix[U.ngroups] = blocks;
  MUON_LAUNCH(KIND_PARAM_UPDATE, stream, launch_param_update(U, param_dtype, blocks, stream));
  return MUON_OK;
}

size_t ns_workspace_size(int batch, int rows, int cols) {
  if (!dims_ok(batch, rows, cols)) return 0;
  size_t cursor = 0;
  make_plan(batch, rows, cols, static_cast<int64_t>(rows) * cols, cursor);
  return cursor;
}

int ns_orthogonalize(const void* in, int in_dtype, uint16_t* out, int batch, int rows, int cols,
                     int64_t batch_stride, int steps, float a, float b, float c, float eps,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!in || !out || !dims_ok(batch, rows, cols)) return MUON_ERR_INVALID_ARG;
  if (in_dtype != MUON_DTYPE_F32 && in_dtype != MUON_DTYPE_BF16) return MUON_ERR_INVALID_ARG;
  if (batch_stride < static_cast<int64_t>(rows) * cols) return MUON_ERR_INVALID_ARG;
  if (steps < 1 || steps > 64 || !(eps >= 0.0f)) return MUON_ERR_INVALID_ARG;
  size_t need = 0;
  std::vector<Plan> plans;
  plans.push_back(make_plan(batch, rows, cols, batch_stride, need));
  if (!workspace || workspace_bytes < need || !aligned(workspace, kAlign)) return MUON_ERR_WORKSPACE;
  Range range("ns_orthogonalize");
  if (small_ok(rows, cols)) {
    const Plan& p = plans[0];
    SmallLaunch S{};
    S.ngroups = 1;
    S.prefix[0] = 0;
    S.prefix[1] = batch;
    SmallGroup& q = S.g[0];
    q.G = in;
    q.bstride = batch_stride;
    q.rows = rows;
    q.cols = cols;
    q.tall = p.tall ? 1 : 0;
    q.m = p.m;
    q.n = p.n;
    q.O = reinterpret_cast<bf16_t*>(out);
    q.o_stride = static_cast<int64_t>(rows) * cols;
    q.o_ld = cols;
    q.inv = at<float>(workspace, p.off_inv);
    q.vec = (cols % 8 == 0) && (batch_stride % 8 == 0) && aligned(in, 16);
    q.ovec = (cols % 8 == 0) && aligned(out, 16);
    S.eps = eps;
    S.steps = steps;
    S.a = a;
    S.b = b;
    S.c = c;
    MUON_LAUNCH(KIND_SMALL_STEP, stream, launch_small_step(S, in_dtype, batch, stream));
    return MUON_OK;
  }
  std::vector<PrepIn> ins{{in, nullptr}};
  int st = launch_prep(plans, ins, in_dtype, 0.0f, 0, workspace, stream);
  if (st != MUON_OK) return st;
  st = launch_finalize(plans, eps, workspace, stream);
  if (st != MUON_OK) return st;
  std::vector<FinalOut> fins{{reinterpret_cast<bf16_t*>(out), static_cast<int64_t>(rows) * cols, cols}};
  return run_ns(plans, steps, a, b, c, workspace, &fins, stream);
}

size_t qkclip_rowmax_workspace_size(int B, int T, int H) {
  if (B < 1 || T < 1 || H < 1) return 0;
  const int nqb = (T + 255) / 256;   // the most query blocks of any head dimension (256 queries each)
  return align_up(static_cast<size_t>(B) * H * nqb * sizeof(float));
}

}  // extern "C"

namespace {
// Argument checks shared by the two row-max entry points; nqb receives the
// number of query blocks per (batch row, head) of the row-max kernel.
int rowmax_args(const uint16_t* Q, const uint16_t* K, int B, int T, int H, int d_head, float logit_scale,
                const float* s_max, int* nqb) {
  if (!Q || !K || !s_max || B < 1 || T < 1 || H < 1 || d_head < 1) return MUON_ERR_INVALID_ARG;
  if (!(logit_scale > 0.0f) || !isfinite(logit_scale)) return MUON_ERR_INVALID_ARG;
  if (d_head != 64 && d_head != 128 && d_head != 256) return MUON_ERR_UNSUPPORTED;
  if (!aligned(Q, 16) || !aligned(K, 16)) return MUON_ERR_INVALID_ARG;
  if (static_cast<int64_t>(B) * T * H * d_head > (int64_t(1) << 40)) return MUON_ERR_INVALID_ARG;
  const int qblk = qk_rowmax_query_block(d_head);
  *nqb = (T + qblk - 1) / qblk;   // query blocks of the row-max kernel
  if (static_cast<int64_t>(B) * H * *nqb > (int64_t(1) << 31) - 1) return MUON_ERR_INVALID_ARG;
  return MUON_OK;
}
}  // namespace

extern "C" {

int qkclip_rowmax(const uint16_t* Q, const uint16_t* K, int B, int T, int H, int d_head, float logit_scale,
                  int causal, float* s_max, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int nqb = 0;
  const int st = rowmax_args(Q, K, B, T, H, d_head, logit_scale, s_max, &nqb);
  if (st != MUON_OK) return st;
  const size_t need = qkclip_rowmax_workspace_size(B, T, H);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return MUON_ERR_WORKSPACE;
  Range range("qkclip_rowmax");
  float* partial = static_cast<float*>(workspace);
  MUON_LAUNCH(KIND_QK_ROWMAX, stream,
              launch_qk_rowmax(reinterpret_cast<const bf16_t*>(Q), reinterpret_cast<const bf16_t*>(K), B, T, H,
                               d_head, causal ? 1 : 0, partial, nqb, stream));
  MUON_LAUNCH(KIND_QK_REDUCE, stream, launch_qk_reduce(partial, B, H, nqb, logit_scale, s_max, stream));
  return MUON_OK;
}

size_t qkclip_rowmax_noalloc_max_partials(void) { return static_cast<size_t>(kNoAllocPartials); }

int qkclip_rowmax_noalloc(const uint16_t* Q, const uint16_t* K, int B, int T, int H, int d_head, float logit_scale,
                          int causal, float* s_max, hipStream_t stream) {
  int nqb = 0;
  const int st = rowmax_args(Q, K, B, T, H, d_head, logit_scale, s_max, &nqb);
  if (st != MUON_OK) return st;
  if (static_cast<int64_t>(B) * H * nqb > kNoAllocPartials) return MUON_ERR_WORKSPACE;
  Range range("qkclip_rowmax_noalloc");
  float* partial = nullptr;
  if (noalloc_partials(&partial) != hipSuccess) return MUON_ERR_HIP;
  // every partial the reduction reads is written by its row-max block first,
  // so the scratch needs no clearing between calls
  MUON_LAUNCH(KIND_QK_ROWMAX, stream,
              launch_qk_rowmax(reinterpret_cast<const bf16_t*>(Q), reinterpret_cast<const bf16_t*>(K), B, T, H,
                               d_head, causal ? 1 : 0, partial, nqb, stream));
  MUON_LAUNCH(KIND_QK_REDUCE, stream, launch_qk_reduce(partial, B, H, nqb, logit_scale, s_max, stream));
  return MUON_OK;
}

int qkclip_rescale_slices(const qkclip_slice_t* slices, int n_slices, int dtype, int H, const float* s_max,
                          float tau, int32_t* clipped, hipStream_t stream) {
  if (!slices || n_slices < 1 || n_slices > QKCLIP_MAX_SLICES || !s_max || H < 1 || H > 65535)
    return MUON_ERR_INVALID_ARG;
  if (dtype != MUON_DTYPE_F32 && dtype != MUON_DTYPE_BF16) return MUON_ERR_INVALID_ARG;
  if (!(tau > 0.0f) || !isfinite(tau)) return MUON_ERR_INVALID_ARG;
  RescaleLaunch L{};
  L.nmat = n_slices;
  for (int z = 0; z < n_slices; ++z) {
    const qkclip_slice_t& q = slices[z];
    if (!q.w || q.rows_per_head < 1 || q.cols < 1 || q.head_pitch < q.rows_per_head) return MUON_ERR_INVALID_ARG;
    if (!(q.exponent >= 0.0f && q.exponent <= 1.0f)) return MUON_ERR_INVALID_ARG;
    if (static_cast<int64_t>(q.rows_per_head) * q.cols > (int64_t(1) << 40)) return MUON_ERR_INVALID_ARG;
    if (q.head_pitch > (int64_t(1) << 40) / q.cols) return MUON_ERR_INVALID_ARG;
    RescaleMat& R = L.m[z];
    R.W = q.w;
    R.head_pitch = q.head_pitch;
    R.rows_per_head = q.rows_per_head;
    R.cols = q.cols;
    R.expo = q.exponent;
    R.vec = (q.cols % 8 == 0) && aligned(q.w, 16);
  }
  Range range("qkclip_rescale");
  MUON_LAUNCH(KIND_QK_RESCALE, stream, launch_qk_rescale(L, dtype, H, s_max, tau, clipped, stream));
  return MUON_OK;
}

int qkclip_rescale(void* Wq, void* Wk, int dtype, int H, int d_head, int d_model, const float* s_max, float tau,
                   float alpha, int32_t* clipped, hipStream_t stream) {
  if (!(alpha >= 0.0f && alpha <= 1.0f)) return MUON_ERR_INVALID_ARG;
  if (d_head < 1) return MUON_ERR_INVALID_ARG;
  const qkclip_slice_t sl[2] = {{Wq, d_head, d_head, d_model, alpha}, {Wk, d_head, d_head, d_model, 1.0f - alpha}};
  return qkclip_rescale_slices(sl, 2, dtype, H, s_max, tau, clipped, stream);
}

int qkclip_rescale_mla(void* Wqc, void* Wkc, void* Wqr, int dtype, int H, int d_c, int d_r, int q_cols,
                       int kv_cols, const float* s_max, float tau, int32_t* clipped, hipStream_t stream) {
  if (d_c < 1 || d_r < 1) return MUON_ERR_INVALID_ARG;
  const qkclip_slice_t sl[3] = {{Wqc, d_c, d_c, q_cols, 0.5f}, {Wkc, d_c, d_c, kv_cols, 0.5f},
                                {Wqr, d_r, d_r, q_cols, 1.0f}};
  return qkclip_rescale_slices(sl, 3, dtype, H, s_max, tau, clipped, stream);
}

int adamw_step(const adamw_tensor_t* tensors, int n_tensors, int dtype, const adamw_hparams_t* hp,
               hipStream_t stream) {
  if (!tensors || n_tensors < 0 || !hp) return MUON_ERR_INVALID_ARG;
  if (dtype != MUON_DTYPE_F32 && dtype != MUON_DTYPE_BF16) return MUON_ERR_INVALID_ARG;
  if (hp->step < 1 || !(hp->beta1 >= 0.0f && hp->beta1 < 1.0f) || !(hp->beta2 >= 0.0f && hp->beta2 < 1.0f) ||
      !(hp->eps > 0.0f) || !isfinite(hp->lr) || !isfinite(hp->weight_decay))
    return MUON_ERR_INVALID_ARG;
  const size_t esz = dtype == MUON_DTYPE_BF16 ? 2 : 4;
  for (int i = 0; i < n_tensors; ++i) {
    const adamw_tensor_t& t = tensors[i];
    if (t.numel < 0 || t.numel > (int64_t(1) << 40)) return MUON_ERR_INVALID_ARG;
    if (t.numel > 0 && (!t.param || !t.grad || !t.exp_avg || !t.exp_avg_sq)) return MUON_ERR_INVALID_ARG;
    if (t.numel > 0 && (!aligned(t.param, esz) || !aligned(t.grad, esz) || !aligned(t.exp_avg, 4) ||
                        !aligned(t.exp_avg_sq, 4)))
      return MUON_ERR_INVALID_ARG;
  }
  Range range("adamw_step");
  AdamWLaunch A{};
  A.lr = hp->lr;
  A.beta1 = hp->beta1;
  A.beta2 = hp->beta2;
  A.eps = hp->eps;
  A.decay = static_cast<float>(1.0 - static_cast<double>(hp->lr) * hp->weight_decay);
  A.c1 = static_cast<float>(1.0 / (1.0 - std::pow(static_cast<double>(hp->beta1), hp->step)));
  A.c2 = static_cast<float>(1.0 / (1.0 - std::pow(static_cast<double>(hp->beta2), hp->step)));
  int i = 0;
  while (i < n_tensors) {
    A.ntensors = 0;
    int64_t blocks = 0;
    for (; i < n_tensors && A.ntensors < kAdamWMaxTensors; ++i) {
      const adamw_tensor_t& t = tensors[i];
      if (t.numel == 0) continue;
      const int64_t nb = (t.numel + 4095) / 4096;   // 4096 elements per block
      if (A.ntensors > 0 && blocks + nb > (int64_t(1) << 30)) break;
      AdamWTensor& T = A.t[A.ntensors];
      T.p = t.param;
      T.g = t.grad;
      T.m = t.exp_avg;
      T.v = t.exp_avg_sq;
      T.n = t.numel;
      T.vec = aligned(t.param, 16) && aligned(t.grad, 16) && aligned(t.exp_avg, 16) && aligned(t.exp_avg_sq, 16);
      A.blk_start[A.ntensors] = static_cast<int>(blocks);
      blocks += nb;
      ++A.ntensors;
    }
    if (A.ntensors == 0) break;
    A.blk_start[A.ntensors] = static_cast<int>(blocks);
    MUON_LAUNCH(KIND_ADAMW, stream, launch_adamw(A, dtype, static_cast<int>(blocks), stream));
  }
  return MUON_OK;
}

size_t attn_fwd_workspace_size(int B, int T, int H) {
  if (B < 1 || T < 1 || H < 1) return 0;
  const int nqb = (T + 127) / 128;
  return align_up(static_cast<size_t>(B) * H * nqb * 4 * sizeof(float));
}

int attn_fwd(const uint16_t* Q, const uint16_t* K, const uint16_t* V, int B, int T, int H, int d_head,
             float logit_scale, int causal, uint16_t* O, float* lse, float* s_max, void* workspace,
             size_t workspace_bytes, hipStream_t stream) {
  if (!Q || !K || !V || !O || !s_max || B < 1 || T < 1 || H < 1) return MUON_ERR_INVALID_ARG;
  if (d_head != 128) return MUON_ERR_UNSUPPORTED;
  if (!(logit_scale > 0.0f) || !isfinite(logit_scale)) return MUON_ERR_INVALID_ARG;
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16)) return MUON_ERR_INVALID_ARG;
  if (lse && !aligned(lse, 4)) return MUON_ERR_INVALID_ARG;
  if (static_cast<int64_t>(B) * T * H * d_head > (int64_t(1) << 40)) return MUON_ERR_INVALID_ARG;
  const int nqb = (T + 127) / 128;
  if (static_cast<int64_t>(B) * H * nqb > (int64_t(1) << 31) - 1) return MUON_ERR_INVALID_ARG;
  const size_t need = attn_fwd_workspace_size(B, T, H);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return MUON_ERR_WORKSPACE;
  Range range("attn_fwd");
  AttnArgs A{};
  A.Q = reinterpret_cast<const bf16_t*>(Q);
  A.K = reinterpret_cast<const bf16_t*>(K);
  A.V = reinterpret_cast<const bf16_t*>(V);
  A.O = reinterpret_cast<bf16_t*>(O);
  A.lse = lse;
  A.partial = static_cast<float*>(workspace);
  A.B = B; A.T = T; A.H = H; A.nqb = nqb;
  A.scale = logit_scale;
  A.c2 = static_cast<float>(static_cast<double>(logit_scale) * 1.4426950408889634);
  MUON_LAUNCH(KIND_ATTN_FWD, stream, launch_attn_fwd(A, causal ? 1 : 0, stream));
  MUON_LAUNCH(KIND_QK_REDUCE, stream, launch_qk_reduce(A.partial, B, H, nqb * 4, logit_scale, s_max, stream));
  return MUON_OK;
}

// ----------------------------------------------------------------------------
// Dion
// ----------------------------------------------------------------------------
}  // extern "C"

namespace {
struct DionPlan {
  int rp, nsplit;
  size_t gram_per;  // doubles per matrix in the Gram region
  size_t off_pa, off_pb, off_r, off_lt, off_inv, off_gram, total;
};

bool dion_dims_ok(int batch, int rows, int cols, int rank) {
  if (batch < 1 || rows < 1 || cols < 1 || rank < 1) return false;
  if (rows > (1 << 20) || cols > (1 << 20)) return false;
  return static_cast<int64_t>(rows) * cols < (int64_t(1) << 31);
}

DionPlan dion_plan(int batch, int rows, int cols, int rank) {
  DionPlan d{};
  d.rp = round_up(rank, 32);
  d.nsplit = (rows + 127) / 128;
  size_t c = 0;
  auto take = [&](size_t bytes) {
    const size_t o = c;
    c = align_up(c + bytes);
    return o;
  };
  const size_t b = static_cast<size_t>(batch), rp = static_cast<size_t>(d.rp);
  d.off_pa = take(b * rows * rp * sizeof(float));
  d.off_pb = take(b * rows * rp * sizeof(float));
  d.off_r = take(b * cols * rp * sizeof(float));
  d.off_lt = take(b * rp * rp * sizeof(float));
  d.off_inv = take(b * rp * sizeof(float));
  // Gram partials, later the column sums of squares of R per 64 rows
  d.gram_per = std::max(static_cast<size_t>(d.nsplit) * rp * rp, static_cast<size_t>((cols + 63) / 64) * rp);
  d.off_gram = take(b * d.gram_per * sizeof(double));
  d.total = c;
  return d;
}
}  // namespace

extern "C" {

size_t dion_workspace_size(int batch, int rows, int cols, int rank) {
  if (!dion_dims_ok(batch, rows, cols, rank)) return 0;
  return dion_plan(batch, rows, cols, rank).total;
}

int dion_step(void* param, int dtype, const void* grad, float* momentum, float* q, int batch, int rows, int cols,
              int rank, int64_t batch_stride, float lr, float mu, void* workspace, size_t workspace_bytes,
              hipStream_t stream) {
  if (!param || !grad || !momentum || !q) return MUON_ERR_INVALID_ARG;
  if (dtype != MUON_DTYPE_F32 && dtype != MUON_DTYPE_BF16) return MUON_ERR_INVALID_ARG;
  if (!dion_dims_ok(batch, rows, cols, rank)) return MUON_ERR_INVALID_ARG;
  if (batch_stride < static_cast<int64_t>(rows) * cols) return MUON_ERR_INVALID_ARG;
  if (!isfinite(lr) || !isfinite(mu)) return MUON_ERR_INVALID_ARG;
  if (rank % 8 != 0 || rank > 128 || rank > std::min(rows, cols) || rows % 8 != 0 || cols % 8 != 0 ||
      batch_stride % 8 != 0 || batch > 65535 || !aligned(param, 16) || !aligned(grad, 16) ||
      !aligned(momentum, 16) || !aligned(q, 16))
    return MUON_ERR_UNSUPPORTED;
  const DionPlan d = dion_plan(batch, rows, cols, rank);
  if (!workspace || workspace_bytes < d.total || !aligned(workspace, kAlign)) return MUON_ERR_WORKSPACE;

  Range range("dion_step");
  DionArgs A{};
  A.G = grad;
  A.M = momentum;
  A.W = param;
  A.Q = q;
  A.bstride = batch_stride;
  A.q_stride = static_cast<int64_t>(cols) * rank;
  A.m = rows;
  A.n = cols;
  A.r = rank;
  A.rp = d.rp;
  A.nsplit = d.nsplit;
  A.mu = mu;
  A.lr = lr;
  float* Pa = at<float>(workspace, d.off_pa);
  float* Pb = at<float>(workspace, d.off_pb);
  const int64_t ps = static_cast<int64_t>(rows) * d.rp;
  A.R = at<float>(workspace, d.off_r);
  A.r_stride = static_cast<int64_t>(cols) * d.rp;
  A.Lt = at<float>(workspace, d.off_lt);
  A.lt_stride = static_cast<int64_t>(d.rp) * d.rp;
  A.inv = at<float>(workspace, d.off_inv);
  A.gram = at<double>(workspace, d.off_gram);
  A.gram_stride = static_cast<int64_t>(d.gram_per);

  // P0 = B Q
  A.dst = Pa;
  A.dst_stride = ps;
  MUON_LAUNCH(KIND_DION_BQ, stream, launch_dion_gemm(A, DION_BQ, dtype, batch, stream));
  // Cholesky-QR, twice: Pa -> Pb -> Pa
  for (int pass = 0; pass < 2; ++pass) {
    float* from = pass == 0 ? Pa : Pb;
    float* to = pass == 0 ? Pb : Pa;
    A.src = from;
    A.src_stride = ps;
    MUON_LAUNCH(KIND_DION_GRAM, stream, launch_dion_gram(A, batch, stream));
    MUON_LAUNCH(KIND_DION_GRAM, stream, launch_dion_gram_reduce(A, batch, stream));
    MUON_LAUNCH(KIND_DION_CHOL, stream, launch_dion_chol(A, batch, stream));
    A.bsrc = A.Lt;
    A.bsrc_stride = A.lt_stride;
    A.dst = to;
    A.dst_stride = ps;
    MUON_LAUNCH(KIND_DION_PL, stream, launch_dion_gemm(A, DION_PL, dtype, batch, stream));
  }
  // R = B^T P
  A.bsrc = Pa;
  A.bsrc_stride = ps;
  A.dst = A.R;
  A.dst_stride = A.r_stride;
  MUON_LAUNCH(KIND_DION_BTP, stream, launch_dion_gemm(A, DION_BTP, dtype, batch, stream));
  // column norms, Q = ColNorm(R)
  MUON_LAUNCH(KIND_DION_COLNORM, stream, launch_dion_colnorm(A, batch, stream));
  // M <- B - (1 - mu) P R^T, W <- W - lr P Q^T
  A.src = Pa;
  A.src_stride = ps;
  A.bsrc = A.R;
  A.bsrc_stride = A.r_stride;
  MUON_LAUNCH(KIND_DION_UPDATE, stream, launch_dion_gemm(A, DION_UPD, dtype, batch, stream));
  return MUON_OK;
}

int muon_mfma_probe(int blocks, int iters, int operands, float* sink, hipStream_t stream) {
  if (blocks < 1 || blocks > (1 << 20) || iters < 1 || iters > (1 << 24) || !sink) return MUON_ERR_INVALID_ARG;
  if (operands != MUON_PROBE_RANDOM && operands != MUON_PROBE_SMOOTH) return MUON_ERR_INVALID_ARG;
  if (launch_mfma_probe(blocks, iters, operands, sink, stream) != hipSuccess) return MUON_ERR_HIP;
  return MUON_OK;
}

int64_t muon_hbm_probe(const void* src, size_t src_bytes, void* dst, size_t dst_bytes, int reads, int writes,
                       int unroll, hipStream_t stream) {
  const bool mix = (reads == 1 && writes == 1) || (reads == 3 && writes == 4) || (reads == 2 && writes == 1);
  if (!src || !dst || !mix || !aligned(src, 16) || !aligned(dst, 16)) return -MUON_ERR_INVALID_ARG;
  if (unroll != 1 && unroll != 4) return -MUON_ERR_INVALID_ARG;
  const int64_t units = static_cast<int64_t>(std::min(src_bytes / (16 * static_cast<size_t>(reads)),
                                                      dst_bytes / (16 * static_cast<size_t>(writes))));
  if (units < 1 || units > (int64_t(1) << 36)) return -MUON_ERR_INVALID_ARG;
  if (launch_hbm_probe(src, dst, units, reads, writes, unroll, stream) != hipSuccess) return -MUON_ERR_HIP;
  return units * 16 * (reads + writes);
}

int muon_profile_enable(int on) {
  for (auto& r : g_prof) {
    g_event_pool.push_back(r.a);
    g_event_pool.push_back(r.b);
  }
  g_prof.clear();
  g_prof_on = on != 0;
  return MUON_OK;
}

int muon_profile_collect(double* total_ms, int64_t* launches, int n_kinds) {
  for (int k = 0; k < n_kinds; ++k) {
    if (total_ms) total_ms[k] = 0.0;
    if (launches) launches[k] = 0;
  }
  for (auto& r : g_prof) {
    if (hipEventSynchronize(r.b) != hipSuccess) return -MUON_ERR_HIP;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return -MUON_ERR_HIP;
    if (r.kind < n_kinds) {
      if (total_ms) total_ms[r.kind] += ms;
      if (launches) launches[r.kind] += 1;
    }
  }
  return KIND_COUNT;
}

const char* muon_kernel_kind_name(int kind) {
  static const char* names[KIND_COUNT] = {"momentum_norm", "norm_finalize", "ns_syrk_xxt", "ns_syrk_poly",
                                          "ns_gemm_bx",    "param_update",  "qk_rowmax",   "qk_reduce",
                                          "qk_rescale",    "adamw",         "attn_fwd",
                                          "ns_syrk_xxt_slices", "ns_syrk_poly_slices", "small_step",
                                          "dion_bq",       "dion_gram",     "dion_chol",   "dion_pl",
                                          "dion_btp",      "dion_colnorm",  "dion_update",
                                          "ns_thin_gram",  "ns_thin_poly",  "ns_thin_bx"};
  if (kind < 0 || kind >= KIND_COUNT) return "unknown";
  return names[kind];
}

}  // extern "C"
