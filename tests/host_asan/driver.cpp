// Host-only driver of libmuon's C ABI for the sanitizer build (see
// stubs.hip): every entry point is called with invalid arguments (each must
// return its documented status and launch nothing) and with valid ones on
// every workload shape and on assorted ragged, thin, tall, small and mixed
// groups (each launch descriptor is checked by the stubs).  Device buffers
// are address ranges that are never dereferenced.  Exits 0 when every check
// holds; a failed check prints a line starting "FAIL".
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <random>
#include <vector>

#include "../../include/muon.h"

extern "C" {
void stub_register(const void* p, uint64_t bytes);
void stub_reset(const char* name);
long stub_launches();
}

static int g_fail = 0;
#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);         \
      ++g_fail;                                                      \
    }                                                                \
  } while (0)

// fake device address space: 1 TiB regions, 256-byte aligned
static uintptr_t g_next = uintptr_t(1) << 40;
static void* fake(uint64_t bytes) {
  const uintptr_t p = g_next;
  g_next += ((bytes + 255) / 256 + 1) * 256;
  stub_register(reinterpret_cast<void*>(p), bytes);
  return reinterpret_cast<void*>(p);
}

static muon_hparams_t hparams(int steps = 5, float c = 2.0315f) {
  muon_hparams_t h{};
  h.lr = 0.02f;
  h.momentum = 0.95f;
  h.weight_decay = 0.1f;
  h.nesterov = 1;
  h.ns_steps = steps;
  h.ns_a = 3.4445f;
  h.ns_b = -4.7750f;
  h.ns_c = c;
  h.ns_eps = 1e-7f;
  h.scale_mode = MUON_SCALE_MOONLIGHT;
  h.rms_target = 0.2f;
  return h;
}

struct Shape {
  int batch, rows, cols;
  int64_t pad;   // extra elements between matrices
};

static void run_step(const char* name, const std::vector<Shape>& shapes, int dtype, int steps, float c = 2.0315f) {
  stub_reset(name);
  const int esz = dtype == MUON_DTYPE_BF16 ? 2 : 4;
  std::vector<muon_group_t> gs;
  for (const Shape& s : shapes) {
    muon_group_t g{};
    g.batch = s.batch;
    g.rows = s.rows;
    g.cols = s.cols;
    g.batch_stride = int64_t(s.rows) * s.cols + s.pad;
    const uint64_t n = uint64_t(s.batch) * g.batch_stride;
    g.param = fake(n * esz);
    g.grad = fake(n * esz);
    g.momentum = static_cast<float*>(fake(n * 4));
    gs.push_back(g);
  }
  const size_t ws = muon_step_workspace_size(gs.data(), int(gs.size()));
  CHECK(ws > 0);
  void* w = fake(ws);
  const muon_hparams_t hp = hparams(steps, c);
  const int st = muon_step(gs.data(), int(gs.size()), dtype, &hp, w, ws, nullptr);
  if (st != MUON_OK) printf("FAIL %s: muon_step returned %d\n", name, st), ++g_fail;
  CHECK(stub_launches() > 0);
  // one byte short of the workspace: refused, nothing launched
  stub_reset(name);
  stub_register(w, ws);
  CHECK(muon_step(gs.data(), int(gs.size()), dtype, &hp, w, ws - 1, nullptr) == MUON_ERR_WORKSPACE);
  CHECK(stub_launches() == 0);
  // the layout query stays inside the workspace
  for (int g = 0; g < int(gs.size()); ++g) {
    muon_ws_layout_t lay{};
    CHECK(muon_step_workspace_layout(gs.data(), int(gs.size()), g, steps, &lay) == MUON_OK);
    const int m = gs[g].rows < gs[g].cols ? gs[g].rows : gs[g].cols;
    const int n = gs[g].rows < gs[g].cols ? gs[g].cols : gs[g].rows;
    const uint64_t o_end = lay.o_offset + 2 * ((gs[g].batch - 1) * lay.o_batch_stride +
                                               (gs[g].rows - 1) * lay.o_ld + gs[g].cols);
    const uint64_t x_end = lay.x0_offset + 2 * ((gs[g].batch - 1) * lay.x0_batch_stride + (m - 1) * lay.x0_ld + n);
    CHECK(o_end <= ws && x_end <= ws && lay.inv_norm_offset + 4 * gs[g].batch <= ws);
  }
}

static void run_ns(const char* name, int batch, int rows, int cols, int dtype, int steps) {
  stub_reset(name);
  const int esz = dtype == MUON_DTYPE_BF16 ? 2 : 4;
  const uint64_t n = uint64_t(batch) * rows * cols;
  void* in = fake(n * esz);
  uint16_t* out = static_cast<uint16_t*>(fake(n * 2));
  const size_t ws = ns_workspace_size(batch, rows, cols);
  CHECK(ws > 0);
  void* w = fake(ws);
  const int st = ns_orthogonalize(in, dtype, out, batch, rows, cols, int64_t(rows) * cols, steps, 3.4445f, -4.775f,
                                  2.0315f, 1e-7f, w, ws, nullptr);
  if (st != MUON_OK) printf("FAIL %s: ns_orthogonalize returned %d\n", name, st), ++g_fail;
}

static void invalid_arguments() {
  stub_reset("invalid arguments");
  const muon_hparams_t hp = hparams();
  muon_group_t g{};
  g.batch = 1;
  g.rows = 8;
  g.cols = 8;
  g.batch_stride = 64;
  g.param = fake(256);
  g.grad = fake(256);
  g.momentum = static_cast<float*>(fake(256));
  void* w = fake(1 << 20);
  CHECK(muon_step(nullptr, 1, 0, &hp, w, 1 << 20, nullptr) == MUON_ERR_INVALID_ARG);
  CHECK(muon_step(&g, 0, 0, &hp, w, 1 << 20, nullptr) == MUON_ERR_INVALID_ARG);
  CHECK(muon_step(&g, MUON_MAX_GROUPS + 1, 0, &hp, w, 1 << 20, nullptr) == MUON_ERR_INVALID_ARG);
  CHECK(muon_step(&g, 1, 7, &hp, w, 1 << 20, nullptr) == MUON_ERR_INVALID_ARG);
  CHECK(muon_step(&g, 1, 0, nullptr, w, 1 << 20, nullptr) == MUON_ERR_INVALID_ARG);
  muon_hparams_t bad = hp;
  bad.ns_steps = 0;
  CHECK(muon_step(&g, 1, 0, &bad, w, 1 << 20, nullptr) == MUON_ERR_INVALID_ARG);
  bad = hp;
  bad.scale_mode = 9;
  CHECK(muon_step(&g, 1, 0, &bad, w, 1 << 20, nullptr) == MUON_ERR_INVALID_ARG);
  bad = hp;
  bad.lr = 1.0f / 0.0f;
  CHECK(muon_step(&g, 1, 0, &bad, w, 1 << 20, nullptr) == MUON_ERR_INVALID_ARG);
  muon_group_t z = g;
  z.rows = 0;
  CHECK(muon_step(&z, 1, 0, &hp, w, 1 << 20, nullptr) == MUON_ERR_INVALID_ARG);
  CHECK(muon_step_workspace_size(&z, 1) == 0);
  z = g;
  z.batch_stride = 63;
  CHECK(muon_step(&z, 1, 0, &hp, w, 1 << 20, nullptr) == MUON_ERR_INVALID_ARG);
  z = g;
  z.reserved = 1;
  CHECK(muon_step(&z, 1, 0, &hp, w, 1 << 20, nullptr) == MUON_ERR_INVALID_ARG);
  z = g;
  z.rows = 1 << 21;
  CHECK(muon_step_workspace_size(&z, 1) == 0);
  z = g;
  z.param = nullptr;
  CHECK(muon_step(&z, 1, 0, &hp, w, 1 << 20, nullptr) == MUON_ERR_INVALID_ARG);
  CHECK(muon_step(&g, 1, 0, &hp, nullptr, 1 << 20, nullptr) == MUON_ERR_WORKSPACE);
  CHECK(muon_step(&g, 1, 0, &hp, static_cast<char*>(w) + 16, 1 << 19, nullptr) == MUON_ERR_WORKSPACE);
  muon_ws_layout_t lay;
  CHECK(muon_step_workspace_layout(&g, 1, 1, 5, &lay) == MUON_ERR_INVALID_ARG);
  CHECK(muon_step_workspace_layout(&g, 1, 0, 5, nullptr) == MUON_ERR_INVALID_ARG);
  uint16_t* o = static_cast<uint16_t*>(fake(256));
  CHECK(ns_orthogonalize(nullptr, 0, o, 1, 8, 8, 64, 5, 1, 1, 1, 0, w, 1 << 20, nullptr) == MUON_ERR_INVALID_ARG);
  CHECK(ns_orthogonalize(g.grad, 0, o, 1, 8, 8, 64, 65, 1, 1, 1, 0, w, 1 << 20, nullptr) == MUON_ERR_INVALID_ARG);
  CHECK(ns_orthogonalize(g.grad, 0, o, 1, 8, 8, 64, 5, 1, 1, 1, -1.0f, w, 1 << 20, nullptr) == MUON_ERR_INVALID_ARG);
  CHECK(ns_orthogonalize(g.grad, 0, o, 1, 8, 8, 64, 5, 1, 1, 1, 0, w, 8, nullptr) == MUON_ERR_WORKSPACE);
  // QK-Clip
  const uint16_t* q = static_cast<const uint16_t*>(fake(1 << 20));
  float* s = static_cast<float*>(fake(1024));
  CHECK(qkclip_rowmax(q, q, 1, 16, 2, 96, 0.1f, 1, s, w, 1 << 20, nullptr) == MUON_ERR_UNSUPPORTED);
  CHECK(qkclip_rowmax(q, q, 1, 16, 2, 64, 0.0f, 1, s, w, 1 << 20, nullptr) == MUON_ERR_INVALID_ARG);
  CHECK(qkclip_rowmax(q, q, 0, 16, 2, 64, 0.1f, 1, s, w, 1 << 20, nullptr) == MUON_ERR_INVALID_ARG);
  CHECK(qkclip_rowmax(q, q, 1, 16, 2, 64, 0.1f, 1, s, w, 0, nullptr) == MUON_ERR_WORKSPACE);
  CHECK(qkclip_rowmax(reinterpret_cast<const uint16_t*>(reinterpret_cast<uintptr_t>(q) + 2), q, 1, 16, 2, 64, 0.1f,
                      1, s, w, 1 << 20, nullptr) == MUON_ERR_INVALID_ARG);
  void* W = fake(1 << 20);
  CHECK(qkclip_rescale(W, W, 1, 2, 64, 8, s, 0.0f, 0.5f, nullptr, nullptr) == MUON_ERR_INVALID_ARG);
  CHECK(qkclip_rescale(W, W, 1, 2, 64, 8, s, 100.0f, 1.5f, nullptr, nullptr) == MUON_ERR_INVALID_ARG);
  CHECK(qkclip_rescale(W, W, 5, 2, 64, 8, s, 100.0f, 0.5f, nullptr, nullptr) == MUON_ERR_INVALID_ARG);
  CHECK(qkclip_rescale(nullptr, W, 1, 2, 64, 8, s, 100.0f, 0.5f, nullptr, nullptr) == MUON_ERR_INVALID_ARG);
  qkclip_slice_t sl[QKCLIP_MAX_SLICES + 1];
  for (auto& x : sl) x = qkclip_slice_t{W, 64, 64, 8, 0.5f};
  CHECK(qkclip_rescale_slices(sl, QKCLIP_MAX_SLICES + 1, 1, 2, s, 100.0f, nullptr, nullptr) == MUON_ERR_INVALID_ARG);
  sl[0].head_pitch = 32;
  CHECK(qkclip_rescale_slices(sl, 1, 1, 2, s, 100.0f, nullptr, nullptr) == MUON_ERR_INVALID_ARG);
  CHECK(qkclip_rescale_mla(W, W, W, 1, 2, 0, 64, 8, 8, s, 100.0f, nullptr, nullptr) == MUON_ERR_INVALID_ARG);
  CHECK(attn_fwd(q, q, q, 1, 16, 2, 64, 0.1f, 1, o, nullptr, s, w, 1 << 20, nullptr) == MUON_ERR_UNSUPPORTED);
  // AdamW
  adamw_hparams_t ah{1e-3f, 0.9f, 0.95f, 1e-8f, 0.1f, 1};
  adamw_tensor_t t{W, W, s, s, 16};
  adamw_hparams_t abad = ah;
  abad.step = 0;
  CHECK(adamw_step(&t, 1, 1, &abad, nullptr) == MUON_ERR_INVALID_ARG);
  abad = ah;
  abad.beta1 = 1.0f;
  CHECK(adamw_step(&t, 1, 1, &abad, nullptr) == MUON_ERR_INVALID_ARG);
  adamw_tensor_t tn = t;
  tn.exp_avg = nullptr;
  CHECK(adamw_step(&tn, 1, 1, &ah, nullptr) == MUON_ERR_INVALID_ARG);
  // Dion
  float* qd = static_cast<float*>(fake(1 << 20));
  CHECK(dion_step(W, 1, W, qd, qd, 1, 64, 64, 12, 4096, 0.02f, 0.95f, w, 1 << 20, nullptr) == MUON_ERR_UNSUPPORTED);
  CHECK(dion_step(W, 1, W, qd, qd, 1, 64, 64, 136, 4096, 0.02f, 0.95f, w, 1 << 20, nullptr) == MUON_ERR_UNSUPPORTED);
  CHECK(dion_step(W, 1, W, qd, qd, 1, 64, 64, 16, 4096, 0.02f, 0.95f, w, 8, nullptr) == MUON_ERR_WORKSPACE);
  CHECK(dion_step(nullptr, 1, W, qd, qd, 1, 64, 64, 16, 4096, 0.02f, 0.95f, w, 1 << 20, nullptr) == MUON_ERR_INVALID_ARG);
  // probe
  CHECK(muon_mfma_probe(0, 1, MUON_PROBE_RANDOM, s, nullptr) == MUON_ERR_INVALID_ARG);
  CHECK(muon_mfma_probe(1, 1, MUON_PROBE_RANDOM, nullptr, nullptr) == MUON_ERR_INVALID_ARG);
  CHECK(muon_mfma_probe(1, 1, 2, s, nullptr) == MUON_ERR_INVALID_ARG);
  CHECK(muon_mfma_probe(1, (1 << 24) + 1, MUON_PROBE_SMOOTH, s, nullptr) == MUON_ERR_INVALID_ARG);
  {
    void* a = fake(4096);
    void* b = fake(4096);
    CHECK(muon_hbm_probe(a, 4096, b, 4096, 2, 2, 1, nullptr) == -MUON_ERR_INVALID_ARG);
    CHECK(muon_hbm_probe(a, 4096, b, 4096, 1, 1, 2, nullptr) == -MUON_ERR_INVALID_ARG);
    CHECK(muon_hbm_probe(nullptr, 4096, b, 4096, 1, 1, 1, nullptr) == -MUON_ERR_INVALID_ARG);
    CHECK(muon_hbm_probe(a, 4096, b, 8, 3, 4, 4, nullptr) == -MUON_ERR_INVALID_ARG);   // no whole unit
    CHECK(muon_hbm_probe(static_cast<char*>(a) + 8, 4000, b, 4096, 1, 1, 1, nullptr) == -MUON_ERR_INVALID_ARG);
  }
  for (int k = 0; k < 5; ++k) CHECK(muon_status_string(k) && strlen(muon_status_string(k)) > 0);
  CHECK(stub_launches() == 0);
}

static void qkclip_and_friends() {
  stub_reset("qkclip / attention / adamw / dion");
  const int B = 2, T = 300, H = 3;
  for (int d : {64, 128, 256}) {
    const uint16_t* q = static_cast<const uint16_t*>(fake(uint64_t(B) * T * H * d * 2));
    const uint16_t* k = static_cast<const uint16_t*>(fake(uint64_t(B) * T * H * d * 2));
    float* s = static_cast<float*>(fake(H * 4));
    const size_t ws = qkclip_rowmax_workspace_size(B, T, H);
    void* w = fake(ws);
    CHECK(qkclip_rowmax(q, k, B, T, H, d, 0.125f, 1, s, w, ws, nullptr) == MUON_OK);
  }
  {
    // the no-allocation variant: within its 262144 partials, and one past
    const uint16_t* q = static_cast<const uint16_t*>(fake(uint64_t(4) * 4096 * 64 * 128 * 2));
    float* s = static_cast<float*>(fake(64 * 4));
    CHECK(qkclip_rowmax_noalloc_max_partials() == 262144);
    const long before = stub_launches();
    CHECK(qkclip_rowmax_noalloc(q, q, 4, 4096, 64, 128, 0.088f, 1, s, nullptr) == MUON_OK);
    CHECK(stub_launches() == before + 2);
    CHECK(qkclip_rowmax_noalloc(q, q, 1, 256 * 4097, 64, 64, 0.125f, 1, s, nullptr) == MUON_ERR_WORKSPACE);
    // head dim 128 runs 512-query blocks: twice the sequence fits the same scratch
    CHECK(qkclip_rowmax_noalloc(q, q, 1, 512 * 4097, 64, 128, 0.088f, 1, s, nullptr) == MUON_ERR_WORKSPACE);
    CHECK(qkclip_rowmax_noalloc(q, q, 1, 16, 2, 96, 0.1f, 1, s, nullptr) == MUON_ERR_UNSUPPORTED);
    CHECK(qkclip_rowmax_noalloc(nullptr, q, 1, 16, 2, 64, 0.1f, 1, s, nullptr) == MUON_ERR_INVALID_ARG);
    CHECK(stub_launches() == before + 2);
    const uint16_t* qb = static_cast<const uint16_t*>(fake(uint64_t(512) * 4096 * 64 * 128 * 2));
    CHECK(qkclip_rowmax_noalloc(qb, qb, 1, 512 * 4096, 64, 128, 0.088f, 1, s, nullptr) == MUON_OK);
    CHECK(stub_launches() == before + 4);
  }
  {
    const uint64_t n = uint64_t(B) * T * H * 128;
    const uint16_t* q = static_cast<const uint16_t*>(fake(n * 2));
    uint16_t* o = static_cast<uint16_t*>(fake(n * 2));
    float* lse = static_cast<float*>(fake(uint64_t(B) * H * T * 4));
    float* s = static_cast<float*>(fake(H * 4));
    const size_t ws = attn_fwd_workspace_size(B, T, H);
    void* w = fake(ws);
    CHECK(attn_fwd(q, q, q, B, T, H, 128, 0.088f, 1, o, lse, s, w, ws, nullptr) == MUON_OK);
  }
  {
    const int Hh = 5, dh = 64, dm = 200;
    void* Wq = fake(uint64_t(Hh) * dh * dm * 2);
    void* Wk = fake(uint64_t(Hh) * dh * dm * 2);
    float* s = static_cast<float*>(fake(Hh * 4));
    int32_t* f = static_cast<int32_t*>(fake(Hh * 4));
    CHECK(qkclip_rescale(Wq, Wk, MUON_DTYPE_BF16, Hh, dh, dm, s, 100.0f, 0.5f, f, nullptr) == MUON_OK);
    void* c = fake(uint64_t(Hh) * 96 * 300 * 4);
    void* kc = fake(uint64_t(Hh) * 96 * 100 * 4);
    void* r = fake(uint64_t(Hh) * 32 * 300 * 4);
    CHECK(qkclip_rescale_mla(c, kc, r, MUON_DTYPE_F32, Hh, 96, 32, 300, 100, s, 100.0f, f, nullptr) == MUON_OK);
    // a fused per-head [content | rotary] layout
    void* fused = fake(uint64_t(Hh) * 160 * 48 * 2);
    qkclip_slice_t sl[2] = {{fused, 160, 128, 48, 0.5f},
                            {static_cast<char*>(fused) + 128 * 48 * 2, 160, 32, 48, 1.0f}};
    CHECK(qkclip_rescale_slices(sl, 2, MUON_DTYPE_BF16, Hh, s, 100.0f, f, nullptr) == MUON_OK);
  }
  {
    std::vector<adamw_tensor_t> ts;
    for (int i = 0; i < 100; ++i) {
      const int64_t n = (i % 7 == 0) ? 0 : 1 + 977 * i;
      ts.push_back({fake(n * 2 + 2), fake(n * 2 + 2), static_cast<float*>(fake(n * 4 + 4)),
                    static_cast<float*>(fake(n * 4 + 4)), n});
    }
    adamw_hparams_t ah{1e-3f, 0.9f, 0.95f, 1e-8f, 0.1f, 3};
    CHECK(adamw_step(ts.data(), int(ts.size()), MUON_DTYPE_BF16, &ah, nullptr) == MUON_OK);
  }
  for (int rank : {8, 16, 128}) {
    const int b = 3, m = 256, n = 136;
    const uint64_t e = uint64_t(b) * m * n;
    void* W = fake(e * 2);
    void* G = fake(e * 2);
    float* M = static_cast<float*>(fake(e * 4));
    float* Q = static_cast<float*>(fake(uint64_t(b) * n * rank * 4));
    const size_t ws = dion_workspace_size(b, m, n, rank);
    void* w = fake(ws);
    CHECK(dion_step(W, MUON_DTYPE_BF16, G, M, Q, b, m, n, rank, int64_t(m) * n, 0.02f, 0.95f, w, ws, nullptr) ==
          MUON_OK);
  }
  {
    float* sink = static_cast<float*>(fake(512 * 4));
    CHECK(muon_mfma_probe(512, 10, MUON_PROBE_RANDOM, sink, nullptr) == MUON_OK);
    CHECK(muon_mfma_probe(512, 10, MUON_PROBE_SMOOTH, sink, nullptr) == MUON_OK);
    // the HBM probe: units from the smaller stream, every chunk inside both
    void* src = fake(3 * 16 * 1000 + 40);
    void* dst = fake(4 * 16 * 1001);
    CHECK(muon_hbm_probe(src, 3 * 16 * 1000 + 40, dst, 4 * 16 * 1001, 3, 4, 4, nullptr) == 1000 * 16 * 7);
    CHECK(muon_hbm_probe(src, 32 * 1000, dst, 16 * 999, 2, 1, 1, nullptr) == 999 * 16 * 3);
    CHECK(muon_hbm_probe(src, 16 * 7, dst, 16 * 7, 1, 1, 4, nullptr) == 7 * 16 * 2);
  }
  // the profiler: on, one call, collect, off
  CHECK(muon_profile_enable(1) == MUON_OK);
  {
    float* sink = static_cast<float*>(fake(4));
    CHECK(muon_mfma_probe(1, 1, MUON_PROBE_RANDOM, sink, nullptr) == MUON_OK);
  }
  double ms[64];
  int64_t cnt[64];
  const int kinds = muon_profile_collect(ms, cnt, 64);
  CHECK(kinds > 0 && kinds <= 64);
  for (int k = 0; k < kinds; ++k) CHECK(muon_kernel_kind_name(k) != nullptr);
  CHECK(strcmp(muon_kernel_kind_name(-1), "unknown") == 0);
  CHECK(muon_profile_enable(0) == MUON_OK);
}

int main() {
  invalid_arguments();
  qkclip_and_friends();
  // the workloads' shape classes, each in one call as the benchmark runs them
  run_step("workload 1", {{1, 256, 128, 0}}, MUON_DTYPE_F32, 5);
  run_step("workload 2", {{4, 2048, 2048, 0}, {2, 8192, 2048, 0}, {1, 2048, 8192, 0}}, MUON_DTYPE_BF16, 5);
  run_step("workload 3", {{48, 4096, 4096, 0}, {48, 1024, 4096, 0}, {48, 14336, 4096, 0}, {24, 4096, 14336, 0}},
           MUON_DTYPE_BF16, 5);
  run_step("workload 4", {{128, 2048, 7168, 0}, {64, 7168, 2048, 0}}, MUON_DTYPE_BF16, 5);
  run_step("workload 5", {{3, 8192, 7168, 0}, {1, 7168, 8192, 0}}, MUON_DTYPE_BF16, 5);
  // ragged, thin, small, tall and mixed groups; 1..6 steps; the cubic
  const std::vector<Shape> mixed = {{2, 1, 37, 0},   {2, 37, 1, 3},    {2, 64, 64, 0},    {2, 130, 70, 1},
                                    {2, 70, 130, 0}, {2, 200, 200, 0}, {2, 256, 100, 0},  {2, 100, 256, 9},
                                    {2, 300, 17, 0}, {2, 17, 300, 0},  {2, 520, 64, 0},   {2, 64, 520, 0},
                                    {2, 96, 160, 0}, {2, 512, 513, 0}, {2, 513, 512, 5},  {2, 33, 777, 0}};
  for (int steps : {1, 2, 5, 6}) {
    run_step("sixteen groups bf16", mixed, MUON_DTYPE_BF16, steps);
    run_step("sixteen groups f32", mixed, MUON_DTYPE_F32, steps);
  }
  run_step("cubic", mixed, MUON_DTYPE_BF16, 3, 0.0f);
  run_step("thin, long", {{3, 1, 100000, 0}, {2, 96, 70000, 0}, {1, 70000, 40, 0}, {2, 97, 1000, 0}},
           MUON_DTYPE_BF16, 5);
  std::mt19937 rng(7);
  for (int k = 0; k < 300; ++k) {
    std::vector<Shape> sh;
    const int ng = 1 + int(rng() % MUON_MAX_GROUPS);
    for (int g = 0; g < ng; ++g) {
      const int kind = int(rng() % 4);
      const int lim = kind == 0 ? 140 : kind == 1 ? 600 : kind == 2 ? 2100 : 5000;
      int r = 1 + int(rng() % lim), c = 1 + int(rng() % lim);
      if (kind == 3) r = 1 + int(rng() % 120);
      if (rng() % 2) std::swap(r, c);
      sh.push_back({1 + int(rng() % 3), r, c, int64_t(rng() % 3) * 8});
    }
    run_step("random groups", sh, (k % 2) ? MUON_DTYPE_BF16 : MUON_DTYPE_F32, 1 + int(rng() % 6));
  }
  for (auto [r, c] : std::vector<std::pair<int, int>>{{1, 37}, {250, 1}, {33, 777}, {777, 33}, {512, 2048},
                                                      {7168, 8192}, {96, 1000}, {1, 5000}, {4096, 256}}) {
    run_ns("ns_orthogonalize", 2, r, c, MUON_DTYPE_F32, 5);
    run_ns("ns_orthogonalize", 1, r, c, MUON_DTYPE_BF16, 2);
  }
  if (g_fail) {
    printf("FAIL: %d checks failed\n", g_fail);
    return 1;
  }
  printf("host checks passed\n");
  return 0;
}
