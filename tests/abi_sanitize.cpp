// Host-side sanitizer run of the C ABI (include/af.h): plan lifecycle,
// workspace sizing and every argument check that precedes device work, with
// fake device pointers that are never dereferenced.  Built with
// -fsanitize=address,undefined (host code only) by tests/test_abi_sanitize.py;
// a failed check prints its line and the program exits non-zero.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "af.h"

static int failures = 0;
#define CHECK(cond)                                                     \
  do {                                                                  \
    if (!(cond)) {                                                      \
      std::printf("FAILED line %d: %s (%s)\n", __LINE__, #cond, af_last_error()); \
      ++failures;                                                       \
    }                                                                   \
  } while (0)

// 16-byte aligned host storage standing in for device buffers
alignas(256) static float fake[64];

struct Weights {
  std::vector<const void*> mats;
  std::vector<const float*> vecs;
  af_block_weights w{};
};

static void fill(Weights& W, int n_layers) {
  const float* f = fake;
  W.vecs.assign(8 * n_layers, f);
  W.mats.assign(4 * n_layers, (const void*)f);
  af_block_weights& w = W.w;
  w.w_in = w.b_in = w.pos = w.ln_f_g = w.ln_f_b = w.w_head = w.b_head = f;
  const float* const* v = W.vecs.data();
  const void* const* m = W.mats.data();
  w.ln1_g = v;
  w.ln1_b = v + n_layers;
  w.b_qkv = v + 2 * n_layers;
  w.b_o = v + 3 * n_layers;
  w.ln2_g = v + 4 * n_layers;
  w.ln2_b = v + 5 * n_layers;
  w.b_1 = v + 6 * n_layers;
  w.b_2 = v + 7 * n_layers;
  w.w_qkv = m;
  w.w_o = m + n_layers;
  w.w_1 = m + 2 * n_layers;
  w.w_2 = m + 3 * n_layers;
}

static af_plan* make(int C, int d, int H, int layers, int max_len, af_dtype dt, int T,
                     af_status* st) {
  static std::vector<Weights> keep;
  keep.emplace_back();
  fill(keep.back(), layers);
  std::vector<af_block_weights> ws(T, keep.back().w);
  af_block_cfg cfg{C, d, H, layers, max_len, dt};
  af_plan* p = nullptr;
  *st = af_plan_create(&cfg, T, ws.data(), &p);
  return p;
}

int main() {
  CHECK(af_abi_version() == AF_ABI_VERSION);
  CHECK(std::strcmp(af_status_str(AF_OK), "AF_OK") == 0);
  CHECK(std::strcmp(af_status_str(AF_ERR_NONFINITE), "AF_ERR_NONFINITE") == 0);

  af_status st;
  // shapes outside the documented ranges
  CHECK(make(0, 64, 2, 1, 64, AF_F32, 1, &st) == nullptr && st == AF_ERR_ARG);
  CHECK(make(16, 96, 2, 1, 64, AF_F32, 1, &st) == nullptr && st == AF_ERR_UNSUPPORTED);
  CHECK(make(16, 64, 4, 1, 64, AF_F32, 1, &st) == nullptr && st == AF_ERR_UNSUPPORTED);
  CHECK(make(16, 128, 2, 1, 64, AF_BF16, 1, &st) == nullptr && st == AF_ERR_UNSUPPORTED);
  CHECK(make(16, 64, 2, 1, 64, (af_dtype)7, 1, &st) == nullptr && st == AF_ERR_ARG);
  CHECK(make(16, 64, 2, 1, 64, AF_F32, 0, &st) == nullptr && st == AF_ERR_ARG);
  {
    af_block_cfg cfg{16, 64, 2, 1, 64, AF_F32};
    af_plan* p = nullptr;
    CHECK(af_plan_create(&cfg, 1, nullptr, &p) == AF_ERR_ARG && p == nullptr);
    CHECK(af_plan_create(nullptr, 1, nullptr, &p) == AF_ERR_ARG);
  }

  // a valid fp32 plan and its validation paths
  af_plan* p = make(16, 64, 2, 1, 64, AF_F32, 1, &st);
  CHECK(st == AF_OK && p != nullptr);
  const size_t big = af_workspace_bytes(p, 1, 64);
  CHECK(big > 0 && af_workspace_bytes(p, 1, 16) < big && af_workspace_bytes(p, 0, 16) == 0);
  CHECK(af_cache_bytes(p, 1) == (size_t)1 * 2 * 2 * 64 * 32 * 4);
  float* buf = fake;
  float* other = fake + 16;
  void* ws = (void*)(uintptr_t)(1u << 20);
  CHECK(af_forward(p, nullptr, other, buf, 1, 64, 1, 0, ws, big, nullptr) == AF_ERR_ARG);
  CHECK(af_forward(p, buf, other, buf, 1, 65, 1, 0, ws, big, nullptr) == AF_ERR_ARG);
  CHECK(af_forward(p, buf, other, buf, 1, 64, 1, 0, ws, 16, nullptr) == AF_ERR_WORKSPACE);
  CHECK(af_forward(p, buf, other, buf, 1, 64, 1, 0, (char*)ws + 4, big, nullptr) == AF_ERR_ARG);
  CHECK(af_forward(p, buf, other, buf, 3, 64, 2, 0, ws, big, nullptr) == AF_ERR_ARG);
  CHECK(af_forward(p, buf, other, buf, 1, 64, 0, 0, ws, big, nullptr) == AF_ERR_ARG);
  CHECK(af_forward(p, buf, other, buf, 1, 64, 1, 8, ws, big, nullptr) == AF_ERR_ARG);
  CHECK(af_forward(p, buf, buf, buf, 1, 64, 1, 0, ws, big, nullptr) == AF_ERR_ARG);
  CHECK(af_forward(p, fake + 1, other, buf, 1, 64, 1, 0, ws, big, nullptr) == AF_ERR_ARG);

  int32_t iters[16];
  auto inv = [&](const float* z, int N, int L, int B, float tau, int init, const float* x_init,
                 int F, int P, const float* x_last, float* x, size_t wsb) {
    return af_inverse_jacobi(p, z, N, L, B, tau, 0, (af_init)init, x_init, F, P, x_last, x,
                             iters, ws, wsb, nullptr);
  };
  CHECK(inv(buf, 1, 64, 16, NAN, 0, nullptr, 0, 0, nullptr, other, big) == AF_ERR_ARG);
  CHECK(inv(buf, 1, 64, 0, 1e-3f, 0, nullptr, 0, 0, nullptr, other, big) == AF_ERR_ARG);
  CHECK(inv(buf, 1, 64, 16, 1e-3f, 9, nullptr, 0, 0, nullptr, other, big) == AF_ERR_ARG);
  CHECK(inv(buf, 1, 64, 16, 1e-3f, 1, nullptr, 0, 0, nullptr, other, big) == AF_ERR_ARG);
  CHECK(inv(buf, 1, 64, 16, 1e-3f, 2, nullptr, 8, 0, nullptr, other, big) == AF_ERR_ARG);
  CHECK(inv(buf, 1, 64, 16, 1e-3f, 0, nullptr, 0, 1, nullptr, other, big) == AF_ERR_ARG);
  CHECK(inv(buf, 1, 64, 16, 1e-3f, 0, nullptr, 0, 10, buf, other, big) == AF_ERR_ARG);
  CHECK(inv(buf, 1, 64, 16, 1e-3f, 0, nullptr, 0, 0, nullptr, buf, big) == AF_ERR_ARG);
  CHECK(inv(buf, 1, 64, 16, 1e-3f, 0, nullptr, 0, 0, nullptr, other, 8) == AF_ERR_WORKSPACE);
  CHECK(inv(buf, 1, 64, 16, 1e-3f, 0, nullptr, 0, 0, nullptr, fake + 33, big) == AF_ERR_ARG);
  CHECK(af_inverse_jacobi(p, buf, 1, 64, 16, 1e-3f, 0, AF_INIT_ZERO, nullptr, 0, 0, nullptr,
                          other, nullptr, ws, big, nullptr) == AF_ERR_ARG);
  CHECK(af_prefill(p, nullptr, 1, 8, ws, big, nullptr) == AF_ERR_ARG);
  CHECK(af_prefill(p, buf, 1, 65, ws, big, nullptr) == AF_ERR_ARG);
  CHECK(af_refresh_kv(p, nullptr, 1, 8, 0, nullptr, ws, big, nullptr) == AF_ERR_ARG);
  CHECK(af_refresh_kv(p, buf, 1, 8, 8, nullptr, ws, big, nullptr) == AF_ERR_ARG);
  CHECK(af_refresh_kv(p, buf, 1, 60, 8, buf, ws, big, nullptr) == AF_ERR_ARG);
  CHECK(af_refresh_kv(p, buf, 1, 8, 0, nullptr, ws, 16, nullptr) == AF_ERR_WORKSPACE);

  // controls and diagnostics
  CHECK(af_profile_enable(p, "nope") == AF_ERR_ARG);
  CHECK(af_profile_enable(p, nullptr) == AF_ERR_ARG);
  CHECK(af_profile_disable(p) == AF_OK);
  int n = -1;
  double ms = -1, work = -1;
  CHECK(af_profile_read(p, &n, &ms, &work) == AF_OK && n == 0 && ms == 0.0 && work == 0.0);
  CHECK(af_profile_read(p, nullptr, &ms, nullptr) == AF_ERR_ARG);
  long long c = -1, r = -1;
  CHECK(af_plan_graph_stats(p, &c, &r) == AF_OK && c == 0 && r == 0);
  CHECK(af_plan_set_graphs(p, 1) == AF_OK && af_plan_set_graphs(p, 0) == AF_OK);
  CHECK(af_plan_set_fused_refresh(p, 1) == AF_OK && af_plan_set_row_split(p, 0) == AF_OK);
  CHECK(af_plan_set_graphs(nullptr, 1) == AF_ERR_ARG);
  float res[4];
  CHECK(af_plan_last_residual(p, 2, res) == AF_ERR_ARG);
  CHECK(af_plan_last_residual(p, 2, nullptr) == AF_ERR_ARG);
  af_plan_destroy(p);
  af_plan_destroy(nullptr);

  // a stack: only zero init and no prefix
  af_plan* s = make(16, 64, 2, 1, 64, AF_F32, 2, &st);
  CHECK(st == AF_OK && s != nullptr);
  const size_t sb = af_workspace_bytes(s, 1, 16);
  CHECK(af_inverse_jacobi(s, buf, 1, 64, 16, 1e-3f, 0, AF_INIT_PREV_FRAME, nullptr, 16, 0,
                          nullptr, other, iters, ws, sb, nullptr) == AF_ERR_UNSUPPORTED);
  CHECK(af_prefill(s, buf, 1, 8, ws, sb, nullptr) == AF_ERR_UNSUPPORTED);
  af_plan_destroy(s);

  // a one-layer bf16 plan at the benchmark width: workspace sizes with the
  // row split (from two layers the scratch of a refresh beside the next
  // block covers the half's at every size)
  af_plan* b = make(48, 1024, 16, 1, 4680, AF_BF16, 1, &st);
  CHECK(st == AF_OK && b != nullptr);
  CHECK(af_workspace_bytes(b, 1, 1024) - af_workspace_bytes(b, 1, 1023) > 20000000u);
  CHECK(af_workspace_bytes(b, 1, 4097) < af_workspace_bytes(b, 1, 4096));
  CHECK(af_cache_bytes(b, 1) == (size_t)1 * 2 * 16 * 4736 * 64 * 2);
  CHECK(af_plan_set_overlap_refresh(b, 0) == AF_OK);
  CHECK(af_plan_set_overlap_refresh(nullptr, 1) == AF_ERR_ARG);
  {
    static int calls = 0;
    af_block_done_fn cb = [](void* user, int, int) { ++*(int*)user; };
    CHECK(af_plan_set_block_done(b, cb, &calls) == AF_OK);
    CHECK(af_plan_set_block_done(b, nullptr, nullptr) == AF_OK);
    CHECK(af_plan_set_block_done(nullptr, cb, &calls) == AF_ERR_ARG);
    CHECK(calls == 0);
  }
  af_plan_destroy(b);
  af_plan* b8 = make(48, 1024, 16, 8, 4680, AF_BF16, 1, &st);
  CHECK(st == AF_OK && b8 != nullptr);
  CHECK(af_workspace_bytes(b8, 1, 4097) > af_workspace_bytes(b8, 1, 4096));
  CHECK(af_cache_bytes(b8, 1) == (size_t)8 * 2 * 16 * 4736 * 64 * 2);
  af_plan_destroy(b8);

  // kernel-level entry points: argument checks
  CHECK(afk_affine_partials_bytes(0, 4, 4) == 0);
  CHECK(afk_affine(2, buf, buf, other, 1, 4, 4, buf, buf, 1024, 0, nullptr) == AF_ERR_ARG);
  CHECK(afk_affine(0, buf, buf, buf, 1, 4, 4, buf, buf, 1024, 0, nullptr) == AF_ERR_ARG);
  CHECK(afk_affine(0, buf, buf, other, 1, 4, 4, buf, buf, 0, 0, nullptr) == AF_ERR_WORKSPACE);
  CHECK(afk_gemm_bf16(buf, buf, nullptr, other, 4, 60, 64, nullptr) == AF_ERR_ARG);
  CHECK(afk_stream_copy(buf, other, 0, nullptr) == AF_OK);
  CHECK(afk_attention_workspace_bytes(1, 100, 4, 64, 300) > 0);
  CHECK(afk_attention_workspace_bytes(1, 100, 4, 48, 300) == 0);
  CHECK(afk_attention(buf, buf, buf, other, 1, 100, 4, 48, 448, 300, buf, 1 << 20, nullptr) == AF_ERR_UNSUPPORTED);
  CHECK(afk_attention(buf, buf, buf, other, 1, 100, 4, 64, 400, 300, buf, 1 << 20, nullptr) == AF_ERR_ARG);
  CHECK(afk_attention(buf, buf, buf, other, 1, 100, 4, 64, 448, 400, buf, 1 << 20, nullptr) == AF_ERR_ARG);
  CHECK(afk_attention(buf, buf, buf, other, 1, 100, 4, 64, 448, 300, buf, 16, nullptr) == AF_ERR_WORKSPACE);
  CHECK(afk_stream_copy(nullptr, other, 16, nullptr) == AF_ERR_ARG);
  CHECK(afk_stream_copy(buf, other, 24, nullptr) == AF_ERR_ARG);
  CHECK(afk_stream_copy((char*)buf + 8, other, 16, nullptr) == AF_ERR_ARG);
  CHECK(afk_stream_copy(buf, (char*)buf + 64, 128, nullptr) == AF_ERR_ARG);

  std::printf("%s: %d failed checks\n", failures ? "FAIL" : "OK", failures);
  return failures ? 1 : 0;
}
