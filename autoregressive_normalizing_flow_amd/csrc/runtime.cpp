// Host runtime of the AF-block library: plan, workspace layout, argument
// validation, the per-pass kernel sequence and the block-wise Jacobi schedule.
//
// Method (STARFlow-V notes, papernotes.org, "STARFlow-V: End-to-End Video
// Generative Modeling with Autoregressive Normalizing Flows"):
//   关键设计 1 - affine AF block z = (x - mu(x*m)) / sigma(x*m), alternating
//                mask directions in a stack;
//   关键设计 3 - Jacobi fixed point x = mu(x*m) + sigma(x*m) z solved block by
//                block with a KV cache, warm start from the previous frame and
//                the residual stop ||dx||^2 / ||x||^2 < tau;
//   一个完整示例 - conditioning by forward-encoding observed tokens into the cache.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/af.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

// Record the failure; a failed HIP call's error is also taken out of the
// runtime's per-thread last-error state, so that it does not surface in the
// caller's next unrelated HIP call.
af_status fail(af_status s, const std::string& msg) {
  g_err = msg;
  if (s == AF_ERR_HIP) (void)hipGetLastError();
  return s;
}

#define AF_HIP(expr)                                                        \
  do {                                                                      \
    hipError_t e_ = (expr);                                                 \
    if (e_ != hipSuccess)                                                   \
      return fail(AF_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// The kernels read weights and token rows as 16-byte vectors.
bool misaligned(const void* q) { return q && ((uintptr_t)q & 15) != 0; }
template <class... P>
bool any_misaligned(const P*... q) {
  return (misaligned(q) || ...);
}

struct LayerW {
  const float *ln1_g, *ln1_b, *b_qkv, *b_o, *ln2_g, *ln2_b, *b_1, *b_2;
  const void *w_qkv, *w_o, *w_1, *w_2;
};

struct BlockW {
  const float *w_in, *b_in, *pos, *ln_f_g, *ln_f_b, *w_head, *b_head;
  std::vector<LayerW> layers;
};

// Byte offsets of the workspace regions for (batch, rows).
struct WsLayout {
  size_t cache_layer;  // bytes of one layer's K (or V) cache
  size_t cache, h, a, q, att, u, hf, head, partials, res, counter, tickets, slab, attn_part, xtmp;
  // lo halves of the split (higher-precision) forward on the bf16 path
  size_t cache_lo, a_lo, q_lo, att_lo, u_lo, total;
};

enum KClass { K_EMBED, K_LN, K_QKV, K_O, K_MLP1, K_MLP2, K_HEAD, K_ATTN, K_AFFINE, K_LOOP,
              K_NCLASS };
const char* kclass_names[K_NCLASS] = {"embed", "layernorm", "gemm_qkv", "gemm_o",
                                      "gemm_mlp1", "gemm_mlp2", "gemm_head",
                                      "attention", "affine", "device_loop"};

// Key of a captured Jacobi update: every host value its launches bake in.
struct GraphKey {
  const void* block;
  const float *src, *x_last, *z;
  float* res_host;
  const char* ws;
  int device, N, L, s, R, P, dir, rows;
  unsigned tag;
  bool operator==(const GraphKey& o) const { return std::memcmp(this, &o, sizeof(*this)) == 0; }
};

static_assert(sizeof(GraphKey) == 6 * sizeof(void*) + 10 * sizeof(int), "GraphKey has padding");

struct GraphEntry {
  GraphKey key;
  hipGraphExec_t exec = nullptr;
  uint64_t used = 0;
};

constexpr int kGraphCacheCap = 128;
constexpr int kProfileLaunches = 16384;   // launches recorded per af_profile_enable

}  // namespace

struct af_plan {
  af_block_cfg cfg;
  int T;
  int dh, dmlp, Lcap;
  bool bf;
  size_t esz;  // bytes per element of the per-layer operand type
  std::vector<BlockW> blocks;
  float* host_res = nullptr;  // pinned [res_cap][2], then one sequence word
  int res_cap = 0;
  float* host_res_dev = nullptr;  // the same memory as the device sees it
  // profiling
  int prof_class = -1;
  std::vector<hipEvent_t> ev;  // pairs
  int prof_n = 0;
  double prof_work = 0.0;      // algorithmic work of the recorded launches
  // a block's cache refresh merged into the next block's first update
  bool fuse_refresh = false;
  // HIP graphs of one Jacobi update, replayed once per iteration
  bool graphs = false;
  hipStream_t cap_stream = nullptr;
  std::vector<GraphEntry> gcache;
  uint64_t gclock = 0;
  long long g_captures = 0, g_replays = 0;
  // row split of a Jacobi update over two streams (see af_inverse_jacobi)
  bool row_split = false;
  // a block's cache refresh on the second stream beside the next block's
  // first update (see af_inverse_jacobi; on by default)
  bool overlap_refresh = true;
  // called on the calling thread once a Jacobi block's tokens are final on
  // the stream (af_plan_set_block_done)
  af_block_done_fn done_fn = nullptr;
  void* done_user = nullptr;
  hipStream_t split_stream = nullptr;
  std::vector<hipEvent_t> split_ev;   // eq[l], ea[l], then affine, fork, join
  // residual pairs of the last update of the last inverse call (halves added)
  std::vector<float> last_res;
  // the Jacobi loop on the device for small fp32 blocks (on by default);
  // pinned block counts and non-finite words of its launches
  bool device_loop = true;
  int loop_lds_max = 0;   // LDS bytes per workgroup for the device loop (0: not queried yet)
  int* loop_host = nullptr;
  int* loop_host_dev = nullptr;
  size_t loop_cap = 0;   // ints
};

namespace {

// Rows of head partial planes needed for any pass of at most M rows:
// max over m <= M of splits(m) * m, for either head kernel (both use one
// split above 16384 rows).
size_t head_plane_rows(size_t M, int n_out, int d) {
  size_t best = M;
  const size_t top = std::min<size_t>(M, 16384);
  for (size_t m = 16; m < top + 16; m += 16) {
    const size_t mm = m < top ? m : top;
    const size_t s = std::max(af::head_splits((int)mm, n_out, d), af::head_mfma_splits((int)mm, d));
    if (s * mm > best) best = s * mm;
  }
  return best;
}

WsLayout layout(const af_plan* p, int N, int rows) {
  WsLayout w{};
  const af_block_cfg& c = p->cfg;
  const size_t M = (size_t)N * rows;
  w.cache_layer = (size_t)N * c.n_heads * p->Lcap * p->dh * p->esz;
  size_t off = 0;
  w.cache = off;
  off += align256(2 * w.cache_layer * c.n_layers);
  w.h = off;        off += align256(M * c.d * 4);
  w.a = off;        off += align256(M * c.d * p->esz);
  w.q = off;        off += align256(M * c.d * p->esz);
  w.att = off;      off += align256(M * c.d * p->esz);
  w.u = off;        off += align256(M * p->dmlp * p->esz);
  w.hf = off;       off += align256(M * c.d * 4);
  w.head = off;     off += align256(head_plane_rows(M, 2 * c.C, c.d) * 2 * c.C * 4);
  w.partials = off; off += align256((size_t)N * af::affine_groups(N, rows, c.C) * 2 * 4);
  w.res = off;      off += align256((size_t)N * 2 * 4);
  // 64 counter words, then the attention merge tickets (zero between
  // launches; cleared with the counters at the start of every call)
  w.counter = off;  off += 256;
  w.tickets = off;  off += align256(p->bf ? af::attention_tickets(N, rows, c.n_heads) * 4 : 0);
  w.slab = off;
  if (p->bf) {
    const int s1 = af::gemm_resid_splits((int)M, c.d, c.d);
    const int s2 = af::gemm_resid_splits((int)M, c.d, p->dmlp);
    const int s = s1 > s2 ? s1 : s2;
    off += align256((size_t)s * M * c.d * 4);
  }
  w.attn_part = off;
  if (p->bf) {
    // key-chunk partials: at most max(1024, N*H*query tiles) units of
    // 128 x (dh + 2) floats
    const size_t units = std::max<size_t>(1024, (size_t)N * c.n_heads * ((rows + 127) / 128));
    off += align256(units * 128 * (p->dh + 2) * 4);
  }
  w.xtmp = off;
  if (p->T > 1) off += align256((size_t)N * c.max_len * c.C * 4);
  w.cache_lo = w.a_lo = w.q_lo = w.att_lo = w.u_lo = 0;
  if (p->bf) {
    w.cache_lo = off; off += align256(2 * w.cache_layer * c.n_layers);
    w.a_lo = off;     off += align256(M * c.d * 2);
    w.q_lo = off;     off += align256(M * c.d * 2);
    w.att_lo = off;   off += align256(M * c.d * 2);
    w.u_lo = off;     off += align256(M * p->dmlp * 2);
  }
  w.total = off;
  return w;
}

// Row split of a Jacobi update over two streams: rows [0, ra) of the block
// (half A) and [ra, R) (half B) run as two passes side by side, so that each
// fills the GPU where the other's launches leave it idle.  The halves'
// kernels are smaller and less efficient, which the overlap repays only when
// attention over a long prefix dominates: the split is used on the bf16 path
// for long blocks of a small batch (split_possible) with at least 8 R keys
// before the block (measured on 1560-token frames: 7% slower after 1 frame of
// prefix, even after 4, 4-13% faster from 8 frames on).  Returns ra, or 0.
constexpr int kSplitPrefixBlocks = 8;
bool split_possible(const af_plan* p, int N, int R) {
  return p->bf && R >= 1024 && (long)N * R <= 4096;
}
int split_rows_a(const af_plan* p, int N, int R, int keys_before) {
  if (!split_possible(p, N, R) || keys_before < kSplitPrefixBlocks * R) return 0;
  return (R / 2) / 128 * 128;
}

// Scratch of half B behind the whole-block layout w (the KV cache region is
// shared), for halves of at most rows / 2 + 128 rows.
WsLayout layout_b(const af_plan* p, int N, int rows, const WsLayout& w) {
  WsLayout b = layout(p, N, rows / 2 + 128);
  // the per-pass scratch runs from h up to xtmp; the stack's token buffer and
  // the higher-precision forward's lo halves are not needed by half B
  const size_t shift = w.total - b.h;
  size_t* f[] = {&b.h, &b.a, &b.q, &b.att, &b.u, &b.hf, &b.head, &b.partials, &b.res,
                 &b.counter, &b.tickets, &b.slab, &b.attn_part};
  for (size_t* x : f) *x += shift;
  b.total = b.xtmp + shift;
  b.xtmp = w.xtmp;
  b.cache_lo = b.a_lo = b.q_lo = b.att_lo = b.u_lo = 0;
  return b;
}

// Scratch of a cache refresh that runs on the second stream beside the next
// block's updates (bf16 plans): the per-pass buffers for `rows` rows placed
// after the main layout (the refresh and the row split never run in one
// call, so they share that space).  The refresh stops after the last layer's
// K/V, so it never touches the head planes, the affine partials or the
// counter words; its attention tickets are its own and are cleared with the
// call's counters.
bool refresh_overlap_possible(const af_plan* p) { return p->bf && p->cfg.n_layers > 1; }

WsLayout layout_r(const af_plan* p, int N, int rows, const WsLayout& w) {
  WsLayout r = layout(p, N, rows);
  const size_t shift = w.total - r.h;
  size_t* f[] = {&r.h, &r.a, &r.q, &r.att, &r.u, &r.hf, &r.head, &r.partials, &r.res,
                 &r.counter, &r.tickets, &r.slab, &r.attn_part};
  for (size_t* x : f) *x += shift;
  r.total = r.xtmp + shift;
  r.xtmp = w.xtmp;
  r.cache_lo = r.a_lo = r.q_lo = r.att_lo = r.u_lo = 0;
  return r;
}

// Launch helper with optional per-class event timing (direct launches only:
// nothing is captured into a graph while a class is profiled).  The bf16
// projection GEMMs are one kernel per launch call, and their events are taken
// by the kernel launch itself, so they time the kernel alone; the other
// classes are bracketed by event records on the stream, which also count the
// gaps before and after the kernels.
struct Launch {
  hipStream_t st;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  bool ext = false;
  Launch(af_plan* p, hipStream_t s, int cls, double work = 0.0) : st(s) {
    if (p->prof_class != cls || p->prof_n >= (int)p->ev.size() / 2) return;
    p->prof_work += work;
    e0 = p->ev[2 * p->prof_n];
    e1 = p->ev[2 * p->prof_n + 1];
    ++p->prof_n;
    ext = p->bf &&
          (cls == K_QKV || cls == K_O || cls == K_MLP1 || cls == K_MLP2);
    if (ext) af::set_gemm_events(e0, e1);
    else (void)hipEventRecord(e0, st);
  }
  ~Launch() {
    if (!e1) return;
    if (ext && !af::gemm_events_pending()) return;   // the kernel took them
    if (ext) {
      // no GEMM launched (an error path): leave an empty interval
      af::set_gemm_events(nullptr, nullptr);
      (void)hipEventRecord(e0, st);
    }
    (void)hipEventRecord(e1, st);
  }
};

// LAUNCHW also states the launch's algorithmic work for the profiler.
#define LAUNCHW(cls, work, call)                          \
  do {                                                    \
    Launch l_(p, st, cls, (work));                        \
    hipError_t e_ = (call);                               \
    if (e_ != hipSuccess)                                 \
      return fail(AF_ERR_HIP, std::string(#call) + ": " + hipGetErrorString(e_)); \
  } while (0)

#define LAUNCH(cls, call)                                 \
  do {                                                    \
    Launch l_(p, st, cls);                                \
    hipError_t e_ = (call);                               \
    if (e_ != hipSuccess)                                 \
      return fail(AF_ERR_HIP, std::string(#call) + ": " + hipGetErrorString(e_)); \
  } while (0)

struct Pass {
  const float* src;     // token tensor [N, L, C] read by the shift (x or iterate)
  const float* x_last;  // token before processing index 0, or NULL
  int N, L, s, R, P, dir;
  bool kv_only;         // stop after the last layer's K/V (cache refresh)
  bool precise;         // bf16 path: carry activations as bf16 pairs (hi + lo)
  int hskip = 0;        // head and affine skip the first hskip rows of each sample
  // PASS_ALL: the whole pass; PASS_PREFIX: shift + embed, first LayerNorm,
  // layer 0's QKV and attention only; PASS_REST: the remainder after a
  // PASS_PREFIX
  int part = 0;
};
constexpr int PASS_ALL = 0, PASS_PREFIX = 1, PASS_REST = 2;

// Cross-stream ordering of a pass that runs beside another one (the halves of
// a row split; a cache refresh and the next block's first update):
// events waited for or recorded on the pass's stream around its embed, its
// QKV GEMMs, its attentions and its affine update (NULL: none).
struct XSync {
  hipEvent_t wait_embed = nullptr;
  hipEvent_t rec_embed = nullptr;
  hipEvent_t wait_affine = nullptr;
  const hipEvent_t* wait_qkv = nullptr;    // [n_layers]
  const hipEvent_t* rec_qkv = nullptr;     // [n_layers]
  const hipEvent_t* wait_attn = nullptr;   // [n_layers]
  const hipEvent_t* rec_attn = nullptr;    // [n_layers]
  hipEvent_t rec_affine = nullptr;
  bool half = false;   // a row-split half (fewer split planes in its residual GEMMs)
};

// One pass of the network over chunk rows [s, s+R) of every sample:
// shift+embed, n_layers pre-LN layers (K/V into the cache), final LN + head.
af_status run_net(af_plan* p, const BlockW& bw, const Pass& ps, char* ws,
                  const WsLayout& w, hipStream_t st, const af::AffineArgs* aa = nullptr,
                  int mode = 0, const XSync* xs = nullptr) {
  auto wait_ev = [&](const hipEvent_t* e, int l) -> hipError_t {
    return (e && e[l]) ? hipStreamWaitEvent(st, e[l], 0) : hipSuccess;
  };
  auto rec_ev = [&](const hipEvent_t* e, int l) -> hipError_t {
    return (e && e[l]) ? hipEventRecord(e[l], st) : hipSuccess;
  };
  const af_block_cfg& c = p->cfg;
  const int M = ps.N * ps.R, d = c.d;
  // a row-split half runs beside the other: its residual GEMMs take fewer
  // split planes than the shape alone gets (measured faster: the output
  // projection one, MLP2 two)
  const bool half = xs && xs->half;
  const int o_planes = half ? 1 : 8, mlp2_planes = half ? 2 : 8;
  float* h = (float*)(ws + w.h);
  void* a = ws + w.a;
  void* q = ws + w.q;
  void* att = ws + w.att;
  void* u = ws + w.u;
  const bool sp = ps.precise && p->bf;
  void* a_lo = sp ? ws + w.a_lo : nullptr;
  void* q_lo = sp ? ws + w.q_lo : nullptr;
  void* att_lo = sp ? ws + w.att_lo : nullptr;
  void* u_lo = sp ? ws + w.u_lo : nullptr;
  float* slab = (float*)(ws + w.slab);
  const int pos_base = ps.P + ps.s;
  const bool pre = ps.part != PASS_REST, post = ps.part != PASS_PREFIX;
  // algorithmic work per launch (2 flops per multiply-add; attention 4 d flops
  // per unmasked (query, key) pair: row t attends to pos_base + t + 1 keys)
  const double Md = (double)M * d, dd = (double)d * d;
  const double w_qkv = 2.0 * M * 3.0 * dd, w_o = 2.0 * M * dd, w_mlp = 2.0 * M * 4.0 * dd;
  const double w_attn = 4.0 * d * ps.N *
                        ((double)ps.R * pos_base + 0.5 * (double)ps.R * (ps.R + 1));
  const double w_embed = 2.0 * Md * c.C;
  (void)Md;
  if (pre && xs && xs->wait_embed) AF_HIP(hipStreamWaitEvent(st, xs->wait_embed, 0));
  if (pre)
    LAUNCHW(K_EMBED, w_embed, af::launch_embed(ps.src, ps.x_last, bw.w_in, bw.b_in, bw.pos, h,
                                     ps.N, ps.R, c.C, d, ps.L, ps.s, ps.dir,
                                     pos_base, st));
  if (pre && xs && xs->rec_embed) AF_HIP(hipEventRecord(xs->rec_embed, st));
  float* hf = (float*)(ws + w.hf);
  if (p->bf) {
    // bf16 path: the O-projection and MLP-down GEMMs write fp32 partial planes
    // and one row-wise kernel adds bias + residual and emits the next LN.
    if (pre)
      LAUNCH(K_LN, af::launch_layernorm(h, bw.layers[0].ln1_g, bw.layers[0].ln1_b, a, true, M,
                                        d, st, a_lo));
    for (int l = 0; l < c.n_layers; ++l) {
      const LayerW& lw = bw.layers[l];
      char* kc = ws + w.cache + (size_t)(2 * l) * w.cache_layer;
      char* vt = ws + w.cache + (size_t)(2 * l + 1) * w.cache_layer;
      char* kc_lo = sp ? ws + w.cache_lo + (size_t)(2 * l) * w.cache_layer : nullptr;
      char* vt_lo = sp ? ws + w.cache_lo + (size_t)(2 * l + 1) * w.cache_layer : nullptr;
      af::QKVDst dst{q, kc, vt, ps.R, d, p->dh, c.n_heads, p->Lcap, pos_base, q_lo, kc_lo, vt_lo};
      if (l > 0 || pre) {
        if (xs) AF_HIP(wait_ev(xs->wait_qkv, l));
        LAUNCHW(K_QKV, w_qkv, af::launch_gemm_qkv(true, a, a_lo, lw.w_qkv, lw.b_qkv, M, 3 * d, d, dst, st));
        if (xs) AF_HIP(rec_ev(xs->rec_qkv, l));
      }
      if (ps.kv_only && l == c.n_layers - 1) return AF_OK;
      af::AttnSplit asp{q_lo, kc_lo, vt_lo, att_lo};
      if (l > 0 || pre) {
        if (xs) AF_HIP(wait_ev(xs->wait_attn, l));
        LAUNCHW(K_ATTN, w_attn, af::launch_attention(true, q, kc, vt, att, (float*)(ws + w.attn_part),
                                            (unsigned*)(ws + w.tickets), ps.N, ps.R,
                                            c.n_heads, p->dh, d, p->Lcap, pos_base,
                                            st, sp ? &asp : nullptr));
        if (xs) AF_HIP(rec_ev(xs->rec_attn, l));
      }
      if (!post) return AF_OK;
      int S = 1;
      LAUNCHW(K_O, w_o, af::launch_gemm_partial(att, att_lo, lw.w_o, slab, M, d, d, &S, st, o_planes));
      LAUNCH(K_LN, af::launch_resid_ln(slab, S, lw.b_o, h, lw.ln2_g, lw.ln2_b, a, true, a_lo,
                                       M, d, st));
      LAUNCHW(K_MLP1, w_mlp, af::launch_gemm_gelu(true, a, a_lo, lw.w_1, lw.b_1, u, u_lo, M, p->dmlp,
                                          d, st));
      LAUNCHW(K_MLP2, w_mlp, af::launch_gemm_partial(u, u_lo, lw.w_2, slab, M, d, p->dmlp, &S, st,
                                                     mlp2_planes));
      if (l + 1 < c.n_layers) {
        const LayerW& nx = bw.layers[l + 1];
        LAUNCH(K_LN, af::launch_resid_ln(slab, S, lw.b_2, h, nx.ln1_g, nx.ln1_b, a, true, a_lo,
                                         M, d, st));
      } else {
        LAUNCH(K_LN, af::launch_resid_ln(slab, S, lw.b_2, h, bw.ln_f_g, bw.ln_f_b, hf, false,
                                         nullptr, M, d, st));
      }
    }
  } else {
    for (int l = 0; l < c.n_layers; ++l) {
      const LayerW& lw = bw.layers[l];
      char* kc = ws + w.cache + (size_t)(2 * l) * w.cache_layer;
      char* vt = ws + w.cache + (size_t)(2 * l + 1) * w.cache_layer;
      af::QKVDst dst{q, kc, vt, ps.R, d, p->dh, c.n_heads, p->Lcap, pos_base, nullptr,
                     nullptr, nullptr};
      if (l > 0 || pre) {
        LAUNCH(K_LN, af::launch_layernorm(h, lw.ln1_g, lw.ln1_b, a, false, M, d, st));
        LAUNCHW(K_QKV, w_qkv, af::launch_gemm_qkv(false, a, nullptr, lw.w_qkv, lw.b_qkv, M, 3 * d, d,
                                          dst, st));
      }
      if (ps.kv_only && l == c.n_layers - 1) return AF_OK;
      if (l > 0 || pre)
        LAUNCHW(K_ATTN, w_attn, af::launch_attention(false, q, kc, vt, att, nullptr, nullptr, ps.N,
                                            ps.R, c.n_heads, p->dh, d, p->Lcap, pos_base, st));
      if (!post) return AF_OK;
      LAUNCHW(K_O, w_o, af::launch_gemm_resid(false, att, nullptr, lw.w_o, lw.b_o, h, M, d, d,
                                        nullptr, st));
      LAUNCH(K_LN, af::launch_layernorm(h, lw.ln2_g, lw.ln2_b, a, false, M, d, st));
      LAUNCHW(K_MLP1, w_mlp, af::launch_gemm_gelu(false, a, nullptr, lw.w_1, lw.b_1, u, nullptr, M,
                                          p->dmlp, d, st));
      LAUNCHW(K_MLP2, w_mlp, af::launch_gemm_resid(false, u, nullptr, lw.w_2, lw.b_2, h, M, d,
                                           p->dmlp, nullptr, st));
    }
    LAUNCH(K_LN, af::launch_layernorm(h, bw.ln_f_g, bw.ln_f_b, hf, false, M, d, st));
  }
  // final head (split-K planes: on the fp32 matrix cores where the shape
  // allows) and the affine update of the caller's AffineArgs
  float* head = (float*)(ws + w.head);
  af::AffineArgs fa = *aa;
  fa.head = head;
  if (af::head_mfma_supported(c.C, d)) {
    const int rh = ps.R - ps.hskip, mh = ps.N * rh;
    fa.head_splits = af::head_mfma_splits(mh, d);
    LAUNCHW(K_HEAD, 4.0 * mh * c.C * d, af::launch_head_mfma(hf, bw.w_head, head, mh, c.C, d, fa.head_splits, st,
                                        rh, ps.R, ps.hskip));
  } else {
    if (ps.hskip != 0) return fail(AF_ERR_UNSUPPORTED, "head row offset needs C % 8 == 0");
    fa.head_splits = af::head_splits(M, 2 * c.C, d);
    LAUNCHW(K_HEAD, 4.0 * M * c.C * d, af::launch_gemm_f32_planes(hf, bw.w_head, head, M, 2 * c.C, d,
                                              fa.head_splits, st));
  }
  if (xs && xs->wait_affine) AF_HIP(hipStreamWaitEvent(st, xs->wait_affine, 0));
  // bytes: mu, raw, z (or x) read and x (or z) written; the inverse also
  // reads the previous iterate
  LAUNCHW(K_AFFINE, (mode == 0 ? 20.0 : 16.0) * c.C * ps.N * (ps.R - ps.hskip),
          af::launch_affine(mode, fa, st));
  if (xs && xs->rec_affine) AF_HIP(hipEventRecord(xs->rec_affine, st));
  return AF_OK;
}

// Zero the counter words and the attention merge tickets behind them.
hipError_t clear_counters(const WsLayout& w, char* ws, hipStream_t st) {
  return af::launch_fill_u32(ws + w.counter, 0u, (w.slab - w.counter) / 4, st);
}

af_status check_ws(const af_plan* p, int N, int rows, void* ws, size_t ws_bytes,
                   WsLayout* out) {
  if (!ws) return fail(AF_ERR_ARG, "ws is NULL");
  if (((uintptr_t)ws & 255) != 0) return fail(AF_ERR_ARG, "ws must be 256-byte aligned");
  // the bf16 GEMMs address activation rows with 32-bit byte offsets
  if (p->bf && (uint64_t)N * rows * std::max(p->dmlp, p->cfg.d) * 2 >= (1ull << 32))
    return fail(AF_ERR_UNSUPPORTED, "batch x rows too large: activations above 4 GiB");
  *out = layout(p, N, rows);
  if (ws_bytes < out->total)
    return fail(AF_ERR_WORKSPACE, "workspace too small: need " +
                                      std::to_string(out->total) + " bytes, got " +
                                      std::to_string(ws_bytes));
  return AF_OK;
}

// Pinned, host-coherent [N][2] residual buffer that the affine kernel writes
// directly, so the stop test needs no copy command.
void destroy_entry(GraphEntry& e);

af_status ensure_host_res(af_plan* p, int N) {
  if (p->res_cap >= N) return AF_OK;
  if (p->host_res) {
    // Captured updates bake in the sequence and tag words at 2 * res_cap
    // floats past the buffer, and a new buffer may land at the old address:
    // let outstanding work finish, then drop every graph with the old buffer.
    AF_HIP(hipDeviceSynchronize());
    for (GraphEntry& e : p->gcache) destroy_entry(e);
    p->gcache.clear();
    (void)hipHostFree(p->host_res);
  }
  p->host_res = p->host_res_dev = nullptr;
  p->res_cap = 0;
  AF_HIP(hipHostMalloc((void**)&p->host_res, ((size_t)N * 2 + 64) * sizeof(float),
                       hipHostMallocMapped | hipHostMallocCoherent));
  AF_HIP(hipHostGetDevicePointer((void**)&p->host_res_dev, p->host_res, 0));
  p->res_cap = N;
  return AF_OK;
}

unsigned* seq_word(const af_plan* p, bool dev) {
  return (unsigned*)((dev ? p->host_res_dev : p->host_res) + 2 * (size_t)p->res_cap);
}

// Wait until the update numbered `want` of this call has published its
// residuals: the affine kernel writes them to pinned memory and then the
// update's number to the sequence word.  Polling that word avoids a stream
// synchronisation per update; the stream is queried now and then so that a
// failed launch is reported instead of waited on.
// With a row split, half B publishes to the next word (want2 updates) and
// both words must have arrived.
af_status wait_update(af_plan* p, unsigned want, hipStream_t st, hipStream_t st2 = nullptr,
                      unsigned want2 = 0) {
  volatile unsigned* f = seq_word(p, false);
  auto done = [&]() { return f[0] == want && (!st2 || f[1] == want2); };
  for (unsigned long it = 1;; ++it) {
    if (done()) break;
    if ((it & 4095) == 0) {
      hipError_t q = hipStreamQuery(st);
      if (q == hipSuccess && st2) q = hipStreamQuery(st2);
      if (q == hipSuccess) {
        if (done()) break;
        return fail(AF_ERR_HIP, "update finished without publishing its residual");
      }
      if (q != hipErrorNotReady)
        return fail(AF_ERR_HIP, std::string("hipStreamQuery: ") + hipGetErrorString(q));
    }
    __builtin_ia32_pause();
  }
  std::atomic_thread_fence(std::memory_order_acquire);
  return AF_OK;
}

// One Jacobi update: the network pass over the block, then the affine update.
af_status jacobi_update(af_plan* p, const BlockW& bw, const Pass& ps, const af::AffineArgs& aa,
                        char* ws, const WsLayout& w, hipStream_t st) {
  return run_net(p, bw, ps, ws, w, st, &aa, 0);
}

void destroy_entry(GraphEntry& e) {
  if (e.exec) (void)hipGraphExecDestroy(e.exec);
  e.exec = nullptr;
}

GraphEntry* graph_lookup(af_plan* p, const GraphKey& key) {
  for (GraphEntry& e : p->gcache)
    if (e.key == key) {
      e.used = ++p->gclock;
      return &e;
    }
  return nullptr;
}

// Capture one Jacobi update on the plan's private stream (nothing runs) and
// instantiate it.  The least recently used entry is dropped when the cache is
// full, after `st` (the only stream this call replays on) has drained.
af_status graph_capture(af_plan* p, const GraphKey& key, const BlockW& bw, const Pass& ps,
                        const af::AffineArgs& aa, char* ws, const WsLayout& w,
                        hipStream_t st, GraphEntry** out) {
  *out = nullptr;
  if (!p->cap_stream) AF_HIP(hipStreamCreateWithFlags(&p->cap_stream, hipStreamNonBlocking));
  GraphEntry e;
  e.key = key;
  hipError_t he = hipStreamBeginCapture(p->cap_stream, hipStreamCaptureModeRelaxed);
  if (he != hipSuccess)
    return fail(AF_ERR_HIP, std::string("hipStreamBeginCapture: ") + hipGetErrorString(he));
  const af_status s = jacobi_update(p, bw, ps, aa, ws, w, p->cap_stream);
  hipGraph_t graph = nullptr;
  he = hipStreamEndCapture(p->cap_stream, &graph);
  if (s != AF_OK || he != hipSuccess) {
    if (graph) (void)hipGraphDestroy(graph);
    return s != AF_OK ? s
                      : fail(AF_ERR_HIP, std::string("hipStreamEndCapture: ") + hipGetErrorString(he));
  }
  he = hipGraphInstantiate(&e.exec, graph, nullptr, nullptr, 0);
  (void)hipGraphDestroy(graph);
  if (he != hipSuccess)
    return fail(AF_ERR_HIP, std::string("hipGraphInstantiate: ") + hipGetErrorString(he));
  if ((int)p->gcache.size() >= kGraphCacheCap) {
    AF_HIP(hipStreamSynchronize(st));
    auto lru = std::min_element(p->gcache.begin(), p->gcache.end(),
                                [](const GraphEntry& a, const GraphEntry& b) { return a.used < b.used; });
    destroy_entry(*lru);
    p->gcache.erase(lru);
  }
  e.used = ++p->gclock;
  p->gcache.push_back(std::move(e));
  ++p->g_captures;
  *out = &p->gcache.back();
  return AF_OK;
}


}  // namespace

int af::record_error(int status, const char* msg) {
  return (int)fail((af_status)status, msg);
}

extern "C" {

const char* af_status_str(af_status s) {
  switch (s) {
    case AF_OK: return "AF_OK";
    case AF_ERR_ARG: return "AF_ERR_ARG";
    case AF_ERR_HIP: return "AF_ERR_HIP";
    case AF_ERR_WORKSPACE: return "AF_ERR_WORKSPACE";
    case AF_ERR_NONFINITE: return "AF_ERR_NONFINITE";
    case AF_ERR_UNSUPPORTED: return "AF_ERR_UNSUPPORTED";
  }
  return "AF_ERR_UNKNOWN";
}

const char* af_last_error(void) { return g_err.c_str(); }
int af_abi_version(void) { return AF_ABI_VERSION; }

af_status af_plan_create(const af_block_cfg* cfg, int n_blocks,
                         const af_block_weights* w, af_plan** out) {
  if (!cfg || !w || !out) return fail(AF_ERR_ARG, "NULL argument");
  *out = nullptr;
  if (n_blocks < 1 || n_blocks > 64) return fail(AF_ERR_ARG, "n_blocks must be 1..64");
  // a C caller may pass any int in the enum field: read its bytes as an int
  // (a C++ load of an out-of-range enum value is undefined)
  int dtype_raw;
  std::memcpy(&dtype_raw, &cfg->dtype, sizeof(dtype_raw));
  if (dtype_raw != AF_F32 && dtype_raw != AF_BF16) return fail(AF_ERR_ARG, "unknown dtype");
  const af_block_cfg& c = *cfg;
  if (c.C < 1 || c.C > 256) return fail(AF_ERR_ARG, "C must be 1..256");
  if (c.n_layers < 1 || c.n_layers > 1024) return fail(AF_ERR_ARG, "n_layers must be >= 1");
  if (c.max_len < 1 || c.max_len > (1 << 24)) return fail(AF_ERR_ARG, "max_len out of range");
  if (c.d < 64 || c.d > 8192 || c.n_heads < 1 || c.d % c.n_heads)
    return fail(AF_ERR_ARG, "d must be 64..8192 and divisible by n_heads");
  const int dh = c.d / c.n_heads;
  if (dh != 32 && dh != 64 && dh != 128)
    return fail(AF_ERR_UNSUPPORTED, "d / n_heads must be 32, 64 or 128");
  const int per_lane = c.d / 64;
  if (c.d % 64 || (per_lane & (per_lane - 1)))
    return fail(AF_ERR_UNSUPPORTED, "d must be 64 times a power of two");
  if (c.dtype == AF_BF16 && c.d % 256)
    return fail(AF_ERR_UNSUPPORTED, "bf16 path needs d % 256 == 0");
  af_plan* p = new (std::nothrow) af_plan();
  if (!p) return fail(AF_ERR_ARG, "out of host memory");
  p->cfg = c;
  p->T = n_blocks;
  p->dh = dh;
  p->dmlp = 4 * c.d;
  p->Lcap = (c.max_len + 63) / 64 * 64;
  p->bf = c.dtype == AF_BF16;
  p->esz = p->bf ? 2 : 4;
  for (int t = 0; t < n_blocks; ++t) {
    const af_block_weights& bw = w[t];
    BlockW b;
    b.w_in = bw.w_in; b.b_in = bw.b_in; b.pos = bw.pos;
    b.ln_f_g = bw.ln_f_g; b.ln_f_b = bw.ln_f_b; b.w_head = bw.w_head; b.b_head = bw.b_head;
    if (!b.w_in || !b.b_in || !b.pos || !b.ln_f_g || !b.ln_f_b || !b.w_head || !b.b_head ||
        !bw.ln1_g || !bw.ln1_b || !bw.w_qkv || !bw.b_qkv || !bw.w_o || !bw.b_o ||
        !bw.ln2_g || !bw.ln2_b || !bw.w_1 || !bw.b_1 || !bw.w_2 || !bw.b_2) {
      delete p;
      return fail(AF_ERR_ARG, "NULL weight pointer in block " + std::to_string(t));
    }
    if (any_misaligned(b.w_in, b.b_in, b.pos, b.ln_f_g, b.ln_f_b, b.w_head, b.b_head)) {
      delete p;
      return fail(AF_ERR_ARG, "weight pointer not 16-byte aligned in block " + std::to_string(t));
    }
    for (int l = 0; l < c.n_layers; ++l) {
      LayerW lw{bw.ln1_g[l], bw.ln1_b[l], bw.b_qkv[l], bw.b_o[l], bw.ln2_g[l],
                bw.ln2_b[l], bw.b_1[l], bw.b_2[l], bw.w_qkv[l], bw.w_o[l],
                bw.w_1[l], bw.w_2[l]};
      if (!lw.ln1_g || !lw.ln1_b || !lw.b_qkv || !lw.b_o || !lw.ln2_g || !lw.ln2_b ||
          !lw.b_1 || !lw.b_2 || !lw.w_qkv || !lw.w_o || !lw.w_1 || !lw.w_2) {
        delete p;
        return fail(AF_ERR_ARG, "NULL layer weight pointer in block " +
                                    std::to_string(t) + " layer " + std::to_string(l));
      }
      if (any_misaligned(lw.ln1_g, lw.ln1_b, lw.b_qkv, lw.b_o, lw.ln2_g, lw.ln2_b, lw.b_1,
                         lw.b_2, lw.w_qkv, lw.w_o, lw.w_1, lw.w_2)) {
        delete p;
        return fail(AF_ERR_ARG, "layer weight pointer not 16-byte aligned in block " +
                                    std::to_string(t) + " layer " + std::to_string(l));
      }
      b.layers.push_back(lw);
    }
    p->blocks.push_back(std::move(b));
  }
  *out = p;
  return AF_OK;
}

void af_plan_destroy(af_plan* p) {
  if (!p) return;
  // an inverse call returns with its last kernels possibly still queued
  (void)hipDeviceSynchronize();
  for (GraphEntry& e : p->gcache) destroy_entry(e);
  if (p->cap_stream) (void)hipStreamDestroy(p->cap_stream);
  if (p->split_stream) (void)hipStreamDestroy(p->split_stream);
  for (hipEvent_t e : p->split_ev) (void)hipEventDestroy(e);
  if (p->host_res) (void)hipHostFree(p->host_res);
  if (p->loop_host) (void)hipHostFree(p->loop_host);
  for (hipEvent_t e : p->ev) (void)hipEventDestroy(e);
  delete p;
}

size_t af_workspace_bytes(const af_plan* p, int batch, int rows) {
  if (!p || batch < 1 || rows < 1) return 0;
  const WsLayout w = layout(p, batch, rows);
  // room for the row split's second half when a block of `rows` rows uses
  // it, and for the scratch of a cache refresh beside the next block's
  // updates (the two share the space after the main layout)
  size_t total = w.total;
  if (split_possible(p, batch, rows)) total = std::max(total, layout_b(p, batch, rows, w).total);
  if (refresh_overlap_possible(p)) total = std::max(total, layout_r(p, batch, rows, w).total);
  return total;
}

size_t af_cache_bytes(const af_plan* p, int batch) {
  if (!p || batch < 1) return 0;
  return align256(2 * layout(p, batch, 1).cache_layer * p->cfg.n_layers);
}

af_status af_forward(af_plan* p, const float* x, float* z, float* logdet, int N,
                     int L, int frames_per_entry, int flags, void* ws_, size_t ws_bytes,
                     void* stream) {
  if (!p || !x || !z || !logdet) return fail(AF_ERR_ARG, "NULL argument");
  if (any_misaligned(x, z)) return fail(AF_ERR_ARG, "x and z must be 16-byte aligned");
  if (N < 1 || L < 1 || L > p->cfg.max_len) return fail(AF_ERR_ARG, "need N >= 1 and 1 <= L <= max_len");
  if (frames_per_entry < 1 || N % frames_per_entry)
    return fail(AF_ERR_ARG, "frames_per_entry must be >= 1 and divide N");
  if (flags & ~(AF_FWD_ACCUMULATE | AF_FWD_CHECK_FINITE)) return fail(AF_ERR_ARG, "unknown flags");
  if (x == z) return fail(AF_ERR_ARG, "x and z may not alias");
  WsLayout w;
  if (af_status s = check_ws(p, N, L, ws_, ws_bytes, &w)) return s;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)ws_;
  const int C = p->cfg.C;
  AF_HIP(clear_counters(w, ws, st));
  if (!(flags & AF_FWD_ACCUMULATE))
    AF_HIP(af::launch_fill_u32(logdet, 0u, (size_t)(N / frames_per_entry), st));
  // the affine kernel tags the first stack block that produced a non-finite z
  unsigned* bad = (unsigned*)(ws + w.counter) + 1;
  float* xtmp = (float*)(ws + w.xtmp);
  const float* cur = x;
  for (int t = 0; t < p->T; ++t) {
    float* dst = ((p->T - 1 - t) % 2 == 0) ? z : xtmp;
    // the forward carries bf16 activations as hi + lo pairs, so that the
    // log-det (a sum of many terms that largely cancel) keeps fp32 accuracy
    Pass ps{cur, nullptr, N, L, 0, L, 0, t & 1, false, true};
    af::AffineArgs aa{(const float*)(ws + w.head), p->blocks[t].b_head,
                      af::head_splits(N * L, 2 * C, p->cfg.d), nullptr,
                      const_cast<float*>(cur), dst,
                      N, L, C, L, 0, t & 1, (float*)(ws + w.partials),
                      (float*)(ws + w.res), (unsigned*)(ws + w.counter), logdet,
                      bad, (unsigned)(t + 1)};
    aa.ld_group = frames_per_entry;
    if (af_status s = run_net(p, p->blocks[t], ps, ws, w, st, &aa, 1)) return s;
    cur = dst;
  }
  if (flags & AF_FWD_CHECK_FINITE) {
    unsigned tag = 0;
    AF_HIP(hipStreamSynchronize(st));
    AF_HIP(hipMemcpy(&tag, bad, sizeof(tag), hipMemcpyDeviceToHost));
    if (tag != 0)
      return fail(AF_ERR_NONFINITE, "non-finite z in stack block " + std::to_string(tag - 1));
  }
  return AF_OK;
}

static af::LoopArgs loop_args(const af_plan* p, const BlockW& bw, char* ws, const WsLayout& w);
static int loop_refresh_rows(af_plan* p, int N, int L);

af_status af_prefill(af_plan* p, const float* x_prefix, int N, int P, void* ws_,
                     size_t ws_bytes, void* stream) {
  if (!p || !x_prefix) return fail(AF_ERR_ARG, "NULL argument");
  if (misaligned(x_prefix)) return fail(AF_ERR_ARG, "x_prefix must be 16-byte aligned");
  if (p->T != 1) return fail(AF_ERR_UNSUPPORTED, "af_prefill needs a single-block plan");
  if (N < 1 || P < 1 || P > p->cfg.max_len) return fail(AF_ERR_ARG, "need N >= 1 and 1 <= P <= max_len");
  WsLayout w;
  if (af_status s = check_ws(p, N, P, ws_, ws_bytes, &w)) return s;
  hipStream_t st = (hipStream_t)stream;
  Pass ps{x_prefix, nullptr, N, P, 0, P, 0, 0, true, false};
  AF_HIP(clear_counters(w, (char*)ws_, st));
  return run_net(p, p->blocks[0], ps, (char*)ws_, w, st);
}

af_status af_refresh_kv(af_plan* p, const float* x, int N, int L, int prefix_len,
                        const float* x_last, void* ws_, size_t ws_bytes, void* stream) {
  if (!p || !x) return fail(AF_ERR_ARG, "NULL argument");
  if (any_misaligned(x, x_last)) return fail(AF_ERR_ARG, "x and x_last must be 16-byte aligned");
  if (p->T != 1) return fail(AF_ERR_UNSUPPORTED, "af_refresh_kv needs a single-block plan");
  if (N < 1 || L < 1 || prefix_len < 0 || prefix_len + L > p->cfg.max_len)
    return fail(AF_ERR_ARG, "need N, L >= 1, prefix_len >= 0 and prefix_len + L <= max_len");
  if (prefix_len > 0 && !x_last) return fail(AF_ERR_ARG, "x_last is required when prefix_len > 0");
  WsLayout w;
  if (af_status s = check_ws(p, N, L, ws_, ws_bytes, &w)) return s;
  hipStream_t st = (hipStream_t)stream;
  // the plan's device loop refreshes the rows of a call's blocks: the rows
  // of its last block come from the same pass here
  if (const int R = loop_refresh_rows(p, N, L)) {
    af::LoopArgs a = loop_args(p, p->blocks[0], (char*)ws_, w);
    a.x_init = x;
    a.refresh = 1;
    a.x_last = x_last;
    a.N = N;
    a.L = L;
    a.B = R;
    a.P = prefix_len;
    // algorithmic flops: embed, every layer but the last, the last one's QKV
    const af_block_cfg& c = p->cfg;
    const double d = c.d, C = c.C, dm = p->dmlp;
    double work = 0.0;
    for (int s0 = 0; s0 < L; s0 += R) {
      const int r = std::min(R, L - s0);
      const double M = (double)N * r;
      const double pairs = (double)N * r * (prefix_len + s0 + (r + 1) / 2.0);
      const double layer = M * (6 * d * d + 2 * d * d + 4 * d * dm) + 4 * d * pairs;
      work += 2 * C * d * M + (c.n_layers - 1) * layer + 6 * d * d * M;
    }
    LAUNCHW(K_LOOP, work, af::launch_jacobi_loop(a, st));
    return AF_OK;
  }
  Pass ps{x, x_last, N, L, 0, L, prefix_len, 0, true, false};
  AF_HIP(clear_counters(w, (char*)ws_, st));
  return run_net(p, p->blocks[0], ps, (char*)ws_, w, st);
}

// The arguments of the device loop that describe AF block bw and its cache.
static af::LoopArgs loop_args(const af_plan* p, const BlockW& bw, char* ws, const WsLayout& w) {
  const af_block_cfg& c = p->cfg;
  af::LoopArgs a{};
  a.w_in = bw.w_in;
  a.b_in = bw.b_in;
  a.pos = bw.pos;
  a.ln_f_g = bw.ln_f_g;
  a.ln_f_b = bw.ln_f_b;
  a.w_head = bw.w_head;
  a.b_head = bw.b_head;
  for (int l = 0; l < c.n_layers; ++l) {
    const LayerW& lw = bw.layers[l];
    a.layers[l] = af::LoopLayer{lw.ln1_g, lw.ln1_b, (const float*)lw.w_qkv, lw.b_qkv,
                                (const float*)lw.w_o, lw.b_o, lw.ln2_g, lw.ln2_b,
                                (const float*)lw.w_1, lw.b_1, (const float*)lw.w_2, lw.b_2};
    a.kc[l] = (float*)(ws + w.cache + (size_t)(2 * l) * w.cache_layer);
    a.vt[l] = (float*)(ws + w.cache + (size_t)(2 * l + 1) * w.cache_layer);
  }
  a.n_layers = c.n_layers;
  a.C = c.C;
  a.d = c.d;
  a.H = c.n_heads;
  a.dh = p->dh;
  a.dmlp = p->dmlp;
  a.Lcap = p->Lcap;
  a.lds_max = p->loop_lds_max;
  return a;
}

// LDS one workgroup of the device loop may take: the current device's limit
// per block (160 KB on gfx950), queried once; 64 KB if the query fails.
static int loop_lds_max(af_plan* p) {
  if (p->loop_lds_max == 0) {
    int dev = 0, v = 0;
    p->loop_lds_max = 65536;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) ==
            hipSuccess &&
        v > 65536)
      p->loop_lds_max = std::min(v, 160 * 1024);
    (void)hipGetLastError();
  }
  return p->loop_lds_max;
}

static bool loop_supported(af_plan* p, int N, int rows) {
  return af::jacobi_loop_supported(N, rows, p->cfg.C, p->cfg.d, p->cfg.n_heads, p->dmlp,
                                   p->cfg.n_layers, p->Lcap, loop_lds_max(p));
}

// Rows per device-loop block for a refresh of N samples (0: not supported).
static int loop_refresh_rows(af_plan* p, int N, int L) {
  if (p->bf || !p->device_loop || p->graphs || p->row_split || p->fuse_refresh || N > 64)
    return 0;
  const int R = std::min(L, 64 / N);
  return loop_supported(p, N, R) ? R : 0;
}

// The whole Jacobi inverse of each AF block of the stack in one launch (small
// fp32 blocks): the loop, its stop tests and the cache refreshes run on the
// device, which writes the block counts, the last residual pairs and a
// non-finite word to pinned memory; the host waits once at the end.
static af_status inverse_on_device(af_plan* p, const float* z, int N, int L, int B, float tau,
                                   int max_iters, af_init init, const float* x_init,
                                   int frame_len, int prefix_len, const float* x_last,
                                   float* x, int32_t* iters, char* ws, const WsLayout& w,
                                   int nb, hipStream_t st) {
  const af_block_cfg& c = p->cfg;
  const size_t need = (size_t)p->T * nb + p->T;
  if (p->loop_cap < need) {
    if (p->loop_host) {
      AF_HIP(hipDeviceSynchronize());
      (void)hipHostFree(p->loop_host);
    }
    p->loop_host = p->loop_host_dev = nullptr;
    p->loop_cap = 0;
    AF_HIP(hipHostMalloc((void**)&p->loop_host, need * sizeof(int),
                         hipHostMallocMapped | hipHostMallocCoherent));
    AF_HIP(hipHostGetDevicePointer((void**)&p->loop_host_dev, p->loop_host, 0));
    p->loop_cap = need;
  }
  volatile int* lh = p->loop_host;
  for (size_t i = 0; i < need; ++i) lh[i] = 0;
  float* xtmp = (float*)(ws + w.xtmp);
  const float* zin = z;
  for (int t = p->T - 1; t >= 0; --t) {
    af::LoopArgs a = loop_args(p, p->blocks[t], ws, w);
    a.z = zin;
    a.x = (t % 2 == 0) ? x : xtmp;
    a.x_init = x_init;
    a.x_last = x_last;
    a.N = N;
    a.L = L;
    a.B = B;
    a.P = prefix_len;
    a.dir = t & 1;
    a.init = (int)init;
    a.F = frame_len;
    a.max_iters = max_iters;
    a.tau = tau;
    a.iters_host = p->loop_host_dev + (size_t)t * nb;
    a.res_host = p->host_res_dev;
    a.bad_host = (unsigned*)(p->loop_host_dev + (size_t)p->T * nb + t);
    LAUNCH(K_LOOP, af::launch_jacobi_loop(a, st));
    // every Jacobi block of this AF block is final once the stream reaches here
    if (p->done_fn)
      for (int b = 0; b < nb; ++b) p->done_fn(p->done_user, t, b);
    zin = a.x;
  }
  AF_HIP(hipStreamSynchronize(st));
  for (int t = 0; t < p->T; ++t)
    for (int b = 0; b < nb; ++b) iters[t * nb + b] = lh[(size_t)t * nb + b];
  if (p->prof_class == K_LOOP) {
    // the launches' algorithmic flops, known once the counts are: per update
    // of a block of R rows, embed 2CdM, per layer QKV 6d^2 M + O 2d^2 M + MLP
    // 4 d dmlp M + attention 4d per (query, key) pair, head 4CdM; a refresh
    // (early stop) is the layers' QKV and attention but the last layer's
    const double d = c.d, C = c.C, dm = p->dmlp;
    for (int t = 0; t < p->T; ++t)
      for (int b = 0; b < nb; ++b) {
        const int s = b * B, R = std::min(B, L - s), k = iters[t * nb + b];
        const double M = (double)N * R;
        const double pairs = (double)N * R * (prefix_len + s + (R + 1) / 2.0);
        const double layer = M * (6 * d * d + 2 * d * d + 4 * d * dm) + 4 * d * pairs;
        const double upd = 2 * C * d * M + c.n_layers * layer + 4 * C * d * M;
        double work = k * upd;
        if (k < R && b + 1 < nb) work += 2 * C * d * M + c.n_layers * layer - (layer - 6 * d * d * M);
        p->prof_work += work;
      }
  }
  p->last_res.assign((size_t)2 * N, 0.f);
  for (int n = 0; n < 2 * N; ++n) p->last_res[n] = p->host_res[n];
  for (int t = p->T - 1; t >= 0; --t) {
    const int tag = lh[(size_t)p->T * nb + t];
    if (tag != 0)
      return fail(AF_ERR_NONFINITE, "non-finite x in stack block " + std::to_string(t) +
                                        ", Jacobi block " + std::to_string(tag - 1));
  }
  return AF_OK;
}

af_status af_inverse_jacobi(af_plan* p, const float* z, int N, int L, int B,
                            float tau, int max_iters, af_init init,
                            const float* x_init, int frame_len, int prefix_len,
                            const float* x_last, float* x, int32_t* iters,
                            void* ws_, size_t ws_bytes, void* stream) {
  if (!p || !z || !x || !iters) return fail(AF_ERR_ARG, "NULL argument");
  if (any_misaligned(z, x, x_init, x_last))
    return fail(AF_ERR_ARG, "z, x, x_init and x_last must be 16-byte aligned");
  if (N < 1 || L < 1 || B < 1) return fail(AF_ERR_ARG, "need N, L, B >= 1");
  if (std::isnan(tau)) return fail(AF_ERR_ARG, "tau is NaN");
  if (init != AF_INIT_ZERO && init != AF_INIT_GIVEN && init != AF_INIT_PREV_FRAME)
    return fail(AF_ERR_ARG, "unknown init");
  if (prefix_len < 0 || (long)prefix_len + L > p->cfg.max_len)
    return fail(AF_ERR_ARG, "need prefix_len >= 0 and prefix_len + L <= max_len");
  if (prefix_len > 0 && !x_last) return fail(AF_ERR_ARG, "x_last is required when prefix_len > 0");
  if (init == AF_INIT_GIVEN && !x_init) return fail(AF_ERR_ARG, "x_init is NULL");
  const int Bc = B < L ? B : L;
  if (init == AF_INIT_PREV_FRAME && frame_len < Bc)
    return fail(AF_ERR_ARG, "PREV_FRAME needs frame_len >= min(B, L)");
  if (x == z || (x_init && x_init == x)) return fail(AF_ERR_ARG, "x may not alias z or x_init");
  if (p->T > 1 && (init != AF_INIT_ZERO || prefix_len != 0))
    return fail(AF_ERR_UNSUPPORTED, "stacks support AF_INIT_ZERO with prefix_len 0 only");
  WsLayout w;
  if (af_status s = check_ws(p, N, Bc, ws_, ws_bytes, &w)) return s;
  if (af_status s = ensure_host_res(p, N)) return s;
  const int C = p->cfg.C;
  const int nb = (L + B - 1) / B;
  if (!p->bf && p->device_loop && !p->graphs && !p->row_split && !p->fuse_refresh &&
      loop_supported(p, N, Bc))
    return inverse_on_device(p, z, N, L, B, tau, max_iters, init, x_init, frame_len, prefix_len,
                             x_last, x, iters, (char*)ws_, w, nb, (hipStream_t)stream);
  // A block that stops early has its cache rows recomputed from its final
  // tokens.  With a workspace for two blocks of rows, that pass is merged into
  // the next block's first update (one pass over both blocks' rows; the head
  // and the affine update cover the new block only), else it runs on its own.
  int rows = Bc;
  bool fuse = false;
  if (p->fuse_refresh && nb > 1 && af::head_mfma_supported(C, p->cfg.d)) {
    const int r2 = std::min(2 * Bc, L);
    WsLayout w2;
    if (check_ws(p, N, r2, ws_, ws_bytes, &w2) == AF_OK) {
      w = w2;
      rows = r2;
      fuse = true;
    } else {
      g_err.clear();
    }
  }
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)ws_;
  int device = 0;
  if (p->graphs) AF_HIP(hipGetDevice(&device));
  // Row split (two streams, see split_rows_a): only with direct launches,
  // without the fused refresh, and when the workspace has room for half B.
  WsLayout wb{};
  bool split_ok = p->row_split && !p->graphs && !fuse && split_possible(p, N, Bc);
  if (split_ok) {
    wb = layout_b(p, N, Bc, w);
    split_ok = ws_bytes >= wb.total;
  }
  // Cache refresh beside the next block (see af_plan_set_overlap_refresh):
  // direct launches, one pass per update, room for the refresh's scratch.
  WsLayout wr{};
  bool overlap_ok = p->overlap_refresh && refresh_overlap_possible(p) && !p->graphs && !fuse &&
                    !split_ok && nb > 1;
  if (overlap_ok) {
    wr = layout_r(p, N, Bc, w);
    overlap_ok = ws_bytes >= wr.total;
  }
  const int nl = p->cfg.n_layers;
  const bool two_streams = split_ok || overlap_ok;
  if (two_streams) {
    if (!p->split_stream)
      AF_HIP(hipStreamCreateWithFlags(&p->split_stream, hipStreamNonBlocking));
    if (p->split_ev.empty()) {
      p->split_ev.resize(2 * nl + 4);
      for (auto& e : p->split_ev) AF_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
    }
    if (split_ok)
      if (af_status e = ensure_host_res(p, 2 * N)) return e;
  }
  hipStream_t sb = p->split_stream;
  // (with the refresh beside the next block, ev_qkv[l] marks the refresh's
  // QKV(l), which the next block's first update waits for before its
  // attention(l))
  const hipEvent_t* ev_qkv = two_streams ? p->split_ev.data() : nullptr;        // A: QKV(l) done
  const hipEvent_t* ev_att = two_streams ? p->split_ev.data() + nl : nullptr;   // B: attention(l) done
  hipEvent_t ev_aff = two_streams ? p->split_ev[2 * nl] : nullptr;        // A: affine done
  hipEvent_t ev_emb = two_streams ? p->split_ev[2 * nl + 1] : nullptr;    // B: embed done
  hipEvent_t ev_fork = two_streams ? p->split_ev[2 * nl + 2] : nullptr;
  hipEvent_t ev_join = two_streams ? p->split_ev[2 * nl + 3] : nullptr;
  // layer 0's K/V of a refreshed block come from the prefix on `stream`
  std::vector<hipEvent_t> ev_refresh_qkv(nl, nullptr);
  if (overlap_ok)
    for (int l = 1; l < nl; ++l) ev_refresh_qkv[l] = ev_qkv[l];
  bool b_busy = false;   // the second stream has work enqueued since the last join
  auto join_b = [&]() -> hipError_t {
    if (!b_busy) return hipSuccess;
    b_busy = false;
    hipError_t e = hipEventRecord(ev_join, sb);
    return e != hipSuccess ? e : hipStreamWaitEvent(st, ev_join, 0);
  };
  // every return, errors included, leaves `stream` ordered after half B's work
  struct JoinAtExit {
    decltype(join_b)& j;
    ~JoinAtExit() { (void)j(); }
  } join_at_exit{join_b};
  float* xtmp = (float*)(ws + w.xtmp);
  float* res = (float*)(ws + w.res);
  // counter word of the affine kernel, the sticky non-finite tag after it,
  // then the count of finished updates, published to the host's sequence word
  unsigned* bad = (unsigned*)(ws + w.counter) + 1;
  unsigned* seq_dev = (unsigned*)(ws + w.counter) + 2;
  AF_HIP(clear_counters(w, ws, st));
  if (split_ok) AF_HIP(clear_counters(wb, ws, st));
  if (overlap_ok) AF_HIP(clear_counters(wr, ws, st));
  // host-mapped words behind the residual pairs: the sequence numbers of
  // halves A and B, then the non-finite tags they report
  volatile unsigned* seq_host_words = seq_word(p, false);
  for (int i = 0; i < 4; ++i) seq_host_words[i] = 0u;   // no update of this plan is in flight
  unsigned n_updates = 0;
  unsigned n_split = 0;   // updates that ran as a row split (half B's publications)
  bool last_split = false;
  p->last_res.clear();
  // keep the residual pairs the host saw last (both halves of a split added)
  auto record_res = [&]() {
    const volatile float* hr = p->host_res;
    p->last_res.assign((size_t)2 * N, 0.f);
    for (int n = 0; n < 2 * N; ++n)
      p->last_res[n] = last_split ? hr[n] + hr[2 * N + n] : hr[n];
  };

  const float* zin = z;
  for (int t = p->T - 1; t >= 0; --t) {
    float* xo = (t % 2 == 0) ? x : xtmp;
    const int dir = t & 1;
    int pending = 0;   // rows of the previous block whose refresh is merged here
    bool refresh_beside = false;   // the previous block's refresh runs on the second stream
    for (int b = 0; b < nb; ++b) {
      const int s = b * B, R = (s + B < L ? s + B : L) - s;
      const int kmax = max_iters <= 0 ? R : (max_iters < R ? max_iters : R);
      AF_HIP(af::launch_init_block(xo, x_init, (int)init, N, R, C, L, s, dir, frame_len, st));
      Pass ps{xo, x_last, N, L, s, R, prefix_len, dir, false, false};
      af::AffineArgs aa{(const float*)(ws + w.head), p->blocks[t].b_head,
                        af::head_splits(N * R, 2 * C, p->cfg.d), zin, xo, nullptr, N, R, C, L, s,
                        dir, (float*)(ws + w.partials), res,
                        (unsigned*)(ws + w.counter), nullptr, bad,
                        (unsigned)(1 + t * nb + b), p->host_res_dev, seq_dev,
                        seq_word(p, true), seq_word(p, true) + 2};
      // the update is the same launch sequence on every iteration of the
      // block: replay it as one graph when there are several to run (or it is
      // cached from an earlier call).  Profiled calls launch directly, as
      // event records inside a graph carry no timing on this runtime.
      GraphEntry* g = nullptr;
      if (p->graphs && p->prof_class < 0) {
        const GraphKey key{&p->blocks[t], xo, x_last, zin, p->host_res_dev, ws, device,
                           N, L, s, R, prefix_len, dir, rows, (unsigned)(1 + t * nb + b)};
        g = graph_lookup(p, key);
        if (!g && kmax >= 2)
          if (af_status e = graph_capture(p, key, p->blocks[t], ps, aa, ws, w, st, &g)) return e;
      }
      // Row split: half A (rows [s, s + ra)) on st, half B on sb.  Every
      // update is enqueued as A's prefix, B's prefix, A's rest, B's rest, so
      // that each wait below finds the record it needs already enqueued: B's
      // attention(l) waits for A's QKV(l) (its keys include A's rows); A's
      // QKV(l) waits for B's attention(l) of the previous update (it rewrites
      // K/V rows B still reads); B's embed waits for A's previous affine
      // update (B's first row reads A's last token) and A's affine update
      // waits for B's embed (it rewrites that token).  Each half publishes its
      // own residual pair; the stop test adds them.
      const int ra = split_ok ? split_rows_a(p, N, R, prefix_len + s) : 0;
      const bool split = ra > 0;
      Pass psa = ps, psb = ps;
      af::AffineArgs aaa = aa, aab = aa;
      XSync xa, xb;
      if (split) {
        psa.R = ra;
        psb.s = s + ra;
        psb.R = R - ra;
        aaa.R = ra;
        aab.R = R - ra;
        aab.s = s + ra;
        aab.partials = (float*)(ws + wb.partials);
        aab.res = (float*)(ws + wb.res);
        aab.counter = (unsigned*)(ws + wb.counter);
        aab.res_host = p->host_res_dev + 2 * (size_t)N;
        aab.seq_dev = (unsigned*)(ws + wb.counter) + 2;
        aab.seq_host = seq_word(p, true) + 1;
        aab.bad_host = seq_word(p, true) + 3;
        xa.half = xb.half = true;
        xa.wait_qkv = ev_att;
        xa.rec_qkv = ev_qkv;
        xa.wait_affine = ev_emb;
        xa.rec_affine = ev_aff;
        xb.wait_embed = ev_aff;
        xb.rec_embed = ev_emb;
        xb.wait_attn = ev_qkv;
        xb.rec_attn = ev_att;
        // half B starts after this block's initial iterate and all earlier work
        AF_HIP(hipEventRecord(ev_fork, st));
        AF_HIP(hipStreamWaitEvent(sb, ev_fork, 0));
        b_busy = true;
      }
      auto split_part = [&](int part) -> af_status {
        Pass pa = psa, pb = psb;
        pa.part = part;
        pb.part = part;
        if (af_status e = run_net(p, p->blocks[t], pa, ws, w, st, &aaa, 0, &xa)) return e;
        return run_net(p, p->blocks[t], pb, ws, wb, sb, &aab, 0, &xb);
      };
      int k = 0;
      bool nonfinite = false;
      bool prefixed = false;   // the next update's first kernels are already enqueued
      for (k = 1; k <= kmax; ++k) {
        if (split) {
          if (!prefixed)
            if (af_status e = split_part(PASS_PREFIX)) return e;
          if (af_status e = split_part(PASS_REST)) return e;
          prefixed = false;
        } else if (prefixed) {
          Pass pr = ps;
          pr.part = PASS_REST;
          if (af_status e = jacobi_update(p, p->blocks[t], pr, aa, ws, w, st)) return e;
          prefixed = false;
        } else if (k == 1 && pending > 0) {
          // previous block's refresh + this block's first update, one pass
          Pass pf = ps;
          pf.s = s - pending;
          pf.R = R + pending;
          pf.hskip = pending;
          if (af_status e = jacobi_update(p, p->blocks[t], pf, aa, ws, w, st)) return e;
        } else if (k == 1 && refresh_beside) {
          // the first update beside the previous block's refresh: its
          // attention(l) reads that block's K/V rows of layer l
          XSync xw;
          xw.wait_attn = ev_refresh_qkv.data();
          if (af_status e = run_net(p, p->blocks[t], ps, ws, w, st, &aa, 0, &xw)) return e;
          refresh_beside = false;
        } else if (g) {
          AF_HIP(hipGraphLaunch(g->exec, st));
          ++p->g_replays;
        } else if (af_status e = jacobi_update(p, p->blocks[t], ps, aa, ws, w, st)) {
          return e;
        }
        ++n_updates;
        if (split) ++n_split;
        last_split = split;
        // the residual is read only for the stop test; at the cap (and in
        // forced-count mode) a non-finite residual is caught through the
        // sticky tag read once at the end
        if (!(tau > 0.f && k < kmax)) continue;
        // While the host waits for the residual, the device runs the next
        // update's first kernels (shift + embed, first LayerNorm, layer 0's
        // QKV and attention).  They write only scratch and this block's
        // layer-0 K/V rows, which the next update would write identically;
        // after an early stop they are what the block's cache refresh needs
        // for layer 0, and the refresh continues from them, so a stop leaves
        // the result unchanged.  (Graph replay keeps whole updates.)
        if (split) {
          if (af_status e = split_part(PASS_PREFIX)) return e;
          prefixed = true;
        } else if (!g) {
          Pass pp = ps;
          pp.part = PASS_PREFIX;
          if (af_status e = run_net(p, p->blocks[t], pp, ws, w, st)) return e;
          prefixed = true;
        }
        if (af_status e = wait_update(p, n_updates, st, split ? sb : nullptr, n_split)) return e;
        const volatile float* hr = p->host_res;
        bool all_below = true;
        for (int n = 0; n < N; ++n) {
          float num = hr[2 * n], den = hr[2 * n + 1];
          if (split) {
            num += hr[2 * (N + n)];
            den += hr[2 * (N + n) + 1];
          }
          if (!std::isfinite(num) || !std::isfinite(den)) nonfinite = true;
          const float r = den > 0.f ? num / den : (num == 0.f ? 0.f : INFINITY);
          if (!(r < tau)) all_below = false;
        }
        if (nonfinite) break;
        if (tau > 0.f && all_below) break;
      }
      AF_HIP(join_b());   // later work on st sees all of half B's writes
      if (nonfinite) {
        record_res();
        iters[t * nb + b] = k;
        return fail(AF_ERR_NONFINITE, "non-finite x in stack block " + std::to_string(t) +
                                          ", Jacobi block " + std::to_string(b));
      }
      if (k > kmax) k = kmax;
      iters[t * nb + b] = k;
      // the block's tokens are final once the stream reaches this point
      if (p->done_fn) p->done_fn(p->done_user, t, b);
      pending = 0;
      if (k < R && b + 1 < nb) {
        if (fuse) {
          pending = R;
        } else {
          Pass pr = ps;
          pr.kv_only = true;
          // After a stop the next update's prefix has already run layer 0 on
          // the final tokens (shift + embed into h, first LayerNorm, layer 0's
          // K/V rows, its attention output): the refresh continues from there
          // with the same launches it would otherwise repeat on the same
          // inputs.  (A split prefix leaves its halves in two scratch areas.)
          if (prefixed && !split) pr.part = PASS_REST;
          if (overlap_ok && pr.part == PASS_REST) {
            // The refresh runs on the second stream, in its own scratch (the
            // prefix's embed output and layer-0 attention output copied
            // there), beside the next block's first update, which waits for
            // its K/V layer by layer.  The same launches on the same inputs:
            // results are unchanged.
            AF_HIP(join_b());   // the previous refresh is done with that scratch
            const size_t M = (size_t)N * R;
            AF_HIP(hipMemcpyAsync(ws + wr.h, ws + w.h, M * p->cfg.d * 4,
                                  hipMemcpyDeviceToDevice, st));
            AF_HIP(hipMemcpyAsync(ws + wr.att, ws + w.att, M * p->cfg.d * p->esz,
                                  hipMemcpyDeviceToDevice, st));
            AF_HIP(hipEventRecord(ev_fork, st));
            AF_HIP(hipStreamWaitEvent(sb, ev_fork, 0));
            b_busy = true;
            XSync xr;
            xr.rec_qkv = ev_qkv;
            if (af_status e = run_net(p, p->blocks[t], pr, ws, wr, sb, nullptr, 0, &xr)) return e;
            refresh_beside = true;
          } else if (af_status e = run_net(p, p->blocks[t], pr, ws, w, st)) {
            return e;
          }
        }
      }
    }
    zin = xo;
  }
  AF_HIP(join_b());
  // An update that finds a non-finite sum writes the first such tag to its
  // half's pinned word before it publishes its number: waiting for the last
  // update's publication (the stop test may have seen it already) replaces
  // draining the stream, so work enqueued behind it (a speculative prefix)
  // keeps running while the call returns.
  if (af_status e = wait_update(p, n_updates, st, n_split ? sb : nullptr, n_split)) return e;
  record_res();
  unsigned tag = seq_host_words[2];
  if (tag == 0) tag = seq_host_words[3];
  if (tag != 0) {
    const int t = (int)(tag - 1) / nb, b = (int)(tag - 1) % nb;
    return fail(AF_ERR_NONFINITE, "non-finite x in stack block " + std::to_string(t) +
                                      ", Jacobi block " + std::to_string(b));
  }
  return AF_OK;
}

af_status af_profile_enable(af_plan* p, const char* kernel_class) {
  if (!p || !kernel_class) return fail(AF_ERR_ARG, "NULL argument");
  int cls = -1;
  for (int i = 0; i < K_NCLASS; ++i)
    if (std::strcmp(kernel_class, kclass_names[i]) == 0) cls = i;
  if (cls < 0) return fail(AF_ERR_ARG, std::string("unknown kernel class ") + kernel_class);
  if (p->ev.empty()) {
    p->ev.resize(2 * kProfileLaunches);
    // timing-only events: no system-scope fence (cache writeback and
    // invalidate) when recorded, which would add its own cost to the
    // bracketed launch
    for (auto& e : p->ev) AF_HIP(hipEventCreateWithFlags(&e, hipEventDisableSystemFence));
  }
  p->prof_class = cls;
  p->prof_n = 0;
  p->prof_work = 0.0;
  return AF_OK;
}

af_status af_profile_disable(af_plan* p) {
  if (!p) return fail(AF_ERR_ARG, "NULL argument");
  p->prof_class = -1;
  return AF_OK;
}

af_status af_profile_read(af_plan* p, int* launches, double* total_ms, double* work) {
  if (!p || !launches || !total_ms) return fail(AF_ERR_ARG, "NULL argument");
  if (work) *work = p->prof_work;
  double tot = 0.0;
  for (int i = 0; i < p->prof_n; ++i) {
    AF_HIP(hipEventSynchronize(p->ev[2 * i + 1]));
    float ms = 0.f;
    AF_HIP(hipEventElapsedTime(&ms, p->ev[2 * i], p->ev[2 * i + 1]));
    tot += ms;
  }
  *launches = p->prof_n;
  *total_ms = tot;
  return AF_OK;
}

af_status af_plan_last_residual(const af_plan* p, int N, float* num_den) {
  if (!p || !num_den) return fail(AF_ERR_ARG, "NULL argument");
  if (p->last_res.empty()) return fail(AF_ERR_ARG, "no inverse call has finished on this plan");
  if ((size_t)2 * N != p->last_res.size())
    return fail(AF_ERR_ARG, "N differs from the batch of the last inverse call");
  std::memcpy(num_den, p->last_res.data(), p->last_res.size() * sizeof(float));
  return AF_OK;
}

af_status af_plan_set_fused_refresh(af_plan* p, int enable) {
  if (!p) return fail(AF_ERR_ARG, "NULL argument");
  p->fuse_refresh = enable != 0;
  return AF_OK;
}

af_status af_plan_set_device_loop(af_plan* p, int enable) {
  if (!p) return fail(AF_ERR_ARG, "NULL argument");
  p->device_loop = enable != 0;
  return AF_OK;
}

af_status af_plan_set_row_split(af_plan* p, int enable) {
  if (!p) return fail(AF_ERR_ARG, "NULL argument");
  p->row_split = enable != 0;
  return AF_OK;
}

af_status af_plan_set_overlap_refresh(af_plan* p, int enable) {
  if (!p) return fail(AF_ERR_ARG, "NULL argument");
  p->overlap_refresh = enable != 0;
  return AF_OK;
}

af_status af_plan_set_block_done(af_plan* p, af_block_done_fn fn, void* user) {
  if (!p) return fail(AF_ERR_ARG, "NULL argument");
  p->done_fn = fn;
  p->done_user = fn ? user : nullptr;
  return AF_OK;
}

af_status af_plan_set_graphs(af_plan* p, int enable) {
  if (!p) return fail(AF_ERR_ARG, "NULL argument");
  p->graphs = enable != 0;
  return AF_OK;
}

af_status af_plan_graph_stats(const af_plan* p, long long* captures, long long* replays) {
  if (!p || !captures || !replays) return fail(AF_ERR_ARG, "NULL argument");
  *captures = p->g_captures;
  *replays = p->g_replays;
  return AF_OK;
}

size_t afk_affine_partials_bytes(int N, int rows_per_sample, int C) {
  if (N < 1 || rows_per_sample < 1 || C < 1) return 0;
  return (size_t)N * af::affine_groups(N, rows_per_sample, C) * 2 * sizeof(float) + 256;
}

af_status afk_affine(int mode, const float* head, const float* src, float* dst,
                     int N, int rows_per_sample, int C, float* res, void* partials,
                     size_t partials_bytes, int check, void* stream) {
  if (mode != 0 && mode != 1) return fail(AF_ERR_ARG, "mode must be 0 or 1");
  if (!head || !src || !dst || !res || !partials) return fail(AF_ERR_ARG, "NULL argument");
  if (src == dst) return fail(AF_ERR_ARG, "src and dst may not alias");
  if (N < 1 || rows_per_sample < 1 || C < 1 || C > 256) return fail(AF_ERR_ARG, "bad sizes");
  const size_t need = afk_affine_partials_bytes(N, rows_per_sample, C);
  if (partials_bytes < need) return fail(AF_ERR_WORKSPACE, "partials too small");
  hipStream_t st = (hipStream_t)stream;
  char* pb = (char*)partials;
  unsigned* counter = (unsigned*)(pb + need - 256);
  AF_HIP(af::launch_fill_u32(counter, 0u, 1, st));
  af::AffineArgs aa{head, nullptr, 1, mode == 0 ? src : nullptr,
                    mode == 0 ? dst : const_cast<float*>(src),
                    mode == 1 ? dst : nullptr, N, rows_per_sample, C,
                    rows_per_sample, 0, 0, (float*)pb, res, counter, nullptr};
  hipError_t e = af::launch_affine(mode, aa, st);
  if (e != hipSuccess) return fail(AF_ERR_HIP, hipGetErrorString(e));
  if (check) {
    AF_HIP(hipStreamSynchronize(st));
    std::vector<float> h((size_t)N * 2);
    AF_HIP(hipMemcpy(h.data(), res, h.size() * sizeof(float), hipMemcpyDeviceToHost));
    for (int n = 0; n < N; ++n) {
      if (!std::isfinite(h[2 * n]) || !std::isfinite(h[2 * n + 1]) ||
          (mode == 1 && h[2 * n + 1] != 0.f))
        return fail(AF_ERR_NONFINITE, "non-finite value in sample " + std::to_string(n));
    }
  }
  return AF_OK;
}

size_t afk_attention_workspace_bytes(int N, int R, int H, int dh, int pos_base) {
  if (N < 1 || R < 1 || H < 1 || pos_base < 0 || (dh != 32 && dh != 64 && dh != 128))
    return 0;
  const size_t part = af::attention_partial_floats(N, R, H, dh, pos_base) * sizeof(float);
  const size_t tick = af::attention_tickets(N, R, H) * sizeof(unsigned);
  return ((part + 255) / 256) * 256 + ((tick + 255) / 256) * 256;
}

af_status afk_attention(const void* q, const void* kc, const void* vt, void* out, int N,
                        int R, int H, int dh, int Lcap, int pos_base, void* ws,
                        size_t ws_bytes, void* stream) {
  if (!q || !kc || !vt || !out || !ws) return fail(AF_ERR_ARG, "NULL argument");
  if (any_misaligned(q, kc, vt, out, ws)) return fail(AF_ERR_ARG, "pointers must be 16-byte aligned");
  if (N < 1 || R < 1 || H < 1 || pos_base < 0) return fail(AF_ERR_ARG, "bad sizes");
  if (dh != 32 && dh != 64 && dh != 128) return fail(AF_ERR_UNSUPPORTED, "dh must be 32, 64 or 128");
  if (Lcap < 64 || Lcap % 64 != 0 || (long)pos_base + R > Lcap)
    return fail(AF_ERR_ARG, "need Lcap % 64 == 0 and pos_base + R <= Lcap");
  if ((long)H * dh > (1 << 16)) return fail(AF_ERR_UNSUPPORTED, "H * dh too large");
  const size_t need = afk_attention_workspace_bytes(N, R, H, dh, pos_base);
  if (ws_bytes < need) return fail(AF_ERR_WORKSPACE, "workspace too small");
  hipStream_t st = (hipStream_t)stream;
  const size_t part = af::attention_partial_floats(N, R, H, dh, pos_base) * sizeof(float);
  unsigned* tickets = (unsigned*)((char*)ws + ((part + 255) / 256) * 256);
  AF_HIP(af::launch_fill_u32(tickets, 0u, af::attention_tickets(N, R, H), st));
  hipError_t e = af::launch_attention(true, q, kc, vt, out, (float*)ws, tickets, N, R, H, dh,
                                      H * dh, Lcap, pos_base, st);
  if (e != hipSuccess) return fail(AF_ERR_HIP, hipGetErrorString(e));
  return AF_OK;
}

af_status afk_stream_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (bytes == 0) return AF_OK;
  if (!src || !dst) return fail(AF_ERR_ARG, "NULL argument");
  if (bytes % 16 != 0) return fail(AF_ERR_ARG, "bytes must be a multiple of 16");
  if (any_misaligned(src, dst)) return fail(AF_ERR_ARG, "src and dst must be 16-byte aligned");
  const char* s = (const char*)src;
  char* d = (char*)dst;
  if (s < d + bytes && d < s + bytes) return fail(AF_ERR_ARG, "src and dst overlap");
  hipError_t e = af::launch_stream_copy(src, dst, bytes, (hipStream_t)stream);
  if (e != hipSuccess) return fail(AF_ERR_HIP, hipGetErrorString(e));
  return AF_OK;
}

af_status afk_gemm_bf16(const void* a, const void* w, const float* bias, float* y,
                        int M, int N, int K, void* stream) {
  if (!a || !w || !y) return fail(AF_ERR_ARG, "NULL argument");
  if (M < 1 || N < 64 || K < 64 || N % 64 || K % 64)
    return fail(AF_ERR_ARG, "need M >= 1, N % 64 == 0, K % 64 == 0");
  if ((uint64_t)std::max(M, N) * K * 2 >= (1ull << 32))
    return fail(AF_ERR_UNSUPPORTED, "a or w above 4 GiB");
  hipError_t e = af::launch_gemm_f32out(true, a, w, bias, y, M, N, K, (hipStream_t)stream);
  if (e != hipSuccess) return fail(AF_ERR_HIP, hipGetErrorString(e));
  return AF_OK;
}

}  // extern "C"
