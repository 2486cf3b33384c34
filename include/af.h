/*
 * af.h - C ABI of the affine autoregressive-flow (AF) block on AMD MI355X (gfx950).
 *
 * The method (STARFlow-V notes, papernotes.org, "STARFlow-V: End-to-End Video
 * Generative Modeling with Autoregressive Normalizing Flows"):
 *   - 关键设计 1, affine AF equation: z = (x - mu(x*m)) / sigma(x*m), sigma > 0,
 *     m the self-exclusive causal mask; blocks alternate L->R / R->L masks.
 *   - 损失函数, L_NF: the forward map's log|det J| = -sum log sigma.
 *   - 关键设计 3, Jacobi fixed-point equation: x^(k+1) = mu(x^(k)*m) +
 *     sigma(x^(k)*m) * z, stopped when ||x^(k+1)-x^(k)||^2/||x^(k+1)||^2 < tau;
 *     blocks of B tokens in sequence, tokens of a block in parallel, finished
 *     blocks feed a KV cache, a new frame warm-starts from the previous one.
 *   - 一个完整示例, I2V: observed tokens are forward-encoded into the KV cache.
 *
 * Network (one AF block): tokens are shifted by one (row t sees x[t-1], row 0
 * sees the token before the sequence or zeros), projected by W_in (d x C) plus
 * b_in plus a learned position row, run through n_layers pre-LN Transformer
 * layers (LayerNorm eps 1e-5, causal attention with scale 1/sqrt(d/n_heads),
 * exact-erf GELU MLP of width 4d), a final LayerNorm and a head W_head (2C x d)
 * whose outputs are [mu (C) | raw (C)]; log sigma = 0.5 * tanh(raw).
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers owned by the caller, row-major and
 *     contiguous.  x, z, x_init, x_last, logdet are fp32.  Token tensors are
 *     [N, L, C] (sample, token, channel).  The library allocates no device
 *     memory: all scratch lives in the caller's workspace.
 *   - Calls return a status and never abort; no exception crosses the ABI.
 *     Arguments are validated before any device work.  af_last_error() gives
 *     a thread-local detail string for the last failure.
 *   - `stream` is a hipStream_t (NULL = the default stream).  af_forward and
 *     af_prefill are stream-ordered and return without waiting.
 *     af_inverse_jacobi blocks: the affine kernel writes each update's
 *     residual (and a sticky non-finite tag) into pinned host memory of the
 *     plan for the stop test, and the call returns once the last update has
 *     published them, so iters and the status are final; x is stream-ordered
 *     (kernels the call enqueued may still be running when it returns).
 */
#ifndef AF_H
#define AF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AF_ABI_VERSION 3

typedef enum {
  AF_OK = 0,
  AF_ERR_ARG = 1,          /* a bad argument: null pointer, size out of range, bad enum */
  AF_ERR_HIP = 2,          /* a HIP runtime call failed (detail in af_last_error) */
  AF_ERR_WORKSPACE = 3,    /* ws_bytes below what the call needs */
  AF_ERR_NONFINITE = 4,    /* an update produced a non-finite x (output unspecified) */
  AF_ERR_UNSUPPORTED = 5   /* a valid request this build does not implement */
} af_status;

/* Operand type of the four per-layer matrices (w_qkv, w_o, w_1, w_2) and of
 * the activations fed to them and the KV cache.  Every other tensor is fp32. */
typedef enum { AF_F32 = 0, AF_BF16 = 1 } af_dtype;

/* Initial iterate x^(0) of each Jacobi block [s, e):
 *   ZERO        zeros
 *   GIVEN       x_init[:, s:e]  (x_init is [N, L, C])
 *   PREV_FRAME  the already-solved x[:, s-F:e-F] if s >= F, else zeros */
typedef enum { AF_INIT_ZERO = 0, AF_INIT_GIVEN = 1, AF_INIT_PREV_FRAME = 2 } af_init;

typedef struct {
  int C;          /* channels per token, 1..256 */
  int d;          /* model width: 64 times a power of two; AF_BF16 needs d % 256 == 0,
                     and batch x rows x 4d x 2 bytes below 4 GiB per call */
  int n_heads;    /* d / n_heads in {32, 64, 128} */
  int n_layers;   /* >= 1; MLP width is 4d */
  int max_len;    /* positions 0..max_len-1 (rows of the position table) */
  af_dtype dtype;
} af_block_cfg;

/* One block's parameters: borrowed device pointers that must outlive the plan
 * and be 16-byte aligned (the kernels read them as 16-byte vectors;
 * af_plan_create returns AF_ERR_ARG otherwise).  Token buffers passed to the
 * calls below (x, z, x_prefix, x_init, x_last) must be 16-byte aligned too.
 * Matrices are row-major [out, in] (y = x W^T + b).  The four per-layer
 * matrices have the element type of cfg.dtype (fp32 or bf16 bit patterns);
 * everything else is fp32.  The per-layer fields are HOST arrays of
 * n_layers device pointers (copied at plan creation).
 *   w_in [d, C]  b_in [d]  pos [max_len, d]
 *   per layer: ln1_g, ln1_b [d]; w_qkv [3d, d] rows [Q | K | V], heads
 *   contiguous inside each; b_qkv [3d]; w_o [d, d]; b_o [d]; ln2_g, ln2_b [d];
 *   w_1 [4d, d]; b_1 [4d]; w_2 [d, 4d]; b_2 [d]
 *   ln_f_g, ln_f_b [d]  w_head [2C, d]  b_head [2C]  */
typedef struct {
  const float *w_in, *b_in, *pos;
  const float *ln_f_g, *ln_f_b, *w_head, *b_head;
  const float *const *ln1_g, *const *ln1_b;
  const void *const *w_qkv;
  const float *const *b_qkv;
  const void *const *w_o;
  const float *const *b_o;
  const float *const *ln2_g, *const *ln2_b;
  const void *const *w_1;
  const float *const *b_1;
  const void *const *w_2;
  const float *const *b_2;
} af_block_weights;

typedef struct af_plan af_plan;

/* Create a plan for a stack of n_blocks AF blocks sharing one shape.  Block t
 * runs left-to-right when t is even and right-to-left when t is odd (STARFlow-V
 * notes, 整体框架 and 关键设计 1: alternating mask directions); a deep block is
 * a stack of one.  w points to n_blocks weight sets.  The plan keeps host
 * metadata only.  Returns AF_ERR_ARG / AF_ERR_UNSUPPORTED for shapes outside
 * the documented ranges. */
af_status af_plan_create(const af_block_cfg *cfg, int n_blocks,
                         const af_block_weights *w, af_plan **out);
/* Release the plan's streams, events, graphs and pinned memory.  Work that a
 * call left queued (see af_inverse_jacobi) may still use them, so this first
 * waits for the current device to finish all outstanding work. */
void af_plan_destroy(af_plan *p);

/* Workspace bytes for `batch` samples when at most `rows` tokens per sample
 * are processed in one pass (L for af_forward, P for af_prefill, B for
 * af_inverse_jacobi).  The first af_cache_bytes(p, batch) bytes hold the KV
 * cache (positions 0..max_len-1 of every layer), so a workspace keeps its
 * cache across calls made with the same batch.  Returns 0 on bad arguments. */
size_t af_workspace_bytes(const af_plan *p, int batch, int rows);
size_t af_cache_bytes(const af_plan *p, int batch);

/* Forward pass of the whole stack (blocks t = 0..n_blocks-1):
 * z = f(x) and the log-determinant log|det dz/dx| = -sum over blocks, tokens
 * and channels of log sigma (STARFlow-V notes, 关键设计 1 and 损失函数).
 * x, z: [N, L, C] (may not alias).  Needs L <= max_len and
 * ws_bytes >= af_workspace_bytes(p, N, L).  For a single block the KV cache
 * of positions 0..L-1 is left in ws.
 *   frames_per_entry G >= 1, dividing N: the N inputs are N / G sequences of
 *     G consecutive frames each, and logdet has N / G entries; entry j receives
 *     the log-dets of samples jG..jG+G-1, added in sample order.  G = 1 gives
 *     one entry per sample.  With G > 1 a shallow stack run over every frame
 *     of a sequence yields the per-sequence sum of its frames' Jacobian
 *     factors (关键设计 1: the deep-shallow likelihood factorises into the deep
 *     term and one shallow factor per frame).
 *   flags: AF_FWD_ACCUMULATE adds into logdet (which then holds the other
 *     factors, e.g. the shallow stack's sum before the deep block's forward);
 *     without it logdet is overwritten.  AF_FWD_CHECK_FINITE makes the call
 *     wait for its kernels and return AF_ERR_NONFINITE if any z (or log-det
 *     term) is not finite; without it the call is stream-ordered and does not
 *     wait, and z then holds the non-finite values unflagged. */
#define AF_FWD_ACCUMULATE 1
#define AF_FWD_CHECK_FINITE 2
af_status af_forward(af_plan *p, const float *x, float *z, float *logdet,
                     int N, int L, int frames_per_entry, int flags,
                     void *ws, size_t ws_bytes, void *stream);

/* Encode observed tokens into the KV cache (STARFlow-V notes, 一个完整示例:
 * I2V / V2V conditioning): runs the single block's network on the shifted
 * x_prefix [N, P, C] at positions 0..P-1 and leaves every layer's K/V in ws.
 * A following af_inverse_jacobi with prefix_len = P and the same ws continues
 * at position P.  Only for n_blocks == 1.  Stream-ordered. */
af_status af_prefill(af_plan *p, const float *x_prefix, int N, int P,
                     void *ws, size_t ws_bytes, void *stream);

/* Recompute the K/V cache rows of positions P..P+L-1 from their final tokens
 * x [N, L, C] (STARFlow-V notes, 关键设计 3: the state of a finished block
 * feeds the cache of the blocks after it; 一个完整示例, streaming: the last
 * overlap latents are re-run through the deep block to rebuild the cache).
 * Positions 0..P-1 must already be in ws; x_last [N, C] is the token at
 * position P-1 (required when P > 0, NULL for zeros when P == 0).  With
 * P == 0 this is af_prefill.  Only for n_blocks == 1.  Needs P + L <= max_len
 * and ws_bytes >= af_workspace_bytes(p, N, L).  Where af_inverse_jacobi runs
 * on the device loop (af_plan_set_device_loop), so does this call, with the
 * pass that refreshes a block after an early stop, so rows refreshed here
 * equal the ones a single call over the longer sequence leaves, bit for bit.
 * Stream-ordered. */
af_status af_refresh_kv(af_plan *p, const float *x, int N, int L, int prefix_len,
                        const float *x_last, void *ws, size_t ws_bytes, void *stream);

/* Invert the stack by video-aware block-wise Jacobi (STARFlow-V notes, 关键设计
 * 3).  Blocks t = n_blocks-1..0 in turn; inside each, Jacobi blocks
 * [s, e) = [b*B, min(L, (b+1)*B)) in sequence.  A Jacobi block repeats
 *   x^(k) = mu(shift(x[:s] ++ x^(k-1))) + exp(0.5 tanh raw(...)) * z[:, s:e]
 * from x^(0) (see af_init) and stops after the first update whose residual
 * r_n = sum (x^(k)-x^(k-1))^2 / sum (x^(k))^2 (per sample n, over the block's
 * tokens and channels; 0/0 = 0) is below tau for every sample, or after
 * min(max_iters, e-s) updates (max_iters <= 0 means e-s).  tau <= 0 forces
 * that many updates.  The finished block's K/V are then recomputed from its
 * final x and kept in the cache (skipped when the block ran e-s updates, as
 * its last inputs were already final, and for the call's last Jacobi block,
 * which nothing in the call reads: a later call that continues after it
 * refreshes those rows with af_refresh_kv; its layer-0 rows may already hold
 * the K/V of its final tokens).
 *   z        [N, L, C]   input
 *   x        [N, L, C]   output (may not alias z)
 *   x_init   [N, L, C]   AF_INIT_GIVEN only, else may be NULL
 *   frame_len F > 0      AF_INIT_PREV_FRAME only
 *   prefix_len P >= 0    positions already in the cache (af_prefill); the new
 *                        tokens take positions P..P+L-1; P + L <= max_len
 *   x_last   [N, C]      the token at position P-1 (shifted input of position
 *                        P); required when P > 0, NULL for zeros when P == 0
 *   iters    HOST int32 [n_blocks][ceil(L/B)]: updates made per Jacobi block,
 *                        row t for stack block t
 * For n_blocks > 1 only AF_INIT_ZERO and P == 0 are supported.  Needs
 * ws_bytes >= af_workspace_bytes(p, N, min(B, L)).  With
 * af_plan_set_fused_refresh(p, 1) and ws_bytes >= af_workspace_bytes(p, N,
 * min(2B, L)) the recomputation of a block's K/V runs in the same network pass
 * as the next block's first update, over the rows of both blocks (the update
 * covers the new block's rows only); results equal those of the separate pass
 * up to floating-point summation order.  Returns AF_ERR_NONFINITE if an update
 * produced a non-finite value. */
af_status af_inverse_jacobi(af_plan *p, const float *z, int N, int L, int B,
                            float tau, int max_iters, af_init init,
                            const float *x_init, int frame_len, int prefix_len,
                            const float *x_last, float *x, int32_t *iters,
                            void *ws, size_t ws_bytes, void *stream);

/* ---- per-kernel timing (measurement only) --------------------------------
 * While enabled, every launch of the named kernel class made by this plan is
 * bracketed by HIP events on the launch stream; af_profile_read synchronises
 * on those events and returns the number of launches and their summed
 * duration in milliseconds since the last enable, and (work may be NULL) the
 * summed algorithmic work of those launches: flops (2 per multiply-add) for
 * "embed", the GEMM classes and "attention" (4 d flops per unmasked (query,
 * key) pair, STARFlow-V notes 关键设计 3: the queries of a block attend to the
 * cached keys up to their own position), bytes for "affine" (20 C per token
 * in an inverse update, 16 C in the forward), 0 for "layernorm".  Classes:
 * "embed", "layernorm", "gemm_qkv", "gemm_o", "gemm_mlp1", "gemm_mlp2",
 * "gemm_head", "attention", "affine", "device_loop" (one launch per AF block
 * of an inverse on the device loop, its work the flops of its updates and
 * refreshes).  At most 16384 launches are recorded per enable. */
af_status af_profile_enable(af_plan *p, const char *kernel_class);
af_status af_profile_disable(af_plan *p);
af_status af_profile_read(af_plan *p, int *launches, double *total_ms, double *work);

/* ---- graph replay of the Jacobi update (opt-in) ---------------------------
 * Every update of a Jacobi block (关键设计 3) runs the same launch sequence on
 * the same buffers.  With graphs enabled, af_inverse_jacobi captures it once
 * into a HIP graph (on a private stream of the plan, where nothing runs) and
 * replays that graph on `stream` once per iteration, which takes the per-kernel
 * launch work off the host thread.  Off by default: where every kernel runs for
 * several microseconds the host already launches ahead of the device, and
 * direct launches measured no slower.  Graphs are cached in the plan (at most 128,
 * least recently used dropped) under every value they depend on: the stack
 * block, the z / x / x_last / workspace pointers, the device, N, L, the block
 * bounds and prefix_len; a later call with the same values replays without
 * capturing.  A block that may run a single update is launched directly
 * unless already cached, and so is every update while a kernel class is
 * profiled (af_profile_enable: the runtime gives no timing for events
 * recorded inside a graph).  Results are identical with and without graphs.
 * A plan must not be used by two calls at once.
 *   af_plan_set_graphs: enable != 0 turns graph replay on, 0 (the default)
 *     launches every kernel directly; AF_ERR_ARG if p is NULL.
 *   af_plan_graph_stats: graphs captured and graph launches made by this plan
 *     since it was created; AF_ERR_ARG on a NULL argument. */
af_status af_plan_set_graphs(af_plan *p, int enable);

/* Merge a Jacobi block's K/V recomputation into the next block's first update
 * when the workspace allows (see af_inverse_jacobi): enable != 0, or 0 (the
 * default) for a pass of its own, which stops after the last layer's K/V and
 * measured faster for full-frame blocks; AF_ERR_ARG if p is NULL. */
af_status af_plan_set_fused_refresh(af_plan *p, int enable);
af_status af_plan_graph_stats(const af_plan *p, long long *captures, long long *replays);

/* Row split of a Jacobi update (STARFlow-V notes, 关键设计 3: the update is
 * one parallel pass over the block's rows).  On the bf16 path, for blocks of
 * R >= 1024 rows with N * R <= 4096 and at least 8 R cached keys before the
 * block (prefix_len + block start >= 8 R: attention over the prefix then
 * dominates the update), af_inverse_jacobi runs each update
 * as two passes over the first and second half of the block's rows, on
 * `stream` and on a second stream of the plan, ordered by events (the second
 * half's attention waits for the first half's K/V of the same update).  The
 * two passes overlap where one leaves the GPU idle; the stop test adds their
 * residuals.  Results equal those of the single pass up to floating-point
 * summation order.  Used only with direct launches (not with graphs or the
 * fused refresh) and when ws_bytes >= af_workspace_bytes(p, N, min(B, L)),
 * which includes the second half's scratch whenever the shape allows a split.
 * The call returns (also on an error) with `stream` ordered after all of the
 * second stream's work.  Like the graph cache, the second stream and its
 * events belong to the plan: a plan must not be used by two calls at once.
 * enable != 0 allows the split, 0 (the default) keeps one pass: with the
 * 32 x 32 attention kernels one pass measured faster; AF_ERR_ARG if p is NULL. */
af_status af_plan_set_row_split(af_plan *p, int enable);

/* Cache refresh beside the next Jacobi block (STARFlow-V notes, 关键设计 3:
 * finished blocks feed the KV cache that later blocks attend to).  On the
 * bf16 path with at least two layers, when a block that is not the call's
 * last stops before e-s updates, its K/V recomputation (which continues from
 * the layer-0 results the next update's speculative first kernels already
 * computed from the final tokens) runs on a second stream of the plan, in
 * scratch of its own, while the next block's first update runs on `stream`;
 * that update's attention at layer l waits (an event) for the refresh's K/V
 * of layer l, and everything after it on `stream` is ordered after the
 * whole refresh.  The same kernels run on the same inputs, so results are
 * identical to the refresh on `stream`.  Used with direct launches, one pass
 * per update (not with graphs, the row split or the fused refresh) and when
 * ws_bytes >= af_workspace_bytes(p, N, min(B, L)), which includes that
 * scratch on the bf16 path.  The call returns (also on an error) with
 * `stream` ordered after all of the second stream's work; a plan must not be
 * used by two calls at once.  enable != 0 (the default) allows it, 0 runs
 * every refresh on `stream`; AF_ERR_ARG if p is NULL. */
af_status af_plan_set_overlap_refresh(af_plan *p, int enable);

/* Block-done notification (STARFlow-V notes, 关键设计 3: the shallow flow
 * inverts each frame as soon as the deep block has produced it).  While
 * af_inverse_jacobi runs, fn(user, t, b) is called on the calling thread once
 * per Jacobi block b of stack block t, right after the work that makes that
 * block's x final has been enqueued on `stream`: an event recorded on `stream`
 * inside fn completes when x[:, b*B : min(L, (b+1)*B)] of stack block t is
 * final (for t = 0, the call's output), so another stream can start on those
 * tokens while the call goes on.  On the device loop (af_plan_set_device_loop)
 * every Jacobi block of an AF block is reported right after that AF block's
 * launch.  A call is not a promise that the block succeeded: the call's
 * return status says so.  fn must not use the plan (it is inside a call) and
 * must return promptly.  fn = NULL (the default) turns it off; AF_ERR_ARG if
 * p is NULL. */
typedef void (*af_block_done_fn)(void *user, int stack_block, int jacobi_block);
af_status af_plan_set_block_done(af_plan *p, af_block_done_fn fn, void *user);

/* The Jacobi loop on the device (STARFlow-V notes, 关键设计 3: the update is
 * repeated until the residual falls below tau).  For fp32 plans whose block
 * fits one workgroup (N * min(B, L) <= 64 rows, d 64 or 128, d / n_heads 32
 * or 64, C % 4 == 0, C <= 64, d_mlp % 64 == 0, at most 8 layers, the block's
 * activations within the LDS one workgroup may take: 160 KB on gfx950) and no
 * graph replay, row split or fused refresh is asked for, af_inverse_jacobi
 * runs the whole inverse of each AF block of the stack as one launch: every
 * Jacobi block in order, every update, the stop test and the cache refresh
 * after an early stop happen on the device, with no host read-back per
 * update; the call waits for the stream once at the end and reads the block
 * counts, the last residual pairs and a non-finite flag from pinned memory.
 * Results and counts follow the same rules as the launch-per-kernel path (its
 * fp32 arithmetic differs only in summation order), and so does the KV cache
 * left in the workspace, but for the rows of the call's last Jacobi block,
 * which neither path refreshes (here every layer's rows hold the K/V of the
 * last update's inputs; af_refresh_kv, which takes the same route for the
 * same shapes, brings them up to date).  enable != 0 (the default) uses it
 * where the shape allows, 0 keeps the launch-per-kernel path; AF_ERR_ARG if p
 * is NULL. */
af_status af_plan_set_device_loop(af_plan *p, int enable);

/* ---- kernel-level entry points (unit parity and bandwidth measurement) ---
 * The fused affine kernel on its own, over N samples of rows_per_sample
 * contiguous rows of C channels (token tensors [N, rows_per_sample, C]).
 * head [N * rows_per_sample, 2C] holds [mu | raw] per row; ls = 0.5 tanh(raw).
 * mode 0 (inverse): src = z, dst = x updated in place:
 *   x <- mu + exp(ls) * z, res[n] = {sum (x_new - x_old)^2, sum x_new^2}.
 * mode 1 (forward): src = x, dst = z written:
 *   z <- (x - mu) * exp(-ls), res[n] = {-sum ls, number of non-finite z}.
 * res is [N][2] fp32 device; partials is device scratch of at least
 * afk_affine_partials_bytes(N, rows_per_sample, C) bytes.  Stream-ordered;
 * with check != 0 it synchronises and returns AF_ERR_NONFINITE if a produced
 * value is not finite. */
size_t afk_affine_partials_bytes(int N, int rows_per_sample, int C);
af_status afk_affine(int mode, const float *head, const float *src, float *dst,
                     int N, int rows_per_sample, int C, float *res,
                     void *partials, size_t partials_bytes, int check,
                     void *stream);

/* The fused affine kernel as afk_affine, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): its partial sums and ticket counter live in a
 * static device array of the library, one per GPU, of AF_NOALLOC_SCRATCH_BYTES
 * (the call needs afk_affine_partials_bytes(N, rows_per_sample, C) of it;
 * larger requests return AF_ERR_WORKSPACE).  The call allocates nothing
 * (no hipMalloc, no host buffer); its first call on a device looks the array
 * up.  Same arguments and results as afk_affine with check = 0; stream-ordered.
 * Calls that overlap on one GPU (two streams, or two threads) share the array
 * and race: order them. */
#define AF_NOALLOC_SCRATCH_BYTES (256 * 1024)
af_status afk_affine_noalloc(int mode, const float *head, const float *src, float *dst,
                             int N, int rows_per_sample, int C, float *res, void *stream);

/* Streaming device copy dst[0, bytes) = src[0, bytes): the bandwidth
 * reference the fused affine kernel is measured against (contiguous range per
 * workgroup, four 16-byte non-temporal loads in flight per thread).  src and
 * dst are device pointers, 16-byte aligned, not overlapping; bytes is a
 * multiple of 16 (0 is a no-op).  AF_ERR_ARG otherwise.  Stream-ordered. */
af_status afk_stream_copy(const void *src, void *dst, size_t bytes, void *stream);

/* One layer's bf16 causal attention over a KV cache (STARFlow-V notes,
 * 关键设计 3: the block's queries attend to every cached key up to their own
 * position), as the Jacobi path runs it, for unit parity at any shape:
 *   out[n, t, h*dh + e] = sum_j softmax_j(q_t . k_j / sqrt(dh)) v_j[e]
 * over keys j = 0 .. pos_base + t of head h.  Layouts (bf16 bit patterns,
 * device pointers):
 *   q    [N, R, H*dh]        holding Q * log2(e) / sqrt(dh), the QKV GEMM's
 *                            storage (the softmax is taken in base 2)
 *   kc   [N][H][Lcap][dh]    keys by position
 *   vt   [N][H][dh][Lcap]    values, transposed
 *   out  [N, R, H*dh]
 * dh is 32, 64 or 128; Lcap % 64 == 0 and pos_base + R <= Lcap; cache rows at
 * or past pos_base + R are not read into the result.  ws is device scratch of
 * afk_attention_workspace_bytes(N, R, H, dh, pos_base) bytes (key-chunk
 * partials and merge tickets, cleared by the call).  Every pointer 16-byte
 * aligned; AF_ERR_ARG / AF_ERR_WORKSPACE otherwise.  Stream-ordered. */
size_t afk_attention_workspace_bytes(int N, int R, int H, int dh, int pos_base);
af_status afk_attention(const void *q, const void *kc, const void *vt, void *out,
                        int N, int R, int H, int dh, int Lcap, int pos_base,
                        void *ws, size_t ws_bytes, void *stream);

/* bf16 MFMA GEMM y[M, N] = a[M, K] * w[N, K]^T + bias[N] (bias may be NULL),
 * fp32 out, for unit parity.  a, w are bf16 bit patterns, row-major;
 * K % 64 == 0, N % 64 == 0; a and w below 4 GiB each (AF_ERR_UNSUPPORTED
 * otherwise).  Stream-ordered. */
af_status afk_gemm_bf16(const void *a, const void *w, const float *bias,
                        float *y, int M, int N, int K, void *stream);

/* Residual of the last Jacobi update made by the last af_inverse_jacobi call
 * of this plan that returned AF_OK or AF_ERR_NONFINITE (STARFlow-V notes,
 * 关键设计 3, residual stop): num_den[2n] = sum (x^(k) - x^(k-1))^2 and
 * num_den[2n+1] = sum (x^(k))^2 of sample n over that Jacobi block, as the
 * stop test used them (a row-split update adds its two halves).  num_den is a
 * HOST float array [N][2]; N must be the batch of that call.  AF_ERR_ARG on a
 * NULL argument, a different N, or before any inverse call. */
af_status af_plan_last_residual(const af_plan *p, int N, float *num_den);

const char *af_status_str(af_status s);
const char *af_last_error(void);
int af_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* AF_H */
