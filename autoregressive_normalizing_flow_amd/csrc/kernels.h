// Internal launchers of the AF-block kernels.  Every launcher validates
// nothing (the runtime does) and returns the launch's hipError_t.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace af {

// ---- token-side kernels ----------------------------------------------------
// h[m, :] = shift(x)[m] W_in^T + b_in + pos[pos_base + t] for the chunk rows
// m = n*R + t (processing index i = s + t); the shifted input of processing
// index i is token i-1 of the same sample, or x_last[n] (zeros if NULL) at i=0.
hipError_t launch_embed(const float* x, const float* x_last, const float* w_in,
                        const float* b_in, const float* pos, float* h, int N,
                        int R, int C, int d, int L, int s, int dir, int pos_base,
                        hipStream_t st);

// out = LayerNorm(h) * g + b over rows of width d (eps 1e-5); out is bf16 when
// out_bf16, else fp32.  With out_lo (bf16 only) the value is also split as
// out + out_lo, both bf16, for the higher-precision forward.
hipError_t launch_layernorm(const float* h, const float* g, const float* b,
                            void* out, bool out_bf16, int M, int d, hipStream_t st,
                            void* out_lo = nullptr);

// h += bias + sum of S split-K planes (slab [S][M][d]); out = LayerNorm(h)
// (bf16 with optional lo half, or fp32).
hipError_t launch_resid_ln(const float* slab, int S, const float* bias, float* h,
                           const float* g, const float* b, void* out, bool out_bf16,
                           void* out_lo, int M, int d, hipStream_t st);

// x^(0) of a Jacobi block: mode 0 zeros, 1 copy of x_init, 2 previous frame.
hipError_t launch_init_block(float* x, const float* x_init, int mode, int N,
                             int R, int C, int L, int s, int dir, int F,
                             hipStream_t st);

hipError_t launch_fill_u32(void* p, uint32_t v, size_t n, hipStream_t st);

struct AffineArgs {
  const float* head;   // head_splits planes of [N*R, 2C]: partial [mu | raw] per row
  const float* head_bias;  // [2C] added to the plane sum, or NULL
  int head_splits;
  const float* z;      // inverse: z tokens [N, L, C]
  float* x;            // inverse: x tokens, updated in place; forward: x tokens (read)
  float* zout;         // forward: z tokens (written)
  int N, R, C, L, s, dir;
  float* partials;     // [N][G][2]
  float* res;          // [N][2]
  unsigned* counter;   // zero before the first launch; the kernel leaves it zero
  float* logdet;       // forward: logdet[n] += -sum log sigma (may be NULL)
  unsigned* bad;       // set to `tag` (if still 0) when a residual sum (inverse) is
  unsigned tag;        // not finite or a z (forward) is not finite; may be NULL
  float* res_host;     // inverse: host-mapped copy of res written at the end, or NULL
  unsigned* seq_dev;   // inverse: device counter of finished updates, or NULL
  unsigned* seq_host;  // inverse: host-mapped word that receives the counter after
                       // res_host is written (the host polls it), or NULL
  unsigned* bad_host;  // inverse: host-mapped word that receives the sticky `bad`
                       // value when this update finds a non-finite sum, or NULL
  int ld_group;        // forward: sample nn adds into logdet[nn / ld_group] (0 or 1:
                       // one entry per sample)
};
// mode 0: inverse update + residual sums; mode 1: forward + log-sigma sums.
hipError_t launch_affine(int mode, const AffineArgs& a, hipStream_t st);
int affine_groups(int N, int R, int C);   // G, the partial slots per sample

// dst[0, bytes) = src[0, bytes) with the streaming form the affine kernel's
// large ranges use (16-byte aligned, bytes % 16 == 0, no overlap).
hipError_t launch_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t st);

// Head GEMM on the fp32 matrix cores: planes[s] = hf W^T over the s-th of
// `splits` equal K ranges, planes [splits][M][2C] as launch_affine reads them.
// Output row m reads hf row (m / r_out) * r_in + off + m % r_out (r_out =
// r_in = M, off = 0: row m), so a pass may cover more rows per sample than
// the head.  Needs head_mfma_supported(C, d) and d % (64 * splits) == 0.
bool head_mfma_supported(int C, int d);
int head_mfma_splits(int M, int d);
hipError_t launch_head_mfma(const float* hf, const float* w, float* planes, int M, int C,
                            int d, int splits, hipStream_t st, int r_out, int r_in, int off);

// ---- GEMMs: y[M, N] = A[M, K] W[N, K]^T + bias -----------------------------
// The bf16 kernels take an optional second activation operand A_lo: with it
// the activations are the bf16 pair A + A_lo (the higher-precision forward),
// and the QKV / GELU epilogues then also write the lo halves of their outputs.
struct QKVDst {
  void* q;        // [M, d]
  void* kc;       // K cache of this layer  [Nb][H][Lcap][dh]
  void* vt;       // V cache (transposed)   [Nb][H][dh][Lcap]
  int R, d, dh, H, Lcap, pos_base;
  void* q_lo;     // lo halves (split mode) or NULL
  void* kc_lo;
  void* vt_lo;
};
// Timing of one bf16 GEMM kernel (profiling only): after set_gemm_events(a, b)
// the next bf16 GEMM launch of this thread records a at the kernel's start and
// b at its end (hipExtLaunchKernelGGL) and clears the pair; gemm_events_pending()
// tells whether it is still unused.
void set_gemm_events(hipEvent_t start, hipEvent_t stop);
bool gemm_events_pending();
// The bf16 path stores Q times log2(e) / sqrt(dh), the base-2 softmax units
// the bf16 attention takes (scaled in fp32 before the one rounding to bf16).
hipError_t launch_gemm_qkv(bool bf16, const void* A, const void* A_lo, const void* W,
                           const float* bias, int M, int N, int K, QKVDst dst,
                           hipStream_t st);
// h += A W^T + bias.  With a non-NULL slab ([S][M][N] fp32, S =
// gemm_resid_splits(M, N, K)) the bf16 path splits K and reduces the partial
// planes in a fixed order in a second kernel.
hipError_t launch_gemm_resid(bool bf16, const void* A, const void* A_lo, const void* W,
                             const float* bias, float* h, int M, int N, int K,
                             float* slab, hipStream_t st);
int gemm_resid_splits(int M, int N, int K);
// The residual GEMMs of the bf16 path write fp32 partial planes only
// (slab [S][M][N], S = the returned split count); launch_resid_ln finishes them.
// At most max_splits planes (a power of two; never more than
// gemm_resid_splits(M, N, K)).
hipError_t launch_gemm_partial(const void* A, const void* A_lo, const void* W,
                               float* slab, int M, int N, int K, int* splits,
                               hipStream_t st, int max_splits = 8);
hipError_t launch_gemm_gelu(bool bf16, const void* A, const void* A_lo, const void* W,
                            const float* bias, void* out, void* out_lo, int M, int N,
                            int K, hipStream_t st);
hipError_t launch_gemm_f32out(bool bf16, const void* A, const void* W,
                              const float* bias, float* out, int M, int N, int K,
                              hipStream_t st);
// fp32 GEMM split over K into `splits` partial planes out[s][M][N] (no bias);
// head_splits(M, N, K) picks the split count.
hipError_t launch_gemm_f32_planes(const float* A, const float* W, float* out, int M,
                                  int N, int K, int splits, hipStream_t st);
int head_splits(int M, int N, int K);

// ---- attention ---------------------------------------------------------------
// out[m, h*dh:(h+1)*dh] = softmax(q k^T / sqrt(dh)) v over cached keys
// 0..pos_base+t (inclusive) for chunk row m = n*R + t.
// bf16: q comes from launch_gemm_qkv already times log2(e) / sqrt(dh), so
// the softmax is 2^(q k^T) normalised; long key ranges are split into chunks
// whose partial results go to `part` (attention_partial_floats(...) floats),
// and the last chunk of a query tile to finish merges them.  `tickets` holds
// attention_tickets(N, R, H) words that must be zero before the first launch;
// every launch leaves them zero again.
struct AttnSplit {   // lo halves of the split (higher-precision) mode
  const void* q_lo;
  const void* kc_lo;
  const void* vt_lo;
  void* out_lo;
};
hipError_t launch_attention(bool bf16, const void* q, const void* kc,
                            const void* vt, void* out, float* part, unsigned* tickets,
                            int N, int R, int H, int dh, int d, int Lcap, int pos_base,
                            hipStream_t st, const AttnSplit* split = nullptr);
size_t attention_partial_floats(int N, int R, int H, int dh, int pos_base);
inline size_t attention_tickets(int N, int R, int H) {
  return (size_t)N * H * ((R + 127) / 128);
}

// ---- the Jacobi loop on the device (small fp32 blocks) -----------------------
constexpr int kLoopMaxLayers = 8;
struct LoopLayer {
  const float *ln1_g, *ln1_b, *w_qkv, *b_qkv, *w_o, *b_o, *ln2_g, *ln2_b, *w_1, *b_1, *w_2, *b_2;
};
struct LoopArgs {
  const float *w_in, *b_in, *pos, *ln_f_g, *ln_f_b, *w_head, *b_head;
  LoopLayer layers[kLoopMaxLayers];
  float* kc[kLoopMaxLayers];   // K cache of each layer  [N][H][Lcap][dh]
  float* vt[kLoopMaxLayers];   // V cache (transposed)   [N][H][dh][Lcap]
  int n_layers, C, d, H, dh, dmlp, Lcap;
  const float* z;        // [N, L, C]
  float* x;              // [N, L, C] written block by block
  const float* x_init;   // init 1 (given); with refresh, the final tokens
  int refresh;           // 1: only recompute the cache rows of x_init's tokens
  int lds_max;           // LDS bytes one workgroup may take (sets the MLP chunk)
  const float* x_last;   // the token before the sequence, [N, C], or NULL (zeros)
  int N, L, B, P, dir, init, F, max_iters;
  float tau;             // <= 0: exactly min(max_iters, block) updates
  int* iters_host;       // host-mapped: the block counts of this stack block
  float* res_host;       // host-mapped: the last update's residual pairs [N][2]
  unsigned* bad_host;    // host-mapped: 1 + the block that met a non-finite sum
};
// Rows N x min(B, L) <= 64, d 64 or 128, d_h 32 or 64, C % 4 == 0, C <= 64,
// d_mlp % 64 == 0, at most kLoopMaxLayers layers, the block's state within
// lds_max bytes of LDS.
bool jacobi_loop_supported(int N, int Bc, int C, int d, int H, int dmlp, int n_layers,
                           int Lcap, int lds_max);
// One workgroup runs the whole Jacobi inverse of one AF block (every block of
// the sequence, the stop tests and the cache refreshes), or with a.refresh the
// cache rows of given tokens in blocks of B rows, by the same pass as the
// refresh after an early stop.
hipError_t launch_jacobi_loop(const LoopArgs& a, hipStream_t st);

// Record a failure for af_last_error() from another translation unit
// (defined with the ABI in runtime.cpp); a HIP failure also clears the
// runtime's last-error state.  Returns status.
int record_error(int status, const char* msg);

}  // namespace af
