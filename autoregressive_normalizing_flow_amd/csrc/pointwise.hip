// Token-side kernels of the AF block: the masked shift + input embedding,
// LayerNorm, Jacobi-block initialisation and the fused affine kernel that
// applies the affine map, reduces log sigma (forward) or the Jacobi residual
// (inverse) per sample.
//
// Method: STARFlow-V notes (papernotes.org), 关键设计 1 (affine AF equation
// z = (x - mu(x*m)) / sigma(x*m) with the self-exclusive causal mask) and
// 关键设计 3 (Jacobi update x = mu + sigma * z and the scale-normalised
// residual ||x^(k+1) - x^(k)||^2 / ||x^(k+1)||^2).
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace af {

// ---------------------------------------------------------------------------
// shift + embed on the fp32 matrix cores.  Per 16-feature x 16-token tile,
// D = W_in . inp^T with v_mfma_f32_16x16x4f32: lane (i = l % 16, g = l / 16)
// feeds W_in row (feature) i and the shifted input of token i at the same k
// slot g, and receives features 4g..4g+3 of token i, so h is stored as float4s.
// The k order is permuted the same way in both operands (slot g of step
// 4t + e is channel 4g + 16t + e), so every lane loads whole float4s of W_in
// and of its token's input.  Block: 4 waves x 64 features, 16 tokens; all
// loads are issued before the first MFMA.
// CP = C rounded up within {16, 32, 48, 64}; C % 4 == 0, d % 64 == 0.  Other
// shapes go through embed_generic_kernel.
// ---------------------------------------------------------------------------
constexpr int EMB_ROWS = 16;    // tokens per block
constexpr int EMB_COLS = 256;   // features per block (64 per wave)

// Address and validity of shifted input element (m, c): token m's input is
// the previous token (in processing order) of its sample, x_last (or zero)
// for the first one.  Invalid elements read x[0] and are masked.
__device__ __forceinline__ const float* shifted_src(const float* __restrict__ x,
                                                   const float* __restrict__ x_last,
                                                   int m, int c, int M, int R, int C,
                                                   int L, int s, int dir, bool& valid) {
  const int mm = min(m, M - 1), cc = min(c, C - 1);
  const int n = mm / R, i = s + (mm - n * R);   // processing index
  const bool first = i == 0;
  valid = m < M && c < C && (!first || x_last != nullptr);
  if (!valid) return x;
  return first ? x_last + (size_t)n * C + cc
               : x + ((size_t)n * L + storage_index(max(i - 1, 0), L, dir)) * C + cc;
}

template <int CP>
__global__ __launch_bounds__(256) void embed_kernel(
    const float* __restrict__ x, const float* __restrict__ x_last,
    const float* __restrict__ w_in, const float* __restrict__ b_in,
    const float* __restrict__ pos, float* __restrict__ h, int N, int R, int C,
    int d, int L, int s, int dir, int pos_base) {
  constexpr int T = CP / 16;   // float4s per lane and operand row (4 k-steps each)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int f0 = blockIdx.x * EMB_COLS + wave * 64;   // first feature of the wave
  if (f0 >= d) return;                                // d % 64 == 0: whole waves
  const int M = N * R;
  const int m = blockIdx.y * EMB_ROWS + i;            // this lane's token

  // B operand: token m's shifted input, channels 4g + 16t .. +3 (zero past C
  // and for an invalid token)
  bool ok;
  const float* src = shifted_src(x, x_last, m, 0, M, R, C, L, s, dir, ok);
  float4 xb[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int c = 4 * g + 16 * t;
    const float4 v = *(const float4*)(src + min(c, C - 4));   // in bounds
    const bool use = ok && c < C;
    xb[t] = use ? v : float4{0.f, 0.f, 0.f, 0.f};
  }
  // A operand: W_in rows f0 + 16 ft + i, the same channels (zero past C)
  float4 wa[4][T];
#pragma unroll
  for (int ft = 0; ft < 4; ++ft) {
    const float* wr = w_in + (size_t)(f0 + 16 * ft + i) * C;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int c = 4 * g + 16 * t;
      const float4 v = *(const float4*)(wr + min(c, C - 4));
      wa[ft][t] = c < C ? v : float4{0.f, 0.f, 0.f, 0.f};
    }
  }
  // bias and position rows of the outputs this lane holds: token m,
  // features f0 + 16 ft + 4g .. +3
  const float* prow = pos + (size_t)(pos_base + min(m, M - 1) % R) * d;
  float4 add[4];
#pragma unroll
  for (int ft = 0; ft < 4; ++ft) {
    const int f = f0 + 16 * ft + 4 * g;
    const float4 bb = *(const float4*)(b_in + f), pp = *(const float4*)(prow + f);
    add[ft] = float4{bb.x + pp.x, bb.y + pp.y, bb.z + pp.z, bb.w + pp.w};
  }

#pragma unroll
  for (int ft = 0; ft < 4; ++ft) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < T; ++t) {
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wa[ft][t].x, xb[t].x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wa[ft][t].y, xb[t].y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wa[ft][t].z, xb[t].z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wa[ft][t].w, xb[t].w, acc, 0, 0, 0);
    }
    if (m < M)
      *(float4*)(h + (size_t)m * d + f0 + 16 * ft + 4 * g) =
          float4{acc[0] + add[ft].x, acc[1] + add[ft].y, acc[2] + add[ft].z, acc[3] + add[ft].w};
  }
}

__device__ __forceinline__ float shifted_input(const float* __restrict__ x,
                                               const float* __restrict__ x_last, int m,
                                               int c, int M, int R, int C, int L, int s,
                                               int dir) {
  bool ok;
  const float v = *shifted_src(x, x_last, m, c, M, R, C, L, s, dir, ok);
  return ok ? v : 0.f;
}

// Any C: one thread per output element, scalar loop (not on the hot path of
// the workloads; kept for generality).
__global__ __launch_bounds__(256) void embed_generic_kernel(
    const float* __restrict__ x, const float* __restrict__ x_last,
    const float* __restrict__ w_in, const float* __restrict__ b_in,
    const float* __restrict__ pos, float* __restrict__ h, int N, int R, int C,
    int d, int L, int s, int dir, int pos_base) {
  const int M = N * R;
  const size_t total = (size_t)M * d;
  for (size_t e = blockIdx.x * 256ull + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
    const int m = (int)(e / d), j = (int)(e - (size_t)m * d);
    float a = b_in[j];
    for (int c = 0; c < C; ++c)
      a += shifted_input(x, x_last, m, c, M, R, C, L, s, dir) * w_in[(size_t)j * C + c];
    h[e] = a + pos[(size_t)(pos_base + m % R) * d + j];
  }
}

hipError_t launch_embed(const float* x, const float* x_last, const float* w_in,
                        const float* b_in, const float* pos, float* h, int N,
                        int R, int C, int d, int L, int s, int dir, int pos_base,
                        hipStream_t st) {
  dim3 grid((d + EMB_COLS - 1) / EMB_COLS, (N * R + EMB_ROWS - 1) / EMB_ROWS);
#define AF_EMB(CP)                                                                    \
  hipLaunchKernelGGL(embed_kernel<CP>, grid, dim3(256), 0, st, x, x_last, w_in, b_in, \
                     pos, h, N, R, C, d, L, s, dir, pos_base)
  const bool mfma = C % 4 == 0 && d % 64 == 0;
  if (mfma && C <= 16) AF_EMB(16);
  else if (mfma && C <= 32) AF_EMB(32);
  else if (mfma && C <= 48) AF_EMB(48);
  else if (mfma && C <= 64) AF_EMB(64);
  else {
    const size_t total = (size_t)N * R * d;
    const int blocks = (int)std::min<size_t>((total + 255) / 256, 8192);
    hipLaunchKernelGGL(embed_generic_kernel, dim3(blocks), dim3(256), 0, st, x, x_last, w_in,
                       b_in, pos, h, N, R, C, d, L, s, dir, pos_base);
  }
#undef AF_EMB
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// LayerNorm: one wave per row, VPL = d / 64 values per lane kept in registers
// (two-pass mean / variance).
// ---------------------------------------------------------------------------
template <int VPL, class OutT>
__global__ __launch_bounds__(256) void layernorm_kernel(
    const float* __restrict__ h, const float* __restrict__ g,
    const float* __restrict__ b, OutT* __restrict__ out, OutT* __restrict__ out_lo,
    int M) {
  constexpr int D = VPL * AF_WAVE;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float* hr = h + (size_t)row * D;
  float v[VPL];
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    v[i] = hr[lane + AF_WAVE * i];
    sum += v[i];
  }
  const float mean = wave_sum(sum) * (1.0f / D);
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    float c = v[i] - mean;
    sq += c * c;
  }
  const float rstd = rsqrtf(wave_sum(sq) * (1.0f / D) + 1e-5f);
  OutT* orow = out + (size_t)row * D;
  OutT* lrow = out_lo ? out_lo + (size_t)row * D : nullptr;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    int j = lane + AF_WAVE * i;
    const float y = (v[i] - mean) * rstd * g[j] + b[j];
    const OutT hi = from_f32<OutT>(y);
    orow[j] = hi;
    if (lrow) lrow[j] = from_f32<OutT>(y - to_f32(hi));   // split: y = hi + lo
  }
}

// ---------------------------------------------------------------------------
// Residual add + LayerNorm, fused: one wave per row.
//   h[m] += bias + sum_s slab[s][m]          (split-K planes added in order)
//   out[m] = LayerNorm(h[m]) * g + b          (bf16, optional lo half; or fp32)
// It finishes the O-projection / MLP-down GEMMs and produces the next
// LayerNorm's output in the same pass over the row.
// ---------------------------------------------------------------------------
template <class OutT>
__device__ __forceinline__ void store4(OutT* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *(float4*)p = float4{a, b, c, d};
}
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, float a, float b, float c, float d) {
  bf16x4 v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
  *(bf16x4*)p = v;
}

// LayerNorm for d % 256 == 0: one wave per row, V4 = d / 256 float4s per lane;
// the row and the gain / shift vectors are loaded before the first use.
template <int V4, class OutT>
__global__ __launch_bounds__(256) void ln4_kernel(
    const float* __restrict__ h, const float* __restrict__ g, const float* __restrict__ b,
    OutT* __restrict__ out, int M) {
  constexpr int D = V4 * 256;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float* hr = h + (size_t)row * D;
  float4 v[V4], gg[V4], be[V4];
#pragma unroll
  for (int i = 0; i < V4; ++i) {
    const int j = 4 * lane + 256 * i;
    v[i] = *(const float4*)(hr + j);
    gg[i] = *(const float4*)(g + j);
    be[i] = *(const float4*)(b + j);
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < V4; ++i) sum += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  const float mean = wave_sum(sum) * (1.0f / D);
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < V4; ++i) {
    const float a0 = v[i].x - mean, a1 = v[i].y - mean, a2 = v[i].z - mean, a3 = v[i].w - mean;
    sq += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
  }
  const float rstd = rsqrtf(wave_sum(sq) * (1.0f / D) + 1e-5f);
#pragma unroll
  for (int i = 0; i < V4; ++i) {
    const int j = 4 * lane + 256 * i;
    store4<OutT>(out + (size_t)row * D + j, (v[i].x - mean) * rstd * gg[i].x + be[i].x,
                 (v[i].y - mean) * rstd * gg[i].y + be[i].y,
                 (v[i].z - mean) * rstd * gg[i].z + be[i].z,
                 (v[i].w - mean) * rstd * gg[i].w + be[i].w);
  }
}

template <class OutT>
static hipError_t ln_dispatch(const float* h, const float* g, const float* b,
                              OutT* out, OutT* out_lo, int M, int d, hipStream_t st) {
  dim3 grid((M + 3) / 4), blk(256);
  const bool lo = out_lo != nullptr;
  if (d % 256 == 0 && !lo) {
    switch (d / 256) {
      case 1: hipLaunchKernelGGL((ln4_kernel<1, OutT>), grid, blk, 0, st, h, g, b, out, M); break;
      case 2: hipLaunchKernelGGL((ln4_kernel<2, OutT>), grid, blk, 0, st, h, g, b, out, M); break;
      case 4: hipLaunchKernelGGL((ln4_kernel<4, OutT>), grid, blk, 0, st, h, g, b, out, M); break;
      case 8: hipLaunchKernelGGL((ln4_kernel<8, OutT>), grid, blk, 0, st, h, g, b, out, M); break;
      case 16: hipLaunchKernelGGL((ln4_kernel<16, OutT>), grid, blk, 0, st, h, g, b, out, M); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (d / AF_WAVE) {
    case 1: hipLaunchKernelGGL((layernorm_kernel<1, OutT>), grid, blk, 0, st, h, g, b, out, out_lo, M); break;
    case 2: hipLaunchKernelGGL((layernorm_kernel<2, OutT>), grid, blk, 0, st, h, g, b, out, out_lo, M); break;
    case 4: hipLaunchKernelGGL((layernorm_kernel<4, OutT>), grid, blk, 0, st, h, g, b, out, out_lo, M); break;
    case 8: hipLaunchKernelGGL((layernorm_kernel<8, OutT>), grid, blk, 0, st, h, g, b, out, out_lo, M); break;
    case 16: hipLaunchKernelGGL((layernorm_kernel<16, OutT>), grid, blk, 0, st, h, g, b, out, out_lo, M); break;
    case 32: hipLaunchKernelGGL((layernorm_kernel<32, OutT>), grid, blk, 0, st, h, g, b, out, out_lo, M); break;
    case 64: hipLaunchKernelGGL((layernorm_kernel<64, OutT>), grid, blk, 0, st, h, g, b, out, out_lo, M); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_layernorm(const float* h, const float* g, const float* b,
                            void* out, bool out_bf16, int M, int d, hipStream_t st,
                            void* out_lo) {
  if (out_bf16) return ln_dispatch(h, g, b, (bf16*)out, (bf16*)out_lo, M, d, st);
  return ln_dispatch(h, g, b, (float*)out, (float*)nullptr, M, d, st);
}

// One wave per row, V4 = d / 256 float4 per lane, S split planes, LO: also
// write the bf16 lo halves.  All loads of a row are issued before the sums.
template <int V4, int S, bool LO, class OutT>
__global__ __launch_bounds__(256) void resid_ln_kernel(
    const float* __restrict__ slab, const float* __restrict__ bias,
    float* __restrict__ h, const float* __restrict__ g, const float* __restrict__ b,
    OutT* __restrict__ out, OutT* __restrict__ out_lo, int M) {
  constexpr int D = V4 * 256;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const size_t plane = (size_t)M * D;
  float* hr = h + (size_t)row * D;
  const float* sr = slab + (size_t)row * D;
  float4 v[V4], pl[S][V4];
#pragma unroll
  for (int i = 0; i < V4; ++i) {
    const int j = 4 * lane + 256 * i;
    v[i] = *(const float4*)(hr + j);
#pragma unroll
    for (int sp = 0; sp < S; ++sp) pl[sp][i] = *(const float4*)(sr + sp * plane + j);
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < V4; ++i) {
    const int j = 4 * lane + 256 * i;
    const float4 bb = *(const float4*)(bias + j);
    float4 acc = pl[0][i];
#pragma unroll
    for (int sp = 1; sp < S; ++sp) {
      acc.x += pl[sp][i].x;
      acc.y += pl[sp][i].y;
      acc.z += pl[sp][i].z;
      acc.w += pl[sp][i].w;
    }
    v[i].x += acc.x + bb.x;
    v[i].y += acc.y + bb.y;
    v[i].z += acc.z + bb.z;
    v[i].w += acc.w + bb.w;
    *(float4*)(hr + j) = v[i];
    sum += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  }
  const float mean = wave_sum(sum) * (1.0f / D);
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < V4; ++i) {
    const float a0 = v[i].x - mean, a1 = v[i].y - mean, a2 = v[i].z - mean, a3 = v[i].w - mean;
    sq += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
  }
  const float rstd = rsqrtf(wave_sum(sq) * (1.0f / D) + 1e-5f);
#pragma unroll
  for (int i = 0; i < V4; ++i) {
    const int j = 4 * lane + 256 * i;
    const float4 gg = *(const float4*)(g + j), be = *(const float4*)(b + j);
    const float y0 = (v[i].x - mean) * rstd * gg.x + be.x;
    const float y1 = (v[i].y - mean) * rstd * gg.y + be.y;
    const float y2 = (v[i].z - mean) * rstd * gg.z + be.z;
    const float y3 = (v[i].w - mean) * rstd * gg.w + be.w;
    store4<OutT>(out + (size_t)row * D + j, y0, y1, y2, y3);
    if (LO)
      store4<OutT>(out_lo + (size_t)row * D + j, y0 - to_f32(from_f32<OutT>(y0)),
                   y1 - to_f32(from_f32<OutT>(y1)), y2 - to_f32(from_f32<OutT>(y2)),
                   y3 - to_f32(from_f32<OutT>(y3)));
  }
}

template <int S, bool LO, class OutT>
static hipError_t rln_v4(const float* slab, const float* bias, float* h, const float* g,
                         const float* b, OutT* out, OutT* out_lo, int M, int d,
                         hipStream_t st) {
  dim3 grid((M + 3) / 4), blk(256);
#define AF_RLN(V)                                                                     \
  hipLaunchKernelGGL((resid_ln_kernel<V, S, LO, OutT>), grid, blk, 0, st, slab, bias, h, \
                     g, b, out, out_lo, M)
  switch (d / 256) {
    case 1: AF_RLN(1); break;
    case 2: AF_RLN(2); break;
    case 4: AF_RLN(4); break;
    case 8: AF_RLN(8); break;
    case 16: AF_RLN(16); break;
    default: return hipErrorInvalidValue;
  }
#undef AF_RLN
  return hipGetLastError();
}

template <class OutT>
static hipError_t rln_dispatch(const float* slab, int S, const float* bias, float* h,
                               const float* g, const float* b, OutT* out, OutT* out_lo,
                               int M, int d, hipStream_t st) {
  if (d % 256) return hipErrorInvalidValue;
  const bool lo = out_lo != nullptr;
  switch (S * 2 + (lo ? 1 : 0)) {
    case 2: return rln_v4<1, false>(slab, bias, h, g, b, out, out_lo, M, d, st);
    case 3: return rln_v4<1, true>(slab, bias, h, g, b, out, out_lo, M, d, st);
    case 4: return rln_v4<2, false>(slab, bias, h, g, b, out, out_lo, M, d, st);
    case 5: return rln_v4<2, true>(slab, bias, h, g, b, out, out_lo, M, d, st);
    case 8: return rln_v4<4, false>(slab, bias, h, g, b, out, out_lo, M, d, st);
    case 9: return rln_v4<4, true>(slab, bias, h, g, b, out, out_lo, M, d, st);
    case 16: return rln_v4<8, false>(slab, bias, h, g, b, out, out_lo, M, d, st);
    case 17: return rln_v4<8, true>(slab, bias, h, g, b, out, out_lo, M, d, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_resid_ln(const float* slab, int S, const float* bias, float* h,
                           const float* g, const float* b, void* out, bool out_bf16,
                           void* out_lo, int M, int d, hipStream_t st) {
  if (out_bf16)
    return rln_dispatch<bf16>(slab, S, bias, h, g, b, (bf16*)out, (bf16*)out_lo, M, d, st);
  return rln_dispatch<float>(slab, S, bias, h, g, b, (float*)out, (float*)nullptr, M, d, st);
}

// ---------------------------------------------------------------------------
// Jacobi-block initial iterate, in processing order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void init_block_kernel(
    float* __restrict__ x, const float* __restrict__ x_init, int mode, int N,
    int R, int C, int L, int s, int dir, int F) {
  const size_t total = (size_t)N * R * C;
  for (size_t e = blockIdx.x * 256ull + threadIdx.x; e < total;
       e += (size_t)gridDim.x * 256) {
    int c = (int)(e % C);
    size_t nt = e / C;
    int t = (int)(nt % R), n = (int)(nt / R);
    int i = s + t;
    size_t dst = ((size_t)n * L + storage_index(i, L, dir)) * C + c;
    float v = 0.f;
    if (mode == 1) {
      v = x_init[dst];
    } else if (mode == 2 && s >= F) {
      v = x[((size_t)n * L + storage_index(i - F, L, dir)) * C + c];
    }
    x[dst] = v;
  }
}

hipError_t launch_init_block(float* x, const float* x_init, int mode, int N,
                             int R, int C, int L, int s, int dir, int F,
                             hipStream_t st) {
  size_t total = (size_t)N * R * C;
  int blocks = (int)std::min<size_t>((total + 255) / 256, 4096);
  hipLaunchKernelGGL(init_block_kernel, dim3(blocks), dim3(256), 0, st, x, x_init,
                     mode, N, R, C, L, s, dir, F);
  return hipGetLastError();
}

__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, size_t n) {
  for (size_t e = blockIdx.x * 256ull + threadIdx.x; e < n; e += (size_t)gridDim.x * 256)
    p[e] = v;
}

hipError_t launch_fill_u32(void* p, uint32_t v, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  int blocks = (int)std::min<size_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(fill_u32_kernel, dim3(blocks), dim3(256), 0, st, (uint32_t*)p, v, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused affine kernel.
//   mode 0 (inverse):  x <- mu + exp(ls) * z,  sums (x_new - x_old)^2, x_new^2
//   mode 1 (forward):  z <- (x - mu) * exp(-ls), sums ls, #non-finite z
// with ls = log sigma = 0.5 tanh(raw) and [mu | raw] = bias + the sum of the
// head GEMM's split-K partial planes, added in plane order.  Work is split
// into per-sample ranges of 4-channel quads (float4 I/O when C % 4 == 0);
// each block reduces its range into partials and the last block to finish
// (atomic ticket) sums the partials in a fixed order, so results do not
// depend on block scheduling.
// ---------------------------------------------------------------------------
int affine_groups(int N, int R, int C) {
  const long quads = ((long)R * C + 3) / 4;
  long g = (quads + 255) / 256;             // one quad per thread per pass
  const long cap = std::max(1, 8192 / std::max(N, 1));
  if (g > cap) g = cap;
  return (int)std::max(1L, g);
}

// Block-wide sums of a and b (red: 2 floats per wave; blocks of 4..16 waves),
// in a fixed order.
__device__ __forceinline__ void block_sum2(float& a, float& b, float* red) {
  a = wave_sum(a);
  b = wave_sum(b);
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  __syncthreads();
  if (lane == 0) {
    red[2 * wv] = a;
    red[2 * wv + 1] = b;
  }
  __syncthreads();
  a = (red[0] + red[2]) + (red[4] + red[6]);
  b = (red[1] + red[3]) + (red[5] + red[7]);
  for (int w = 4; w < nw; ++w) {
    a += red[2 * w];
    b += red[2 * w + 1];
  }
}

// Run by the last block to finish: the per-sample sums of the G partial
// pairs of every sample, added in a fixed order, into res (and res_host, the
// sticky non-finite tag, or the log-det); then the ticket counter is reset.
template <int MODE>
__device__ void finish_sums(const AffineArgs& a, const float* partials, int G, float* red) {
  for (int nn = 0; nn < a.N; ++nn) {
    float p0 = 0.f, p1 = 0.f;
    for (int gg = threadIdx.x; gg < G; gg += blockDim.x) {
      p0 += coherent_load(&partials[((size_t)nn * G + gg) * 2]);
      p1 += coherent_load(&partials[((size_t)nn * G + gg) * 2 + 1]);
    }
    block_sum2(p0, p1, red);
    if (threadIdx.x == 0) {
      if (MODE == 0) {
        a.res[2 * nn] = p0;
        a.res[2 * nn + 1] = p1;
        if (a.res_host) {
          system_store(&a.res_host[2 * nn], p0);
          system_store(&a.res_host[2 * nn + 1], p1);
        }
        if (a.bad && !(isfinite(p0) && isfinite(p1))) {
          // the first tag set stays; the host reads it beside the sequence word
          const unsigned first = atomicCAS(a.bad, 0u, a.tag);
          if (a.bad_host) system_store(a.bad_host, first ? first : a.tag);
        }
      } else {
        a.res[2 * nn] = -p0;
        a.res[2 * nn + 1] = p1;
        // samples in order: a group's entry adds its frames in a fixed order
        if (a.logdet) a.logdet[a.ld_group > 1 ? nn / a.ld_group : nn] += -p0;
        if (a.bad && p1 != 0.f) atomicCAS(a.bad, 0u, a.tag);
      }
    }
  }
  if (threadIdx.x == 0) {
    if (MODE == 0 && a.seq_host) {
      // publish the update's number once its residuals (and a non-finite
      // tag) have reached the host
      wait_stores();
      system_store(a.seq_host, atomicAdd(a.seq_dev, 1u) + 1u);
    }
    atomicExch(a.counter, 0u);
  }
}

// Global loads and stores of the affine kernel; NT marks them non-temporal
// (streamed past the caches), for inputs read once and outputs not re-read.
template <bool NT>
__device__ __forceinline__ float4 ld4(const float* p) {
  if (NT) {
    const f32x4 v = __builtin_nontemporal_load((const f32x4*)p);
    return float4{v[0], v[1], v[2], v[3]};
  }
  return *(const float4*)p;
}
template <bool NT>
__device__ __forceinline__ void st4(float* p, float4 v) {
  if (NT) __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w}, (f32x4*)p);
  else *(float4*)p = v;
}

// U items per thread and pass (VEC only): the loads of all U items are issued
// before the first is used, so each thread keeps U rows in flight.
template <int MODE, bool VEC, int U = 1, bool NT = false>
__global__ __launch_bounds__(256) void affine_kernel(AffineArgs a, int G) {
  static_assert(VEC || U == 1, "scalar path takes one item per pass");
  __shared__ float red[8];
  __shared__ unsigned ticket;
  const int n = blockIdx.y, g = blockIdx.x;
  const int C = a.C;
  const int W = VEC ? 4 : 1;                      // channels per item
  const unsigned CW = (unsigned)(C / W);          // items per token
  const unsigned items = (unsigned)a.R * CW;
  const unsigned chunk = (items + G - 1) / G;
  const unsigned i_end = min(items, (g + 1) * chunk);
  const size_t plane = (size_t)a.N * a.R * 2 * C;
  float s0 = 0.f, s1 = 0.f;
  for (unsigned base = g * chunk + threadIdx.x; base < i_end; base += 256 * U) {
    float mu[U][W], raw[U][W], in[U][W], out[U][W];
    size_t xi[U];
    const float* hp[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const unsigned it = base + 256 * u;
      ok[u] = it < i_end;
      const unsigned t = ok[u] ? it / CW : 0u;
      const int c = ok[u] ? (int)(it - t * CW) * W : 0;
      const size_t row = (size_t)n * a.R + t;
      xi[u] = ((size_t)n * a.L + storage_index(a.s + (int)t, a.L, a.dir)) * C + c;
      hp[u] = a.head + row * 2 * C + c;
#pragma unroll
      for (int q = 0; q < W; ++q) {
        mu[u][q] = a.head_bias ? a.head_bias[c + q] : 0.f;
        raw[u][q] = a.head_bias ? a.head_bias[C + c + q] : 0.f;
      }
    }
    // issue every load of the pass before the first use: the x (and z) rows
    // first, then the head planes in plane order
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!ok[u]) continue;
      const float* src = a.x;   // inverse: x_old; forward: x
      if (VEC) {
        const float4 v = ld4<NT>(src + xi[u]);
        in[u][0] = v.x; in[u][1 % W] = v.y; in[u][2 % W] = v.z; in[u][3 % W] = v.w;
        if (MODE == 0) {
          const float4 zz = ld4<NT>(a.z + xi[u]);
          out[u][0] = zz.x; out[u][1 % W] = zz.y; out[u][2 % W] = zz.z; out[u][3 % W] = zz.w;
        }
      } else {
        in[u][0] = src[xi[u]];
        if (MODE == 0) out[u][0] = a.z[xi[u]];
      }
    }
#pragma unroll 4
    for (int sp = 0; sp < a.head_splits; ++sp) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (!ok[u]) continue;
        const float* hs = hp[u] + sp * plane;
        if (VEC) {
          const float4 m4 = ld4<NT>(hs);
          const float4 r4 = ld4<NT>(hs + C);
          mu[u][0] += m4.x; mu[u][1 % W] += m4.y; mu[u][2 % W] += m4.z; mu[u][3 % W] += m4.w;
          raw[u][0] += r4.x; raw[u][1 % W] += r4.y; raw[u][2 % W] += r4.z; raw[u][3 % W] += r4.w;
        } else {
          mu[u][0] += hs[0];
          raw[u][0] += hs[C];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!ok[u]) continue;
      if (MODE == 0) {
        // in = x_old, out = z on entry
#pragma unroll
        for (int q = 0; q < W; ++q) {
          const float xn = mu[u][q] + expf(0.5f * tanhf(raw[u][q])) * out[u][q];
          const float df = xn - in[u][q];
          s0 += df * df;
          s1 += xn * xn;
          out[u][q] = xn;
        }
        if (VEC)
          st4<NT>(a.x + xi[u], float4{out[u][0], out[u][1 % W], out[u][2 % W], out[u][3 % W]});
        else
          a.x[xi[u]] = out[u][0];
      } else {
#pragma unroll
        for (int q = 0; q < W; ++q) {
          const float ls = 0.5f * tanhf(raw[u][q]);
          const float zv = (in[u][q] - mu[u][q]) * expf(-ls);
          out[u][q] = zv;
          s0 += ls;
          s1 += isfinite(zv) ? 0.f : 1.f;
        }
        if (VEC)
          st4<NT>(a.zout + xi[u], float4{out[u][0], out[u][1 % W], out[u][2 % W], out[u][3 % W]});
        else
          a.zout[xi[u]] = out[u][0];
      }
    }
  }
  block_sum2(s0, s1, red);
  if (threadIdx.x == 0) {
    coherent_store(&a.partials[((size_t)n * G + g) * 2], s0);
    coherent_store(&a.partials[((size_t)n * G + g) * 2 + 1], s1);
    wait_stores();
    ticket = atomicAdd(a.counter, 1u);
  }
  __syncthreads();
  if (ticket != (unsigned)(gridDim.x * gridDim.y) - 1) return;
  finish_sums<MODE>(a, a.partials, G, red);
}

// Large ranges, where even four items per thread leave the block cap
// binding, stream: four items in flight per thread and non-temporal loads
// and stores (5.0 -> 5.56 TB/s at 2^22 tokens of 48 channels, the rate of a
// plain streaming copy).  Smaller ones (the Jacobi path's frames, resident in
// L2) take one item per thread over more blocks: four per thread there cut
// the grid to a quarter and ran 8 -> 12 us at 1560 rows.
static bool affine_streaming(int N, int R, int C) {
  const long quads = ((long)R * C + 3) / 4;
  const long cap = std::max(1, 8192 / std::max(N, 1));
  return (C % 4) == 0 && quads >= cap * 256L * 4;
}

hipError_t launch_affine(int mode, const AffineArgs& a, hipStream_t st) {
  const int G = affine_groups(a.N, a.R, a.C);
  dim3 grid(G, a.N);
  const bool vec = (a.C % 4) == 0;
  const bool stream = affine_streaming(a.N, a.R, a.C);
  if (mode == 0) {
    if (stream) hipLaunchKernelGGL((affine_kernel<0, true, 4, true>), grid, dim3(256), 0, st, a, G);
    else if (vec) hipLaunchKernelGGL((affine_kernel<0, true>), grid, dim3(256), 0, st, a, G);
    else hipLaunchKernelGGL((affine_kernel<0, false>), grid, dim3(256), 0, st, a, G);
  } else {
    if (stream) hipLaunchKernelGGL((affine_kernel<1, true, 4, true>), grid, dim3(256), 0, st, a, G);
    else if (vec) hipLaunchKernelGGL((affine_kernel<1, true>), grid, dim3(256), 0, st, a, G);
    else hipLaunchKernelGGL((affine_kernel<1, false>), grid, dim3(256), 0, st, a, G);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Streaming copy: the bandwidth reference of the fused affine kernel.  Each
// block copies one contiguous range with four 16-byte non-temporal loads in
// flight per thread before their stores.  Measured against other forms on
// this GPU (2 GiB each way): grid-stride single loads 4.5-5.4 TB/s, the
// runtime's device-to-device copy 4.9 TB/s, this form 5.6 TB/s.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void stream_copy_kernel(const float4* __restrict__ src,
                                                          float4* __restrict__ dst,
                                                          size_t n4, size_t chunk) {
  const size_t b0 = (size_t)blockIdx.x * chunk;
  const size_t b1 = min(n4, b0 + chunk);
  for (size_t base = b0 + threadIdx.x; base < b1; base += 256 * 4) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (base + u * 256 < b1) v[u] = ld4<true>((const float*)&src[base + u * 256]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (base + u * 256 < b1) st4<true>((float*)&dst[base + u * 256], v[u]);
  }
}

hipError_t launch_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t st) {
  const size_t n4 = bytes / 16;
  if (n4 == 0) return hipSuccess;
  // 32768 blocks measured best for gigabyte copies; at least 1024 items each
  const size_t blocks = std::min<size_t>(32768, (n4 + 1023) / 1024);
  const size_t chunk = (n4 + blocks - 1) / blocks;
  hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     (const float4*)src, (float4*)dst, n4, chunk);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Head GEMM on the fp32 matrix cores: planes[s][m][:] = hf[m] W_head^T over
// the s-th of S equal K ranges (the affine kernel adds bias and planes).
// One wave per (16-row tile, K range): it computes all 2C = 16 NT columns of
// its rows with v_mfma_f32_16x16x4f32.  Lane (i = l % 16, g = l / 16) feeds
// hf row i and W row i of each column tile with the float4 at k + 4g; the four
// components are four MFMA steps, so both operands load 16 contiguous bytes
// per lane, and the loads of U steps of 16 are issued before their MFMAs.
// ---------------------------------------------------------------------------
bool head_mfma_supported(int C, int d) {
  const int nt = C / 8;
  return C % 8 == 0 && d % 64 == 0 &&
         (nt == 1 || nt == 2 || nt == 3 || nt == 4 || nt == 6 || nt == 8 || nt == 12 || nt == 16);
}

// Output row m (sample m / r_out, row m % r_out) reads hf row
// (m / r_out) * r_in + off + m % r_out: the last r_out of every r_in rows.
template <int NT>
__global__ __launch_bounds__(64) void head_mfma_kernel(const float* __restrict__ hf,
                                                       const float* __restrict__ w,
                                                       float* __restrict__ planes, int M,
                                                       int d, int k_len, int r_out, int r_in,
                                                       int off) {
  // U steps of 16 loaded at a time: all of a 128-long K range when 2C <= 96
  // (fewer than one wave per SIMD here, so registers are plentiful)
  constexpr int NC = 16 * NT, U = NT <= 6 ? 8 : NT <= 12 ? 4 : 2;
  const int tiles = (M + 15) / 16;
  const int s = blockIdx.x / tiles, m0 = (blockIdx.x - s * tiles) * 16;
  const int lane = threadIdx.x, l16 = lane & 15, g = lane >> 4;
  const int kb = s * k_len + 4 * g;
  // rows past M read row M-1; their results are not stored
  const int mr = min(m0 + l16, M - 1), smp = mr / r_out;
  const float* ap = hf + ((size_t)smp * r_in + off + (mr - smp * r_out)) * d + kb;
  const float* wp = w + (size_t)l16 * d + kb;
  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < k_len; k += 16 * U) {
    float4 av[U], bv[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool on = k + 16 * u < k_len;
      av[u] = on ? *(const float4*)(ap + k + 16 * u) : float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < NT; ++t)
        bv[u][t] = on ? *(const float4*)(wp + (size_t)t * 16 * d + k + 16 * u)
                      : float4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u].x, bv[u][t].x, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u].y, bv[u][t].y, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u].z, bv[u][t].z, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u].w, bv[u][t].w, acc[t], 0, 0, 0);
      }
  }
  // lane (l16, g) holds rows 4g..4g+3 of column l16 of every column tile
  float* out = planes + (size_t)s * M * NC;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = m0 + 4 * g + r;
    if (m < M) {
#pragma unroll
      for (int t = 0; t < NT; ++t) out[(size_t)m * NC + t * 16 + l16] = acc[t][r];
    }
  }
}

hipError_t launch_head_mfma(const float* hf, const float* w, float* planes, int M, int C,
                            int d, int splits, hipStream_t st, int r_out, int r_in, int off) {
  const dim3 grid(((M + 15) / 16) * splits);
  const int k_len = d / splits;
#define AF_HM(NT)                                                                        \
  hipLaunchKernelGGL((head_mfma_kernel<NT>), grid, dim3(64), 0, st, hf, w, planes, M, d, \
                     k_len, r_out, r_in, off);                                           \
  break;
  switch (C / 8) {
    case 1: AF_HM(1)
    case 2: AF_HM(2)
    case 3: AF_HM(3)
    case 4: AF_HM(4)
    case 6: AF_HM(6)
    case 8: AF_HM(8)
    case 12: AF_HM(12)
    case 16: AF_HM(16)
    default: return hipErrorInvalidValue;
  }
#undef AF_HM
  return hipGetLastError();
}

int head_mfma_splits(int M, int d) {
  const long tiles = (M + 15) / 16;
  int S = 1;
  // K ranges of at least 64 (four steps), grid of at most ~1024 waves
  while (S < 8 && tiles * S * 2 <= 1024 && d % (64 * S * 2) == 0) S *= 2;
  return S;
}

}  // namespace af
