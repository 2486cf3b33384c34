// Jacobi inverse of one affine AF block with the whole loop on the device, for
// small fp32 blocks (STARFlow-V notes, 关键设计 3: block-wise Jacobi with a KV
// cache and a residual stop; 关键设计 1: the affine AF update).
//
// One workgroup runs every Jacobi block of the sequence in order: the
// shifted embedding, every layer (LayerNorm, QKV with K/V into the cache,
// causal attention over the cache, output projection, LayerNorm, GELU MLP),
// the final LayerNorm and head, the affine update and the per-sample residual
// sums; then it takes the stop test itself (every sample's
// sum (x' - x)^2 / sum x'^2 below tau, or the update cap) and refreshes the
// block's cache rows from its final tokens after an early stop (but the last
// block's, which nothing in the launch reads).  No kernel launch and no host
// read-back per update: the host launches once per AF block and reads the
// iteration counts at the end.  In refresh mode a launch runs only that
// refresh pass, over given tokens (the rows a later call needs of an earlier
// call's last block), so both come from the same arithmetic.
//
// The block's activations live in LDS (rows M = N x B <= 64, d 64 or 128);
// the projections run on the fp32 matrix cores, one wave per 16 x 16 output
// tile, the weights read from global memory (L2-resident at these sizes) in
// whole float4s per lane; the KV cache is the workspace's, in the layout the
// other kernels use, so a later call continues from it.  Attention runs one wave per (sample, head, four
// rows): the lanes take 64 keys at a time for the scores of the rows, then
// the value dimensions for P V, so each K row and V^T chunk is loaded once
// for the four rows.  Arithmetic is fp32 throughout, sums in a fixed order
// (results do not depend on scheduling).
#include "common.h"
#include "kernels.h"

namespace af {

namespace {

constexpr int LT = 512;   // threads
constexpr int NW = LT / 64;   // waves
constexpr int RG = 4;     // attention rows per wave pass
constexpr int KT = 64;    // attention keys per wave pass (one per lane)

// Shared-memory carve-up of one block's state (floats).  uc = MLP hidden
// columns per chunk: the whole hidden width when it fits in lds_max bytes,
// else the largest halving of it (a multiple of 64) that does.
struct LoopLds {
  int xb, zb, prev, h, a, q, o, u, hd, ps, red, fin;
  int uc, total;
};

__host__ __device__ LoopLds loop_lds(int M, int N, int C, int d, int dmlp, int lds_max) {
  LoopLds l{};
  for (int uc = dmlp;; uc /= 2) {
    int off = 0;
    auto take = [&](int n) { const int o = off; off += (n + 3) & ~3; return o; };
    l.xb = take(M * C);
    l.zb = take(M * C);
    l.prev = take(N * C);
    l.h = take(M * (d + 4));   // rows padded by 4 floats: the 16 rows an MFMA
    l.a = take(M * (d + 4));   // operand read spans fall on distinct banks
    l.q = take(M * (d + 4));
    l.o = take(M * (d + 4));
    l.u = take(M * (uc + 4));
    l.hd = take(M * 2 * C);
    l.ps = take(NW * RG * KT);   // one probability strip per wave
    l.red = take(NW * N * 2);    // per-wave residual partials
    l.fin = take(N * 2);         // each sample's residual pair
    l.uc = uc;
    l.total = off;
    if (off * 4 <= lds_max || uc % 128 != 0) return l;
  }
}

// y[m][n] = X[m] . W[n] (+ bias[n]) for m < M, n < Nout, contraction length K
// (a multiple of 16); X in LDS with row stride ldx, W row-major with row
// stride ldw (global).  On the fp32 matrix cores (v_mfma_f32_16x16x4f32), one
// wave per 16-token x 16-feature tile: lane (i = l % 16, g = l / 16) feeds W
// row f0 + i and token m0 + i at k slot g, with the k order permuted alike in
// both operands (slot g of step 4t + e is k = 4g + 16t + e), so every lane
// loads whole float4s, up to KG of K per load round; it receives features
// f0 + 4g .. f0 + 4g + 3 of token m0 + i, and epi(m, n, value) consumes
// each.  Padding rows and features past M and Nout read valid ones and are
// not stored.
template <int KG, class Epi>
__device__ void linear(const float* X, int ldx, int M, const float* W, int ldw,
                       const float* bias, int Nout, int K, Epi epi) {
  static_assert(KG % 16 == 0, "k group");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = lane & 15, g = lane >> 4;
  const int tm = (M + 15) / 16, tn = (Nout + 15) / 16;
  for (int tile = wave; tile < tm * tn; tile += NW) {
    const int m0 = (tile % tm) * 16, f0 = (tile / tm) * 16;
    const float* xr = X + min(m0 + i, M - 1) * ldx + 4 * g;
    const float* wr = W + (size_t)min(f0 + i, Nout - 1) * ldw + 4 * g;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma clang loop unroll(disable)
    for (int k0 = 0; k0 < K; k0 += KG) {
      float4 wa[KG / 16], xb[KG / 16];
#pragma unroll
      for (int t = 0; t < KG / 16; ++t)
        if (k0 + 16 * t < K) {
          wa[t] = *(const float4*)(wr + k0 + 16 * t);
          xb[t] = *(const float4*)(xr + k0 + 16 * t);
        }
#pragma unroll
      for (int t = 0; t < KG / 16; ++t)
        if (k0 + 16 * t < K) {
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wa[t].x, xb[t].x, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wa[t].y, xb[t].y, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wa[t].z, xb[t].z, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wa[t].w, xb[t].w, acc, 0, 0, 0);
        }
    }
    if (m0 + i < M) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = f0 + 4 * g + r;
        if (n < Nout) epi(m0 + i, n, acc[r] + (bias ? bias[n] : 0.f));
      }
    }
  }
}

// out[m] = LayerNorm(in[m]) * g + b over rows of width d and stride ld (eps
// 1e-5), one wave per row.
__device__ void layernorm_rows(const float* in, float* out, int M, int d, int ld,
                               const float* g, const float* b) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int m = wave; m < M; m += LT / 64) {
    const float* r = in + m * ld;
    float s = 0.f;
    for (int e = lane; e < d; e += 64) s += r[e];
    const float mean = wave_sum(s) / d;
    float v = 0.f;
    for (int e = lane; e < d; e += 64) {
      const float t = r[e] - mean;
      v += t * t;
    }
    const float rstd = rsqrtf(wave_sum(v) / d + 1e-5f);
    for (int e = lane; e < d; e += 64) out[m * ld + e] = (r[e] - mean) * rstd * g[e] + b[e];
  }
}

// Causal attention of the block rows over the cache, one wave per (sample,
// head, group of RG rows) at a time: for KT keys per pass, lane j scores key j0 + j
// against each row (its K row in registers, the rows' q from LDS), the online
// softmax per row keeps (max, sum) in registers of every lane, then lane l
// adds sum_j p_rj V^T[e][j] over its share of the pass's keys for dimension
// e = l % d_h (its V^T chunk in registers; with d_h 32 the two halves of the
// wave take the two halves of the keys and are added at the end).
// Keys past a row's position are masked; cache rows past the last key are
// never multiplied (their p is 0 and their V is replaced by 0).
template <int D, int DH>
__device__ void loop_attention(const LoopArgs& a, const float* q, float* o, float* ps,
                               const float* kc, const float* vt, int s, int R) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int N = a.N, H = a.H;
  // scores in base-2 units: p = 2^(s log2(e) / sqrt(dh) - m)
  const float scale = 1.4426950408889634f / sqrtf((float)DH);
  // P V: lane l takes dimension l % DH over key part l / DH of each 64-key
  // pass (NP parts of KP keys); the parts are added at the end
  constexpr int NP = 64 / DH, KP = KT / NP;
  const int ve = lane % DH, vpart = lane / DH;
  float* pw = ps + wave * RG * KT;
  const int ngrp = (R + RG - 1) / RG;
  for (int item = wave; item < N * H * ngrp; item += LT / 64) {
    const int pair = item / ngrp, t0 = (item - pair * ngrp) * RG;
    const int nn = pair / H, head = pair - nn * H;
    const size_t base = (size_t)nn * H + head;
    const float* kr = kc + base * a.Lcap * DH;
    const float* vr = vt + base * DH * a.Lcap;
    {
      const int rows = min(RG, R - t0);
      const int nkmax = a.P + s + t0 + rows;   // keys of the group's last row
      float om[RG], ol[RG], oacc[RG];
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        om[r] = -INFINITY;
        ol[r] = 0.f;
        oacc[r] = 0.f;
      }
      for (int j0 = 0; j0 < nkmax; j0 += KT) {
        const int j = j0 + lane;
        const bool kv = j < nkmax;
        float4 kreg[DH / 4];
#pragma unroll
        for (int e = 0; e < DH / 4; ++e)
          kreg[e] = kv ? *(const float4*)(kr + (size_t)j * DH + 4 * e) : float4{0.f, 0.f, 0.f, 0.f};
        // this lane's V^T chunk (dimension ve, keys of part vpart), zero past
        // the last key
        float vv[KP];
        {
          const int k0 = j0 + vpart * KP;
          const float* vp = vr + (size_t)ve * a.Lcap + k0;
#pragma unroll
          for (int jj = 0; jj < KP; jj += 4) {
            const float4 v4 = *(const float4*)(vp + jj);
            vv[jj] = k0 + jj < nkmax ? v4.x : 0.f;
            vv[jj + 1] = k0 + jj + 1 < nkmax ? v4.y : 0.f;
            vv[jj + 2] = k0 + jj + 2 < nkmax ? v4.z : 0.f;
            vv[jj + 3] = k0 + jj + 3 < nkmax ? v4.w : 0.f;
          }
        }
#pragma unroll
        for (int r = 0; r < RG; ++r) {
          if (r >= rows) continue;
          const float* qr = q + (nn * R + t0 + r) * (D + 4) + head * DH;
          float sv = 0.f;
#pragma unroll
          for (int e = 0; e < DH / 4; ++e) {
            const float4 q4 = *(const float4*)(qr + 4 * e);
            sv = fmaf(q4.x, kreg[e].x, sv);
            sv = fmaf(q4.y, kreg[e].y, sv);
            sv = fmaf(q4.z, kreg[e].z, sv);
            sv = fmaf(q4.w, kreg[e].w, sv);
          }
          sv = (kv && j <= a.P + s + t0 + r) ? sv * scale : -INFINITY;
          const float mn = fmaxf(om[r], wave_max(sv));
          const float al = __builtin_amdgcn_exp2f(om[r] - mn);
          const float pv = __builtin_amdgcn_exp2f(sv - mn);
          ol[r] = ol[r] * al + wave_sum(pv);
          om[r] = mn;
          oacc[r] *= al;
          pw[r * KT + lane] = pv;
        }
        // the strip is complete before any lane reads it (one wave: LDS
        // accesses stay in order; the barrier keeps the compiler from
        // reordering them)
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int r = 0; r < RG; ++r) {
          if (r >= rows) continue;
          float acc = oacc[r];
#pragma unroll
          for (int jj = 0; jj < KP; jj += 4) {
            const float4 p4 = *(const float4*)(pw + r * KT + vpart * KP + jj);
            acc = fmaf(p4.x, vv[jj], acc);
            acc = fmaf(p4.y, vv[jj + 1], acc);
            acc = fmaf(p4.z, vv[jj + 2], acc);
            acc = fmaf(p4.w, vv[jj + 3], acc);
          }
          oacc[r] = acc;
        }
        __builtin_amdgcn_wave_barrier();
      }
      if constexpr (NP == 2) {
        // the two key parts, lanes l and l + 32: low part first in both
#pragma unroll
        for (int r = 0; r < RG; ++r) {
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(oacc[r]),
                                                           __float_as_uint(oacc[r]), false, false);
          const unsigned lo = sw[0], hi = sw[1];
          oacc[r] = __uint_as_float(lo) + __uint_as_float(hi);
        }
      }
      if (lane < DH) {
#pragma unroll
        for (int r = 0; r < RG; ++r) {
          if (r >= rows) continue;
          o[(nn * R + t0 + r) * (D + 4) + head * DH + lane] = oacc[r] / ol[r];
        }
      }
    }
  }
}

}  // namespace

// One Jacobi update (or, with kv_only, the cache refresh: every layer's K/V of
// the block rows from the current tokens) of block [s, s + R).
template <int D, int DH>
__device__ void loop_pass(const LoopArgs& a, float* sm, const LoopLds& L, int s, int R,
                          bool kv_only) {
  const int N = a.N, C = a.C, H = a.H, M = N * R;
  const int tid = threadIdx.x;
  const float* xb = sm + L.xb;
  const float* prev = sm + L.prev;
  float* h = sm + L.h;
  float* act = sm + L.a;
  float* q = sm + L.q;
  float* o = sm + L.o;
  float* u = sm + L.u;
  constexpr int LD = D + 4;   // row stride of h, act, q, o
  // shift + embed: row m = n R + t takes token t - 1 of the block (the token
  // before the block at t = 0), position P + s + t
  for (int idx = tid; idx < M * D; idx += LT) {
    const int m = idx / D, e = idx - m * D, n = m / R, t = m - n * R;
    const float* in = t == 0 ? prev + n * C : xb + (m - 1) * C;
    const float* w = a.w_in + (size_t)e * C;
    float acc = a.b_in[e] + a.pos[(size_t)(a.P + s + t) * D + e];
    for (int c = 0; c < C; c += 4) {
      const float4 w4 = *(const float4*)(w + c);
      acc = fmaf(in[c], w4.x, acc);
      acc = fmaf(in[c + 1], w4.y, acc);
      acc = fmaf(in[c + 2], w4.z, acc);
      acc = fmaf(in[c + 3], w4.w, acc);
    }
    h[m * LD + e] = acc;
  }
  __syncthreads();
  for (int l = 0; l < a.n_layers; ++l) {
    const LoopLayer& w = a.layers[l];
    float* kc = a.kc[l];
    float* vt = a.vt[l];
    layernorm_rows(h, act, M, D, LD, w.ln1_g, w.ln1_b);
    __syncthreads();
    // QKV: Q into LDS, K and V of the block rows into the cache
    linear<D>(act, LD, M, w.w_qkv, D, w.b_qkv, 3 * D, D, [&](int m, int n, float v) {
      const int which = n / D, hd = n - which * D;
      if (which == 0) {
        q[m * LD + hd] = v;
        return;
      }
      const int nn = m / R, t = m - nn * R, p = a.P + s + t;
      const int head = hd / DH, e = hd - head * DH;
      const size_t base = (size_t)nn * H + head;
      if (which == 1) kc[(base * a.Lcap + p) * DH + e] = v;
      else vt[(base * DH + e) * a.Lcap + p] = v;
    });
    __syncthreads();   // the cache rows are written (workgroup scope)
    if (kv_only && l == a.n_layers - 1) return;
    loop_attention<D, DH>(a, q, o, sm + L.ps, kc, vt, s, R);
    __syncthreads();
    // output projection into the residual stream
    linear<D>(o, LD, M, w.w_o, D, w.b_o, D, D, [&](int m, int n, float v) { h[m * LD + n] += v; });
    __syncthreads();
    layernorm_rows(h, act, M, D, LD, w.ln2_g, w.ln2_b);
    __syncthreads();
    // MLP in hidden chunks of UC columns: u = GELU(a W1^T + b1), h += u W2^T
    // (+ b2 with the first chunk)
    const int UC = L.uc, LU = UC + 4;
    for (int c0 = 0; c0 < a.dmlp; c0 += UC) {
      linear<D>(act, LD, M, w.w_1 + (size_t)c0 * D, D, w.b_1 + c0, UC, D,
                [&](int m, int n, float v) { u[m * LU + n] = gelu_erf(v); });
      __syncthreads();
      linear<128>(u, LU, M, w.w_2 + c0, a.dmlp, c0 == 0 ? w.b_2 : nullptr, D, UC,
                  [&](int m, int n, float v) { h[m * LD + n] += v; });
      __syncthreads();
    }
  }
}

// The affine update of the block from the head output, with each sample's
// residual pair in fin[2n], fin[2n + 1] (per thread, then per wave, then over
// the waves in order: a fixed summation order).
template <int D>
__device__ void loop_affine(const LoopArgs& a, float* sm, const LoopLds& L, int R) {
  const int N = a.N, C = a.C, M = N * R, tid = threadIdx.x;
  float* xb = sm + L.xb;
  const float* zb = sm + L.zb;
  float* h = sm + L.h;
  float* act = sm + L.a;
  float* hd = sm + L.hd;
  float* red = sm + L.red;
  float* fin = sm + L.fin;
  const int wave = tid >> 6, lane = tid & 63;
  constexpr int LD = D + 4;
  layernorm_rows(h, act, M, D, LD, a.ln_f_g, a.ln_f_b);
  __syncthreads();
  linear<D>(act, LD, M, a.w_head, D, a.b_head, 2 * C, D,
            [&](int m, int n, float v) { hd[m * 2 * C + n] = v; });
  __syncthreads();
  for (int n = 0; n < N; ++n) {
    float s0 = 0.f, s1 = 0.f;
    for (int idx = tid; idx < R * C; idx += LT) {
      const int m = n * R + idx / C, c = idx % C;
      const float mu = hd[m * 2 * C + c];
      const float ls = 0.5f * tanhf(hd[m * 2 * C + C + c]);
      const float xn = mu + expf(ls) * zb[m * C + c];
      const float df = xn - xb[m * C + c];
      s0 += df * df;
      s1 += xn * xn;
    }
    s0 = wave_sum(s0);
    s1 = wave_sum(s1);
    if (lane == 0) {
      red[(wave * N + n) * 2] = s0;
      red[(wave * N + n) * 2 + 1] = s1;
    }
  }
  __syncthreads();
  if (tid < 2 * N) {
    float t = 0.f;
    for (int w = 0; w < NW; ++w) t += red[w * N * 2 + tid];
    fin[tid] = t;
  }
  __syncthreads();
  // the new iterate (after every thread read the old one)
  for (int idx = tid; idx < M * C; idx += LT) {
    const int m = idx / C, c = idx % C;
    const float mu = hd[m * 2 * C + c];
    const float ls = 0.5f * tanhf(hd[m * 2 * C + C + c]);
    xb[idx] = mu + expf(ls) * zb[idx];
  }
  __syncthreads();
}

template <int D, int DH>
__global__ __launch_bounds__(LT) void jacobi_loop_kernel(LoopArgs a) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  const int N = a.N, C = a.C, tid = threadIdx.x;
  const int nb = (a.L + a.B - 1) / a.B;
  const LoopLds L = loop_lds(N * min(a.B, a.L), N, C, D, a.dmlp, a.lds_max);
  float* xb = sm + L.xb;
  float* zb = sm + L.zb;
  float* prev = sm + L.prev;
  float* fin = sm + L.fin;
  // the token before the sequence
  for (int idx = tid; idx < N * C; idx += LT)
    prev[idx] = a.x_last ? a.x_last[idx] : 0.f;
  for (int b = 0; b < nb; ++b) {
    const int s = b * a.B, R = min(a.B, a.L - s), M = N * R;
    if (a.refresh) {
      // the block's tokens, then the pass that writes their cache rows
      for (int idx = tid; idx < M * C; idx += LT) {
        const int m = idx / C, c = idx - m * C, n = m / R, t = m - n * R;
        xb[idx] = a.x_init[((size_t)n * a.L + storage_index(s + t, a.L, a.dir)) * C + c];
      }
      __syncthreads();
      loop_pass<D, DH>(a, sm, L, s, R, true);
      for (int idx = tid; idx < N * C; idx += LT) {
        const int n = idx / C, c = idx - n * C;
        prev[idx] = xb[((n + 1) * R - 1) * C + c];
      }
      __syncthreads();
      continue;
    }
    // z of the block and the first iterate
    for (int idx = tid; idx < M * C; idx += LT) {
      const int m = idx / C, c = idx - m * C, n = m / R, t = m - n * R, i = s + t;
      const size_t g = ((size_t)n * a.L + storage_index(i, a.L, a.dir)) * C + c;
      zb[idx] = a.z[g];
      float x0 = 0.f;
      if (a.init == 1) x0 = a.x_init[g];
      else if (a.init == 2 && s >= a.F)
        x0 = a.x[((size_t)n * a.L + storage_index(i - a.F, a.L, a.dir)) * C + c];
      xb[idx] = x0;
    }
    __syncthreads();
    const int kmax = a.max_iters <= 0 ? R : min(a.max_iters, R);
    int k = 0;
    bool bad = false;
    while (k < kmax) {
      loop_pass<D, DH>(a, sm, L, s, R, false);
      loop_affine<D>(a, sm, L, R);
      ++k;
      bool all = true;
      for (int n = 0; n < N; ++n) {
        const float num = fin[2 * n], den = fin[2 * n + 1];
        if (!(isfinite(num) && isfinite(den))) bad = true;
        const float r = den > 0.f ? num / den : (num == 0.f ? 0.f : INFINITY);
        all = all && r < a.tau;
      }
      if (bad || (a.tau > 0.f && all)) break;
    }
    // the last update's residual pairs and the block's count
    if (tid == 0) {
      for (int n = 0; n < 2 * N; ++n) system_store(&a.res_host[n], fin[n]);
      system_store((unsigned*)&a.iters_host[b], (unsigned)k);
      if (bad) system_store(a.bad_host, (unsigned)(1 + b));
    }
    if (bad) return;
    // an early stop leaves the cache rows from the previous iterate: recompute
    // them from the final tokens (not for the last block, which nothing in
    // this launch reads; a later call refreshes it with the same pass)
    if (k < R && b + 1 < nb) {
      __syncthreads();
      loop_pass<D, DH>(a, sm, L, s, R, true);
    }
    // the block's tokens out, and each sample's last token for the next block
    for (int idx = tid; idx < M * C; idx += LT) {
      const int m = idx / C, c = idx - m * C, n = m / R, t = m - n * R;
      a.x[((size_t)n * a.L + storage_index(s + t, a.L, a.dir)) * C + c] = xb[idx];
    }
    __syncthreads();
    for (int idx = tid; idx < N * C; idx += LT) {
      const int n = idx / C, c = idx - n * C;
      prev[idx] = xb[((n + 1) * R - 1) * C + c];
    }
    __syncthreads();
  }
}

bool jacobi_loop_supported(int N, int Bc, int C, int d, int H, int dmlp, int n_layers,
                           int Lcap, int lds_max) {
  if (N < 1 || Bc < 1 || H < 1 || (d != 64 && d != 128) || d % H != 0) return false;
  const int dh = d / H;
  if (dh != 32 && dh != 64) return false;
  const int M = N * Bc;
  if (M > 64 || C % 4 != 0 || C > 64 || Lcap % 64 != 0) return false;
  if (dmlp % 64 != 0 || n_layers < 1 || n_layers > kLoopMaxLayers) return false;
  return loop_lds(M, N, C, d, dmlp, lds_max).total * sizeof(float) <= (size_t)lds_max;
}

hipError_t launch_jacobi_loop(const LoopArgs& a, hipStream_t st) {
  const int Bc = a.B < a.L ? a.B : a.L;
  const size_t lds = loop_lds(a.N * Bc, a.N, a.C, a.d, a.dmlp, a.lds_max).total * sizeof(float);
  const dim3 g(1), b(LT);
  // more than 64 KB of dynamic LDS is asked for explicitly
  auto go = [&](const void* k, auto launch) {
    if (lds > 65536) {
      const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)lds);
      if (e != hipSuccess) return e;
    }
    launch();
    return hipGetLastError();
  };
  if (a.d == 64 && a.dh == 32)
    return go((const void*)jacobi_loop_kernel<64, 32>,
              [&] { hipLaunchKernelGGL((jacobi_loop_kernel<64, 32>), g, b, lds, st, a); });
  if (a.d == 64 && a.dh == 64)
    return go((const void*)jacobi_loop_kernel<64, 64>,
              [&] { hipLaunchKernelGGL((jacobi_loop_kernel<64, 64>), g, b, lds, st, a); });
  if (a.d == 128 && a.dh == 32)
    return go((const void*)jacobi_loop_kernel<128, 32>,
              [&] { hipLaunchKernelGGL((jacobi_loop_kernel<128, 32>), g, b, lds, st, a); });
  if (a.d == 128 && a.dh == 64)
    return go((const void*)jacobi_loop_kernel<128, 64>,
              [&] { hipLaunchKernelGGL((jacobi_loop_kernel<128, 64>), g, b, lds, st, a); });
  return hipErrorInvalidValue;
}

}  // namespace af
