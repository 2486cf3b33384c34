// Projection GEMMs of the AF block's Transformer: y[M, N] = A[M, K] W[N, K]^T
// + bias with a fused epilogue (QKV scatter into the KV cache, residual add
// into the fp32 stream, exact GELU, or plain fp32 store).
//
//  * bf16 path: MFMA kernel for gfx950 (v_mfma_f32_16x16x32_bf16), both
//    operands K-contiguous, LDS double-buffered with register prefetch.
//  * fp32 path: LDS-tiled SIMT kernel (also used for the fp32 head).
#include "common.h"
#include "kernels.h"

#include <hip/hip_ext.h>

#include <algorithm>

namespace af {

// ---------------------------------------------------------------------------
// epilogues.  operator() takes one element (fp32 SIMT kernel); store4 takes
// four consecutive output features n..n+3 of row m (bf16 MFMA kernel).
// ---------------------------------------------------------------------------
template <class T>
__device__ __forceinline__ void store_vec4(T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store_vec4<float>(float* p, float a, float b, float c, float d) {
  *(float4*)p = float4{a, b, c, d};
}
template <>
__device__ __forceinline__ void store_vec4<bf16>(bf16* p, float a, float b, float c, float d) {
  bf16x4 v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
  *(bf16x4*)p = v;
}

template <class T>
struct EpiQKV {
  const float* bias;
  T* q;
  T* kc;
  T* vt;
  int M, R, d, dh, H, Lcap, pos_base;
  int log2d, log2dh;   // d and dh are powers of two
  T* q_lo;    // split outputs (bf16 hi + lo) of the higher-precision forward, or NULL
  T* kc_lo;
  T* vt_lo;
  float qscale;  // Q is stored times qscale (rounded once, after the scaling)
  __device__ __forceinline__ void operator()(int m, int n, float v, int = 0) const {
    if (m >= M) return;
    v += bias[n];
    const int which = n / d, hd = n - which * d;
    if (which == 0) {
      q[(size_t)m * d + hd] = from_f32<T>(v * qscale);
      return;
    }
    const int nn = m / R, t = m - nn * R, p = pos_base + t;
    const int head = hd / dh, e = hd - head * dh;
    const size_t base = (size_t)nn * H + head;
    if (which == 1)
      kc[(base * Lcap + p) * dh + e] = from_f32<T>(v);
    else
      vt[(base * dh + e) * Lcap + p] = from_f32<T>(v);
  }
  __device__ __forceinline__ void at_split(int) {}
  __device__ __forceinline__ float4 bias4(int n) const { return *(const float4*)(bias + n); }
  __device__ __forceinline__ void store4(int m, int n, f32x4 v, float4 b) const {
    if (m >= M) return;
    const int which = n >> log2d, hd = n & (d - 1);
    const float sc = which == 0 ? qscale : 1.0f;
    const float v0 = (v[0] + b.x) * sc, v1 = (v[1] + b.y) * sc, v2 = (v[2] + b.z) * sc,
                v3 = (v[3] + b.w) * sc;
    const T h0 = from_f32<T>(v0), h1 = from_f32<T>(v1), h2 = from_f32<T>(v2),
            h3 = from_f32<T>(v3);
    const bool split = q_lo != nullptr;
    const float l0 = v0 - to_f32(h0), l1 = v1 - to_f32(h1), l2 = v2 - to_f32(h2),
                l3 = v3 - to_f32(h3);
    if (which == 0) {
      store_vec4(q + (size_t)m * d + hd, v0, v1, v2, v3);
      if (split) store_vec4(q_lo + (size_t)m * d + hd, l0, l1, l2, l3);
      return;
    }
    const int nn = m / R, t = m - nn * R, p = pos_base + t;
    const int head = hd >> log2dh, e = hd & (dh - 1);
    const size_t base = (size_t)nn * H + head;
    if (which == 1) {
      store_vec4(kc + (base * Lcap + p) * dh + e, v0, v1, v2, v3);
      if (split) store_vec4(kc_lo + (base * Lcap + p) * dh + e, l0, l1, l2, l3);
    } else {
      const size_t o = (base * dh + e) * Lcap + p;
      vt[o] = h0;
      vt[o + Lcap] = h1;
      vt[o + 2 * (size_t)Lcap] = h2;
      vt[o + 3 * (size_t)Lcap] = h3;
      if (split) {
        vt_lo[o] = from_f32<T>(l0);
        vt_lo[o + Lcap] = from_f32<T>(l1);
        vt_lo[o + 2 * (size_t)Lcap] = from_f32<T>(l2);
        vt_lo[o + 3 * (size_t)Lcap] = from_f32<T>(l3);
      }
    }
  }
};

struct EpiResid {
  const float* bias;
  float* h;
  int M, N;
  __device__ __forceinline__ void operator()(int m, int n, float v, int = 0) const {
    if (m >= M) return;
    float* p = h + (size_t)m * N + n;
    *p = *p + (v + bias[n]);
  }
  __device__ __forceinline__ void at_split(int) {}
  __device__ __forceinline__ float4 bias4(int n) const { return *(const float4*)(bias + n); }
  __device__ __forceinline__ void store4(int m, int n, f32x4 v, float4 b) const {
    if (m >= M) return;
    float4* p = (float4*)(h + (size_t)m * N + n);
    float4 o = *p;
    o.x += v[0] + b.x;
    o.y += v[1] + b.y;
    o.z += v[2] + b.z;
    o.w += v[3] + b.w;
    *p = o;
  }
};

template <class T>
struct EpiGelu {
  const float* bias;
  T* out;
  int M, N;
  T* out_lo;   // split output of the higher-precision forward, or NULL
  __device__ __forceinline__ void operator()(int m, int n, float v, int = 0) const {
    if (m >= M) return;
    out[(size_t)m * N + n] = from_f32<T>(gelu_erf(v + bias[n]));
  }
  __device__ __forceinline__ void at_split(int) {}
  __device__ __forceinline__ float4 bias4(int n) const { return *(const float4*)(bias + n); }
  __device__ __forceinline__ void store4(int m, int n, f32x4 v, float4 b) const {
    if (m >= M) return;
    const float g0 = gelu_erf(v[0] + b.x), g1 = gelu_erf(v[1] + b.y),
                g2 = gelu_erf(v[2] + b.z), g3 = gelu_erf(v[3] + b.w);
    store_vec4(out + (size_t)m * N + n, g0, g1, g2, g3);
    if (out_lo)
      store_vec4(out_lo + (size_t)m * N + n, g0 - to_f32(from_f32<T>(g0)),
                 g1 - to_f32(from_f32<T>(g1)), g2 - to_f32(from_f32<T>(g2)),
                 g3 - to_f32(from_f32<T>(g3)));
  }
};

struct EpiF32 {
  const float* bias;
  float* out;
  int M, N;
  __device__ __forceinline__ void operator()(int m, int n, float v, int = 0) const {
    if (m >= M) return;
    out[(size_t)m * N + n] = v + (bias ? bias[n] : 0.f);
  }
  __device__ __forceinline__ void at_split(int) {}
  __device__ __forceinline__ float4 bias4(int n) const {
    return bias ? *(const float4*)(bias + n) : float4{0.f, 0.f, 0.f, 0.f};
  }
  __device__ __forceinline__ void store4(int m, int n, f32x4 v, float4 b) const {
    if (m >= M) return;
    *(float4*)(out + (size_t)m * N + n) =
        float4{v[0] + b.x, v[1] + b.y, v[2] + b.z, v[3] + b.w};
  }
};

// fp32 split-K partial planes out[s][M][N] (the consumer sums them).
struct EpiPlane {
  float* out;
  int M, N;
  __device__ __forceinline__ void operator()(int m, int n, float v, int split) const {
    if (m >= M) return;
    out[((size_t)split * M + m) * N + n] = v;
  }
};

// Split-K partial: fp32 slab [S][M][N]; a reduce kernel adds the slabs in a
// fixed order (deterministic) and applies the residual epilogue.
struct EpiSlab {
  float* slab;   // plane s of split s at slab + s * M * N
  int M, N;
  __device__ __forceinline__ void at_split(int s) { slab += (size_t)s * M * N; }
  __device__ __forceinline__ float4 bias4(int) const { return float4{0.f, 0.f, 0.f, 0.f}; }
  __device__ __forceinline__ void store4(int m, int n, f32x4 v, float4) const {
    if (m >= M) return;
    *(float4*)(slab + (size_t)m * N + n) = float4{v[0], v[1], v[2], v[3]};
  }
};

// ---------------------------------------------------------------------------
// bf16 MFMA GEMM (gfx950 v_mfma_f32_16x16x32_bf16, wave64).
//
// Computes the transposed product D = W A^T tile by tile so that each lane's
// accumulator holds four consecutive output features of one row, which the
// epilogues store as one vector.  Fragment layout of the MFMA: lane l
// supplies A-operand row l%16 / B-operand column l%16 with k = 8*(l/16)..+8,
// and receives D[4*(l/16) + r][l%16], r = 0..3.  Here the A operand is a W
// row (output feature) and the B operand an activation row (token).
//
// Block tile BM = 32*TM tokens x BN = 32*TN features x 64, 4 waves in 2 x 2,
// wave tile 16*TM x 16*TN.  TM = 7 gives 224-row tiles: a 1560-token frame
// (and every multiple of it) then pads by only 0.5%.  Two LDS buffers (rows
// padded to 144 B: conflict-free 16-byte fragment reads).  Blocks are mapped
// XCD-aware by gemm_unit_of (each XCD works on one split's K range and one
// column group of tiles, keeping its operand panels in its own L2).
// One register stage: the global loads of tile k+1 are in flight while tile
// k is multiplied (a second stage costs more registers than it hides).
// The grid holds tiles * S blocks; split s covers K range [s*k_len,
// (s+1)*k_len).  Requirements: N % BN == 0, k_len % 64 == 0.
// ---------------------------------------------------------------------------
template <int TM_, int TN_>
struct GemmCfg {
  static constexpr int TM = TM_, TN = TN_;
  static constexpr int NT = 256, BK = 64, LDS = BK + 8, CPR = BK / 8;
  static constexpr int WM = 16 * TM, WN = 16 * TN, BM = 2 * WM, BN = 2 * WN;
  static constexpr int CA = BM * CPR / NT, CB = BN * CPR / NT;
  static_assert(BM * CPR % NT == 0 && BN * CPR % NT == 0, "tile/threads");
};

template <class G, bool SPLIT>
__device__ __forceinline__ void gemm_gload(u32x4 (&ra)[G::CA], u32x4 (&ral)[G::CA],
                                           u32x4 (&rb)[G::CB],
                                           const bf16* __restrict__ A,
                                           const bf16* __restrict__ Alo,
                                           const bf16* __restrict__ W, int m0,
                                           int n0, int M, int K, int k0, int tid) {
#pragma unroll
  for (int i = 0; i < G::CA; ++i) {
    const int c = tid + i * G::NT, row = c / G::CPR, kc = c - row * G::CPR;
    const int gm = min(m0 + row, M - 1);
    ra[i] = *(const u32x4*)(A + (size_t)gm * K + k0 + kc * 8);
    if (SPLIT) ral[i] = *(const u32x4*)(Alo + (size_t)gm * K + k0 + kc * 8);
  }
#pragma unroll
  for (int i = 0; i < G::CB; ++i) {
    const int c = tid + i * G::NT, row = c / G::CPR, kc = c - row * G::CPR;
    rb[i] = *(const u32x4*)(W + (size_t)(n0 + row) * K + k0 + kc * 8);
  }
}

template <class G, bool SPLIT>
__device__ __forceinline__ void gemm_lstore(const u32x4 (&ra)[G::CA],
                                            const u32x4 (&ral)[G::CA],
                                            const u32x4 (&rb)[G::CB], bf16* sA,
                                            bf16* sAl, bf16* sB, int tid) {
#pragma unroll
  for (int i = 0; i < G::CA; ++i) {
    const int c = tid + i * G::NT, row = c / G::CPR, kc = c - row * G::CPR;
    *(u32x4*)(sA + row * G::LDS + kc * 8) = ra[i];
    if (SPLIT) *(u32x4*)(sAl + row * G::LDS + kc * 8) = ral[i];
  }
#pragma unroll
  for (int i = 0; i < G::CB; ++i) {
    const int c = tid + i * G::NT, row = c / G::CPR, kc = c - row * G::CPR;
    *(u32x4*)(sB + row * G::LDS + kc * 8) = rb[i];
  }
}

// SPLIT: the activation tile is a bf16 pair (hi + lo) and both halves are
// multiplied by the (exact bf16) weights into the same accumulator.
template <class G, bool SPLIT>
__device__ __forceinline__ void gemm_compute(f32x4 (&acc)[G::TN][G::TM],
                                             const bf16* sA, const bf16* sAl,
                                             const bf16* sB, int wm, int wn, int lane) {
  const int fr = lane & 15, fk = (lane >> 4) * 8;
#pragma unroll
  for (int ks = 0; ks < G::BK / 32; ++ks) {
    bf16x8 wf[G::TN], af[G::TM];
#pragma unroll
    for (int j = 0; j < G::TN; ++j)
      wf[j] = *(const bf16x8*)(sB + (wn * G::WN + j * 16 + fr) * G::LDS + ks * 32 + fk);
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
      af[i] = *(const bf16x8*)(sA + (wm * G::WM + i * 16 + fr) * G::LDS + ks * 32 + fk);
#pragma unroll
    for (int j = 0; j < G::TN; ++j)
#pragma unroll
      for (int i = 0; i < G::TM; ++i)
        acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j], af[i], acc[j][i], 0, 0, 0);
    if (SPLIT) {
#pragma unroll
      for (int i = 0; i < G::TM; ++i)
        af[i] = *(const bf16x8*)(sAl + (wm * G::WM + i * 16 + fr) * G::LDS + ks * 32 + fk);
#pragma unroll
      for (int j = 0; j < G::TN; ++j)
#pragma unroll
        for (int i = 0; i < G::TM; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j], af[i], acc[j][i], 0, 0, 0);
    }
  }
}

// Split index and tile (tm, tn) of block b among S splits of a
// tiles_m x tiles_n grid.  Consecutive block ids go to different XCDs (b & 7),
// so when the splits and the tile columns divide over the 8 XCDs, XCD x takes
// split x / (8 / S) and column group x % (8 / S) of it: each XCD then reads
// one split's K range of the activations and one column group's rows of W,
// and keeps them in its own L2.  Other shapes are mapped row-major.
__device__ __forceinline__ void gemm_unit_of(int b, int S, int tiles_m, int tiles_n,
                                             int& tm, int& tn, int& split) {
  if (S <= 8 && (8 % S) == 0 && tiles_n % (8 / S) == 0) {
    const int xcd = b & 7, local = b >> 3, G = 8 / S, gw = tiles_n / G;
    split = xcd / G;
    tm = local / gw;
    tn = (xcd - split * G) * gw + (local - tm * gw);
  } else {
    const int tiles = tiles_m * tiles_n;
    split = b / tiles;
    const int p = b - split * tiles;
    tm = p / tiles_n;
    tn = p - tm * tiles_n;
  }
}

template <int TM, int TN, bool SPLIT, class Epi>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ Alo,
    const bf16* __restrict__ W, int M, int N, int K, int k_len, Epi epi) {
  using G = GemmCfg<TM, TN>;
  __shared__ __attribute__((aligned(16))) bf16 sA[2][G::BM * G::LDS];
  __shared__ __attribute__((aligned(16))) bf16 sAl[2][SPLIT ? G::BM * G::LDS : 8];
  __shared__ __attribute__((aligned(16))) bf16 sB[2][G::BN * G::LDS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_n = N / G::BN;
  const int tiles_m = (M + G::BM - 1) / G::BM;
  int tm, tn, split;
  gemm_unit_of(blockIdx.x, gridDim.x / (tiles_m * tiles_n), tiles_m, tiles_n, tm, tn, split);
  epi.at_split(split);
  const int m0 = tm * G::BM, n0 = tn * G::BN;
  const int kb = split * k_len;
  const int KT = k_len / G::BK;

  f32x4 acc[G::TN][G::TM];
#pragma unroll
  for (int j = 0; j < G::TN; ++j)
#pragma unroll
    for (int i = 0; i < G::TM; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  {
    u32x4 ra[G::CA], ral[G::CA], rb[G::CB];
    gemm_gload<G, SPLIT>(ra, ral, rb, A, Alo, W, m0, n0, M, K, kb, tid);
    gemm_lstore<G, SPLIT>(ra, ral, rb, sA[0], sAl[0], sB[0], tid);
    __syncthreads();
#pragma clang loop unroll(disable)
    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < KT)
        gemm_gload<G, SPLIT>(ra, ral, rb, A, Alo, W, m0, n0, M, K, kb + (kt + 1) * G::BK, tid);
      gemm_compute<G, SPLIT>(acc, sA[cur], sAl[cur], sB[cur], wm, wn, lane);
      if (kt + 1 < KT)
        gemm_lstore<G, SPLIT>(ra, ral, rb, sA[cur ^ 1], sAl[cur ^ 1], sB[cur ^ 1], tid);
      __syncthreads();
    }
  }

  const int mb = m0 + wm * G::WM + (lane & 15);
  const int nb = n0 + wn * G::WN + 4 * (lane >> 4);
#pragma unroll
  for (int j = 0; j < G::TN; ++j)
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
      epi.store4(mb + i * 16, nb + j * 16, acc[j][i], epi.bias4(nb + j * 16));
}

// ---------------------------------------------------------------------------
// bf16 MFMA GEMM with direct global->LDS loads (gfx950 global_load_lds_dwordx4).
//
// Same block tiles, fragment layout and epilogues as gemm_bf16_kernel, with
// 8 waves (two per SIMD).  The per-CU rate of LDS DMA grows with the number
// of waves issuing it (about 26 B/clk with four waves, 37 with eight, from an
// L2-resident source), so all eight waves load, and they split the work of a
// k-tile instead of the output tile: waves 0-3 (group 0) multiply k-slice
// 0..31 of every 64-wide k-tile and waves 4-7 (group 1) slice 32..63, each
// over the full 2 x 2 wave-tile grid.  The two partial accumulators are added
// through LDS at the end (fixed order: deterministic).
//
// Operand tiles go from global memory straight into LDS through a 3-stage
// ring (tiles kt+1 and kt+2 in flight while kt is multiplied).  A DMA
// wave-instruction writes 64 consecutive 16-byte LDS slots (lane i -> slot
// i); each lane therefore chooses which global chunk lands in its slot, and
// the tile is stored XOR-swizzled: chunk c of row r sits at slot
// 8r + (c ^ (r & 7)), which makes the 16-byte fragment reads (16 rows, one
// chunk) conflict-free without padding.  One instruction moves 8 rows; the
// BM/8 + BN/8 instructions of a stage are dealt round-robin to the 8 waves.
//
// The DMA is issued from inline asm (saddr form: 64-bit uniform base in SGPRs
// + 32-bit per-lane byte offset) and every wait on it is explicit; with the
// builtin, the compiler's own wait insertion cannot tell the ring buffers
// apart across the loop back-edge and drains every DMA at the loop head.
// Only these asm statements write M0 in the kernel.
// Requirements: N % BN == 0, k_len % 64 == 0, M * K * 2 and N * K * 2 below
// 4 GiB (32-bit offsets).
// ---------------------------------------------------------------------------

template <int TM_, int TN_>
struct DmaCfg {
  static constexpr int TM = TM_, TN = TN_;
  static constexpr int WM = 16 * TM, WN = 16 * TN, BM = 2 * WM, BN = 2 * WN, BK = 64;
  static constexpr int NA = BM / 8, NB = BN / 8;       // DMA instructions per stage
  static_assert(NA % 4 == 0 && NB % 4 == 0, "instructions split evenly per wave group");
  static constexpr int CA = (NA + 7) / 8, CB = (NB + 7) / 8;   // per wave, at most
  // instructions per stage of a wave in group 0 / group 1
  static constexpr int IPW0 = (NA + 7) / 8 + (NB + 7) / 8;
  static constexpr int IPW1 = (NA + 3) / 8 + (NB + 3) / 8;
  static constexpr int STAGE = (BM + BN) * BK;         // bf16 elements per stage
};


// Wait until at most N of this wave's vector-memory loads are outstanding and
// all its LDS reads have returned, then barrier.  The asm is a compiler memory
// barrier as well, so no LDS access moves across it.
template <int N>
__device__ __forceinline__ void dma_sync() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(N) : "memory");
}

// The same with the vmcnt of this wave's group; PENDING = stages issued
// after the one waited for.
template <class G, int PENDING>
__device__ __forceinline__ void dma_sync_group(int grp) {
  if (grp == 0) dma_sync<PENDING * G::IPW0>();
  else dma_sync<PENDING * G::IPW1>();
}

// Per-lane byte offsets of this wave's DMA chunks (k offset 0).
template <class G>
__device__ __forceinline__ void dma_offsets(uint32_t (&va)[G::CA], uint32_t (&vb)[G::CB],
                                            int m0, int n0, int M, int K, int wave,
                                            int lane) {
#pragma unroll
  for (int i = 0; i < G::CA; ++i) {
    const int q = min(wave + 8 * i, G::NA - 1);
    const int r = 8 * q + (lane >> 3), c = (lane & 7) ^ (r & 7);
    va[i] = ((uint32_t)min(m0 + r, M - 1) * (uint32_t)K + c * 8) * 2u;
  }
#pragma unroll
  for (int i = 0; i < G::CB; ++i) {
    const int q = min(wave + 8 * i, G::NB - 1);
    const int r = 8 * q + (lane >> 3), c = (lane & 7) ^ (r & 7);
    vb[i] = ((uint32_t)(n0 + r) * (uint32_t)K + c * 8) * 2u;
  }
}

// This wave's share of the DMA of the k-tile at column k0 into the stage at
// LDS address st.
template <class G>
__device__ __forceinline__ void dma_issue(const bf16* A, const bf16* W,
                                          const uint32_t (&va)[G::CA],
                                          const uint32_t (&vb)[G::CB], uint32_t st, int k0,
                                          int wave) {
  const bf16* ak = A + k0;
  const bf16* wk = W + k0;
#pragma unroll
  for (int i = 0; i < G::CA; ++i)
    if (wave + 8 * i < G::NA) dma16(ak, va[i], st + (wave + 8 * i) * 1024);
#pragma unroll
  for (int i = 0; i < G::CB; ++i)
    if (wave + 8 * i < G::NB) dma16(wk, vb[i], st + G::BM * 128 + (wave + 8 * i) * 1024);
}

template <class G>
struct Frags {
  bf16x8 w[G::TN], a[G::TM];
};

// Fragments of k-slice ks (0 or 1) of a stage.
template <class G>
__device__ __forceinline__ void frag_load(Frags<G>& f, const bf16* stage, int ks, int wm,
                                          int wn, int lane) {
  const bf16* sA = stage;
  const bf16* sB = stage + G::BM * G::BK;
  const int fr = lane & 15, c = ks * 4 + (lane >> 4), sw = (c ^ (lane & 7)) << 3;
#pragma unroll
  for (int j = 0; j < G::TN; ++j)
    f.w[j] = *(const bf16x8*)(sB + (wn * G::WN + j * 16 + fr) * 64 + sw);
#pragma unroll
  for (int i = 0; i < G::TM; ++i)
    f.a[i] = *(const bf16x8*)(sA + (wm * G::WM + i * 16 + fr) * 64 + sw);
}

template <class G>
__device__ __forceinline__ void frag_mma(f32x4 (&acc)[G::TN][G::TM], const Frags<G>& f) {
#pragma unroll
  for (int j = 0; j < G::TN; ++j)
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
      acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.w[j], f.a[i], acc[j][i], 0, 0, 0);
}

// One k-step: wait for tile kt, issue tile kt+2 into the buffer of tile kt-1,
// multiply this group's k-slice of tile kt.
template <class G, int PENDING>
__device__ __forceinline__ void dma_step(f32x4 (&acc)[G::TN][G::TM], const bf16* A,
                                         const bf16* W, const uint32_t (&va)[G::CA],
                                         const uint32_t (&vb)[G::CB], const bf16* cur,
                                         const bf16* nxt, int k_issue, bool issue, int wave,
                                         int grp, int wm, int wn, int lane) {
  dma_sync_group<G, PENDING>(grp);
  if (issue) dma_issue<G>(A, W, va, vb, lds_address(nxt), k_issue, wave);
  Frags<G> f;
  frag_load<G>(f, cur, grp, wm, wn, lane);
  // raised wave priority while this wave multiplies: its MFMAs issue ahead
  // of the other waves' loads and fragment reads (the QKV GEMM alone at 1560
  // rows: 18.7 -> 17.9 us)
  __builtin_amdgcn_s_setprio(1);
  frag_mma<G>(acc, f);
  __builtin_amdgcn_s_setprio(0);
}

template <int TM, int TN, class Epi>
__global__ __launch_bounds__(512) void gemm_bf16_dma_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ W, int M, int N, int K,
    int k_len, Epi epi) {
  using G = DmaCfg<TM, TN>;
  __shared__ __attribute__((aligned(1024))) bf16 ring[3 * G::STAGE];
  bf16* const s0 = ring;
  bf16* const s1 = ring + G::STAGE;
  bf16* const s2 = ring + 2 * G::STAGE;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wm = (wave >> 1) & 1, wn = wave & 1;
  const int tiles_n = N / G::BN;
  const int tiles_m = (M + G::BM - 1) / G::BM;
  int tm, tn, split;
  gemm_unit_of(blockIdx.x, gridDim.x / (tiles_m * tiles_n), tiles_m, tiles_n, tm, tn, split);
  epi.at_split(split);
  const int m0 = tm * G::BM, n0 = tn * G::BN;
  const int kb = split * k_len;
  const int KT = k_len / G::BK;

  f32x4 acc[G::TN][G::TM];
#pragma unroll
  for (int j = 0; j < G::TN; ++j)
#pragma unroll
    for (int i = 0; i < G::TM; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint32_t va[G::CA], vb[G::CB];
  dma_offsets<G>(va, vb, m0, n0, M, K, wave, lane);
  dma_issue<G>(A, W, va, vb, lds_address(s0), kb, wave);
  if (KT > 1) dma_issue<G>(A, W, va, vb, lds_address(s1), kb + G::BK, wave);

  // steady state: tile kt + 1 stays in flight while waiting for tile kt
  int kt = 0;
#pragma clang loop unroll(disable)
  for (; kt + 3 < KT; kt += 3) {
    dma_step<G, 1>(acc, A, W, va, vb, s0, s2, kb + (kt + 2) * G::BK, true, wave, grp, wm, wn, lane);
    dma_step<G, 1>(acc, A, W, va, vb, s1, s0, kb + (kt + 3) * G::BK, true, wave, grp, wm, wn, lane);
    dma_step<G, 1>(acc, A, W, va, vb, s2, s1, kb + (kt + 4) * G::BK, kt + 4 < KT, wave, grp, wm, wn, lane);
  }
  // tail; the buffer of tile t is t % 3
  for (; kt < KT; ++kt) {
    const int b = kt % 3;
    const bf16* cur = b == 0 ? s0 : b == 1 ? s1 : s2;
    const bf16* nxt = b == 0 ? s2 : b == 1 ? s0 : s1;
    if (kt + 1 < KT)
      dma_step<G, 1>(acc, A, W, va, vb, cur, nxt, kb + (kt + 2) * G::BK, kt + 2 < KT, wave, grp, wm, wn, lane);
    else
      dma_step<G, 0>(acc, A, W, va, vb, cur, nxt, 0, false, wave, grp, wm, wn, lane);
  }

  // Add the two groups' partial sums: group 0 finishes column fragments
  // j < JH, group 1 the rest; each hands the other half to its partner wave
  // (same wm, wn) through LDS, which the ring no longer needs.  The epilogue's
  // bias values are loaded first, so their latency hides under the exchange.
  constexpr int JH = (G::TN + 1) / 2;
  static_assert(G::TN * G::TM * 4 * 64 * 16 <= 3 * G::STAGE * 2, "reduction fits the ring");
  float4* red = (float4*)ring;
  const int wq = wave & 3;
  const int mb = m0 + wm * G::WM + (lane & 15);
  const int nb = n0 + wn * G::WN + 4 * (lane >> 4);
  float4 bv[JH];
#pragma unroll
  for (int jl = 0; jl < JH; ++jl) {
    const int j = grp == 0 ? jl : min(JH + jl, G::TN - 1);
    bv[jl] = epi.bias4(nb + j * 16);
  }
  dma_sync<0>();   // every wave is done reading the ring
#pragma unroll
  for (int j = 0; j < G::TN; ++j) {
    if ((j < JH) == (grp == 0)) continue;
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
      red[((wq * G::TN + j) * G::TM + i) * 64 + lane] =
          float4{acc[j][i][0], acc[j][i][1], acc[j][i][2], acc[j][i][3]};
  }
  dma_sync<0>();
#pragma unroll
  for (int j = 0; j < G::TN; ++j) {
    if ((j < JH) != (grp == 0)) continue;
    // j is a compile-time constant here: group 0 holds j < JH in bv[j],
    // group 1 holds j >= JH in bv[j - JH]
    const float4 b = j < JH ? bv[j < JH ? j : 0] : bv[j >= JH ? j - JH : 0];
#pragma unroll
    for (int i = 0; i < G::TM; ++i) {
      const float4 o = red[((wq * G::TN + j) * G::TM + i) * 64 + lane];
      f32x4 v = acc[j][i];
      // group 0's partial first: the same order in both halves
      if (grp == 0) v = f32x4{v[0] + o.x, v[1] + o.y, v[2] + o.z, v[3] + o.w};
      else v = f32x4{o.x + v[0], o.y + v[1], o.z + v[2], o.w + v[3]};
      epi.store4(mb + i * 16, nb + j * 16, v, b);
    }
  }
}

// h[m, n] += bias[n] + sum_s slab[s][m][n], summed in split order.
__global__ __launch_bounds__(256) void splitk_resid_kernel(
    const float* __restrict__ slab, const float* __restrict__ bias,
    float* __restrict__ h, int M, int N, int S) {
  const size_t total4 = (size_t)M * N / 4;
  const size_t plane = (size_t)M * N;
  for (size_t e = blockIdx.x * 256ull + threadIdx.x; e < total4; e += (size_t)gridDim.x * 256) {
    const size_t o = e * 4;
    const int n = (int)(o % N);
    float4 acc = *(const float4*)(slab + o);
    for (int s = 1; s < S; ++s) {
      const float4 v = *(const float4*)(slab + s * plane + o);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    const float4 b = *(const float4*)(bias + n);
    float4 hv = *(float4*)(h + o);
    hv.x += acc.x + b.x;
    hv.y += acc.y + b.y;
    hv.z += acc.z + b.z;
    hv.w += acc.w + b.w;
    *(float4*)(h + o) = hv;
  }
}

// ---------------------------------------------------------------------------
// fp32 SIMT GEMM: 64 x 64 block tile, BK = 16, 4 x 4 outputs per thread.
// Requirements: K % 16 == 0; M, N arbitrary.
// ---------------------------------------------------------------------------
template <class Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(
    const float* __restrict__ A, const float* __restrict__ W, int M, int N,
    int K, int k_len, Epi epi) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float sA[BK][BM + 4];
  __shared__ float sB[BK][BN + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int tiles_n = (N + BN - 1) / BN;
  const int tiles = ((M + BM - 1) / BM) * tiles_n;
  const int split = blockIdx.x / tiles, tile = blockIdx.x - split * tiles;
  const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  float acc[4][4] = {};
  const int lrow = tid >> 2, lk = (tid & 3) * 4;
  const int gm = min(m0 + lrow, M - 1), gn = min(n0 + lrow, N - 1);
  for (int k0 = split * k_len; k0 < (split + 1) * k_len; k0 += BK) {
    const float4 va = *(const float4*)(A + (size_t)gm * K + k0 + lk);
    const float4 vb = *(const float4*)(W + (size_t)gn * K + k0 + lk);
    __syncthreads();
    sA[lk + 0][lrow] = va.x;
    sA[lk + 1][lrow] = va.y;
    sA[lk + 2][lrow] = va.z;
    sA[lk + 3][lrow] = va.w;
    sB[lk + 0][lrow] = vb.x;
    sB[lk + 1][lrow] = vb.y;
    sB[lk + 2][lrow] = vb.z;
    sB[lk + 3][lrow] = vb.w;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sB[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx + 16 * j;
      if (n < N) epi(m0 + ty + 16 * i, n, acc[i][j], split);
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
// Tile configurations (TM, TN) of the bf16 GEMM, and the choice per shape:
// the fewest "rounds" of 256 blocks (one per CU) weighted by the work per
// block, with K splits allowed only where the epilogue can reduce them.
struct TileChoice {
  int tm, tn, splits;
};
static const int kTileCfgs[][2] = {{7, 4}, {7, 3}, {7, 2}, {4, 4}, {4, 2}};

// Tile and split choice from a cost model fitted to measured launches at
// 1560 rows (bf16, d = 1024): a block's time grows with its operand bytes,
// (BM + BN) * K / S (the per-CU load path sets the pace), and with its output
// tile, BM * BN (epilogue); blocks beyond 256 take another round; each extra
// split plane costs its consumer one more fp32 [M, N] read (0.82 us per plane
// at 1560 x 1024, from the residual + LayerNorm kernel with one and with four
// planes).  At 1560 rows this makes MLP2 (K = 4096) two planes of 128 x 128
// tiles rather than four of 224 x 128: 2% faster per Jacobi update.  The
// halves of a row-split update (two 780-row passes side by side) cap the
// planes at two: MLP2 as (4, 4) split 2 rather than the model's (4, 4) split
// 4 made the 21-frame video inverse 1.8% faster (the model, which gives each
// launch the whole chip, also preferred (7, 4) split 4 when given half of it:
// +0.7% only).
TileChoice gemm_choose(int M, int N, int K, bool allow_split, bool split_a = false,
                       int max_splits = 8) {
  TileChoice best{4, 2, 1};
  double best_cost = 1e300;
  for (auto& c : kTileCfgs) {
    if (split_a && c[0] > 4) continue;   // hi + lo activation tiles must fit LDS
    const int BM = 32 * c[0], BN = 32 * c[1];
    if (N % BN) continue;
    const long tiles = (long)((M + BM - 1) / BM) * (N / BN);
    for (int s = 1; s <= (allow_split ? max_splits : 1); s *= 2) {
      if (K % (64 * s) || (s > 1 && K / s < 256)) break;
      const long rounds = (tiles * s + 255) / 256;
      const double per_block = 4.28e-5 * (BM + BN) * (double)(K / s) + 4.66e-4 * BM * BN;
      const double cost = rounds * per_block + 6.7e-7 * (s - 1) * (double)M * N;
      if (cost < best_cost) {
        best_cost = cost;
        best = TileChoice{c[0], c[1], s};
      }
    }
  }
  return best;
}

namespace {
thread_local hipEvent_t g_ev_start = nullptr, g_ev_stop = nullptr;
}

void set_gemm_events(hipEvent_t start, hipEvent_t stop) {
  g_ev_start = start;
  g_ev_stop = stop;
}

bool gemm_events_pending() { return g_ev_start != nullptr; }

template <int TM, int TN, bool SPLIT, class Epi>
static void launch_cfg(const void* A, const void* Alo, const void* W, int M, int N,
                       int K, int splits, const Epi& epi, hipStream_t st) {
  using G = GemmCfg<TM, TN>;
  const int tiles = ((M + G::BM - 1) / G::BM) * (N / G::BN);
  // events bracketing this kernel alone, when the profiler asked for them
  const hipEvent_t e0 = g_ev_start, e1 = g_ev_stop;
  g_ev_start = g_ev_stop = nullptr;
  if (SPLIT)
    hipExtLaunchKernelGGL((gemm_bf16_kernel<TM, TN, SPLIT, Epi>), dim3(tiles * splits),
                          dim3(256), 0, st, e0, e1, 0, (const bf16*)A, (const bf16*)Alo,
                          (const bf16*)W, M, N, K, K / splits, epi);
  else
    hipExtLaunchKernelGGL((gemm_bf16_dma_kernel<TM, TN, Epi>), dim3(tiles * splits),
                          dim3(512), 0, st, e0, e1, 0, (const bf16*)A, (const bf16*)W, M,
                          N, K, K / splits, epi);
}

// Alo != NULL selects the split (hi + lo) activation kernel.
template <class Epi>
static hipError_t run_bf16_cfg(const void* A, const void* Alo, const void* W, int M,
                               int N, int K, TileChoice c, const Epi& epi,
                               hipStream_t st) {
  if (Alo) {
    if (c.tm == 4 && c.tn == 4) launch_cfg<4, 4, true>(A, Alo, W, M, N, K, c.splits, epi, st);
    else launch_cfg<4, 2, true>(A, Alo, W, M, N, K, c.splits, epi, st);
    return hipGetLastError();
  }
  if (c.tm == 7 && c.tn == 4) launch_cfg<7, 4, false>(A, Alo, W, M, N, K, c.splits, epi, st);
  else if (c.tm == 7 && c.tn == 3) launch_cfg<7, 3, false>(A, Alo, W, M, N, K, c.splits, epi, st);
  else if (c.tm == 7 && c.tn == 2) launch_cfg<7, 2, false>(A, Alo, W, M, N, K, c.splits, epi, st);
  else if (c.tm == 4 && c.tn == 4) launch_cfg<4, 4, false>(A, Alo, W, M, N, K, c.splits, epi, st);
  else launch_cfg<4, 2, false>(A, Alo, W, M, N, K, c.splits, epi, st);
  return hipGetLastError();
}

template <class Epi>
static hipError_t run_bf16(const void* A, const void* Alo, const void* W, int M, int N,
                           int K, const Epi& epi, hipStream_t st) {
  TileChoice c = gemm_choose(M, N, K, false, Alo != nullptr);
  return run_bf16_cfg(A, Alo, W, M, N, K, c, epi, st);
}

int gemm_resid_splits(int M, int N, int K) {
  const int a = gemm_choose(M, N, K, true).splits, b = gemm_choose(M, N, K, true, true).splits;
  return a > b ? a : b;
}

static int ilog2(int v) {
  int r = 0;
  while ((1 << (r + 1)) <= v) ++r;
  return r;
}

template <class Epi>
static hipError_t run_f32(const void* A, const void* W, int M, int N, int K,
                          const Epi& epi, hipStream_t st, int splits = 1) {
  const int tiles = ((M + 63) / 64) * ((N + 63) / 64);
  hipLaunchKernelGGL((gemm_f32_kernel<Epi>), dim3(tiles * splits), dim3(256), 0, st,
                     (const float*)A, (const float*)W, M, N, K, K / splits, epi);
  return hipGetLastError();
}

int head_splits(int M, int N, int K) {
  const int tiles = ((M + 63) / 64) * ((N + 63) / 64);
  int s = 1;
  while (s < 16 && tiles * s * 2 <= 512 && K % (16 * s * 2) == 0 && K / (s * 2) >= 64) s *= 2;
  return s;
}

hipError_t launch_gemm_f32_planes(const float* A, const float* W, float* out, int M,
                                  int N, int K, int splits, hipStream_t st) {
  EpiPlane e{out, M, N};
  return run_f32(A, W, M, N, K, e, st, splits);
}

hipError_t launch_gemm_qkv(bool bf, const void* A, const void* Alo, const void* W,
                           const float* bias, int M, int N, int K, QKVDst d,
                           hipStream_t st) {
  if (bf) {
    // the bf16 attention takes Q in base-2 softmax units: Q / sqrt(dh) * log2(e)
    EpiQKV<bf16> e{bias, (bf16*)d.q, (bf16*)d.kc, (bf16*)d.vt, M, d.R, d.d, d.dh, d.H,
                   d.Lcap, d.pos_base, ilog2(d.d), ilog2(d.dh), (bf16*)d.q_lo,
                   (bf16*)d.kc_lo, (bf16*)d.vt_lo,
                   1.4426950408889634f / sqrtf((float)d.dh)};
    return run_bf16(A, Alo, W, M, N, K, e, st);
  }
  EpiQKV<float> e{bias, (float*)d.q, (float*)d.kc, (float*)d.vt, M, d.R, d.d, d.dh, d.H,
                  d.Lcap, d.pos_base, ilog2(d.d), ilog2(d.dh), nullptr, nullptr, nullptr,
                  1.0f};
  return run_f32(A, W, M, N, K, e, st);
}

hipError_t launch_gemm_resid(bool bf, const void* A, const void* Alo, const void* W,
                             const float* bias, float* h, int M, int N, int K,
                             float* slab, hipStream_t st) {
  if (!bf) {
    EpiResid e{bias, h, M, N};
    return run_f32(A, W, M, N, K, e, st);
  }
  TileChoice c = gemm_choose(M, N, K, slab != nullptr, Alo != nullptr);
  if (c.splits == 1) {
    EpiResid e{bias, h, M, N};
    return run_bf16_cfg(A, Alo, W, M, N, K, c, e, st);
  }
  EpiSlab es{slab, M, N};
  hipError_t err = run_bf16_cfg(A, Alo, W, M, N, K, c, es, st);
  if (err != hipSuccess) return err;
  const size_t total4 = (size_t)M * N / 4;
  const int blocks = (int)std::min<size_t>((total4 + 255) / 256, 2048);
  hipLaunchKernelGGL(splitk_resid_kernel, dim3(blocks), dim3(256), 0, st, slab, bias, h,
                     M, N, c.splits);
  return hipGetLastError();
}

hipError_t launch_gemm_partial(const void* A, const void* Alo, const void* W,
                               float* slab, int M, int N, int K, int* splits,
                               hipStream_t st, int max_splits) {
  TileChoice c = gemm_choose(M, N, K, true, Alo != nullptr, max_splits);
  *splits = c.splits;
  EpiSlab es{slab, M, N};
  return run_bf16_cfg(A, Alo, W, M, N, K, c, es, st);
}

hipError_t launch_gemm_gelu(bool bf, const void* A, const void* Alo, const void* W,
                            const float* bias, void* out, void* out_lo, int M, int N,
                            int K, hipStream_t st) {
  if (bf) {
    EpiGelu<bf16> e{bias, (bf16*)out, M, N, (bf16*)out_lo};
    return run_bf16(A, Alo, W, M, N, K, e, st);
  }
  EpiGelu<float> e{bias, (float*)out, M, N, nullptr};
  return run_f32(A, W, M, N, K, e, st);
}

hipError_t launch_gemm_f32out(bool bf, const void* A, const void* W,
                              const float* bias, float* out, int M, int N, int K,
                              hipStream_t st) {
  EpiF32 e{bias, out, M, N};
  return bf ? run_bf16(A, nullptr, W, M, N, K, e, st) : run_f32(A, W, M, N, K, e, st);
}

}  // namespace af
