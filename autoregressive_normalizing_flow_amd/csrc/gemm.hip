// Projection GEMMs of the AF block's Transformer: y[M, N] = A[M, K] W[N, K]^T
// + bias with a fused epilogue (QKV scatter into the KV cache, residual add
// into the fp32 stream, exact GELU, or plain fp32 store).
//
//  * bf16 path: MFMA kernel for gfx950 (v_mfma_f32_16x16x32_bf16), both
//    operands K-contiguous, LDS double-buffered with register prefetch.
//  * fp32 path: LDS-tiled SIMT kernel (also used for the fp32 head).
#include "common.h"
#include "kernels.h"

namespace af {

// ---------------------------------------------------------------------------
// epilogues: called once per output element with the fp32 accumulator
// ---------------------------------------------------------------------------
template <class T>
struct EpiQKV {
  const float* bias;
  T* q;
  T* kc;
  T* vt;
  int M, R, d, dh, H, Lcap, pos_base;
  __device__ __forceinline__ void operator()(int m, int n, float v) const {
    if (m >= M) return;
    v += bias[n];
    const int which = n / d, hd = n - which * d;
    if (which == 0) {
      q[(size_t)m * d + hd] = from_f32<T>(v);
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
};

struct EpiResid {
  const float* bias;
  float* h;
  int M, N;
  __device__ __forceinline__ void operator()(int m, int n, float v) const {
    if (m >= M) return;
    float* p = h + (size_t)m * N + n;
    *p = *p + (v + bias[n]);
  }
};

template <class T>
struct EpiGelu {
  const float* bias;
  T* out;
  int M, N;
  __device__ __forceinline__ void operator()(int m, int n, float v) const {
    if (m >= M) return;
    out[(size_t)m * N + n] = from_f32<T>(gelu_erf(v + bias[n]));
  }
};

struct EpiF32 {
  const float* bias;
  float* out;
  int M, N;
  __device__ __forceinline__ void operator()(int m, int n, float v) const {
    if (m >= M) return;
    out[(size_t)m * N + n] = v + (bias ? bias[n] : 0.f);
  }
};

// ---------------------------------------------------------------------------
// bf16 MFMA GEMM.  Block tile BM x BN x 64, waves arranged (BM/WM) x (BN/WN),
// each wave owns a WM x WN sub-tile of 16x16 MFMA accumulators.
// Requirements: N % BN == 0, K % 64 == 0; M arbitrary (rows clamped on load,
// masked on store).
// Fragment layout of v_mfma_f32_16x16x32_bf16 (wave64): lane l supplies
// A[l%16][8*(l/16) .. +8] and B[8*(l/16) .. +8][l%16], and receives
// D[4*(l/16) + r][l%16] for r = 0..3.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, class Epi>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void gemm_bf16_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ W, int M, int N, int K,
    Epi epi) {
  constexpr int WAVES_N = BN / WN;
  constexpr int NT = (BM / WM) * WAVES_N * 64;
  constexpr int BK = 64;
  constexpr int LDS = BK + 8;  // padded row stride (bf16 elements, 144 B)
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int CPR = BK / 8;  // 16-byte chunks per tile row
  constexpr int CA = BM * CPR / NT, CB = BN * CPR / NT;
  static_assert((BM * CPR) % NT == 0 && (BN * CPR) % NT == 0, "tile/threads");
  __shared__ __attribute__((aligned(16))) bf16 sA[2][BM * LDS];
  __shared__ __attribute__((aligned(16))) bf16 sB[2][BN * LDS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave - wm * WAVES_N;
  const int tiles_n = N / BN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;

  uint4 ra[CA], rb[CB];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int c = tid + i * NT, row = c / CPR, kc = c - row * CPR;
      const int gm = min(m0 + row, M - 1);
      ra[i] = *(const uint4*)(A + (size_t)gm * K + k0 + kc * 8);
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int c = tid + i * NT, row = c / CPR, kc = c - row * CPR;
      rb[i] = *(const uint4*)(W + (size_t)(n0 + row) * K + k0 + kc * 8);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int c = tid + i * NT, row = c / CPR, kc = c - row * CPR;
      *(uint4*)(&sA[buf][row * LDS + kc * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int c = tid + i * NT, row = c / CPR, kc = c - row * CPR;
      *(uint4*)(&sB[buf][row * LDS + kc * 8]) = rb[i];
    }
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KT = K / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  const int frag_row = lane & 15, frag_k = (lane >> 4) * 8;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *(const bf16x8*)(&sA[cur][(wm * WM + i * 16 + frag_row) * LDS +
                                          ks * 32 + frag_k]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *(const bf16x8*)(&sB[cur][(wn * WN + j * 16 + frag_row) * LDS +
                                           ks * 32 + frag_k]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j],
                                                              acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) lstore(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * WM + i * 16 + (lane >> 4) * 4 + r;
        const int n = n0 + wn * WN + j * 16 + (lane & 15);
        epi(m, n, acc[i][j][r]);
      }
}

// ---------------------------------------------------------------------------
// fp32 SIMT GEMM: 64 x 64 block tile, BK = 16, 4 x 4 outputs per thread.
// Requirements: K % 16 == 0; M, N arbitrary.
// ---------------------------------------------------------------------------
template <class Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(
    const float* __restrict__ A, const float* __restrict__ W, int M, int N,
    int K, Epi epi) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float sA[BK][BM + 4];
  __shared__ float sB[BK][BN + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int tiles_n = (N + BN - 1) / BN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  float acc[4][4] = {};
  const int lrow = tid >> 2, lk = (tid & 3) * 4;
  const int gm = min(m0 + lrow, M - 1), gn = min(n0 + lrow, N - 1);
  for (int k0 = 0; k0 < K; k0 += BK) {
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
      if (n < N) epi(m0 + ty + 16 * i, n, acc[i][j]);
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <class Epi>
static hipError_t run_bf16(const void* A, const void* W, int M, int N, int K,
                           const Epi& epi, hipStream_t st) {
  constexpr int BM = 128;
  if (N % 128 == 0) {
    const int tiles = ((M + BM - 1) / BM) * (N / 128);
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, 128, 64, 64, Epi>), dim3(tiles),
                       dim3(256), 0, st, (const bf16*)A, (const bf16*)W, M, N, K, epi);
  } else {
    const int tiles = ((M + BM - 1) / BM) * (N / 64);
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, 64, 32, 64, Epi>), dim3(tiles),
                       dim3(256), 0, st, (const bf16*)A, (const bf16*)W, M, N, K, epi);
  }
  return hipGetLastError();
}

template <class Epi>
static hipError_t run_f32(const void* A, const void* W, int M, int N, int K,
                          const Epi& epi, hipStream_t st) {
  const int tiles = ((M + 63) / 64) * ((N + 63) / 64);
  hipLaunchKernelGGL((gemm_f32_kernel<Epi>), dim3(tiles), dim3(256), 0, st,
                     (const float*)A, (const float*)W, M, N, K, epi);
  return hipGetLastError();
}

hipError_t launch_gemm_qkv(bool bf, const void* A, const void* W,
                           const float* bias, int M, int N, int K, QKVDst d,
                           hipStream_t st) {
  if (bf) {
    EpiQKV<bf16> e{bias, (bf16*)d.q, (bf16*)d.kc, (bf16*)d.vt, M, d.R, d.d,
                   d.dh, d.H, d.Lcap, d.pos_base};
    return run_bf16(A, W, M, N, K, e, st);
  }
  EpiQKV<float> e{bias, (float*)d.q, (float*)d.kc, (float*)d.vt, M, d.R, d.d,
                  d.dh, d.H, d.Lcap, d.pos_base};
  return run_f32(A, W, M, N, K, e, st);
}

hipError_t launch_gemm_resid(bool bf, const void* A, const void* W,
                             const float* bias, float* h, int M, int N, int K,
                             hipStream_t st) {
  EpiResid e{bias, h, M, N};
  return bf ? run_bf16(A, W, M, N, K, e, st) : run_f32(A, W, M, N, K, e, st);
}

hipError_t launch_gemm_gelu(bool bf, const void* A, const void* W,
                            const float* bias, void* out, int M, int N, int K,
                            hipStream_t st) {
  if (bf) {
    EpiGelu<bf16> e{bias, (bf16*)out, M, N};
    return run_bf16(A, W, M, N, K, e, st);
  }
  EpiGelu<float> e{bias, (float*)out, M, N};
  return run_f32(A, W, M, N, K, e, st);
}

hipError_t launch_gemm_f32out(bool bf, const void* A, const void* W,
                              const float* bias, float* out, int M, int N, int K,
                              hipStream_t st) {
  EpiF32 e{bias, out, M, N};
  return bf ? run_bf16(A, W, M, N, K, e, st) : run_f32(A, W, M, N, K, e, st);
}

}  // namespace af
