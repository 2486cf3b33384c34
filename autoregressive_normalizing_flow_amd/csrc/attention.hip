// Causal attention of the current chunk's queries over the KV cache.
//
// The keys are every cached position up to the query's own position (the
// finished blocks' K/V plus the chunk's, written by the QKV GEMM).  This is
// the "finished blocks feed a KV cache" step of the block-wise Jacobi schedule
// (STARFlow-V notes, papernotes.org, 关键设计 3) and the inclusive causal mask
// that follows the one-token shift (关键设计 1, self-exclusive mask).
//
// Cache layouts (per layer): K [N][H][Lcap][dh] (key rows contiguous) and V
// transposed, Vt [N][H][dh][Lcap] (keys contiguous per dimension), so that
// both MFMA operands below read contiguous runs from LDS.
#include "common.h"
#include "kernels.h"

namespace af {

// ---------------------------------------------------------------------------
// bf16 MFMA flash attention.  A workgroup owns 128 queries of one (sample,
// head); each of its 4 waves owns 32 queries (two 16-query blocks).  Per
// 64-key tile:  S^T = K Q^T  (A = K rows from LDS, B = Q held in registers),
// online softmax in fp32 along the key axis (the 4 lanes sharing a query
// combine with two xor-shuffles), then  O^T += Vt P^T  where P^T is already in
// the B-operand layout of the lanes that hold the scores: the 8 k-slots of
// lane l are keys {4(l/16)+j, 16+4(l/16)+j}, j < 4, of each 32-key step, and
// the Vt fragment reads the same keys (two 8-byte LDS reads).
// ---------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(256) void attn_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ kc,
    const bf16* __restrict__ vt, bf16* __restrict__ out, int R, int H, int d,
    int Lcap, int pos_base, float scale_log2) {
  constexpr int QWAVE = 32, QB = QWAVE / 16, QTILE = 4 * QWAVE;
  constexpr int KT = 64, KB = KT / 16, KS = DH / 32, DB = DH / 16;
  constexpr int KLDS = DH + 8, VLDS = KT + 8;
  constexpr int CK = KT * DH / 8 / 256;  // 16-byte chunks per thread per tile
  __shared__ __attribute__((aligned(16))) bf16 sK[2][KT * KLDS];
  __shared__ __attribute__((aligned(16))) bf16 sV[2][DH * VLDS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int head = blockIdx.y, n = blockIdx.z;
  const int q_lo = blockIdx.x * QTILE;
  const int q_hi = min(R, q_lo + QTILE);
  const int nk = pos_base + q_hi;  // keys 0..nk-1 can be attended
  const int n_tiles = (nk + KT - 1) / KT;
  const size_t hb = (size_t)n * H + head;
  const bf16* kbase = kc + hb * Lcap * DH;
  const bf16* vbase = vt + hb * DH * Lcap;
  const int l16 = lane & 15, lg = lane >> 4;

  bf16x8 qf[QB][KS];
  int qpos[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int t = q_lo + wave * QWAVE + qb * 16 + l16;
    qpos[qb] = pos_base + t;
    const bf16* qrow = q + ((size_t)n * R + min(t, R - 1)) * d + head * DH;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[qb][ks] = *(const bf16x8*)(qrow + ks * 32 + lg * 8);
  }

  float m_run[QB], l_run[QB];
  f32x4 acc_o[DB][QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -1e30f;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc_o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  uint4 rk[CK], rv[CK];
  auto gload = [&](int kt) {
    const int k0 = kt * KT;
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      const int c = tid + i * 256;
      const int key = c / (DH / 8), dc = c - key * (DH / 8);
      const int kk = k0 + key;
      rk[i] = kk < nk ? *(const uint4*)(kbase + (size_t)kk * DH + dc * 8)
                      : uint4{0u, 0u, 0u, 0u};
      const int drow = c / (KT / 8), kc8 = c - drow * (KT / 8);
      const int kk0 = k0 + kc8 * 8;  // k0 + 64 <= Lcap: always in bounds
      uint4 v = *(const uint4*)(vbase + (size_t)drow * Lcap + kk0);
      if (kk0 + 8 > nk) {
        union { uint4 u; unsigned short s[8]; } tmp;
        tmp.u = v;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (kk0 + e >= nk) tmp.s[e] = 0;
        v = tmp.u;
      }
      rv[i] = v;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      const int c = tid + i * 256;
      const int key = c / (DH / 8), dc = c - key * (DH / 8);
      *(uint4*)(&sK[buf][key * KLDS + dc * 8]) = rk[i];
      const int drow = c / (KT / 8), kc8 = c - drow * (KT / 8);
      *(uint4*)(&sV[buf][drow * VLDS + kc8 * 8]) = rv[i];
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < n_tiles; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < n_tiles) gload(kt + 1);

    f32x4 s[KB][QB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 kf =
            *(const bf16x8*)(&sK[cur][(kb * 16 + l16) * KLDS + ks * 32 + lg * 8]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qb][ks],
                                                              s[kb][qb], 0, 0, 0);
      }

    // online softmax (base 2) per query
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kt * KT + kb * 16 + lg * 4 + r;
          float v = s[kb][qb][r] * scale_log2;
          if (key > qpos[qb] || key >= nk) v = -INFINITY;
          s[kb][qb][r] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, AF_WAVE));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, AF_WAVE));
      const float m_new = fmaxf(m_run[qb], tmax);
      const float alpha = exp2f(m_run[qb] - m_new);
      m_run[qb] = m_new;
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = exp2f(s[kb][qb][r] - m_new);
          s[kb][qb][r] = p;
          lsum += p;
        }
      l_run[qb] = l_run[qb] * alpha + lsum;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc_o[db][qb] *= alpha;
    }

    // O^T += Vt P^T over two 32-key steps
#pragma unroll
    for (int c = 0; c < KT / 32; ++c) {
      bf16x8 pf[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pf[qb][r] = (bf16)s[2 * c][qb][r];
          pf[qb][4 + r] = (bf16)s[2 * c + 1][qb][r];
        }
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16* vrow = &sV[cur][(db * 16 + l16) * VLDS + c * 32 + lg * 4];
        const bf16x4 lo = *(const bf16x4*)vrow;
        const bf16x4 hi = *(const bf16x4*)(vrow + 16);
        const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          acc_o[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              vf, pf[qb], acc_o[db][qb], 0, 0, 0);
      }
    }
    if (kt + 1 < n_tiles) lstore(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float l = l_run[qb];
    l += __shfl_xor(l, 16, AF_WAVE);
    l += __shfl_xor(l, 32, AF_WAVE);
    const float inv = 1.0f / l;
    const int t = q_lo + wave * QWAVE + qb * 16 + l16;
    if (t < R) {
      bf16* orow = out + ((size_t)n * R + t) * d + head * DH;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        bf16x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = (bf16)(acc_o[db][qb][r] * inv);
        *(bf16x4*)(orow + db * 16 + lg * 4) = o;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 attention: one thread per query, online softmax over its keys.
// ---------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(64) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kc,
    const float* __restrict__ vt, float* __restrict__ out, int R, int H, int d,
    int Lcap, int pos_base, float scale) {
  const int t = blockIdx.x * 64 + threadIdx.x;
  const int head = blockIdx.y, n = blockIdx.z;
  if (t >= R) return;
  const size_t hb = (size_t)n * H + head;
  const float* kbase = kc + hb * Lcap * DH;
  const float* vbase = vt + hb * DH * Lcap;
  const float* qrow = q + ((size_t)n * R + t) * d + head * DH;
  float qv[DH], acc[DH];
#pragma unroll
  for (int e = 0; e < DH; ++e) {
    qv[e] = qrow[e] * scale;
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int p = pos_base + t;
  for (int key = 0; key <= p; ++key) {
    const float* krow = kbase + (size_t)key * DH;
    float sc = 0.f;
#pragma unroll
    for (int e = 0; e < DH; ++e) sc += qv[e] * krow[e];
    const float m_new = fmaxf(m, sc);
    const float alpha = expf(m - m_new);
    const float w = expf(sc - m_new);
    l = l * alpha + w;
#pragma unroll
    for (int e = 0; e < DH; ++e) acc[e] = acc[e] * alpha + w * vbase[(size_t)e * Lcap + key];
    m = m_new;
  }
  float* orow = out + ((size_t)n * R + t) * d + head * DH;
  const float inv = 1.0f / l;
#pragma unroll
  for (int e = 0; e < DH; ++e) orow[e] = acc[e] * inv;
}

hipError_t launch_attention(bool bf, const void* q, const void* kc,
                            const void* vt, void* out, int N, int R, int H,
                            int dh, int d, int Lcap, int pos_base, hipStream_t st) {
  const float scale = 1.0f / sqrtf((float)dh);
  if (bf) {
    dim3 grid((R + 127) / 128, H, N);
    const float sl2 = scale * 1.4426950408889634f;
    switch (dh) {
      case 64:
        hipLaunchKernelGGL(attn_bf16_kernel<64>, grid, dim3(256), 0, st,
                           (const bf16*)q, (const bf16*)kc, (const bf16*)vt,
                           (bf16*)out, R, H, d, Lcap, pos_base, sl2);
        break;
      case 128:
        hipLaunchKernelGGL(attn_bf16_kernel<128>, grid, dim3(256), 0, st,
                           (const bf16*)q, (const bf16*)kc, (const bf16*)vt,
                           (bf16*)out, R, H, d, Lcap, pos_base, sl2);
        break;
      case 32:
        hipLaunchKernelGGL(attn_bf16_kernel<32>, grid, dim3(256), 0, st,
                           (const bf16*)q, (const bf16*)kc, (const bf16*)vt,
                           (bf16*)out, R, H, d, Lcap, pos_base, sl2);
        break;
      default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  dim3 grid((R + 63) / 64, H, N);
  switch (dh) {
    case 32:
      hipLaunchKernelGGL(attn_f32_kernel<32>, grid, dim3(64), 0, st, (const float*)q,
                         (const float*)kc, (const float*)vt, (float*)out, R, H, d,
                         Lcap, pos_base, scale);
      break;
    case 64:
      hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(64), 0, st, (const float*)q,
                         (const float*)kc, (const float*)vt, (float*)out, R, H, d,
                         Lcap, pos_base, scale);
      break;
    case 128:
      hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(64), 0, st, (const float*)q,
                         (const float*)kc, (const float*)vt, (float*)out, R, H, d,
                         Lcap, pos_base, scale);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace af
