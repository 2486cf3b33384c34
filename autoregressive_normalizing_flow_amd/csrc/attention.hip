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

#include <algorithm>

namespace af {

// ---------------------------------------------------------------------------
// bf16 MFMA flash attention with key-range splitting.
//
// Work unit = (sample, head, 128-query tile, key chunk of KC keys).  Long key
// ranges (a long KV-cache prefix, or the last query tiles of a frame) are cut
// into chunks processed by separate workgroups, so the grid fills the chip
// and no workgroup walks the whole prefix; a query tile with one chunk writes
// its normalised output directly, otherwise each chunk writes its unnormalised
// output and running (max, sum) to a partial slot, takes a ticket of its query
// tile, and the chunk that takes the last ticket merges the tile's slots (in
// chunk order, so the result does not depend on which chunk merges).  Units
// are numbered sample-head major, then query tile, then chunk.
//
// Inside a unit each of the 4 waves owns 32 queries (two 16-query blocks).
// Per 64-key tile:  S^T = K Q^T  (A = K rows from LDS, B = Q held in
// registers), online softmax in fp32 along the key axis (the 4 lanes sharing
// a query combine with two xor-shuffles), then  O^T += Vt P^T  where P^T is
// already in the B-operand layout of the lanes that hold the scores: the 8
// k-slots of lane l are keys {4(l/16)+j, 16+4(l/16)+j}, j < 4, of each
// 32-key step, and the Vt fragment reads the same keys (two 8-byte reads).
// ---------------------------------------------------------------------------
constexpr int ATT_QT = 128;   // queries per unit
constexpr int ATT_KT = 64;    // keys per tile
// Lazy softmax reference: p = 2^(s - m) with m moved only when the tile's
// largest score leaves [m - RESCALE_LOW, m + RESCALE_LOG2], so p of a row's
// largest score stays in [2^-32, 2^8] (no overflow, no underflow to zero).
constexpr float RESCALE_LOG2 = 8.0f;
constexpr float RESCALE_LOW = 32.0f;
// Chunk slots merged per memory round trip.
constexpr int ATT_MAXC = 4;
// Cache-policy operand of the buffer builtins: sc1, agent-coherent access.
constexpr int ATT_SC1 = 16;

// Raw buffer resource over one partial slot (byte offsets from its start).
template <int DH>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slot_rsrc_dh(const float* slot) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(slot), 0,
                                           ATT_QT * (DH + 2) * 4, 0x00020000);
}

struct AttnArgs {
  const bf16* q;
  const bf16* kc;
  const bf16* vt;
  bf16* out;
  // split mode (higher-precision forward): lo halves of q, K, Vt and the
  // output, so that every operand is the bf16 pair hi + lo; NULL otherwise
  const bf16* q_lo;
  const bf16* kc_lo;
  const bf16* vt_lo;
  bf16* out_lo;
  float* part;     // partial slots: [unit][ATT_QT][DH] O, then [ATT_QT] m, [ATT_QT] l
  unsigned* tickets;   // [sample * H + head][query tile], zero between launches
  int R, H, d, Lcap, pos_base, KC, U_nh, n_qt;
  int xcd_map;     // 1: deal (sample, head) pairs to XCDs (needs N*H % 8 == 0)
};

__device__ __forceinline__ int att_chunks(int qt, int R, int pos_base, int KC) {
  const int nk = pos_base + min(R, (qt + 1) * ATT_QT);
  return (nk + KC - 1) / KC;
}

// SPLIT: products of bf16 pairs keep three of the four partial products,
// (a + a')(b + b') ~ ab + a'b + ab', for both S = K Q^T and O = P V.
template <int DH, bool SPLIT>
__device__ __forceinline__ void attn_bf16_body(const AttnArgs& a) {
  constexpr int QWAVE = 32, QB = QWAVE / 16;
  constexpr int KB = ATT_KT / 16, KS = DH / 32, DB = DH / 16;
  // K rows padded to DH + 8 (16-byte fragment reads of 16 rows hit distinct
  // banks); Vt rows padded to 68 bf16 = 136 B so the 8-byte fragment reads of
  // 16 consecutive rows are conflict-free (rows then are 8-byte aligned only).
  constexpr int KLDS = DH + 8, VLDS = ATT_KT + 4;
  constexpr int CK = ATT_KT * DH / 8 / 256;  // 16-byte chunks per thread per tile
  __shared__ __attribute__((aligned(16))) bf16 sK[2][ATT_KT * KLDS];
  __shared__ __attribute__((aligned(16))) bf16 sV[2][DH * VLDS];
  __shared__ __attribute__((aligned(16))) bf16 sKl[2][SPLIT ? ATT_KT * KLDS : 8];
  __shared__ __attribute__((aligned(16))) bf16 sVl[2][SPLIT ? DH * VLDS : 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // unit -> (sample, head, query tile, chunk).  Block ids go round-robin over
  // the 8 XCDs; when N*H is a multiple of 8, (sample, head) pairs are dealt so
  // that all units of one head run on one XCD and share its K/V in that L2.
  int u = blockIdx.x;
  if (a.xcd_map) {
    const int xcd = u & 7, local = u >> 3;
    const int j = local / a.U_nh;
    u = (j * 8 + xcd) * a.U_nh + (local - j * a.U_nh);
  }
  const int nh = u / a.U_nh;
  int rem = u - nh * a.U_nh;
  const int n = nh / a.H, head = nh - n * a.H;
  int qt = 0, n_chunks = att_chunks(0, a.R, a.pos_base, a.KC);
  while (rem >= n_chunks) {
    rem -= n_chunks;
    ++qt;
    n_chunks = att_chunks(qt, a.R, a.pos_base, a.KC);
  }
  const int chunk = rem;
  const int R = a.R, d = a.d, Lcap = a.Lcap, pos_base = a.pos_base;
  const int q_lo = qt * ATT_QT;
  const int nk = pos_base + min(R, q_lo + ATT_QT);   // keys of the tile: 0..nk-1
  const int k_begin = chunk * a.KC;
  const int k_end = min(nk, k_begin + a.KC);
  const int t_begin = k_begin / ATT_KT;
  const int n_tiles = (k_end - k_begin + ATT_KT - 1) / ATT_KT;
  const size_t hb = (size_t)n * a.H + head;
  const bf16* kbase = a.kc + hb * Lcap * DH;
  const bf16* vbase = a.vt + hb * DH * Lcap;
  const bf16* klbase = SPLIT ? a.kc_lo + hb * Lcap * DH : nullptr;
  const bf16* vlbase = SPLIT ? a.vt_lo + hb * DH * Lcap : nullptr;
  const int l16 = lane & 15, lg = lane >> 4;

  bf16x8 qf[QB][KS], qfl[QB][KS];
  int qpos[QB];
  const int wave_qmin = pos_base + q_lo + wave * QWAVE;   // smallest query position
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int t = q_lo + wave * QWAVE + qb * 16 + l16;
    qpos[qb] = pos_base + t;
    const size_t qo = ((size_t)n * R + min(t, R - 1)) * d + head * DH;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[qb][ks] = *(const bf16x8*)(a.q + qo + ks * 32 + lg * 8);
      if (SPLIT) qfl[qb][ks] = *(const bf16x8*)(a.q_lo + qo + ks * 32 + lg * 8);
    }
  }

  float m_run[QB];
  f32x4 acc_o[DB][QB], acc_l[QB];
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (bf16)1.0f;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = 0.f;
    acc_l[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < DB; ++db) acc_o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Two register stages: tile kt+2 is loaded while kt is multiplied and
  // tile kt+1 waits in registers to be stored into the other LDS buffer.
  struct Stage {
    u32x4 k[CK], v[CK], kl[CK], vl[CK];
  } ra, rb;
  // This thread's 16-byte chunks of a tile, the same in every tile: chunk
  // c = tid + 256 i is K row c / (DH/8), columns 8 (c % (DH/8)).., and Vt row
  // c / (ATT_KT/8), keys 8 (c % (ATT_KT/8)).. of the tile.  Element offsets
  // from the tile's (uniform) base.
  uint32_t koff[CK], voff[CK];
#pragma unroll
  for (int i = 0; i < CK; ++i) {
    const int c = tid + i * 256;
    const int key = c / (DH / 8), dc = c - key * (DH / 8);
    const int drow = c / (ATT_KT / 8), kc8 = c - drow * (ATT_KT / 8);
    koff[i] = (uint32_t)(key * DH + dc * 8);
    voff[i] = (uint32_t)(drow * Lcap + kc8 * 8);
  }
  auto gload = [&](Stage& st, int kt) {
    u32x4(&rk)[CK] = st.k;
    u32x4(&rv)[CK] = st.v;
    u32x4(&rkl)[CK] = st.kl;
    u32x4(&rvl)[CK] = st.vl;
    const int k0 = (t_begin + kt) * ATT_KT;
    const bf16* kp = kbase + (size_t)k0 * DH;
    const bf16* vp = vbase + k0;
    const bf16* klp = SPLIT ? klbase + (size_t)k0 * DH : nullptr;
    const bf16* vlp = SPLIT ? vlbase + k0 : nullptr;
    // every address is inside the allocation (k0 + 64 <= Lcap)
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      rk[i] = *(const u32x4*)(kp + koff[i]);
      rv[i] = *(const u32x4*)(vp + voff[i]);
      if (SPLIT) {
        rkl[i] = *(const u32x4*)(klp + koff[i]);
        rvl[i] = *(const u32x4*)(vlp + voff[i]);
      }
    }
    if (k0 + ATT_KT > k_end) {
      // ragged last tile: keys at or past k_end become zeros (in place, so
      // that only this rare branch waits for the loads)
#pragma unroll
      for (int i = 0; i < CK; ++i) {
        const int c = tid + i * 256;
        if (k0 + c / (DH / 8) >= k_end) {
          rk[i] = u32x4{0u, 0u, 0u, 0u};
          if (SPLIT) rkl[i] = u32x4{0u, 0u, 0u, 0u};
        }
        const int kk0 = k0 + (c % (ATT_KT / 8)) * 8;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const unsigned lo_ok = (kk0 + 2 * e) < k_end ? 0xFFFFu : 0u;
          const unsigned hi_ok = (kk0 + 2 * e + 1) < k_end ? 0xFFFF0000u : 0u;
          rv[i][e] &= (lo_ok | hi_ok);
          if (SPLIT) rvl[i][e] &= (lo_ok | hi_ok);
        }
      }
    }
  };
  auto lstore = [&](const Stage& st, int buf) {
    const u32x4(&rk)[CK] = st.k;
    const u32x4(&rv)[CK] = st.v;
    const u32x4(&rkl)[CK] = st.kl;
    const u32x4(&rvl)[CK] = st.vl;
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      const int c = tid + i * 256;
      const int key = c / (DH / 8), dc = c - key * (DH / 8);
      *(u32x4*)(&sK[buf][key * KLDS + dc * 8]) = rk[i];
      if (SPLIT) *(u32x4*)(&sKl[buf][key * KLDS + dc * 8]) = rkl[i];
      const int drow = c / (ATT_KT / 8), kc8 = c - drow * (ATT_KT / 8);
      {
        uint2* dv = (uint2*)(&sV[buf][drow * VLDS + kc8 * 8]);
        dv[0] = uint2{rv[i][0], rv[i][1]};
        dv[1] = uint2{rv[i][2], rv[i][3]};
      }
      if (SPLIT) {
        uint2* dv = (uint2*)(&sVl[buf][drow * VLDS + kc8 * 8]);
        dv[0] = uint2{rvl[i][0], rvl[i][1]};
        dv[1] = uint2{rvl[i][2], rvl[i][3]};
      }
    }
  };

  // -m of each query, the accumulator seed of S: the MFMAs then produce
  // s - m directly
  f32x4 negm[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) negm[qb] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int kt, int cur) {
    const int key0 = (t_begin + kt) * ATT_KT;

    f32x4 s[KB][QB];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 kf =
            *(const bf16x8*)(&sK[cur][(kb * 16 + l16) * KLDS + ks * 32 + lg * 8]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              kf, qf[qb][ks], ks == 0 ? negm[qb] : s[kb][qb], 0, 0, 0);
        if (SPLIT) {
          const bf16x8 kfl =
              *(const bf16x8*)(&sKl[cur][(kb * 16 + l16) * KLDS + ks * 32 + lg * 8]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            s[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qfl[qb][ks],
                                                                s[kb][qb], 0, 0, 0);
            s[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfl, qf[qb][ks],
                                                                s[kb][qb], 0, 0, 0);
          }
        }
      }

    // online softmax (base 2; q carries log2(e) / sqrt(dh)) per query.  The
    // reference m is lazy: it moves only when some row's largest score in the
    // tile leaves [m - RESCALE_LOW, m + RESCALE_LOG2]; until then p = 2^(s - m)
    // is at most 2^RESCALE_LOG2 (harmless in fp32 and in bf16) and the
    // accumulators are not touched.  The same m scales O and the row sum, so
    // the result is that of the exact update.  Tiles wholly below every query
    // of the wave and inside [k_begin, k_end) skip the masking; both tests are
    // wave-uniform branches (the empty asm keeps the compiler from turning
    // them into per-element selects).
    const bool need_mask = (key0 + ATT_KT - 1 > wave_qmin) || (key0 + ATT_KT > k_end);
    if (need_mask) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = key0 + kb * 16 + lg * 4 + r;
            if (key > qpos[qb] || key >= k_end) s[kb][qb][r] = -INFINITY;
          }
    }
    float tmax[QB];   // largest s - m of the row in this tile
    bool move = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float t = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) t = fmaxf(t, s[kb][qb][r]);
      t = fmaxf(t, __shfl_xor(t, 16, AF_WAVE));
      t = fmaxf(t, __shfl_xor(t, 32, AF_WAVE));
      tmax[qb] = t;
      // (a row with every key masked, t = -inf, keeps its reference)
      move |= t > RESCALE_LOG2 || (t < -RESCALE_LOW && t > -INFINITY);
    }
    if (__builtin_amdgcn_ballot_w64(move) != 0) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float t = tmax[qb];
        const float dm = (t > RESCALE_LOG2 || (t < -RESCALE_LOW && t > -INFINITY)) ? t : 0.f;
        const float alpha = __builtin_amdgcn_exp2f(-dm);
        m_run[qb] += dm;
        negm[qb] = f32x4{-m_run[qb], -m_run[qb], -m_run[qb], -m_run[qb]};
        acc_l[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc_o[db][qb] *= alpha;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) s[kb][qb][r] -= dm;
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) s[kb][qb][r] = __builtin_amdgcn_exp2f(s[kb][qb][r]);

    // O^T += Vt P^T over two 32-key steps
#pragma unroll
    for (int c = 0; c < ATT_KT / 32; ++c) {
      bf16x8 pf[QB], pfl[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pf[qb][r] = (bf16)s[2 * c][qb][r];
          pf[qb][4 + r] = (bf16)s[2 * c + 1][qb][r];
          if (SPLIT) {
            pfl[qb][r] = (bf16)(s[2 * c][qb][r] - (float)pf[qb][r]);
            pfl[qb][4 + r] = (bf16)(s[2 * c + 1][qb][r] - (float)pf[qb][4 + r]);
          }
        }
      }
      // row sums: an all-ones A operand sums P^T over the keys
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        acc_l[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[qb], acc_l[qb], 0, 0, 0);
        if (SPLIT)
          acc_l[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pfl[qb], acc_l[qb], 0, 0, 0);
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
        if (SPLIT) {
          const bf16* vlrow = &sVl[cur][(db * 16 + l16) * VLDS + c * 32 + lg * 4];
          const bf16x4 llo = *(const bf16x4*)vlrow;
          const bf16x4 lhi = *(const bf16x4*)(vlrow + 16);
          const bf16x8 vfl = {llo[0], llo[1], llo[2], llo[3], lhi[0], lhi[1], lhi[2], lhi[3]};
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            acc_o[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                vf, pfl[qb], acc_o[db][qb], 0, 0, 0);
            acc_o[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                vfl, pf[qb], acc_o[db][qb], 0, 0, 0);
          }
        }
      }
    }
  };

  gload(ra, 0);
  if (n_tiles > 1) gload(rb, 1);
  lstore(ra, 0);
  __syncthreads();
  // the buffer of tile t is t & 1
#pragma clang loop unroll(disable)
  for (int kt = 0; kt < n_tiles; kt += 2) {
    if (kt + 2 < n_tiles) gload(ra, kt + 2);
    compute(kt, 0);
    if (kt + 1 < n_tiles) lstore(rb, 1);
    __syncthreads();
    if (kt + 1 >= n_tiles) break;
    if (kt + 3 < n_tiles) gload(rb, kt + 3);
    compute(kt + 1, 1);
    if (kt + 2 < n_tiles) lstore(ra, 0);
    __syncthreads();
  }

  // bf16 hi + lo of the normalised output row of query t, dimensions
  // db*16 + lg*4 .. +3
  auto store_out = [&](int t, int db, const f32x4& v, float inv) {
    const size_t oo = ((size_t)n * R + t) * d + head * DH + db * 16 + lg * 4;
    bf16x4 o, ol;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float y = v[r] * inv;
      o[r] = (bf16)y;
      ol[r] = (bf16)(y - (float)o[r]);
    }
    *(bf16x4*)(a.out + oo) = o;
    if (SPLIT) *(bf16x4*)(a.out_lo + oo) = ol;
  };

  if (n_chunks == 1) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int t = q_lo + wave * QWAVE + qb * 16 + l16;
      if (t < R) {
        const float inv = 1.0f / acc_l[qb][0];
#pragma unroll
        for (int db = 0; db < DB; ++db) store_out(t, db, acc_o[db][qb], inv);
      }
    }
    return;
  }

  // Partial slot of this chunk, written with agent-coherent (sc1) stores so
  // that the merging block reads it from any XCD without an L2 writeback.
  constexpr int SLOT = ATT_QT * (DH + 2);
  {
    const __amdgpu_buffer_rsrc_t rs = slot_rsrc_dh<DH>(a.part + (size_t)u * SLOT);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float l = acc_l[qb][0];
      const int tq = wave * QWAVE + qb * 16 + l16;   // query within the tile
#pragma unroll
      for (int db = 0; db < DB; ++db)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc_o[db][qb]), rs,
                                               (tq * DH + db * 16 + lg * 4) * 4, 0, ATT_SC1);
      if (lg == 0) {
        // a row with no key in this chunk (l = 0) must not set the merge's max
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l > 0.f ? m_run[qb] : -1e30f),
                                              rs, (ATT_QT * DH + tq) * 4, 0, ATT_SC1);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l), rs,
                                              (ATT_QT * DH + ATT_QT + tq) * 4, 0, ATT_SC1);
      }
    }
  }
  wait_stores();
  __syncthreads();   // every store of the block is complete before the ticket
  __shared__ unsigned s_last;
  if (tid == 0) {
    unsigned* tk = a.tickets + (size_t)nh * a.n_qt + qt;
    const unsigned last = atomicAdd(tk, 1u) + 1u == (unsigned)n_chunks;
    if (last) __hip_atomic_store(tk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;

  // Merge: O = sum_c 2^(m_c - m) O_c / sum_c 2^(m_c - m) l_c over the chunks in
  // order, MC chunks per memory round trip (every load of a group, for both
  // query blocks, is issued before the first use; this block's own chunk comes
  // from its registers), with a running max across groups.
  constexpr int MC = DH <= 64 ? ATT_MAXC : ATT_MAXC / 2;
  const float* tile0 = a.part + (size_t)(u - chunk) * SLOT;   // the tile's chunk 0
  float m[QB], l[QB];
  f32x4 o[QB][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -1e30f;
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int c0 = 0; c0 < n_chunks; c0 += MC) {
    float mc[MC][QB], lc[MC][QB];
    f32x4 oc[MC][QB][DB];
#pragma unroll
    for (int c = 0; c < MC; ++c) {
      const int cc = min(c0 + c, n_chunks - 1);
      if (cc == chunk) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          lc[c][qb] = acc_l[qb][0];
          mc[c][qb] = lc[c][qb] > 0.f ? m_run[qb] : -1e30f;
#pragma unroll
          for (int db = 0; db < DB; ++db) oc[c][qb][db] = acc_o[db][qb];
        }
      } else {
        const __amdgpu_buffer_rsrc_t rs = slot_rsrc_dh<DH>(tile0 + (size_t)cc * SLOT);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int tq = wave * QWAVE + qb * 16 + l16;
          mc[c][qb] = __uint_as_float(
              __builtin_amdgcn_raw_buffer_load_b32(rs, (ATT_QT * DH + tq) * 4, 0, ATT_SC1));
          lc[c][qb] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
              rs, (ATT_QT * DH + ATT_QT + tq) * 4, 0, ATT_SC1));
#pragma unroll
          for (int db = 0; db < DB; ++db)
            oc[c][qb][db] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                rs, (tq * DH + db * 16 + lg * 4) * 4, 0, ATT_SC1));
        }
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mg = m[qb];
#pragma unroll
      for (int c = 0; c < MC; ++c)
        if (c0 + c < n_chunks) mg = fmaxf(mg, mc[c][qb]);
      const float alpha = __builtin_amdgcn_exp2f(m[qb] - mg);
      l[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[qb][db] *= alpha;
#pragma unroll
      for (int c = 0; c < MC; ++c) {
        if (c0 + c >= n_chunks) break;
        const float w = __builtin_amdgcn_exp2f(mc[c][qb] - mg);
        l[qb] = fmaf(w, lc[c][qb], l[qb]);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[qb][db][r] = fmaf(w, oc[c][qb][db][r], o[qb][db][r]);
      }
      m[qb] = mg;
    }
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int t = q_lo + wave * QWAVE + qb * 16 + l16;
    if (t < R) {
      const float inv = 1.0f / l[qb];
#pragma unroll
      for (int db = 0; db < DB; ++db) store_out(t, db, o[qb][db], inv);
    }
  }
}

// Two waves per SIMD are the target: the compiler then keeps the MFMA
// results in VGPRs (with a 512-register budget it moves them through AGPRs
// around every VALU step of the softmax).  The wider variants need more than
// 256 registers and keep the default budget.
template <int DH, bool SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void
attn_bf16_kernel_o2(AttnArgs a) {
  attn_bf16_body<DH, SPLIT>(a);
}

template <int DH, bool SPLIT>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnArgs a) {
  attn_bf16_body<DH, SPLIT>(a);
}

// Key chunk length.  For the two-blocks-per-CU kernel (d_h <= 64, not split)
// the smallest chunk of 448..1024 keys (a multiple of the 64-key tile) that
// keeps every unit in one round of two blocks per CU, when there is one (448
// keys at 1560 tokens: 512 units of at most 7 tiles, against 448 units of 8
// tiles with 512-key chunks).  Otherwise the smallest multiple of 512 keys
// that keeps the number of units at most 1024 (four per CU); whole ranges when
// that is already enough.
static int att_units(int R, int pos_base, int KC, int n_qt) {
  int s = 0;
  for (int qt = 0; qt < n_qt; ++qt) {
    const int nk = pos_base + std::min(R, (qt + 1) * ATT_QT);
    s += (nk + KC - 1) / KC;
  }
  return s;
}

int attention_chunk(int N, int R, int H, int dh, bool split, int pos_base) {
  const int n_qt = (R + ATT_QT - 1) / ATT_QT;
  const int nk_max = pos_base + R;
  if (dh <= 64 && !split)
    for (int kc = 448; kc <= 1024 && kc < nk_max; kc += ATT_KT)
      if ((long)N * H * att_units(R, pos_base, kc, n_qt) <= 512) return kc;
  int KC = 512;
  while (KC < nk_max && (long)N * H * att_units(R, pos_base, KC, n_qt) > 1024) KC *= 2;
  return KC;
}

size_t attention_partial_floats(int N, int R, int H, int dh, int pos_base) {
  const int n_qt = (R + ATT_QT - 1) / ATT_QT;
  // the larger of the two chunk rules' unit counts
  const int KC = std::min(attention_chunk(N, R, H, dh, false, pos_base),
                          attention_chunk(N, R, H, dh, true, pos_base));
  return (size_t)N * H * att_units(R, pos_base, KC, n_qt) * ATT_QT * (dh + 2);
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

template <int DH, bool SPLIT>
static void attn_launch(const AttnArgs& a, dim3 grid, hipStream_t st) {
  if constexpr (DH <= 64 && !SPLIT)
    hipLaunchKernelGGL((attn_bf16_kernel_o2<DH, SPLIT>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<DH, SPLIT>), grid, dim3(256), 0, st, a);
}

hipError_t launch_attention(bool bf, const void* q, const void* kc,
                            const void* vt, void* out, float* part, unsigned* tickets,
                            int N, int R, int H, int dh, int d, int Lcap, int pos_base,
                            hipStream_t st, const AttnSplit* split) {
  const float scale = 1.0f / sqrtf((float)dh);
  if (bf) {
    const int n_qt = (R + ATT_QT - 1) / ATT_QT;
    const int KC = attention_chunk(N, R, H, dh, split != nullptr, pos_base);
    const int U_nh = att_units(R, pos_base, KC, n_qt);
    AttnArgs a{(const bf16*)q, (const bf16*)kc, (const bf16*)vt, (bf16*)out,
               split ? (const bf16*)split->q_lo : nullptr,
               split ? (const bf16*)split->kc_lo : nullptr,
               split ? (const bf16*)split->vt_lo : nullptr,
               split ? (bf16*)split->out_lo : nullptr, part, tickets,
               R, H, d, Lcap, pos_base, KC, U_nh, n_qt, (N * H) % 8 == 0 ? 1 : 0};
    if (U_nh > n_qt && (!part || !tickets)) return hipErrorInvalidValue;
    const dim3 grid(N * H * U_nh);
    switch (dh * 2 + (split ? 1 : 0)) {
      case 128: attn_launch<64, false>(a, grid, st); break;
      case 129: attn_launch<64, true>(a, grid, st); break;
      case 256: attn_launch<128, false>(a, grid, st); break;
      case 257: attn_launch<128, true>(a, grid, st); break;
      case 64: attn_launch<32, false>(a, grid, st); break;
      case 65: attn_launch<32, true>(a, grid, st); break;
      default: return hipErrorInvalidValue;
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
