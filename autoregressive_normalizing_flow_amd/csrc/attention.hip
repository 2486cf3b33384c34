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
// Lazy softmax reference: p = 2^(s - m) with m moved up only when a tile's
// largest score exceeds m + RESCALE_LOG2 (p stays at most 2^8: no overflow),
// and down, to the tile's largest score, only while the row has no mass yet
// (its first tile with a key may lie far below the initial m = 0).  A row
// with mass never moves down: a later tile far below it would otherwise
// rescale O by 2^(-dm), beyond fp32 once dm < -128, and its keys' weights
// are negligible against the mass anyway.
constexpr float RESCALE_LOG2 = 8.0f;
constexpr float RESCALE_LOW = 32.0f;
// The same window as fp32 bit patterns of p: 2^8 and 2^-32.
constexpr unsigned F32_2P8 = 0x43800000u;
constexpr unsigned F32_2M32 = 0x2F800000u;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
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
    // tile exceeds m + RESCALE_LOG2, or lies below m - RESCALE_LOW while the
    // row has no mass yet; until then p = 2^(s - m) is at most 2^RESCALE_LOG2
    // (harmless in fp32 and in bf16) and the accumulators are not touched.
    // The same m scales O and the row sum, so
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
      move |= t > RESCALE_LOG2 ||
              (t < -RESCALE_LOW && t > -INFINITY && acc_l[qb][0] == 0.f);
    }
    if (__builtin_amdgcn_ballot_w64(move) != 0) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float t = tmax[qb];
        const bool up = t > RESCALE_LOG2;
        const bool down = t < -RESCALE_LOW && t > -INFINITY && acc_l[qb][0] == 0.f;
        const float dm = (up || down) ? t : 0.f;
        // a downward move finds O and l still zero: nothing to rescale
        const float alpha = up ? __builtin_amdgcn_exp2f(-dm) : 1.0f;
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

// Merge of a query tile's key-chunk partials in chunk order, MC slots per
// memory round trip (run by the chunk that took the tile's last ticket): lane
// (j, hh) of wave w combines query tq = 32 w + j, dimensions db*32 + 8g + 4hh
// .. +3, and writes row t_q of the output if it is a real row.
template <int DH>
__device__ __forceinline__ void attn32_merge(const AttnArgs& a, int unit0, int n_chunks,
                                             int tq, int t_q, int n, int head, int hh) {
  constexpr int DB = DH / 32;
  constexpr int SLOT = ATT_QT * (DH + 2);
  constexpr int MC = DH <= 64 ? ATT_MAXC : ATT_MAXC / 2;
  const float* tile0 = a.part + (size_t)unit0 * SLOT;
  float m = -1e30f, l = 0.f;
  f32x4 o[DB][4];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) o[db][g] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < n_chunks; c0 += MC) {
    float mc[MC], lc[MC];
    f32x4 oc[MC][DB][4];
#pragma unroll
    for (int c = 0; c < MC; ++c) {
      const int cc = min(c0 + c, n_chunks - 1);
      const __amdgpu_buffer_rsrc_t rs = slot_rsrc_dh<DH>(tile0 + (size_t)cc * SLOT);
      mc[c] = __uint_as_float(
          __builtin_amdgcn_raw_buffer_load_b32(rs, (ATT_QT * DH + tq) * 4, 0, ATT_SC1));
      lc[c] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          rs, (ATT_QT * DH + ATT_QT + tq) * 4, 0, ATT_SC1));
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          oc[c][db][g] = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                         rs, (tq * DH + db * 32 + 8 * g + 4 * hh) * 4, 0, ATT_SC1));
    }
    float mg = m;
#pragma unroll
    for (int c = 0; c < MC; ++c)
      if (c0 + c < n_chunks) mg = fmaxf(mg, mc[c]);
    const float alpha = __builtin_amdgcn_exp2f(m - mg);
    l *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) o[db][g] *= alpha;
#pragma unroll
    for (int c = 0; c < MC; ++c) {
      if (c0 + c >= n_chunks) break;
      const float w = __builtin_amdgcn_exp2f(mc[c] - mg);
      l = fmaf(w, lc[c], l);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) o[db][g][e] = fmaf(w, oc[c][db][g][e], o[db][g][e]);
    }
    m = mg;
  }
  if (t_q < a.R) {
    const float inv = 1.0f / l;
    bf16* orow = a.out + ((size_t)n * a.R + t_q) * a.d + head * DH + 4 * hh;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 ob;
#pragma unroll
        for (int e = 0; e < 4; ++e) ob[e] = (bf16)(o[db][g][e] * inv);
        *(bf16x4*)(orow + db * 32 + 8 * g) = ob;
      }
  }
}

// ---------------------------------------------------------------------------
// bf16 attention on the 32 x 32 x 16 matrix cores (v_mfma_f32_32x32x16_bf16),
// the path of every Jacobi update.  Same work units, chunk merge and cache
// layouts as above; per 64-key tile and wave (32 queries) it issues 8 MFMAs
// for the scores, 4 for the row sums and 4 DH/32 for P V, each doing twice the
// work of a 16 x 16 x 32 step for the same operand bytes.
//
// Lane l of a wave holds query j = l % 32 of the wave's 32 (the two halves
// h = l / 32 hold the same query).  Operand layouts of the 32 x 32 x 16 step:
// A lane l gives row l % 32, k = 8h .. 8h+7; B lane l gives column l % 32,
// the same k; the accumulator's element r of lane l is row 8 (r / 4) + 4h +
// r % 4 of column l % 32.
//   S^T = K Q^T:  A = 32 key rows of K (16 contiguous bytes of a row), B = Q^T
//                 (the lane's query, held in registers); lane l gets the scores
//                 of its query for keys 8 (r / 4) + 4h + r % 4 of the block.
//   O^T += Vt P^T: B = P^T straight from those registers: of each 16-key step
//                 g the lane holds keys {16g + 4h + i, 16g + 8 + 4h + i}, i < 4,
//                 as its 8 k-slots; the Vt tile is stored in LDS with each
//                 16-key group permuted to [0-3, 8-11, 4-7, 12-15], so that the
//                 A fragment of those keys is one 16-byte read at 16g + 8h.
//   row sums:     an all-ones A operand sums the same bf16 P^T over the keys.
// ---------------------------------------------------------------------------
template <int DH>
__device__ __forceinline__ void attn32_body(const AttnArgs& a) {
  constexpr int KS = DH / 16;                   // k-steps of the scores
  constexpr int DB = DH / 32;                   // 32-dimension blocks of O^T
  constexpr int KROW = DH + 8;                  // K tile row in LDS (bf16)
  constexpr int VROW = ATT_KT + 8;              // Vt tile row in LDS (bf16)
  constexpr int CK = ATT_KT * DH / 8 / 256;     // 16-byte chunks per thread per tile
  typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
  __shared__ __attribute__((aligned(16))) bf16 sK[2][ATT_KT * KROW];
  __shared__ __attribute__((aligned(16))) bf16 sV[2][DH * VROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 31, hh = lane >> 5;
  // unit -> (sample, head, query tile, chunk), as in attn_bf16_body
  int u = blockIdx.x;
  if (a.xcd_map) {
    const int xcd = u & 7, local = u >> 3;
    const int jj = local / a.U_nh;
    u = (jj * 8 + xcd) * a.U_nh + (local - jj * a.U_nh);
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
  const int nk = pos_base + min(R, q_lo + ATT_QT);
  const int k_begin = chunk * a.KC;
  const int k_end = min(nk, k_begin + a.KC);
  const int t_begin = k_begin / ATT_KT;
  const int n_tiles = (k_end - k_begin + ATT_KT - 1) / ATT_KT;
  const size_t hb = (size_t)n * a.H + head;
  const bf16* kbase = a.kc + hb * Lcap * DH;
  const bf16* vbase = a.vt + hb * DH * Lcap;
  // a wave whose 32 queries all lie past the last row only loads and syncs
  const bool active = q_lo + wave * 32 < R;
  const int t_q = q_lo + wave * 32 + j;             // this lane's query row
  const int qpos = pos_base + t_q;
  const int wave_qmin = pos_base + q_lo + wave * 32;

  bf16x8 qf[KS];
  {
    const size_t qo = ((size_t)n * R + min(t_q, R - 1)) * d + head * DH + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const bf16x8*)(a.q + qo + ks * 16);
  }
  float m_run = 0.f;
  // accumulator seed of the scores: -m_run in every element
  f32x16 acc_o[DB], acc_l, negm;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    acc_l[e] = 0.f;
    negm[e] = 0.f;
  }
#pragma unroll
  for (int db = 0; db < DB; ++db) acc_o[db] = acc_l;
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (bf16)1.0f;

  // register stages: tile kt+2 loads while kt is multiplied and kt+1 waits
  // to be stored into the other LDS buffer
  struct Stage {
    u32x4 k[CK], v[CK];
  } ra, rb;
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
    const int k0 = (t_begin + kt) * ATT_KT;
    const bf16* kp = kbase + (size_t)k0 * DH;
    const bf16* vp = vbase + k0;
    // every address is inside the allocation (k0 + 64 <= Lcap)
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      st.k[i] = *(const u32x4*)(kp + koff[i]);
      st.v[i] = *(const u32x4*)(vp + voff[i]);
    }
    if (k0 + ATT_KT > k_end) {
      // ragged last tile: keys at or past k_end become zeros
#pragma unroll
      for (int i = 0; i < CK; ++i) {
        const int c = tid + i * 256;
        if (k0 + c / (DH / 8) >= k_end) st.k[i] = u32x4{0u, 0u, 0u, 0u};
        const int kk0 = k0 + (c % (ATT_KT / 8)) * 8;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const unsigned lo_ok = (kk0 + 2 * e) < k_end ? 0xFFFFu : 0u;
          const unsigned hi_ok = (kk0 + 2 * e + 1) < k_end ? 0xFFFF0000u : 0u;
          st.v[i][e] &= (lo_ok | hi_ok);
        }
      }
    }
  };
  auto lstore = [&](const Stage& st, int buf) {
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      const int c = tid + i * 256;
      const int key = c / (DH / 8), dc = c - key * (DH / 8);
      *(u32x4*)(&sK[buf][key * KROW + dc * 8]) = st.k[i];
      // keys 8 kc8 .. +7 of the tile: 16-key group g = kc8 / 2, half kc8 % 2;
      // keys 0-3 / 4-7 of the half go to physical 4 half / 8 + 4 half
      const int drow = c / (ATT_KT / 8), kc8 = c - drow * (ATT_KT / 8);
      const int g = kc8 >> 1, half = kc8 & 1;
      bf16* row = &sV[buf][drow * VROW + 16 * g + 4 * half];
      *(uint2*)row = uint2{st.v[i][0], st.v[i][1]};
      *(uint2*)(row + 8) = uint2{st.v[i][2], st.v[i][3]};
    }
  };

  auto compute = [&](int kt, int cur) {
    const int key0 = (t_begin + kt) * ATT_KT;
    f32x16 s[2];
    {
      bf16x8 kf[2][KS];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          kf[kb][ks] = *(const bf16x8*)(&sK[cur][(kb * 32 + j) * KROW + ks * 16 + 8 * hh]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kb][0], qf[0], negm, 0, 0, 0);
#pragma unroll
        for (int ks = 1; ks < KS; ++ks)
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kb][ks], qf[ks], s[kb], 0, 0, 0);
      }
    }
    // the P V operands, read while the score MFMAs run (d_h <= 64; the
    // wider head reads them at their use, within its register budget)
    constexpr int VPRE = DH <= 64 ? 4 : 1;
    auto vread = [&](int db, int g) {
      return *(const bf16x8*)(&sV[cur][(db * 32 + j) * VROW + 16 * g + 8 * hh]);
    };
    bf16x8 vf[DB][VPRE];
    if constexpr (DH <= 64) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int db = 0; db < DB; ++db) vf[db][g] = vread(db, g);
    }
    const bool need_mask = (key0 + ATT_KT - 1 > wave_qmin) || (key0 + ATT_KT > k_end);
    if (need_mask) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (key > qpos || key >= k_end) s[kb][r] = -INFINITY;
        }
    }
    // The exponentials are taken against the current reference first and
    // the reference check (a max tree over the tile, the two halves of the
    // query combined by a lane swap) runs beside them; in the rare tile that
    // moves the reference they are taken again.
    bf16x8 pf[4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        pf[g][i] = (bf16)__builtin_amdgcn_exp2f(s[g >> 1][8 * (g & 1) + i]);
    float tm[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x16& v = s[c >> 1];
      const int o = 8 * (c & 1);
      tm[c] = fmaxf(fmaxf(fmaxf(v[o], v[o + 1]), v[o + 2]),
                    fmaxf(fmaxf(v[o + 3], v[o + 4]), fmaxf(fmaxf(v[o + 5], v[o + 6]), v[o + 7])));
    }
    float t = fmaxf(fmaxf(tm[0], tm[1]), fmaxf(tm[2], tm[3]));
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t),
                                                       false, false);
      t = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const bool up = t > RESCALE_LOG2;
    const bool move = up || (t < -RESCALE_LOW && t > -INFINITY && acc_l[0] == 0.f);
    if (__builtin_amdgcn_ballot_w64(move) != 0) {
      asm volatile("" ::: "memory");
      const float dm = move ? t : 0.f;
      // a downward move finds O and l still zero: nothing to rescale
      const float alpha = up ? __builtin_amdgcn_exp2f(-dm) : 1.0f;
      m_run += dm;
#pragma unroll
      for (int e = 0; e < 16; ++e) negm[e] = -m_run;
      acc_l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc_o[db] *= alpha;
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          pf[g][i] = (bf16)__builtin_amdgcn_exp2f(s[g >> 1][8 * (g & 1) + i] - dm);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      acc_l = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, pf[g], acc_l, 0, 0, 0);
#pragma unroll
      for (int db = 0; db < DB; ++db)
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            DH <= 64 ? vf[db][g % VPRE] : vread(db, g), pf[g], acc_o[db], 0, 0, 0);
    }
  };

  gload(ra, 0);
  if (n_tiles > 1) gload(rb, 1);
  lstore(ra, 0);
  __syncthreads();
#pragma clang loop unroll(disable)
  for (int kt = 0; kt < n_tiles; kt += 2) {
    if (kt + 2 < n_tiles) gload(ra, kt + 2);
    if (active) compute(kt, 0);
    if (kt + 1 < n_tiles) lstore(rb, 1);
    __syncthreads();
    if (kt + 1 >= n_tiles) break;
    if (kt + 3 < n_tiles) gload(rb, kt + 3);
    if (active) compute(kt + 1, 1);
    if (kt + 2 < n_tiles) lstore(ra, 0);
    __syncthreads();
  }

  // lane (j, hh) holds dimensions db*32 + 8g + 4hh .. +3 of its query in
  // acc_o[db][4g .. 4g+3]
  if (n_chunks == 1) {
    if (active && t_q < R) {
      const float inv = 1.0f / acc_l[0];
      bf16* orow = a.out + ((size_t)n * R + t_q) * d + head * DH + 4 * hh;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (bf16)(acc_o[db][4 * g + e] * inv);
          *(bf16x4*)(orow + db * 32 + 8 * g) = o;
        }
    }
    return;
  }

  constexpr int SLOT = ATT_QT * (DH + 2);
  const int tq = wave * 32 + j;   // query within the tile
  if (active) {
    const __amdgpu_buffer_rsrc_t rs = slot_rsrc_dh<DH>(a.part + (size_t)u * SLOT);
    const float l = acc_l[0];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 v = {acc_o[db][4 * g], acc_o[db][4 * g + 1], acc_o[db][4 * g + 2],
                         acc_o[db][4 * g + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs,
                                               (tq * DH + db * 32 + 8 * g + 4 * hh) * 4, 0,
                                               ATT_SC1);
      }
    if (hh == 0) {
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l > 0.f ? m_run : -1e30f), rs,
                                            (ATT_QT * DH + tq) * 4, 0, ATT_SC1);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l), rs,
                                            (ATT_QT * DH + ATT_QT + tq) * 4, 0, ATT_SC1);
    }
  }
  wait_stores();
  __syncthreads();
  __shared__ unsigned s_last;
  if (tid == 0) {
    unsigned* tk = a.tickets + (size_t)nh * a.n_qt + qt;
    const unsigned last = atomicAdd(tk, 1u) + 1u == (unsigned)n_chunks;
    if (last) __hip_atomic_store(tk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  if (!s_last || !active) return;

  attn32_merge<DH>(a, u - chunk, n_chunks, tq, t_q, n, head, hh);
}

template <int DH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void
attn32_kernel(AttnArgs a) {
  attn32_body<DH>(a);
}

// ---------------------------------------------------------------------------
// The same computation with the K and Vt tiles moved from global memory
// straight into LDS (global_load_lds_dwordx4): no staging registers and no
// LDS stores in the loop.  Tiles are kept in a ring of STAGES buffers (tile x
// in buffer x % STAGES), each a K tile [64 keys][DH] and a Vt tile [DH][64
// keys] in rows of whole 16-byte chunks, XOR-swizzled so that the 16-byte
// fragment reads are free of bank conflicts: LDS serves a 16-byte read to 16
// lanes per cycle over its 64 banks, and the 16 lanes of a fragment read take
// one chunk of 16 consecutive rows.  Rows of 128 bytes (Vt, and K at d_h 64)
// put even and odd rows on opposite bank halves, so chunk c of row r sits at
// slot c ^ ((r >> 1) & 7); rows of 256 bytes (K at d_h 128) start on the same
// bank, so at slot c ^ (r & 15).  (Keyed on r & 7, rows r and r + 8 collided:
// half of the LDS cycles were conflicts, though removing them gained little at
// d_h 64 and 7% at d_h 128.)  Vt is stored in key order; the P operand is
// brought to the same key order instead: of each 16-key step the lane pair
// (j, j + 32) swaps the middle 8 bytes of their P fragments
// (v_permlane32_swap), after which lane half h holds keys 16g + 8h .. +7, the
// keys of its Vt fragment.  Iteration t issues the loads of tile
// t + STAGES - 1 into the buffer of tile t - 1 (free since the barrier that
// ended iteration t - 1), computes tile t, then waits for its share of tile
// t + 1 and meets the other waves at the barrier.  The P V MFMAs run at raised
// wave priority, so they issue ahead of the other waves' softmax work.  Keys
// of the last tile at or past the chunk end are zeroed in LDS before use (the
// cache holds stale rows there).
// ---------------------------------------------------------------------------
// One unit of the DMA kernel: keys [k_begin, k_end) of query tile qt of
// (sample, head) pair nh.  With n_chunks == 1 the unit covers the tile's whole
// key range and writes the normalised output; otherwise it writes its partial
// to slot `slot`, and the last of the tile's n_chunks units to finish (slots
// first_slot .. first_slot + n_chunks - 1, in key order) merges them.
// G = 2: a block of 8 waves, two key groups of 4 waves with a ring each; group
// 0 takes the first half of the unit's key tiles and group 1 the rest, both
// over the same 128 queries, and group 1 hands its row state (reference, row
// sum, O) to group 0 through LDS at the end, which adds it in a fixed order:
// the unit's chain of dependent tiles is half as long, for launches with few
// long units.
template <int DH, int G>
__device__ __forceinline__ void attn_dma_unit(const AttnArgs& a, const int nh, const int qt,
                                             const int k_begin, const int k_end_unit,
                                             const int slot, const int first_slot,
                                             const int n_chunks) {
  static_assert(G == 1 || G == 2, "key groups");
  static_assert(DH == 64 || DH == 128, "head width");
  constexpr int KS = DH / 16, DB = DH / 32;
  constexpr int STAGES = DH <= 64 ? 3 : 2;
  constexpr int KBYTES = ATT_KT * DH * 2;           // K tile bytes (= Vt tile bytes)
  constexpr int NI = DH / 8;                        // K (and Vt) instructions per tile
  constexpr int IPW = 2 * NI / 4;                   // instructions per wave per tile
  constexpr int CPR = DH / 8;                       // K chunks per row
  // 16-byte slot of chunk c in row r of a K (or Q) tile and of a Vt tile
  auto swzk = [](int c, int r) { return CPR == 8 ? (c ^ ((r >> 1) & 7)) : (c ^ (r & 15)); };
  auto swzv = [](int c, int r) { return c ^ ((r >> 1) & 7); };
  // Key held by LDS row r of a K tile: bits 2 and 3 of the row swapped.  The
  // scores of LDS rows {16g + 4h + i, 16g + 8 + 4h + i} (i < 4) sit in lane
  // half h, and with this order they are keys 16g + 8h .. 16g + 8h + 7, the
  // keys of that lane half's Vt fragment: the scores feed the P V MFMAs as
  // they are, with Vt in plain key order.
  auto krow = [](int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); };
  typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
  __shared__ __attribute__((aligned(1024))) char smem_all[G][STAGES][2 * KBYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform (the DMA takes its LDS address in a scalar register)
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = G == 1 ? 0 : wave_all >> 2;   // key group
  const int wave = wave_all & 3;                 // wave within the group
  char (&smem)[STAGES][2 * KBYTES] = smem_all[grp];
  const int j = lane & 31, hh = lane >> 5;
  const int n = nh / a.H, head = nh - n * a.H;
  const int R = a.R, d = a.d, Lcap = a.Lcap, pos_base = a.pos_base;
  const int q_lo = qt * ATT_QT;
  // the unit's key tiles, the first `half` of them to group 0; every group
  // runs n_iter loop trips (the barriers are the block's)
  const int t_unit = (k_end_unit - k_begin + ATT_KT - 1) / ATT_KT;
  const int half = G == 1 ? t_unit : (t_unit + 1) / 2;
  const int n_iter = half;
  const int t_begin = k_begin / ATT_KT + (grp == 0 ? 0 : half);
  const int n_tiles = grp == 0 ? half : t_unit - half;
  const int k_end = grp == 0 ? min(k_end_unit, k_begin + half * ATT_KT) : k_end_unit;
  // tile kt of group g ends past its key range (its Vt tail is zeroed)
  auto tail_of = [&](int g, int kt) {
    const int tb = k_begin / ATT_KT + (g == 0 ? 0 : half);
    const int nt = g == 0 ? half : t_unit - half;
    const int ke = g == 0 ? min(k_end_unit, k_begin + half * ATT_KT) : k_end_unit;
    return kt < nt && (tb + kt) * ATT_KT + ATT_KT > ke;
  };
  const size_t hb = (size_t)n * a.H + head;
  const bf16* kbase = a.kc + hb * Lcap * DH;
  const bf16* vbase = a.vt + hb * DH * Lcap;
  const bool active = q_lo + wave * 32 < R;
  const int t_q = q_lo + wave * 32 + j;
  const int qpos = pos_base + t_q;
  const int wave_qmin = pos_base + q_lo + wave * 32;

  // this wave's DMA lanes: K instruction q = wave + 4i covers rows
  // (64 / CPR) q .. ; Vt instruction q covers dimensions 8q .. 8q + 7
  uint32_t koff[NI / 4], voff[NI / 4];
#pragma unroll
  for (int i = 0; i < NI / 4; ++i) {
    const int q = wave + 4 * i;
    {
      // LDS row r holds key krow(r) of the tile (see the P operand below)
      const int r = q * (64 / CPR) + lane / CPR, s = lane % CPR, c = swzk(s, r);
      koff[i] = (uint32_t)((krow(r) * DH + c * 8) * 2);
    }
    {
      const int r = 8 * q + (lane >> 3), s = lane & 7, c = swzv(s, r);
      voff[i] = (uint32_t)((r * Lcap + c * 8) * 2);
    }
  }
  const uint32_t lds0 = lds_address(&smem[0][0]);
  auto issue = [&](int kt) {
    const int k0 = (t_begin + kt) * ATT_KT;
    const uint32_t st = lds0 + (uint32_t)((kt % STAGES) * 2 * KBYTES);
    const bf16* kp = kbase + (size_t)k0 * DH;
    const bf16* vp = vbase + k0;
#pragma unroll
    for (int i = 0; i < NI / 4; ++i) {
      const int q = wave + 4 * i;
      dma16(kp, koff[i], st + q * 1024);
      dma16(vp, voff[i], st + KBYTES + q * 1024);
    }
  };
  // LDS byte offsets of this lane's fragments within a stage
  auto kfrag = [&](int kb, int ks) {
    const int r = kb * 32 + j, c = 2 * ks + hh;
    return r * DH * 2 + 16 * swzk(c, r);
  };
  auto vfrag = [&](int db, int g) {
    const int r = db * 32 + j, c = 2 * g + hh;
    return KBYTES + r * 128 + 16 * swzv(c, r);
  };

  bf16x8 qf[KS];   // this lane's query fragments, read from LDS in the prologue
  float m_run = 0.f;
  f32x16 acc_o[DB], negm;
#pragma unroll
  for (int e = 0; e < 16; ++e) negm[e] = 0.f;
#pragma unroll
  for (int db = 0; db < DB; ++db) acc_o[db] = negm;
  // this lane's share of its row's sum of p (its lane half's keys), in two
  // chains; the halves are added at the end
  float lsum[2] = {0.f, 0.f};
  bool row_mass = false;   // the row's running sum is no longer zero

  // scores of tile kt minus the current reference (K from its buffer)
  auto scores = [&](f32x16 (&s)[2], int kt) {
    const char* stg = &smem[kt % STAGES][0];
    bf16x8 kf[2][KS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[kb][ks] = *(const bf16x8*)(stg + kfrag(kb, ks));
    // the two 32-key halves' chains interleaved, at raised wave priority (one
    // below the P V MFMAs': a wave that reaches either MFMA phase issues it
    // ahead of the other waves' softmax, which then fills the matrix pipe's
    // busy cycles)
    __builtin_amdgcn_s_setprio(1);
    s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[0][0], qf[0], negm, 0, 0, 0);
    s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[1][0], qf[0], negm, 0, 0, 0);
#pragma unroll
    for (int ks = 1; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kb][ks], qf[ks], s[kb], 0, 0, 0);
    __builtin_amdgcn_s_setprio(0);
  };
  // softmax of tile kt's scores and its row-sum and P V MFMAs (V from its
  // buffer)
  auto finish = [&](f32x16 (&s)[2], int kt) {
    const char* stg = &smem[kt % STAGES][0];
    const int key0 = (t_begin + kt) * ATT_KT;
    // the Vt fragments of the first two P V steps read before the softmax, so
    // that the P V phase does not start on an LDS wait (at d_h 64, where the
    // registers are there; at 128 they would spill)
    constexpr int NPRE = DH == 64 ? 2 : 0;
    bf16x8 vpre[NPRE > 0 ? NPRE : 1][DB];
#pragma unroll
    for (int g = 0; g < NPRE; ++g)
#pragma unroll
      for (int db = 0; db < DB; ++db) vpre[g][db] = *(const bf16x8*)(stg + vfrag(db, g));
    const bool need_mask = (key0 + ATT_KT - 1 > wave_qmin) || (key0 + ATT_KT > k_end);
    auto mask = [&]() {
      if (need_mask) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + krow(kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3));
            if (key > qpos || key >= k_end) s[kb][r] = -INFINITY;
          }
      }
    };
    mask();
    // p = 2^(s - m) against the current reference, and the row's largest p of
    // the tile from the fp32 bit patterns (p >= 0, so their unsigned order is
    // the value order: integer maxima, which run beside the exponentials)
    bf16x8 pf[4];
    unsigned pm = 0u;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float e = __builtin_amdgcn_exp2f(s[g >> 1][8 * (g & 1) + i]);
        pm = max(pm, __float_as_uint(e));
        pf[g][i] = (bf16)e;
      }
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(pm, pm, false, false);
      pm = max(sw[0], sw[1]);
    }
    // The reference moves up when the row's largest p exceeds 2^8 (an
    // overflow to inf included), and down while the row has no mass yet when
    // it is below 2^-32; a row whose keys of this tile are all masked (keys
    // key0 .. key0 + 63, all above its position) keeps it.
    const bool up = pm > F32_2P8;
    const bool move = up || (!row_mass && key0 <= qpos && pm < F32_2M32);
    if (__builtin_amdgcn_ballot_w64(move) != 0) {
      asm volatile("" ::: "memory");
      // the scores again (K is still in this tile's buffer) and the row maximum
      scores(s, kt);
      mask();
      float tm[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x16& v = s[c >> 1];
        const int o = 8 * (c & 1);
        tm[c] = fmaxf(fmaxf(fmaxf(v[o], v[o + 1]), v[o + 2]),
                      fmaxf(fmaxf(v[o + 3], v[o + 4]), fmaxf(fmaxf(v[o + 5], v[o + 6]), v[o + 7])));
      }
      float t = fmaxf(fmaxf(tm[0], tm[1]), fmaxf(tm[2], tm[3]));
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t),
                                                         false, false);
        t = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const float dm = move ? t : 0.f;
      // a downward move finds O and l still zero: nothing to rescale
      const float alpha = up ? __builtin_amdgcn_exp2f(-dm) : 1.0f;
      m_run += dm;
#pragma unroll
      for (int e = 0; e < 16; ++e) negm[e] = -m_run;
      lsum[0] *= alpha;
      lsum[1] *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc_o[db] *= alpha;
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          pf[g][i] = (bf16)__builtin_amdgcn_exp2f(s[g >> 1][8 * (g & 1) + i] - dm);
    }
    // the row has mass once a tile put p >= 2^-32 into it (a moved reference
    // makes the tile's largest p 1)
    row_mass = row_mass || move || pm >= F32_2M32;
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            g < NPRE ? vpre[g < NPRE ? g : 0][db] : *(const bf16x8*)(stg + vfrag(db, g)), pf[g],
            acc_o[db], 0, 0, 0);
      // row sums of the same bf16 p: 2-term dot products with (1, 1)
      const u32x4 pw = __builtin_bit_cast(u32x4, pf[g]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // (a variable of its own: clang mis-reads __builtin_bit_cast of a
        // vector element, taking element 0)
        const unsigned pair = pw[w];
        lsum[w & 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair),
                                                      bf16x2{(bf16)1.0f, (bf16)1.0f},
                                                      lsum[w & 1], false);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // zero the Vt columns of keys at or past k_end in tile kt's buffer
  auto zero_tail = [&](int kt) {
    const int kvalid = k_end - (t_begin + kt) * ATT_KT;
    char* stg = &smem[kt % STAGES][0];
    for (int idx = tid & 255; idx < DH * ATT_KT; idx += 256) {   // the group's 256 threads
      const int r = idx / ATT_KT, kk = idx - r * ATT_KT;
      if (kk >= kvalid) {
        const int c = kk >> 3, e = kk & 7;
        *(bf16*)(stg + KBYTES + r * 128 + 16 * swzv(c, r) + 2 * e) = (bf16)0.0f;
      }
    }
  };

  // prologue: the query tile into the last ring buffer and tiles
  // 0 .. STAGES-2 into the first ones, all in flight together.  The query
  // tile is stored like a K tile (rows of DH, swizzled); its rows past the
  // last one read that row.
  {
    const uint32_t qst = lds0 + (uint32_t)((STAGES - 1) * 2 * KBYTES);
    const bf16* qb = a.q + head * DH;
#pragma unroll
    for (int i = 0; i < 2 * NI / 4; ++i) {
      const int q = wave + 4 * i;   // 2 NI instructions of 64 / CPR rows
      const int r = q * (64 / CPR) + lane / CPR, sl = lane % CPR, c = swzk(sl, r);
      const int t = min(q_lo + r, R - 1);
      dma16(qb, (uint32_t)(((size_t)n * R + t) * d * 2 + c * 16), qst + q * 1024);
    }
  }
#pragma unroll
  for (int kt = 0; kt < STAGES - 1; ++kt)
    if (kt < n_tiles) issue(kt);
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  {
    const char* qs = &smem[STAGES - 1][0];
    const int r = wave * 32 + j;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = 2 * ks + hh;
      qf[ks] = *(const bf16x8*)(qs + r * DH * 2 + 16 * swzk(c, r));
    }
  }
  // every wave has its query fragments before tile STAGES-1 reuses the buffer
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  f32x16 s[2];
#pragma clang loop unroll(disable)
  for (int kt = 0; kt < n_iter; ++kt) {
    const bool more = kt + STAGES - 1 < n_tiles;
    if (more) issue(kt + STAGES - 1);
    const bool tail0 = tail_of(0, kt), tail1 = G == 2 && tail_of(1, kt);
    if (tail0 || tail1) {   // block-uniform
      if (grp == 0 ? tail0 : tail1) zero_tail(kt);
      __syncthreads();
    }
    if (active && kt < n_tiles) {
      scores(s, kt);
      finish(s, kt);
    }
    // tile kt + 1 has landed once at most the later tiles' loads are pending
    if (more) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"((STAGES - 2) * IPW) : "memory");
    else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }

  // the row sum: both chains, both lane halves
  float l_row = lsum[0] + lsum[1];
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_row),
                                                     __float_as_uint(l_row), false, false);
    l_row = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  if constexpr (G == 2) {
    // group 1's (reference, row sum, O) into the free rings, as arrays of 256
    // lanes; group 0 adds them to its own, group 0's terms first.  A group
    // with no key of the row (l = 0) contributes nothing.
    float* xs = (float*)&smem_all[0][0][0];
    const int sl = wave * 64 + lane;
    if (grp == 1) {
      xs[sl] = l_row > 0.f ? m_run : -1e30f;
      xs[256 + sl] = l_row;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) xs[(2 + 16 * db + e) * 256 + sl] = acc_o[db][e];
    }
    __syncthreads();
    if (grp == 0) {
      const float m0 = l_row > 0.f ? m_run : -1e30f, m1 = xs[sl], l1 = xs[256 + sl];
      const float mg = fmaxf(m0, m1);
      const float a0 = __builtin_amdgcn_exp2f(m0 - mg), a1 = __builtin_amdgcn_exp2f(m1 - mg);
      l_row = l_row * a0 + l1 * a1;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          acc_o[db][e] = acc_o[db][e] * a0 + xs[(2 + 16 * db + e) * 256 + sl] * a1;
      m_run = mg;
    }
  }
  // group 0 holds the block's result
  const bool out_wave = active && grp == 0;
  if (n_chunks == 1) {
    if (out_wave && t_q < R) {
      const float inv = 1.0f / l_row;
      bf16* orow = a.out + ((size_t)n * R + t_q) * d + head * DH + 4 * hh;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (bf16)(acc_o[db][4 * g + e] * inv);
          *(bf16x4*)(orow + db * 32 + 8 * g) = o;
        }
    }
    return;
  }

  constexpr int SLOT = ATT_QT * (DH + 2);
  const int tq = wave * 32 + j;
  if (out_wave) {
    const __amdgpu_buffer_rsrc_t rs = slot_rsrc_dh<DH>(a.part + (size_t)slot * SLOT);
    const float l = l_row;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 v = {acc_o[db][4 * g], acc_o[db][4 * g + 1], acc_o[db][4 * g + 2],
                         acc_o[db][4 * g + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs,
                                               (tq * DH + db * 32 + 8 * g + 4 * hh) * 4, 0,
                                               ATT_SC1);
      }
    if (hh == 0) {
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l > 0.f ? m_run : -1e30f), rs,
                                            (ATT_QT * DH + tq) * 4, 0, ATT_SC1);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l), rs,
                                            (ATT_QT * DH + ATT_QT + tq) * 4, 0, ATT_SC1);
    }
  }
  wait_stores();
  __syncthreads();
  __shared__ unsigned s_last;
  if (tid == 0) {
    unsigned* tk = a.tickets + (size_t)nh * a.n_qt + qt;
    const unsigned last = atomicAdd(tk, 1u) + 1u == (unsigned)n_chunks;
    if (last) __hip_atomic_store(tk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  if (!s_last || !out_wave) return;
  attn32_merge<DH>(a, first_slot, n_chunks, tq, t_q, n, head, hh);
}

template <int DH, int G>
__device__ __forceinline__ void attn_dma_body(const AttnArgs& a) {
  // unit -> (sample, head, query tile, chunk).  Block ids go round-robin over
  // the 8 XCDs; when N*H is a multiple of 8, (sample, head) pairs are dealt so
  // that all units of one head run on one XCD and share its K/V in that L2.
  int u = blockIdx.x;
  if (a.xcd_map) {
    const int xcd = u & 7, local = u >> 3;
    const int jj = local / a.U_nh;
    u = (jj * 8 + xcd) * a.U_nh + (local - jj * a.U_nh);
  }
  const int nh = u / a.U_nh;
  int rem = u - nh * a.U_nh;
  // Within a pair the blocks run chunk-major: chunk j of every query tile that
  // has one, then chunk j + 1, so that the units that read one key range are
  // dispatched together and share it in L2 (the partial slots stay numbered
  // query tile by query tile, chunks in key order).  Against query-tile-major
  // order, on one box: attention 132 -> 128 us per launch on average over the
  // 21-frame video, +1.8% tokens/s.
  int j = 0, q0 = 0;
  for (;;) {
    while (q0 < a.n_qt && att_chunks(q0, a.R, a.pos_base, a.KC) <= j) ++q0;
    if (rem < a.n_qt - q0) break;
    rem -= a.n_qt - q0;
    ++j;
  }
  const int qt = q0 + rem;
  int before = 0;
  for (int q = 0; q < qt; ++q) before += att_chunks(q, a.R, a.pos_base, a.KC);
  const int nk = a.pos_base + min(a.R, (qt + 1) * ATT_QT);
  const int slot0 = nh * a.U_nh + before;
  attn_dma_unit<DH, G>(a, nh, qt, j * a.KC, min(nk, (j + 1) * a.KC), slot0 + j, slot0,
                   att_chunks(qt, a.R, a.pos_base, a.KC));
}

// Three blocks per CU at d_h 64 (at most 168 registers), two at d_h 128.
template <int DH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DH <= 64 ? 3 : 2))) void
attn_dma_kernel(AttnArgs a) {
  attn_dma_body<DH, 1>(a);
}

// Two key groups per block (8 waves): one block per CU (two rings).
template <int DH>
__global__ __launch_bounds__(512) void attn_dma2_kernel(AttnArgs a) {
  attn_dma_body<DH, 2>(a);
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

// Key chunk of the 32 x 32 kernels: the multiple of the 64-key tile that
// minimises the modelled time rounds x (tiles of the longest unit + a fixed
// cost of UNIT_COST tiles per unit: its prologue, output or partial store and
// merge share), where rounds = ceil(units / slots) and slots = 256 CUs x the
// blocks one CU holds, plus ATT_MERGE_COST tiles per chunk of the longest
// query tile (each chunk's partial store, ticket and share of the merge); at
// most max(1024, N H query tiles) units (the partial slots of the workspace).
// Candidates are the chunk lengths that cut the longest key range into c
// equal parts; results are memoised per shape.  The merge cost was fitted to
// a sweep of c at every frame of the 21-frame video (1560 queries, 16 heads
// of 64, caches evicted between launches): with 16 the model picks the
// fastest c at all 20 frames (2 chunks at frames 1 to 3, 3 from frame 4 on;
// with 1 it took 4 at frames 1 and 2, 12% and 8% slower there).
constexpr int ATT_UNIT_COST = 3;
constexpr int ATT_MERGE_COST = 16;
static int chunk_for_slots(int N, int R, int H, int pos_base, int slots) {
  struct Entry { int N, R, H, pos_base, slots, kc; };
  thread_local Entry memo[64];
  thread_local int memo_n = 0;
  for (int i = 0; i < memo_n; ++i) {
    const Entry& e = memo[i];
    if (e.N == N && e.R == R && e.H == H && e.pos_base == pos_base && e.slots == slots)
      return e.kc;
  }
  const int n_qt = (R + ATT_QT - 1) / ATT_QT;
  const int max_tiles = (pos_base + R + ATT_KT - 1) / ATT_KT;
  const long cap = std::max<long>(1024, (long)N * H * n_qt);
  long best_cost = -1;
  int best = max_tiles * ATT_KT;
  int prev_kt = -1;
  for (int c = 1; c <= max_tiles; ++c) {
    const int kt = (max_tiles + c - 1) / c;
    if (kt == prev_kt) continue;
    prev_kt = kt;
    const long units = (long)N * H * att_units(R, pos_base, kt * ATT_KT, n_qt);
    if (units > cap) break;
    const long rounds = (units + slots - 1) / slots;
    // the chunk that merges reads every chunk of its query tile in turn
    const long cost = rounds * (kt + ATT_UNIT_COST) + ATT_MERGE_COST * c;
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = kt * ATT_KT;
    }
  }
  memo[memo_n % 64] = Entry{N, R, H, pos_base, slots, best};
  ++memo_n;
  if (memo_n >= 64) memo_n = 64;
  return best;
}

// blocks of the 32 x 32 kernels one CU holds (registers and LDS)
static int att_blocks_per_cu(int dh) { return dh == 128 ? 2 : 3; }

// Kernel of a bf16 launch.  The split (higher-precision forward) mode runs
// the 16 x 16 kernel; d_h = 32 the register-staged 32 x 32 kernel.  At d_h 64
// a launch of at most 256 query tiles over at most 100 key tiles (the first
// frames of a 1560-token video, or a frame with no cached prefix) runs the
// two-key-group DMA kernel over whole key ranges, one unit per CU with the
// chain of each unit halved (at 1560 tokens and 16 heads: 24.2 against 27.4
// us with no prefix, 41.1 against 45.9 after one cached frame; from 5 cached
// frames on it is slower); a frame with no cached prefix and fewer than 64
// (sample, head) pairs otherwise the 16 x 16 kernel (26.7 against 35 us for
// the DMA kernel at 1560 tokens and 16 heads, where every unit is a few
// tiles of the causal triangle); everything else the DMA-fed 32 x 32 kernel.
enum AttKind { ATT_SPLIT16, ATT_SMALL16, ATT_REG32, ATT_DMA32, ATT_DMA2 };
static AttKind att_kind(int N, int R, int H, int dh, bool split, int pos_base) {
  if (split) return ATT_SPLIT16;
  if (dh == 32) return ATT_REG32;
  const long n_qt = (R + ATT_QT - 1) / ATT_QT;
  if (dh == 64 && (long)N * H * n_qt <= 256 && (long)pos_base + R <= 100 * ATT_KT)
    return ATT_DMA2;
  if (dh == 64 && pos_base == 0 && N * H < 64) return ATT_SMALL16;
  return ATT_DMA32;
}

int attention_chunk(int N, int R, int H, int dh, bool split, int pos_base) {
  const int n_qt = (R + ATT_QT - 1) / ATT_QT;
  const int nk_max = pos_base + R;
  const AttKind kind = att_kind(N, R, H, dh, split, pos_base);
  if (kind == ATT_DMA2) return (nk_max + ATT_KT - 1) / ATT_KT * ATT_KT;   // whole ranges
  if (kind == ATT_REG32 || kind == ATT_DMA32)
    return chunk_for_slots(N, R, H, pos_base, 256 * att_blocks_per_cu(dh));
  if (kind == ATT_SMALL16)
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
static void attn_launch(const AttnArgs& a, dim3 grid, AttKind kind, hipStream_t st) {
  if constexpr (SPLIT) {
    hipLaunchKernelGGL((attn_bf16_kernel<DH, true>), grid, dim3(256), 0, st, a);
  } else if constexpr (DH == 32) {
    hipLaunchKernelGGL((attn32_kernel<32>), grid, dim3(256), 0, st, a);
  } else {
    if constexpr (DH == 64) {
      if (kind == ATT_SMALL16) {
        hipLaunchKernelGGL((attn_bf16_kernel_o2<64, false>), grid, dim3(256), 0, st, a);
        return;
      }
      if (kind == ATT_DMA2) {
        hipLaunchKernelGGL((attn_dma2_kernel<64>), grid, dim3(512), 0, st, a);
        return;
      }
    }
    hipLaunchKernelGGL((attn_dma_kernel<DH>), grid, dim3(256), 0, st, a);
  }
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
    const AttKind kind = att_kind(N, R, H, dh, split != nullptr, pos_base);
    switch (dh * 2 + (split ? 1 : 0)) {
      case 128: attn_launch<64, false>(a, grid, kind, st); break;
      case 129: attn_launch<64, true>(a, grid, kind, st); break;
      case 256: attn_launch<128, false>(a, grid, kind, st); break;
      case 257: attn_launch<128, true>(a, grid, kind, st); break;
      case 64: attn_launch<32, false>(a, grid, kind, st); break;
      case 65: attn_launch<32, true>(a, grid, kind, st); break;
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
