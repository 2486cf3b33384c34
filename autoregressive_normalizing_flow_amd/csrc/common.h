// Shared device-side definitions for the AF-block kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;

#define AF_WAVE 64

// Storage conversion helpers: fp32 <-> storage type of the per-layer matrices.
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
template <class T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

// Reductions over the 64 lanes of a wave, the result in every lane: within
// each row of 16 lanes by DPP (quad permutes, then rotations by 4 and 8),
// then the four row values read from lanes 0, 16, 32 and 48 and combined in
// that order (a fixed order, and no LDS round trips as a permute-based
// butterfly takes).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_value(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_mov<0xB1>(v);    // quad_perm 1,0,3,2
  v += dpp_mov<0x4E>(v);    // quad_perm 2,3,0,1
  v += dpp_mov<0x124>(v);   // row_ror 4
  v += dpp_mov<0x128>(v);   // row_ror 8
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));
  v = fmaxf(v, dpp_mov<0x4E>(v));
  v = fmaxf(v, dpp_mov<0x124>(v));
  v = fmaxf(v, dpp_mov<0x128>(v));
  return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)),
               fmaxf(lane_value(v, 32), lane_value(v, 48)));
}

// GELU u * Phi(u) = 0.5 u (1 + erf(u / sqrt 2)), with erfc from Abramowitz &
// Stegun, Handbook of Mathematical Functions, formula 7.1.26:
//   erfc(x) = (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2),
//   t = 1 / (1 + p x), x >= 0, |error| <= 1.5e-7.
// With Q = 0.5 erfc(|u| / sqrt 2), Phi(u) is 1 - Q for u >= 0 and Q for
// u < 0, so u Phi(u) = max(u, 0) - |u| Q: one reciprocal, one exponential and
// a few FMAs, and no cancellation in the negative tail.
__device__ __forceinline__ float gelu_erf(float u) {
  const float au = fabsf(u);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f * 0.70710678118654752f, au, 1.0f));
  const float half_poly =
      t * (0.5f * 0.254829592f +
           t * (0.5f * -0.284496736f +
                t * (0.5f * 1.421413741f + t * (0.5f * -1.453152027f + t * (0.5f * 1.061405429f)))));
  // exp(-u^2 / 2) = 2^(-u^2 log2(e) / 2)
  const float e = __builtin_amdgcn_exp2f(u * (u * (-0.5f * 1.4426950408889634f)));
  return fmaf(-au, half_poly * e, fmaxf(u, 0.0f));
}

// Storage index of processing index i in a sequence of length L: right-to-left
// blocks process the sequence flipped.
__device__ __forceinline__ int storage_index(int i, int L, int dir) {
  return dir ? (L - 1 - i) : i;
}

// Cross-workgroup hand-off without L2 maintenance.  The L2 of each XCD is not
// coherent with the others, and an agent-scope fence (__threadfence) writes
// back and invalidates the whole L2 of the XCD, which costs every other block
// there its cached data.  Data passed between blocks therefore goes through
// agent-scope (sc1) stores and loads, and the writer waits for its stores to
// be acknowledged before it takes the ticket.
__device__ __forceinline__ void coherent_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// store that bypasses the device caches, for host-mapped memory the host
// reads once the stream has drained
__device__ __forceinline__ void system_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void system_store(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
// this lane's outstanding memory operations (stores included) are complete
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }


// Direct global -> LDS loads (gfx950 global_load_lds_dwordx4).  One
// wave-instruction writes 64 consecutive 16-byte LDS slots (lane i -> slot i)
// at the LDS address in m0; each lane chooses the global chunk that lands in
// its slot.  Issued from inline asm (saddr form: 64-bit uniform base in SGPRs
// plus a 32-bit per-lane byte offset), with every wait on it explicit: the
// load has no result register, and completion is counted by vmcnt.
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void_t*)p;
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane from base + voff into LDS at m0 + 16 * lane.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop
