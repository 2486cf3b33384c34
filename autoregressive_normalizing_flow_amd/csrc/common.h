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

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, AF_WAVE);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, AF_WAVE));
  return v;
}

// GELU u * Phi(u) = 0.5 u (1 + erf(u / sqrt 2)), with erf from Abramowitz &
// Stegun, Handbook of Mathematical Functions, formula 7.1.26:
//   erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2),
//   t = 1 / (1 + p x), x >= 0, |error| <= 1.5e-7; erf(-x) = -erf(x).
// One reciprocal, one exponential and a few FMAs, against the bf16 output
// rounding of 2^-9.
__device__ __forceinline__ float erf_as7126(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * ax);
  const float poly =
      t * (0.254829592f +
           t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  const float y = 1.0f - poly * __expf(-ax * ax);
  return copysignf(y, x);
}
__device__ __forceinline__ float gelu_erf(float u) {
  return 0.5f * u * (1.0f + erf_as7126(u * 0.70710678118654752f));
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
// this lane's outstanding memory operations (stores included) are complete
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

