// arx_prims.h — device-side building blocks of libarx for gfx950 (HIP).
//
// Memory-scope vocabulary used throughout (HIP / LLVM AMDGPU memory model):
//   agent  = every workgroup of this GPU, across its 8 XCDs (each XCD has its
//            own L2; agent-scope release writes the L2 back, agent-scope
//            acquire invalidates it, and the compiler emits both);
//   system = agent plus the host CPU and other devices, used for the pinned
//            host words (flags, control block) and for the signal pads.
// The barrier building blocks (signal pads, counters, epochs) are in
// arx_sync.h.
// Waits poll with relaxed loads and order once with a fence afterwards, so
// a poll loop does not invalidate caches on every iteration.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace arx {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---- scoped atomics -------------------------------------------------------

template <typename T>
__device__ __forceinline__ T load_relaxed_system(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
template <typename T>
__device__ __forceinline__ T load_relaxed_agent(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void store_relaxed_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void store_relaxed_system(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
// Releases. A release fence writes the issuing XCD's L2 back (buffer_wbl2)
// and must wait for that write-back to finish before the releasing access
// is issued, or the access can reach memory ahead of the data it publishes.
// The compiler emits that wait as a relaxable one, and merges it away when an
// earlier wait has already drained the counters (seen on gfx950 for a
// release atomic issued right after a load it needed: buffer_wbl2 followed
// directly by the atomic). So every release here is an explicit fence, then
// a hard wait for all outstanding memory operations (s_waitcnt 0), then a
// relaxed access.
__device__ __forceinline__ void fence_release_system() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "");
  __builtin_amdgcn_s_waitcnt(0);
}
__device__ __forceinline__ void fence_release_agent() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __builtin_amdgcn_s_waitcnt(0);
}
template <typename T>
__device__ __forceinline__ void store_release_agent(T* p, T v) {
  fence_release_agent();
  store_relaxed_agent(p, v);
}
template <typename T>
__device__ __forceinline__ void store_release_system(T* p, T v) {
  fence_release_system();
  store_relaxed_system(p, v);
}
__device__ __forceinline__ uint32_t fetch_add_release_system(uint32_t* p, uint32_t v) {
  fence_release_system();
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
// The arrival counter takes system-scope atomics only (with or without a
// release before them), so every arrival is performed at the same place.
__device__ __forceinline__ uint32_t fetch_add_relaxed_system(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ uint32_t fetch_add_relaxed_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void fence_acquire_system() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, ""); }
// Acquire and release in one fence (L2 write-back and invalidate), with the
// same hard wait as the releases above.
__device__ __forceinline__ void fence_acq_rel_system() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "");
  __builtin_amdgcn_s_waitcnt(0);
}
__device__ __forceinline__ void fence_acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

// Constant-rate clock (the wall clock; its rate is a device attribute).
__device__ __forceinline__ uint64_t now_ticks() { return (uint64_t)wall_clock64(); }

// ---- 16-byte loads and stores --------------------------------------------

// Plain cached 16-byte load.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Streaming 16-byte load (nontemporal: the line is not kept in the caches),
// used for slots another agent wrote and for the one-pass HBM stream.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void st16_stream(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// ---- bf16 <-> binary32 ----------------------------------------------------

// The two bf16 values packed in a 32-bit word, widened exactly.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// binary32 -> bf16 with round to nearest, ties to even, returned in the upper
// 16 bits: adding 0x7FFF plus the last kept bit carries into the kept part
// exactly when the dropped 16 bits exceed one half, or equal one half with an
// odd kept part. Overflow carries into the exponent and gives +-Inf. Every
// NaN becomes the canonical 0x7FC0.
__device__ __forceinline__ uint32_t round_bf16_hi(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t r = u + 0x7FFFu + ((u >> 16) & 1u);
  return (f != f) ? 0x7FC00000u : r;
}

// Two binary32 values -> one word of two bf16 (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const uint32_t a = round_bf16_hi(lo), b = round_bf16_hi(hi);
  return __builtin_amdgcn_perm(b, a, 0x07060302u);   // bytes: a.b2 a.b3 b.b2 b.b3
}

// Rank-ordered sum of W vectors of 8 bf16: acc starts with partial 0 (the
// same as -0.0 + x0 for every x0), then adds partials 1..W-1 in order.
template <int W>
__device__ __forceinline__ u32x4 sum_bf16x8(const u32x4 (&x)[W]) {
  float acc[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    acc[2 * k] = bf16_lo(x[0][k]);
    acc[2 * k + 1] = bf16_hi(x[0][k]);
  }
#pragma unroll
  for (int src = 1; src < W; ++src) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc[2 * k] = acc[2 * k] + bf16_lo(x[src][k]);
      acc[2 * k + 1] = acc[2 * k + 1] + bf16_hi(x[src][k]);
    }
  }
  u32x4 o;
#pragma unroll
  for (int k = 0; k < 4; ++k) o[k] = pack_bf16x2(acc[2 * k], acc[2 * k + 1]);
  return o;
}

// One element of the same sum, for the tail.
template <int W>
__device__ __forceinline__ uint16_t sum_bf16x1(const uint16_t (&x)[W]) {
  float acc = __uint_as_float((uint32_t)x[0] << 16);
#pragma unroll
  for (int src = 1; src < W; ++src) acc = acc + __uint_as_float((uint32_t)x[src] << 16);
  return (uint16_t)(round_bf16_hi(acc) >> 16);
}

}  // namespace arx
