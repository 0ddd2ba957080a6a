// arx_kernel_util.h — helpers shared by the kernels of libarx: buffer
// loads with an explicit gfx950 cache policy, and the device-side error
// report into the pinned control block.
#pragma once

#include <hip/hip_runtime.h>

#include "arx_prims.h"
#include "arx_internal.h"

namespace arx {

// ---- buffer loads and stores with an explicit cache policy ---------------

// Cache-policy bits of a gfx950 buffer instruction: sc0 = 1, nt = 2, sc1 = 16.
enum : int {
  CP_SYS = 1 | 16,  // sc0 sc1: coherent at system scope, no stale cached copy
  CP_NT = 2,        // nontemporal: streamed, not kept in the caches
  CP_DEV = 16,      // sc1: coherent at device scope; a store writes through
                    // the L2 instead of staying dirty there
};

// Buffer resource over `bytes` bytes at `base` (raw buffer, stride 0; loads
// past `bytes` return zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

template <int CP>
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, CP);
}

template <int CP>
__device__ __forceinline__ uint16_t bload2(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, byte_off, 0, CP);
}

template <int CP>
__device__ __forceinline__ void bstore16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, CP);
}

// Replica k of the one-shot kernel's go word (WORD_GO, one 256-byte line
// per replica).
__device__ __forceinline__ uint64_t* go_word(uint32_t* words, uint32_t k) {
  return reinterpret_cast<uint64_t*>(words + WORD_GO + 64u * k);
}

__device__ __forceinline__ uint32_t slot_bytes(uint64_t stride) {
  return (uint32_t)(stride * 2u);
}

// Reports a device-side wait timeout to the host through the pinned control
// block (first writer wins only loosely: any writer leaves a valid report).
__device__ __forceinline__ void report_error(Ctl* ctl, uint64_t kind, uint64_t seq) {
  store_relaxed_system(&ctl->err_seq, seq);
  store_release_system(&ctl->err, kind);
}

}  // namespace arx
