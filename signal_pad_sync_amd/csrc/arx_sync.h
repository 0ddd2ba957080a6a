// arx_sync.h — device-side synchronisation building blocks of libarx for
// gfx950: the counter barrier and per-block epochs (page "common.cuh"), and
// the barrier tags that check what a barrier makes visible. The blockwise
// signal-pad barrier (page "triton_barrier.py") is the public one of
// include/arx_device.h. Scopes and ordering follow the conventions stated in
// arx_prims.h.
#pragma once

#include <stddef.h>

#include "arx_device.h"
#include "arx_prims.h"

namespace arx {

// ---- barrier tags -----------------------------------------------------------

// The value workgroup `block` of rank `rank` writes before round `rnd` of a
// tagged barrier launch; never zero, distinct per (rank, block, round).
__device__ __forceinline__ uint32_t barrier_tag(int rank, uint32_t block, int rnd) {
  return 0x80000000u | ((uint32_t)rnd << 16) | (block << 4) | (uint32_t)rank;
}

// ---- counter barrier and per-block epochs --------------------------------

// Page "common.cuh", struct Semaphore: a flag every rank adds to and a base
// count only the owning rank reads and writes, on a 128-byte line of its
// own. end_flag / end_base are a second such pair in the same line, used
// only by the split-stage design (start stages count on flag, end stages on
// end_flag).
struct alignas(128) Semaphore {
  uint32_t flag;
  uint32_t base;
  uint32_t pad0[14];
  uint32_t end_flag;
  uint32_t end_base;
  uint32_t pad1[14];
};
static_assert(sizeof(Semaphore) == 128, "Semaphore layout");
static_assert(offsetof(Semaphore, end_flag) == 64, "Semaphore layout");

__device__ __forceinline__ Semaphore* select_sem(Semaphore* const (&sem)[8], int i) {
  Semaphore* r = sem[0];
#pragma unroll
  for (int k = 1; k < 8; ++k) r = (i == k) ? sem[k] : r;
  return r;
}

// Page "common.cuh", PullController::sync, one stage: lane `lane` < world
// adds 1 to block `block_id`'s flag of rank `lane`; the lane whose index is
// the caller's rank then waits until its own flag minus its base reaches a
// target and advances its base.
//   page design (split = false): one flag for both stages; the start stage
//     waits for world, the end stage for 2 * world and then advances the
//     base by 2 * world. Flags only grow, so no reset is needed.
//   split design (split = true, not the page's): start stages count on
//     flag / base, end stages on end_flag / end_base, each stage waits for
//     world and advances its own base by world. An add made for one stage
//     can then never stand in for an add still due on the other, which the
//     single flag allows at world >= 3 over several rounds.
// `fence` makes the add a release and the wait an acquire (system scope);
// the page allows it on end stages only. The caller places the workgroup
// barriers: before a fenced or end stage, after a start stage. Returns false
// if the wait gave up after `timeout` wall-clock ticks.
__device__ __forceinline__ bool counter_sync(Semaphore* const (&sem)[8], int world, uint32_t block_id, int rank,
                                             int lane, bool fence, bool start, bool split, uint64_t timeout) {
  if (lane >= world) return true;
  const bool second = split && !start;
  Semaphore* const peer = select_sem(sem, lane) + block_id;
  uint32_t* flag = second ? &peer->end_flag : &peer->flag;
  if (fence) fence_release_system();
  __hip_atomic_fetch_add(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  if (lane != rank) return true;
  Semaphore* own = select_sem(sem, rank) + block_id;
  uint32_t* const own_flag = second ? &own->end_flag : &own->flag;
  uint32_t* const own_base = second ? &own->end_base : &own->base;
  const uint32_t target = (uint32_t)world * ((split || start) ? 1u : 2u);
  const uint32_t base = *own_base;          // owner-only: a plain load
  const uint64_t t0 = now_ticks();
  while (load_relaxed_system(own_flag) - base < target) {
    if (now_ticks() - t0 > timeout) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  if (fence) fence_acquire_system();
  if (split || !start) *own_base = base + target;   // owner-only: a plain store
  return true;
}

__device__ __forceinline__ uint32_t* select_epochs(uint32_t* const (&e)[8], int i) {
  uint32_t* r = e[0];
#pragma unroll
  for (int k = 1; k < 8; ++k) r = (i == k) ? e[k] : r;
  return r;
}

// Page "common.cuh", PushController: a per-block epoch that alternates
// between 0 and 1 at every kernel exit, so consecutive launches can pick
// alternate buffers per block with no host involvement.
__device__ __forceinline__ uint32_t block_epoch(const uint32_t* epochs, uint32_t block_id) {
  return epochs[block_id];
}
// Call from one thread after the block's last access of its epoch-selected
// buffers (behind a workgroup barrier).
__device__ __forceinline__ void block_epoch_flip(uint32_t* epochs, uint32_t block_id) {
  epochs[block_id] = (epochs[block_id] + 1u) % 2u;
}

}  // namespace arx
