// arx_sync.h — device-side synchronisation building blocks of libarx for
// gfx950: the blockwise signal-pad barrier (page "triton_barrier.py"), the
// counter barrier and per-block epochs (page "common.cuh"). Scopes and
// ordering follow the conventions stated in arx_device.h.
#pragma once

#include "arx_device.h"

namespace arx {

// ---- blockwise signal-pad barrier ----------------------------------------

// The pads of one group: pad[r] is rank r's u32[num_blocks][world] array;
// slot (b, s) of rank r's pad carries the signal of rank s for block b.
struct Pads {
  uint32_t* pad[8];
  int world;
};

// One lane's part of the barrier, on its two slots: signal by a CAS 0 -> 1
// on `send_slot` (retried while the slot still holds an unconsumed 1), then
// consume by a CAS 1 -> 0 on `wait_slot`. With acq_rel the signal is a
// release and the consume an acquire; relaxed uses neither. The CASes are
// relaxed and the release / acquire are fences placed before the first
// signal attempt and after the successful consume, which orders the same
// accesses as a release CAS and an acquire CAS while keeping the cache
// write-back and invalidate out of the retry loops. Each wait gives up after
// `timeout` wall-clock ticks; returns false if one did.
__device__ __forceinline__ bool barrier_signal_wait(uint32_t* send_slot, uint32_t* wait_slot, bool acq_rel,
                                                    uint64_t timeout) {
  if (acq_rel) fence_release_system();
  const uint64_t t0 = now_ticks();
  while (!cas_system(send_slot, 0u, 1u, __ATOMIC_RELAXED)) {
    if (now_ticks() - t0 > timeout) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  const uint64_t t1 = now_ticks();
  while (!cas_system(wait_slot, 1u, 0u, __ATOMIC_RELAXED)) {
    if (now_ticks() - t1 > timeout) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  if (acq_rel) fence_acquire_system();
  return true;
}

// Element i of an array of 8 pointers for a per-lane i, picked by selects:
// indexing the array with a per-lane value would move it to memory and turn
// the CASes into slower generic-address atomics.
__device__ __forceinline__ uint32_t* select_pad(uint32_t* const (&pad)[8], int i) {
  uint32_t* r = pad[0];
#pragma unroll
  for (int k = 1; k < 8; ++k) r = (i == k) ? pad[k] : r;
  return r;
}

// Page "triton_barrier.py", blockwise_barrier: lane `lane` < world of the
// calling group (rank `rank`, block id `block_id`) signals rank `lane` on
// slot (block_id, rank) of that rank's pad, then consumes rank `lane`'s
// signal on slot (block_id, lane) of its own pad (barrier_signal_wait gives
// the CAS and ordering rules). Every successful barrier leaves the slots it
// used at zero. Lanes >= world return true at once. The caller adds the
// workgroup barriers that a usage pattern needs (before for publishing,
// after for acquiring).
__device__ __forceinline__ bool barrier_blockwise(const Pads& p, uint32_t block_id, int rank, int lane,
                                                  bool acq_rel, uint64_t timeout) {
  if (lane >= p.world) return true;
  const size_t row = (size_t)block_id * p.world;
  return barrier_signal_wait(select_pad(p.pad, lane) + row + rank, select_pad(p.pad, rank) + row + lane, acq_rel,
                             timeout);
}

// ---- counter barrier and per-block epochs --------------------------------

// Page "common.cuh", struct Semaphore: a flag every rank adds to and a base
// count only the owning rank reads and writes, on a 128-byte line of its own.
struct alignas(128) Semaphore {
  uint32_t flag;
  uint32_t base;
  uint32_t pad[30];
};
static_assert(sizeof(Semaphore) == 128, "Semaphore layout");

__device__ __forceinline__ Semaphore* select_sem(Semaphore* const (&sem)[8], int i) {
  Semaphore* r = sem[0];
#pragma unroll
  for (int k = 1; k < 8; ++k) r = (i == k) ? sem[k] : r;
  return r;
}

// Page "common.cuh", PullController::sync, one stage: lane `lane` < world
// adds 1 to block `block_id`'s flag of rank `lane`; the lane whose index is
// the caller's rank then waits until its own flag minus its base reaches
// world (start stage) or 2 * world (end stage), and an end stage advances
// the base by 2 * world. Flags only grow, so no reset is needed between
// rounds. `fence` makes the add a release and the wait an acquire (system
// scope); the page allows it on end stages only. The caller places the
// workgroup barriers: before a fenced or end stage, after a start stage.
// Returns false if the wait gave up after `timeout` wall-clock ticks.
__device__ __forceinline__ bool counter_sync(Semaphore* const (&sem)[8], int world, uint32_t block_id, int rank,
                                             int lane, bool fence, bool start, uint64_t timeout) {
  if (lane >= world) return true;
  uint32_t* flag = &(select_sem(sem, lane) + block_id)->flag;
  if (fence) __hip_atomic_fetch_add(flag, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
  else __hip_atomic_fetch_add(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  if (lane != rank) return true;
  Semaphore* own = select_sem(sem, rank) + block_id;
  const uint32_t target = (uint32_t)world * (start ? 1u : 2u);
  const uint32_t base = own->base;          // owner-only: a plain load
  const uint64_t t0 = now_ticks();
  while (load_relaxed_system(&own->flag) - base < target) {
    if (now_ticks() - t0 > timeout) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  if (fence) fence_acquire_system();
  if (!start) own->base = base + target;    // owner-only: a plain store
  return true;
}

// Page "common.cuh", PushController: a per-block epoch that alternates
// between 0 and 1 at every kernel exit, so consecutive launches can pick
// alternate buffers per block with no host involvement.
__device__ __forceinline__ uint32_t block_epoch(const uint32_t* epochs, uint32_t block_id) {
  return epochs[block_id];
}
// Call after the block's last access of its epoch-selected buffers: a
// workgroup barrier, then thread 0 flips the epoch.
__device__ __forceinline__ void block_epoch_exit(uint32_t* epochs, uint32_t block_id) {
  __syncthreads();
  if (threadIdx.x == 0) epochs[block_id] = (epochs[block_id] + 1u) % 2u;
}

}  // namespace arx
