/*
 * arx_device.h — device-side API of libarx for HIP kernels on gfx950: the
 * blockwise signal-pad barrier (page "triton_barrier.py": blockwise_barrier,
 * send_signal, wait_signal), for a caller's own kernels.
 *
 * Header-only: device code is inlined into the calling kernel's code object,
 * so a kernel built with hipcc --offload-arch=gfx950 includes this file and
 * needs nothing else from libarx. libarx's own kernels use the same code.
 *
 * The barrier. W ranks each hold a pad: u32 [nblocks][W] in memory every rank
 * can reach (on one GPU, any device memory; across GPUs, peer-mapped memory).
 * Slot (b, s) of rank r's pad carries rank s's signal to rank r for block id
 * b. All pads start zero-filled. barrier_blockwise(pad, b), called by every
 * thread of a workgroup of rank `pad.rank`, returns in each thread once the
 * workgroups with block id b of all W ranks have called it: thread t < W
 *   1. signals rank t: compare-and-swap slot (b, rank) of rank t's pad from 0
 *      to 1, retried while it still holds rank `rank`'s previous, unconsumed
 *      signal;
 *   2. consumes rank t's signal: compare-and-swap slot (b, t) of its own pad
 *      from 1 to 0, retried until the signal is there.
 * Threads t >= W return at once. Each successful barrier leaves every slot it
 * used at zero again, so consecutive barriers (and hipGraph replays) need no
 * reset.
 *
 * Memory semantics (page "triton_barrier.py", sem argument and usage
 * patterns): with ARX_SEM_ACQ_REL the signal is a release and the consume an
 * acquire, at system scope, so writes the workgroup made before the barrier
 * are visible to the matching workgroups after it; with ARX_SEM_RELAXED the
 * barrier only orders arrival. The function places no workgroup barrier: a
 * caller that publishes writes puts __syncthreads() before it, and one that
 * reads peers' writes puts __syncthreads() after it (the page's pattern 1:
 * __syncthreads, acq_rel barrier, __syncthreads).
 *
 * Every wait is bounded: after pad.timeout wall-clock ticks (the device's
 * constant-rate clock, hipDeviceAttributeWallClockRate kHz) a thread gives up
 * and barrier_blockwise returns false in it; true otherwise. A barrier that
 * timed out leaves signals in the pads; zero-fill them before the next use.
 *
 * All workgroups that wait on each other must be resident on the device at
 * the same time (a grid within the kernel's occupancy per CU times the CU
 * count), or the waits run into their timeout.
 */
#ifndef ARX_DEVICE_H
#define ARX_DEVICE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef ARX_SEM_RELAXED
#define ARX_SEM_RELAXED 0 /* relaxed system-scope CAS on both sides */
#define ARX_SEM_ACQ_REL 1 /* release to signal, acquire to consume */
#endif

/* Default bound of each wait: 2 s of the 100 MHz wall clock. */
#define ARX_PAD_DEFAULT_TIMEOUT 200000000ull

/* The pads of one group as one rank sees them (page "triton_barrier.py":
 * signal_pad_ptrs, rank, world_size, sem). */
typedef struct arx_pad {
  uint32_t* ptr[8];  /* ptr[r]: rank r's pad, u32 [nblocks][W], slot (b, s) at b * W + s; r < W */
  int rank;          /* the calling workgroup's rank, 0 <= rank < W */
  int W;             /* ranks in the group, 2..8 */
  int sem;           /* ARX_SEM_RELAXED or ARX_SEM_ACQ_REL */
  uint64_t timeout;  /* bound of each wait in wall-clock ticks; 0 = ARX_PAD_DEFAULT_TIMEOUT */
} arx_pad_t;

namespace arx_detail {

/* Element i of an array of 8 pointers for a per-lane i, picked by selects:
 * indexing the array with a per-lane value would move it to memory and turn
 * the compare-and-swaps into slower generic-address atomics. */
__device__ __forceinline__ uint32_t* select_pad(uint32_t* const (&p)[8], int i) {
  uint32_t* r = p[0];
#pragma unroll
  for (int k = 1; k < 8; ++k) r = (i == k) ? p[k] : r;
  return r;
}

__device__ __forceinline__ bool cas_system_relaxed(uint32_t* p, uint32_t expect, uint32_t desired) {
  return __hip_atomic_compare_exchange_strong(p, &expect, desired, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_SYSTEM);
}

/* System-scope release fence that has finished when it returns: the fence
 * writes the L2 back (buffer_wbl2), and the explicit wait for every
 * outstanding memory operation (s_waitcnt 0) keeps the next access from being
 * issued before that write-back completes. The compiler's own wait after the
 * write-back is relaxable and can be merged away when an earlier wait already
 * drained the counters, which would let a signal overtake the data it
 * publishes. */
__device__ __forceinline__ void release_system() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "");
  __builtin_amdgcn_s_waitcnt(0);
}

/* One lane's part of a barrier on its two slots: signal by a CAS 0 -> 1 on
 * `send_slot`, then consume by a CAS 1 -> 0 on `wait_slot`. The CASes are
 * relaxed; with acq_rel a system-scope release fence precedes the first
 * signal attempt and an acquire fence follows the successful consume. That
 * orders the same accesses as a release CAS and an acquire CAS, and keeps the
 * cache write-back and invalidate out of the retry loops. Each wait gives up
 * after `timeout` ticks; returns false if one did. */
__device__ __forceinline__ bool signal_wait(uint32_t* send_slot, uint32_t* wait_slot, bool acq_rel,
                                            uint64_t timeout) {
  if (acq_rel) release_system();
  const uint64_t t0 = (uint64_t)wall_clock64();
  while (!cas_system_relaxed(send_slot, 0u, 1u)) {
    if ((uint64_t)wall_clock64() - t0 > timeout) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  const uint64_t t1 = (uint64_t)wall_clock64();
  while (!cas_system_relaxed(wait_slot, 1u, 0u)) {
    if ((uint64_t)wall_clock64() - t1 > timeout) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  if (acq_rel) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
  return true;
}

/* The barrier for lane `lane` of rank `rank`'s block `block_id`: lane < W
 * signals rank `lane` on slot (block_id, rank) of that rank's pad and
 * consumes rank `lane`'s signal on slot (block_id, lane) of its own pad. */
__device__ __forceinline__ bool barrier_lane(uint32_t* const (&ptr)[8], int W, int rank, uint32_t block_id, int lane,
                                             bool acq_rel, uint64_t timeout) {
  if (lane >= W) return true;
  const size_t row = (size_t)block_id * (size_t)W;
  return signal_wait(select_pad(ptr, lane) + row + rank, select_pad(ptr, rank) + row + lane, acq_rel, timeout);
}

}  // namespace arx_detail

/* The blockwise barrier on block id `block_id` for the calling workgroup (see
 * the top of this file). Call from every thread of the workgroup; thread
 * t = threadIdx.x + blockDim.x * (threadIdx.y + blockDim.y * threadIdx.z)
 * takes part if t < pad.W. Returns false in a thread whose wait timed out. */
__device__ __forceinline__ bool barrier_blockwise(arx_pad_t pad, uint32_t block_id) {
  const int t = (int)(threadIdx.x + blockDim.x * (threadIdx.y + blockDim.y * threadIdx.z));
  const uint64_t timeout = pad.timeout ? pad.timeout : ARX_PAD_DEFAULT_TIMEOUT;
  return arx_detail::barrier_lane(pad.ptr, pad.W, pad.rank, block_id, t, pad.sem == ARX_SEM_ACQ_REL, timeout);
}

#endif /* ARX_DEVICE_H */
