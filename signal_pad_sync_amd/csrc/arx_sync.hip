// arx_sync.hip — the synchronisation kernels of libarx for gfx950, each for
// W virtual ranks on this GPU:
//   barrier_kernel           the blockwise signal-pad barrier (page
//                            "triton_barrier.py", blockwise_barrier)
//   counter_barrier_kernel   the counter barrier and per-block epochs (page
//                            "common.cuh", PullController, PushController)
//   symm_allreduce_kernel    an all-reduce through symmetric buffers fenced
//                            by the pad barrier's usage patterns
#include <hip/hip_runtime.h>

#include "arx_device.h"
#include "arx_internal.h"
#include "arx_kernel_util.h"
#include "arx_sync.h"

namespace arx {

// ---- blockwise signal-pad barrier for W virtual ranks ----------------------

// Workgroup b is one wave; its lanes [v * W, v * W + W) play virtual rank v,
// lane v * W + s being that rank's lane s, and call the barrier on block id b
// `rounds` times. A wave runs its lanes' signal loop to completion before
// their consume loop, so every consume finds its signal and no lane waits on
// a lane that has not run. One wave per rank group also means one release
// and one acquire fence per workgroup, not one per virtual rank. With acq_rel
// each round follows usage pattern 1 of the page (workgroup barrier, acq_rel
// barrier, workgroup barrier); relaxed rounds follow pattern 0. The timeout
// only guards against pads that were not zero-filled.
__global__ __launch_bounds__(64) void barrier_kernel(BarrierArgs a) {
  const int W = a.world;
  const int t = threadIdx.x;
  const int v = t / W, s = t - v * W;
  const bool active = t < W * W;
  const size_t row = (size_t)blockIdx.x * W;
  uint32_t* const send_slot = select_pad(a.pad, s) + row + v;   // slot v of rank s's pad
  uint32_t* const wait_slot = select_pad(a.pad, v) + row + s;   // slot s of rank v's pad
  for (int r = 0; r < a.rounds; ++r) {
    if (a.acq_rel) __syncthreads();
    const bool ok = !active || barrier_signal_wait(send_slot, wait_slot, a.acq_rel != 0, a.timeout);
    if (__syncthreads_or(!ok)) {
      if (threadIdx.x == 0) report_error(a.ctl, ERR_BARRIER_TIMEOUT, (uint64_t)blockIdx.x);
      return;
    }
  }
}

hipError_t launch_barrier(const BarrierArgs& a, int nblocks, hipStream_t s) {
  hipLaunchKernelGGL(barrier_kernel, dim3(nblocks), dim3(64), 0, s, a);
  return hipGetLastError();
}

// ---- counter barrier and per-block epochs for W virtual ranks -------------

// Workgroup b is one wave; lanes [v * W, v * W + W) play virtual rank v. The
// block reads its epoch first, runs `rounds` rounds of a start stage
// (unfenced) and an end stage (fenced) on block id b as the page's
// PullController does, then flips its epoch as PushController::exit does.
__global__ __launch_bounds__(64) void counter_barrier_kernel(CounterArgs a) {
  const int W = a.world;
  const int t = threadIdx.x;
  const int v = t / W, s = t - v * W;
  const bool active = t < W * W;
  if (threadIdx.x == 0 && a.seen) a.seen[blockIdx.x] = block_epoch(a.epochs, blockIdx.x);
  for (int r = 0; r < a.rounds; ++r) {
    // start stage: no fence, workgroup barrier after
    bool ok = !active || counter_sync(a.sem, W, blockIdx.x, v, s, false, true, a.timeout);
    if (__syncthreads_or(!ok)) {
      if (threadIdx.x == 0) report_error(a.ctl, ERR_COUNTER_TIMEOUT, (uint64_t)blockIdx.x);
      return;
    }
    // end stage: workgroup barrier before, fenced
    __syncthreads();
    ok = !active || counter_sync(a.sem, W, blockIdx.x, v, s, true, false, a.timeout);
    if (__syncthreads_or(!ok)) {
      if (threadIdx.x == 0) report_error(a.ctl, ERR_COUNTER_TIMEOUT, (uint64_t)blockIdx.x);
      return;
    }
  }
  block_epoch_exit(a.epochs, blockIdx.x);
}

hipError_t launch_counter_barrier(const CounterArgs& a, int nblocks, hipStream_t s) {
  hipLaunchKernelGGL(counter_barrier_kernel, dim3(nblocks), dim3(64), 0, s, a);
  return hipGetLastError();
}

// ---- symmetric-buffer exchange fenced by the pad barrier's patterns --------

// W virtual ranks of `blocks` workgroups each (all resident together):
// workgroup (v, b) is rank v's block b and owns vector slice b of every
// buffer. Page "triton_barrier.py", usage patterns of blockwise_barrier:
//   kernel start:   pattern 0 (relaxed barrier, workgroup barrier) so writes
//                   of earlier kernels to the buffers are visible;
//   each iteration: write this rank's partial into its symmetric buffer;
//                   pattern 1 (workgroup barrier, acq_rel barrier, workgroup
//                   barrier) publishes it to the matching blocks; read slice
//                   b of every rank's buffer and sum in rank order;
//                   pattern 2 (workgroup barrier, relaxed barrier) so the
//                   next iteration's write cannot clobber a slice a peer
//                   still reads.
// The barrier lanes are threads 0..W-1 of each workgroup, as on the page.
template <int W>
__global__ __launch_bounds__(kBlock) void symm_allreduce_kernel(SymmArgs a) {
  const int v = blockIdx.x / a.blocks, b = blockIdx.x - v * a.blocks;
  const uint32_t nv = a.n >> 3, tail = a.n & 7u;
  const uint32_t per = (nv + a.blocks - 1) / a.blocks;
  const uint32_t lo = b * per, hi = min(nv, lo + per);
  uint16_t* const mine = a.symm + (size_t)v * a.stride;
  __amdgpu_buffer_rsrc_t rs[W];
#pragma unroll
  for (int src = 0; src < W; ++src) rs[src] = make_rsrc(a.symm + (size_t)src * a.stride, slot_bytes(a.stride));
  const bool tail_block = b == a.blocks - 1;
  // pattern 0
  bool ok = (int)threadIdx.x >= W ||
            barrier_signal_wait(select_pad(a.pad, threadIdx.x) + (size_t)b * W + v,
                                select_pad(a.pad, v) + (size_t)b * W + threadIdx.x, false, a.timeout);
  if (__syncthreads_or(!ok)) goto fail;
  for (int k = 0; k < a.iters; ++k) {
    const uint16_t* in = a.inputs + ((size_t)k * W + v) * a.ld;
    uint16_t* out = a.outputs + ((size_t)k * W + v) * a.ld;
    for (uint32_t x = lo + threadIdx.x; x < hi; x += kBlock) st16(mine + 8u * (size_t)x, ld16(in + 8u * (size_t)x));
    if (tail_block && threadIdx.x < tail) mine[8u * (size_t)nv + threadIdx.x] = in[8u * (size_t)nv + threadIdx.x];
    // pattern 1
    __syncthreads();
    ok = (int)threadIdx.x >= W ||
         barrier_signal_wait(select_pad(a.pad, threadIdx.x) + (size_t)b * W + v,
                             select_pad(a.pad, v) + (size_t)b * W + threadIdx.x, true, a.timeout);
    if (__syncthreads_or(!ok)) goto fail;
    for (uint32_t x = lo + threadIdx.x; x < hi; x += kBlock) {
      u32x4 y[W];
#pragma unroll
      for (int src = 0; src < W; ++src) y[src] = bload16<CP_SYS>(rs[src], x * 16u);
      st16(out + 8u * (size_t)x, sum_bf16x8<W>(y));
    }
    if (tail_block && threadIdx.x < tail) {
      const uint32_t i = 8u * nv + threadIdx.x;
      uint16_t y[W];
#pragma unroll
      for (int src = 0; src < W; ++src) y[src] = bload2<CP_SYS>(rs[src], i * 2u);
      out[i] = sum_bf16x1<W>(y);
    }
    // pattern 2
    __syncthreads();
    ok = (int)threadIdx.x >= W ||
         barrier_signal_wait(select_pad(a.pad, threadIdx.x) + (size_t)b * W + v,
                             select_pad(a.pad, v) + (size_t)b * W + threadIdx.x, false, a.timeout);
    if (__syncthreads_or(!ok)) goto fail;
  }
  return;
fail:
  if (threadIdx.x == 0) report_error(a.ctl, ERR_SYMM_TIMEOUT, (uint64_t)blockIdx.x);
}

// Workgroups per rank, G: aim for about 128 workgroups in all (W * G),
// between 2 and 8 vectors per thread, at most 64 per rank, and few enough
// that all W * G workgroups are resident together (occupancy per CU times
// the CU count, queried once per W). Every iteration passes two pad
// barriers over all W * G workgroups, whose release and acquire fences
// serialise per XCD, so fewer, fuller workgroups win until the per-thread
// work dominates. Measured on MI355X for W = 2, 4 and 8 and n from 8 Ki to
// 1 Mi elements, the rule is within a few percent of the best G at every
// point; at W = 8, n = 128 Ki it takes 8.3 us per iteration where two
// vectors per thread (32 per rank) took 10.6 us.
template <int W>
static int symm_blocks_w(uint32_t n, int cus) {
  static const int per_cu = [] {
    int o = 0;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
               &o, reinterpret_cast<const void*>(symm_allreduce_kernel<W>), kBlock, 0) == hipSuccess
               ? o
               : 0;
  }();
  const long long nv = n >> 3;
  const long long most = (nv + 2 * kBlock - 1) / (2 * kBlock);   // at least 2 vectors per thread
  const long long least = (nv + 8 * kBlock - 1) / (8 * kBlock);  // at most 8 vectors per thread
  long long g = 128 / W > least ? 128 / W : least;
  if (g > most) g = most;
  if (g > 64) g = 64;
  if (g < 1) g = 1;
  const long long cap = (long long)per_cu * cus / W;
  if (g > cap) g = cap;
  return (int)g;
}

int symm_blocks(uint32_t n, int world, int cus) {
  switch (world) {
    case 2: return symm_blocks_w<2>(n, cus);
    case 3: return symm_blocks_w<3>(n, cus);
    case 4: return symm_blocks_w<4>(n, cus);
    case 5: return symm_blocks_w<5>(n, cus);
    case 6: return symm_blocks_w<6>(n, cus);
    case 7: return symm_blocks_w<7>(n, cus);
    case 8: return symm_blocks_w<8>(n, cus);
    default: return 0;
  }
}

template <int W>
static hipError_t launch_symm_w(const SymmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((symm_allreduce_kernel<W>), dim3(W * a.blocks), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_symm_allreduce(const SymmArgs& a, hipStream_t s) {
  if (a.blocks < 1) return hipErrorInvalidConfiguration;
  switch (a.world) {
    case 2: return launch_symm_w<2>(a, s);
    case 3: return launch_symm_w<3>(a, s);
    case 4: return launch_symm_w<4>(a, s);
    case 5: return launch_symm_w<5>(a, s);
    case 6: return launch_symm_w<6>(a, s);
    case 7: return launch_symm_w<7>(a, s);
    case 8: return launch_symm_w<8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace arx
