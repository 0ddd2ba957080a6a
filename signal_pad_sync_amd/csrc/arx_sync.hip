// arx_sync.hip — the synchronisation kernels of libarx for gfx950, each for
// W virtual ranks on this GPU:
//   barrier_groups_kernel    the blockwise signal-pad barrier (page
//                            "triton_barrier.py", blockwise_barrier), one
//                            workgroup per rank and block
//   barrier_lanes_kernel     the same, the W ranks as lane groups of a wave
//   counter_groups_kernel    the counter barrier and per-block epochs (page
//                            "common.cuh", PullController, PushController)
//   counter_lanes_kernel     the same, as lane groups
//   symm_allreduce_kernel    an all-reduce through symmetric buffers fenced
//                            by the pad barrier's usage patterns
#include <hip/hip_runtime.h>

#include <mutex>

#include "arx.h"
#include "arx_prims.h"
#include "arx_internal.h"
#include "arx_kernel_util.h"
#include "arx_sync.h"

namespace arx {

// ---- blockwise signal-pad barrier for W virtual ranks ----------------------

// One workgroup per rank and block (the default launch): workgroup g plays
// rank v = g % W's block b = g / W, so the W workgroups that synchronise on
// block id b are consecutive and the dispatcher deals them to different XCDs
// (workgroups go round robin to the 8 XCDs), whose L2 caches are not shared:
// a missing release or acquire shows up as a stale tag. Each round follows
// the page's usage pattern 1 with acq_rel (workgroup barrier, barrier,
// workgroup barrier) and pattern 0 with relaxed. With tags, thread 0 writes
// this block's tag for the round into rank v's tag row before the barrier,
// and after it thread p < W reads rank p's tag for the same block and round
// into seen; each round has tag slots of its own, so nothing is overwritten
// while a peer may still read it.
__global__ __launch_bounds__(64) void barrier_groups_kernel(BarrierArgs a) {
  const int W = a.world;
  const int v = (int)(blockIdx.x % (uint32_t)W);
  const uint32_t b = blockIdx.x / (uint32_t)W;
  const size_t nb = (size_t)a.nblocks;
  for (int r = 0; r < a.rounds; ++r) {
    if (a.tags && threadIdx.x == 0) a.tags[((size_t)v * a.rounds + r) * nb + b] = barrier_tag(v, b, r);
    if (a.acq_rel) __syncthreads();
    const bool ok = arx_detail::barrier_lane(a.pad, W, v, b, (int)threadIdx.x, a.acq_rel != 0, a.timeout);
    if (__syncthreads_or(!ok)) {
      if (threadIdx.x == 0) report_error(a.ctl, ERR_BARRIER_TIMEOUT, (uint64_t)blockIdx.x);
      return;
    }
    if (a.seen && (int)threadIdx.x < W)
      a.seen[(((size_t)v * a.rounds + r) * nb + b) * W + threadIdx.x] =
          a.tags[((size_t)threadIdx.x * a.rounds + r) * nb + b];
  }
}

// Lane groups (the named variant): workgroup b is one wave whose lanes
// [v * W, v * W + W) play virtual rank v, lane v * W + s being that rank's
// lane s, and call the barrier on block id b `rounds` times. A wave runs its
// lanes' signal loop to completion before their consume loop, so every
// consume finds its signal and no workgroup waits on another: this launch
// measures the barrier's atomics and fences without cross-workgroup waiting.
__global__ __launch_bounds__(64) void barrier_lanes_kernel(BarrierArgs a) {
  const int W = a.world;
  const int t = threadIdx.x;
  const int v = t / W, s = t - v * W;
  const bool active = t < W * W;
  const size_t row = (size_t)blockIdx.x * W;
  uint32_t* const send_slot = arx_detail::select_pad(a.pad, s) + row + v;   // slot v of rank s's pad
  uint32_t* const wait_slot = arx_detail::select_pad(a.pad, v) + row + s;   // slot s of rank v's pad
  for (int r = 0; r < a.rounds; ++r) {
    if (a.acq_rel) __syncthreads();
    const bool ok = !active || arx_detail::signal_wait(send_slot, wait_slot, a.acq_rel != 0, a.timeout);
    if (__syncthreads_or(!ok)) {
      if (threadIdx.x == 0) report_error(a.ctl, ERR_BARRIER_TIMEOUT, (uint64_t)blockIdx.x);
      return;
    }
  }
}

hipError_t launch_barrier(const BarrierArgs& a, bool lanes, hipStream_t s) {
  if (lanes) hipLaunchKernelGGL(barrier_lanes_kernel, dim3(a.nblocks), dim3(64), 0, s, a);
  else hipLaunchKernelGGL(barrier_groups_kernel, dim3(a.world * a.nblocks), dim3(64), 0, s, a);
  return hipGetLastError();
}

// ---- counter barrier and per-block epochs for W virtual ranks -------------

// One round: a start stage (unfenced) then an end stage (fenced) on block id
// b, as the page's PullController does, for rank v with its lanes 0..W-1.
// With tags, thread 0 writes the block's tag between the two stages and
// thread p < W reads rank p's tag after the end stage (fresh slots per
// round, as in the pad barrier's check). Returns false on a timeout.
__device__ __forceinline__ bool counter_round(const CounterArgs& a, int v, uint32_t b, int lane, bool active,
                                              int r) {
  const int W = a.world;
  const size_t nb = (size_t)a.nblocks;
  // start stage: no fence, workgroup barrier after
  bool ok = !active || counter_sync(a.sem, W, b, v, lane, false, true, a.split != 0, a.timeout);
  if (__syncthreads_or(!ok)) return false;
  if (a.tags && lane == 0 && active) a.tags[((size_t)v * a.rounds + r) * nb + b] = barrier_tag(v, b, r);
  // end stage: workgroup barrier before, fenced
  __syncthreads();
  ok = !active || counter_sync(a.sem, W, b, v, lane, true, false, a.split != 0, a.timeout);
  if (__syncthreads_or(!ok)) return false;
  if (a.tag_seen && active && lane < W)
    a.tag_seen[(((size_t)v * a.rounds + r) * nb + b) * W + lane] = a.tags[((size_t)lane * a.rounds + r) * nb + b];
  return true;
}

// One workgroup per rank and block (the default launch), placed as in
// barrier_groups_kernel. The workgroup reads its rank's epoch for the block
// first, runs `rounds` rounds, then flips the epoch as PushController's exit
// does.
__global__ __launch_bounds__(64) void counter_groups_kernel(CounterArgs a) {
  const int W = a.world;
  const int v = (int)(blockIdx.x % (uint32_t)W);
  const uint32_t b = blockIdx.x / (uint32_t)W;
  uint32_t* const epochs = select_epochs(a.epochs, v);
  if (threadIdx.x == 0 && a.seen) a.seen[(size_t)v * a.nblocks + b] = block_epoch(epochs, b);
  for (int r = 0; r < a.rounds; ++r) {
    if (!counter_round(a, v, b, (int)threadIdx.x, true, r)) {
      if (threadIdx.x == 0) report_error(a.ctl, ERR_COUNTER_TIMEOUT, (uint64_t)blockIdx.x);
      return;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) block_epoch_flip(epochs, b);
}

// Lane groups (the named variant): workgroup b is one wave; lanes
// [v * W, v * W + W) play virtual rank v, so every add precedes every wait
// in one instruction stream and no workgroup waits on another.
__global__ __launch_bounds__(64) void counter_lanes_kernel(CounterArgs a) {
  const int W = a.world;
  const int t = threadIdx.x;
  const int v = t / W, s = t - v * W;
  const bool active = t < W * W;
  const uint32_t b = blockIdx.x;
  if (a.seen && active && s == 0) a.seen[(size_t)v * a.nblocks + b] = block_epoch(select_epochs(a.epochs, v), b);
  for (int r = 0; r < a.rounds; ++r) {
    bool ok = !active || counter_sync(a.sem, W, b, v, s, false, true, a.split != 0, a.timeout);
    if (__syncthreads_or(!ok)) {
      if (threadIdx.x == 0) report_error(a.ctl, ERR_COUNTER_TIMEOUT, (uint64_t)blockIdx.x);
      return;
    }
    __syncthreads();
    ok = !active || counter_sync(a.sem, W, b, v, s, true, false, a.split != 0, a.timeout);
    if (__syncthreads_or(!ok)) {
      if (threadIdx.x == 0) report_error(a.ctl, ERR_COUNTER_TIMEOUT, (uint64_t)blockIdx.x);
      return;
    }
  }
  __syncthreads();
  if (active && s == 0) block_epoch_flip(select_epochs(a.epochs, v), b);
}

hipError_t launch_counter_barrier(const CounterArgs& a, bool lanes, hipStream_t s) {
  if (lanes) hipLaunchKernelGGL(counter_lanes_kernel, dim3(a.nblocks), dim3(64), 0, s, a);
  else hipLaunchKernelGGL(counter_groups_kernel, dim3(a.world * a.nblocks), dim3(64), 0, s, a);
  return hipGetLastError();
}

// Workgroups of barrier_groups_kernel (or counter_groups_kernel) the device
// holds at once: occupancy per CU, queried once per kernel, times the CU
// count; 0 if the query fails.
long long barrier_groups_cap(bool counter, int cus) {
  static const int per_cu_pad = [] {
    int o = 0;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, reinterpret_cast<const void*>(barrier_groups_kernel), 64,
                                                         0) == hipSuccess
               ? o
               : 0;
  }();
  static const int per_cu_counter = [] {
    int o = 0;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, reinterpret_cast<const void*>(counter_groups_kernel), 64,
                                                         0) == hipSuccess
               ? o
               : 0;
  }();
  return (long long)(counter ? per_cu_counter : per_cu_pad) * cus;
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
// Copy and sum move kSymmU vectors per thread per pass with every load in
// flight before the first use: 9.2 -> 8.0 us per iteration at W=8,
// n = 128 Ki on MI355X, where one vector per pass paid a memory round trip
// per vector (2 vectors per pass: 8.1 us). The copy's and the sum's stores
// write through the L2 (device scope) instead of staying dirty there, so
// the release fence of pattern 1 finds nothing of theirs to write back:
// 8.78-8.82 -> 7.49-7.58 us per iteration at W=8, n = 128 Ki (the copy's
// stores alone: 7.56-7.66; nontemporal copy stores: 9.2), 4.16 -> 3.62 us
// at W=2 and 5.32 -> 4.74 us at W=4. From W = 6 on, the sum's stores are
// nontemporal instead (the outputs are never read back here; the wider
// sums stream more): at n = 128 Ki, W=6 8.65 -> 8.16-8.20 us, W=7
// 9.45-9.49 -> 8.41-8.47, W=8 7.34-7.42 -> 7.05; at W = 5 and below they
// tie or lose (W=5, n = 512 Ki: 10.6 -> 11.0 us).
template <int W>
constexpr int kSymmOutPolicy = W >= 6 ? CP_NT : CP_DEV;
constexpr int kSymmU = 4;

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
  const __amdgpu_buffer_rsrc_t rmine = make_rsrc(mine, slot_bytes(a.stride));
  // pattern 0
  bool ok = arx_detail::barrier_lane(a.pad, W, v, b, (int)threadIdx.x, false, a.timeout);
  if (__syncthreads_or(!ok)) goto fail;
  for (int k = 0; k < a.iters; ++k) {
    const uint16_t* in = a.inputs + ((size_t)k * W + v) * a.ld;
    uint16_t* out = a.outputs + ((size_t)k * W + v) * a.ld;
    // the slice moves kSymmU vectors per thread at a time, all loads issued
    // before the first store (one memory round trip per kSymmU vectors)
    for (uint32_t x0 = lo + threadIdx.x; x0 < hi; x0 += kSymmU * kBlock) {
      u32x4 t[kSymmU];
#pragma unroll
      for (int u = 0; u < kSymmU; ++u) {
        const uint32_t x = x0 + (uint32_t)u * kBlock;
        if (x < hi) t[u] = ld16(in + 8u * (size_t)x);
      }
#pragma unroll
      for (int u = 0; u < kSymmU; ++u) {
        const uint32_t x = x0 + (uint32_t)u * kBlock;
        if (x < hi) bstore16<CP_DEV>(rmine, x * 16u, t[u]);
      }
    }
    if (tail_block && threadIdx.x < tail) mine[8u * (size_t)nv + threadIdx.x] = in[8u * (size_t)nv + threadIdx.x];
    // pattern 1
    __syncthreads();
    ok = arx_detail::barrier_lane(a.pad, W, v, b, (int)threadIdx.x, true, a.timeout);
    if (__syncthreads_or(!ok)) goto fail;
    const __amdgpu_buffer_rsrc_t rout = make_rsrc(out, a.n * 2u);
    for (uint32_t x0 = lo + threadIdx.x; x0 < hi; x0 += kSymmU * kBlock) {
      u32x4 y[kSymmU][W];
#pragma unroll
      for (int u = 0; u < kSymmU; ++u) {
        const uint32_t x = x0 + (uint32_t)u * kBlock;
        if (x < hi) {
#pragma unroll
          for (int src = 0; src < W; ++src) y[u][src] = bload16<CP_SYS>(rs[src], x * 16u);
        }
      }
#pragma unroll
      for (int u = 0; u < kSymmU; ++u) {
        const uint32_t x = x0 + (uint32_t)u * kBlock;
        if (x < hi) bstore16<kSymmOutPolicy<W>>(rout, x * 16u, sum_bf16x8<W>(y[u]));
      }
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
    ok = arx_detail::barrier_lane(a.pad, W, v, b, (int)threadIdx.x, false, a.timeout);
    if (__syncthreads_or(!ok)) goto fail;
  }
  return;
fail:
  if (threadIdx.x == 0) {
    if (a.ctl) report_error(a.ctl, ERR_SYMM_TIMEOUT, (uint64_t)blockIdx.x);
    if (a.status) store_relaxed_system(a.status, 1u);
  }
}

// Workgroups per rank, G: aim for about 128 workgroups in all (W * G),
// between 2 and 8 vectors per thread, at most 64 per rank, and few enough
// that all W * G workgroups are resident together (occupancy per CU times
// the CU count, queried once per W). Every iteration passes two pad
// barriers over all W * G workgroups, whose release and acquire fences
// serialise per XCD, so fewer, fuller workgroups win until the per-thread
// work dominates. Measured on MI355X for W = 2, 4 and 8 and n from 8 Ki to
// 1 Mi elements, the rule is within a few percent of the best G at every
// point; at W = 8, n = 128 Ki it took 8.3 us per iteration where two
// vectors per thread (32 per rank) took 10.6 us. Swept again with the
// write-through stores (targets of 64, 128 and 256 workgroups in all, W =
// 2, 4, 8, n = 32 Ki to 512 Ki): 128 stays the best or within noise, the
// others winning single points by at most 0.4 us (at W = 8, n = 128 Ki:
// 7.38-7.46 us, against 9.6 for 64 and 8.3 for 256).
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

// ---- the symmetric exchange with no allocation -----------------------------

// For callers that cannot allocate (code under hipGraph capture, tight
// serving loops, harnesses that forbid allocation): the symmetric buffers
// and signal pads of the exchange live in this fixed array, which the
// library's code object holds on every GPU it is loaded on until the process
// ends. Layout: W symmetric buffers of kNoAllocMaxN bf16 (rank v's at
// v * kNoAllocMaxN elements), then the pads, rank r's u32 [kSymmMaxBlocks][W]
// at r * kSymmMaxBlocks * W words after the buffers.
constexpr size_t kNoAllocMaxN = ARX_NOALLOC_MAX_N;
constexpr size_t kSymmMaxBlocks = 64;
constexpr size_t kScratchBufBytes = (size_t)ARX_MAX_WORLD * kNoAllocMaxN * sizeof(uint16_t);
constexpr size_t kScratchPadWords = (size_t)ARX_MAX_WORLD * kSymmMaxBlocks * ARX_MAX_WORLD;
constexpr size_t kScratchBytes = kScratchBufBytes + kScratchPadWords * sizeof(uint32_t);
static_assert(kNoAllocMaxN % 128 == 0, "symmetric buffers start on 256-byte boundaries");

static __device__ __align__(256) uint32_t scratch[kScratchBytes / sizeof(uint32_t)];

// Zero-fills the pads of one exchange before it runs: a completed exchange
// leaves them zero, one that timed out may not.
__global__ __launch_bounds__(kBlock) void clear_words_kernel(uint32_t* p, uint32_t n) {
  for (uint32_t i = threadIdx.x; i < n; i += kBlock) p[i] = 0u;
}

namespace {

// Per device: the array's device address (hipGetSymbolAddress, taken with
// that device current), its CU count and its wall-clock rate.
struct ScratchDev {
  void* ptr = nullptr;
  int cus = 0;
  uint64_t khz = 0;
};
constexpr int kMaxDevices = 64;
ScratchDev g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_for_device(ScratchDev* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(ARX_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return set_error(ARX_EINVAL, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> g(g_scratch_mu);
  ScratchDev& d = g_scratch[dev];
  if (!d.ptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return set_error(ARX_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    int cus = 0, khz = 0;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess ||
        (e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev)) != hipSuccess)
      return set_error(ARX_EHIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
    d.cus = cus;
    d.khz = khz > 0 ? (uint64_t)khz : 100000u;
    d.ptr = p;
  }
  *out = d;
  return ARX_OK;
}

}  // namespace

}  // namespace arx

extern "C" int arx_symm_allreduce_noalloc(int world, const void* inputs, void* outputs, size_t n, size_t ld,
                                          int iters, uint32_t* status, hipStream_t stream) {
  using namespace arx;
  if (world < 2 || world > ARX_MAX_WORLD) return set_error(ARX_EINVAL, "world %d not in [2, %d]", world, ARX_MAX_WORLD);
  if (n > kNoAllocMaxN) return set_error(ARX_EINVAL, "n %zu exceeds ARX_NOALLOC_MAX_N %zu", n, kNoAllocMaxN);
  if (ld < n || (ld & 7u)) return set_error(ARX_EINVAL, "ld %zu must be >= n and a multiple of 8", ld);
  if (iters < 1 || iters > 65536) return set_error(ARX_EINVAL, "iters %d not in [1, 65536]", iters);
  if (n > 0 && (inputs == nullptr || outputs == nullptr)) return set_error(ARX_EINVAL, "null inputs or outputs");
  if (((uintptr_t)inputs & 15u) || ((uintptr_t)outputs & 15u) || ((uintptr_t)status & 3u))
    return set_error(ARX_EINVAL, "inputs and outputs must be 16-byte aligned, status 4-byte aligned");
  const size_t extent = (size_t)iters * world * ld * sizeof(uint16_t);
  const uintptr_t x = (uintptr_t)inputs, y = (uintptr_t)outputs;
  if (inputs != outputs && n > 0 && x < y + extent && y < x + extent)
    return set_error(ARX_EINVAL, "inputs and outputs overlap without being the same buffer");
  ScratchDev d;
  int rc = scratch_for_device(&d);
  if (rc != ARX_OK) return rc;
  SymmArgs a;
  a.inputs = (const uint16_t*)inputs;
  a.outputs = (uint16_t*)outputs;
  a.symm = (uint16_t*)d.ptr;
  a.stride = kNoAllocMaxN;
  a.ld = ld;
  a.n = (uint32_t)n;
  a.iters = iters;
  a.world = world;
  a.blocks = symm_blocks(a.n, world, d.cus);
  if (a.blocks < 1 || (size_t)a.blocks > kSymmMaxBlocks)
    return set_error(ARX_EHIP, "no workgroup count for the exchange (occupancy query failed?)");
  uint32_t* const pads = reinterpret_cast<uint32_t*>(static_cast<char*>(d.ptr) + kScratchBufBytes);
  for (int i = 0; i < 8; ++i) a.pad[i] = i < world ? pads + (size_t)i * kSymmMaxBlocks * world : nullptr;
  a.timeout = 2000000ull * d.khz / 1000u;   // 2 s
  a.ctl = nullptr;
  a.status = status;
  hipLaunchKernelGGL(clear_words_kernel, dim3(1), dim3(kBlock), 0, stream, pads,
                     (uint32_t)((size_t)world * kSymmMaxBlocks * world));
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = launch_symm_allreduce(a, stream);
  if (e != hipSuccess) return set_error(ARX_EHIP, "launching the exchange: %s", hipGetErrorString(e));
  return ARX_OK;
}
