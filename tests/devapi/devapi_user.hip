// devapi_user.hip — a caller's kernel built against include/arx_device.h
// alone (nothing else of libarx), used by the GPU tests to check that the
// public device-side blockwise barrier synchronises workgroups and publishes
// their writes (page "triton_barrier.py": blockwise_barrier and its usage
// pattern 1, exercised as the page's barrier test does, with many blocks on
// every rank).
//
// The kernel plays W ranks on one GPU: workgroup g is rank g % W's block
// g / W, so the W workgroups of one block id are consecutive and land on
// different XCDs. Each round, thread 0 writes the block's tag
// 0x80000000 | round << 16 | block << 4 | rank into its rank's tag row, the
// workgroup passes __syncthreads, barrier_blockwise, __syncthreads, and then
// thread p < W reads rank p's tag for the same block and round into seen.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "arx_device.h"

namespace {

struct UserArgs {
  arx_pad_t pad;     // rank field unused: each workgroup sets its own
  uint32_t* tags;    // [W][rounds][nblocks]
  uint32_t* seen;    // [W][rounds][nblocks][W]
  uint32_t* status;  // device u32: 1 once any wait timed out
  int nblocks;
  int rounds;
};

__global__ __launch_bounds__(64) void user_barrier_kernel(UserArgs a) {
  const int W = a.pad.W;
  arx_pad_t pad = a.pad;
  pad.rank = (int)(blockIdx.x % (uint32_t)W);
  const uint32_t b = blockIdx.x / (uint32_t)W;
  const size_t nb = (size_t)a.nblocks;
  for (int r = 0; r < a.rounds; ++r) {
    if (threadIdx.x == 0)
      a.tags[((size_t)pad.rank * a.rounds + r) * nb + b] =
          0x80000000u | ((uint32_t)r << 16) | (b << 4) | (uint32_t)pad.rank;
    __syncthreads();
    const bool ok = barrier_blockwise(pad, b);
    if (__syncthreads_or(!ok)) {
      if (threadIdx.x == 0) __hip_atomic_store(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    if ((int)threadIdx.x < W)
      a.seen[(((size_t)pad.rank * a.rounds + r) * nb + b) * W + threadIdx.x] =
          a.tags[((size_t)threadIdx.x * a.rounds + r) * nb + b];
  }
}

}  // namespace

extern "C" {

// Launches W * nblocks workgroups on `stream`. pads: host array of W device
// pointers, rank r's pad u32 [nblocks][W] (zero-filled by the caller).
// Returns 0, -1 for a bad argument (including a grid the device cannot hold
// at once), -4 for a HIP error.
int devapi_barrier(uint32_t* const* pads, int W, int nblocks, int sem, int rounds, uint32_t* tags, uint32_t* seen,
                   uint32_t* status, uint64_t timeout, hipStream_t stream) {
  if (W < 2 || W > 8 || nblocks < 1 || rounds < 1 || !pads || !tags || !seen || !status) return -1;
  if (sem != ARX_SEM_RELAXED && sem != ARX_SEM_ACQ_REL) return -1;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(user_barrier_kernel), 64,
                                                   0) != hipSuccess)
    return -4;
  if ((long long)W * nblocks > (long long)per_cu * cus) return -1;
  UserArgs a{};
  for (int r = 0; r < 8; ++r) a.pad.ptr[r] = r < W ? pads[r] : nullptr;
  for (int r = 0; r < W; ++r)
    if (!pads[r]) return -1;
  a.pad.W = W;
  a.pad.sem = sem;
  a.pad.timeout = timeout;
  a.tags = tags;
  a.seen = seen;
  a.status = status;
  a.nblocks = nblocks;
  a.rounds = rounds;
  hipLaunchKernelGGL(user_barrier_kernel, dim3(W * nblocks), dim3(64), 0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
