// arx_reduce.hip — the reduction kernels of libarx for gfx950.
//
//   oneshot_kernel     one call of the one-shot path: copy into the send
//                      slot, arrival count and publish, flag wait in a
//                      poll workgroup, go broadcast, W-way reduction,
//                      last-block-out (page "arx.cu", arx_kernel)
//   reduce_kernel      the W-way reduction alone, streaming from HBM
//   round_test_kernel  the reduction's binary32 -> bf16 rounding alone
//
// Data layout in HBM: send slots [2][stride] bf16, recv slots [2][W][stride]
// bf16 (stride = max_n rounded up to 128 elements, so every slot starts on a
// 256-byte boundary); element i of a slot is at byte 2 * i. A thread moves
// 8 bf16 (16 bytes) per access: lanes of a wave touch 1 KiB of consecutive
// bytes per instruction.
#include <hip/hip_runtime.h>

#include "arx_prims.h"
#include "arx_internal.h"
#include "arx_kernel_util.h"

namespace arx {

// ---- one-shot kernel --------------------------------------------------------

// The grid is a poll workgroup and G = gridDim.x - 1 >= 1 reducing
// workgroups. The poll workgroup (blockIdx 0, dispatched first)
// only reads the peers' flags and releases go (page "arx.cu", arx_kernel:
// flag polling is confined to one block, and go reaches the rest through a
// device word); it neither copies nor reduces, so its reads over PCIe hold
// up no copy, and a peer that is already ahead is seen about one PCIe read
// after the kernel starts. Reducing workgroup r = blockIdx.x - 1 copies (if
// r < ncopy), counts arrival, waits for go and sums its share of vectors.
//
// The last of the arrivals (the copying workgroups' and the poll
// workgroup's) publishes seq to the host proxy with a release store, tells
// the poll workgroup so in the published word, and resets the arrival
// counter (the next call's kernel starts after this one ends).
__device__ __forceinline__ void publish_seq(const OneShotArgs& a, uint64_t seq, uint32_t* cnt0, uint64_t* published) {
  fence_acquire_system();
  store_release_system(&a.ctl->seq, seq);
  store_relaxed_agent(published, seq);
  store_relaxed_agent(cnt0, 0u);
}

// ONE_PASS: the G reducing workgroups have a thread for every 16-byte
// vector. When every one of them copies (ncopy == G), each thread keeps
// its own partial's vector in registers from the copy to the sum. Every
// reducing workgroup reads its own partial from `in` (the send slot is what
// the peers receive, and its copy is complete before the publish). ncopy <
// G only when `in` and `out` do not overlap.
template <int W, bool ONE_PASS, int BLOCK>
__global__ __launch_bounds__(BLOCK) void oneshot_kernel(OneShotArgs a) {
  static_assert(BLOCK >= 128, "the poll workgroup uses two waves");
  __shared__ uint32_t s_abort;
  __shared__ uint32_t s_arrived;
  uint64_t* const seq_dev = reinterpret_cast<uint64_t*>(a.words + WORD_SEQ);
  uint64_t* const published = reinterpret_cast<uint64_t*>(a.words + WORD_PUBLISHED);
  uint32_t* const cnt0 = a.words + WORD_CNT0;
  uint32_t* const cnt1 = a.words + WORD_CNT1;

  // ---- the poll workgroup: two waves
  if (blockIdx.x == 0) {
    if (threadIdx.x == 0) s_arrived = 0u;
    __syncthreads();
    // The second wave keeps this call's size for the proxy in
    // ctl.bytes[par] and counts one arrival, so the last arriver's release
    // before the publish waits for no store to pinned memory (a PCIe write
    // is acknowledged about 0.56 us after it is issued). The size shadow
    // holds both slots as last stored: when the slot already holds this
    // size (the same n as two calls ago) nothing is stored, and the
    // arrival, carrying nothing, is relaxed and comes well before the
    // copiers'; otherwise the wave stores the size and its arrival's
    // release carries it. It runs beside the first wave's flag wait; the
    // first wave counts the workgroup finished only after it has arrived
    // (below).
    if (threadIdx.x == 64) {
      uint64_t* const shadow = reinterpret_cast<uint64_t*>(a.words + WORD_BYTES_SHADOW);
      const uint64_t b0 = load_relaxed_agent(shadow), b1 = load_relaxed_agent(shadow + 1);
      const uint64_t s1 = load_relaxed_agent(seq_dev) + 1u;
      const uint32_t p1 = (uint32_t)s1 & 1u;
      const uint64_t nb = (uint64_t)a.n * 2u;
      uint32_t old;
      if ((p1 ? b1 : b0) == nb) {
        old = fetch_add_relaxed_system(cnt0, 1u);
      } else {
        store_relaxed_system(&a.ctl->bytes[p1], nb);
        store_relaxed_agent(shadow + p1, nb);
        old = fetch_add_release_system(cnt0, 1u);
      }
      if (old == a.ncopy) publish_seq(a, s1, cnt0, published);
      __hip_atomic_store(&s_arrived, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if (threadIdx.x >= 64) return;
    const uint32_t lane = threadIdx.x;
    const bool peer = (int)lane < W && (int)lane != a.rank;
    // The lane of each peer rank reads that peer's pinned flag once, at
    // once (in flight with the seq load). If the peer is not yet at seq,
    // the lane waits until the published word says this rank has published
    // seq, and only then reads the flag again until it reaches seq: flag
    // reads in flight around the GPU's store of seq to pinned memory, which
    // the proxy (and every peer) waits for, delay that store on some hosts.
    // The published word is a hint only: what lets the wave on is the flag.
    // Without early_go the wave also waits for the published word when the
    // flag was already there, so go never precedes the publish.
    uint64_t f = 0;
    if (peer) f = load_relaxed_system(a.flags + lane);
    const uint64_t seq = load_relaxed_agent(seq_dev) + 1u;
    bool ok = true;
    if (peer && (f < seq || !a.early_go)) {
      const uint64_t t0 = now_ticks();
      while (load_relaxed_agent(published) < seq && now_ticks() - t0 <= a.timeout) __builtin_amdgcn_s_sleep(1);
      while (f < seq && load_relaxed_system(a.flags + lane) < seq) {
        if (now_ticks() - t0 > a.timeout) {
          ok = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    // One fence acquires what the flags publish and releases it further;
    // the first 8 lanes then store the go value into 8 replicas of the go
    // word, one 256-byte line each. Reducing workgroup b polls replica
    // b % 8, so the workgroups of each XCD (dealt round robin) share a line.
    const bool bad = __any(!ok);
    fence_acq_rel_system();
    if (lane < kGoReplicas) store_relaxed_agent(go_word(a.words, lane), (seq << 1) | (bad ? 1u : 0u));
    if (lane == 0) {
      if (bad) report_error(a.ctl, ERR_FLAG_TIMEOUT, seq);
      // The finish count, after the flag wait (see below) and after the
      // second wave's arrival: with a peer ahead, go and every other count
      // can come before that wave has even read the seq, and a call
      // recorded finished would let it read the next seq, arrive for that
      // call and publish it before its copies. The wave has no wait of its
      // own, so this one ends; the bound is only a guard.
      const uint64_t t1 = now_ticks();
      while (__hip_atomic_load(&s_arrived, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0u &&
             now_ticks() - t1 <= a.timeout)
        __builtin_amdgcn_s_sleep(1);
      // the last workgroup to count records the call as finished
      if (fetch_add_relaxed_agent(cnt1, 1u) == gridDim.x - 1u) {
        store_relaxed_agent(cnt1, 0u);
        store_relaxed_agent(seq_dev, seq);
        store_relaxed_system(&a.ctl->done, seq);
      }
    }
    return;
  }

  // ---- the reducing workgroups
  const uint32_t nred = gridDim.x - 1u;
  const uint32_t r = blockIdx.x - 1u;
  const uint32_t nv = a.n >> 3, tail = a.n & 7u;
  const uint32_t tid = r * BLOCK + threadIdx.x;
  const uint32_t nthr = nred * BLOCK;
  const bool copier = r < a.ncopy;
  const bool keep_own = ONE_PASS && a.ncopy == nred;

  // This rank's vector is loaded before the seq: only where it is stored
  // depends on the parity, so the two loads are in flight together.
  u32x4 own = {0u, 0u, 0u, 0u};
  if (keep_own && tid < nv) own = ld16(a.in + 8u * (size_t)tid);

  // seq and parity: one more than the last completed call. seq is 64-bit
  // like the host's flags. The go word holds 2 * seq, plus 1 when the call
  // is aborted, so one load tells a workgroup both that it may go on and
  // whether to sum; it is never zero for a call (seq >= 1), the value the
  // word starts at.
  const uint64_t seq = load_relaxed_agent(seq_dev) + 1u;
  const uint32_t par = (uint32_t)seq & 1u;
  uint16_t* const mine = a.send + (size_t)par * a.stride;

  // 1. the first ncopy reducing workgroups copy this rank's partial into
  //    send[par], each thread a stride of ncopy * BLOCK vectors. The
  //    stores write through the L2 (device scope), so the release before
  //    the arrival has none of them left dirty to write back: at W=8 on
  //    MI355X, 6.45-6.49 -> 6.30-6.33 us per call at n = 128 Ki, 9.6 ->
  //    9.3 us at 1 Mi, 22.7 -> 20.8 us at 4 Mi and 76.4 -> 75.5 us at 16 Mi
  //    (lockstep). Once the peers' partials outgrow the last-level cache
  //    (nt_copy, set by oneshot_shape) they are nontemporal instead; the
  //    grid then always loops, so only the loop has the choice.
  if (copier) {
    const __amdgpu_buffer_rsrc_t rmine = make_rsrc(mine, slot_bytes(a.stride));
    if (keep_own) {
      if (tid < nv) bstore16<CP_DEV>(rmine, tid * 16u, own);
    } else {
      const uint32_t cthr = a.ncopy * BLOCK;
      if (a.nt_copy)
        for (uint32_t v = tid; v < nv; v += cthr) bstore16<CP_NT>(rmine, v * 16u, ld16(a.in + 8u * (size_t)v));
      else
        for (uint32_t v = tid; v < nv; v += cthr) bstore16<CP_DEV>(rmine, v * 16u, ld16(a.in + 8u * (size_t)v));
    }
    if (tid < tail) mine[8u * (size_t)nv + tid] = a.in[8u * (size_t)nv + tid];
  }
  __syncthreads();

  // 2. arrival count: one system-scope release per copying workgroup
  //    carries all its waves' copies (they precede it through the workgroup
  //    barrier); with the poll workgroup's arrival there are ncopy + 1, and
  //    the last of them acquires them all and publishes (publish_seq)
  if (copier && threadIdx.x == 0) {
    if (fetch_add_release_system(cnt0, 1u) == a.ncopy) publish_seq(a, seq, cnt0, published);
  }

  // The finish count. It has to follow every workgroup's read of seq_dev
  // (the last workgroup to count advances it) and, so that the recorded
  // finished seq means the peers' flags were seen, the flag wait; nothing
  // else. So the reducing workgroups count themselves finished here, where
  // their atomic overlaps the flag round trip, and the poll workgroup right
  // after its flag wait; the last to count is then nearly always the poll
  // workgroup, uncontended. (On the page every block counts after its
  // reduction; moving the count took 0.8-1.0 us off a 256 KiB call on
  // MI355X.)
  uint32_t finished = 0;
  if (threadIdx.x == 0) finished = fetch_add_relaxed_agent(cnt1, 1u);

  // 3. wait for go from the poll workgroup, then an agent-scope acquire
  if (threadIdx.x == 0) {
    const uint64_t* const go = go_word(a.words, blockIdx.x % kGoReplicas);
    const uint64_t t0 = now_ticks();
    bool timed = false;
    uint64_t g;
    while (((g = load_relaxed_agent(go)) >> 1) < seq) {
      if (now_ticks() - t0 > 2u * a.timeout) {
        timed = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    fence_acquire_agent();
    if (timed) report_error(a.ctl, ERR_GO_TIMEOUT, seq);
    s_abort = (timed || (g & 1u) != 0u) ? 1u : 0u;
  }
  __syncthreads();
  const bool abort = s_abort != 0u;

  // 4. rank-ordered W-way sum; peer slots are read with system-coherent
  //    loads, since another agent wrote them
  if (!abort) {
    __amdgpu_buffer_rsrc_t rs[W];
#pragma unroll
    for (int src = 0; src < W; ++src)
      rs[src] = make_rsrc(a.recv + ((size_t)par * W + src) * a.stride, slot_bytes(a.stride));
    if (ONE_PASS) {
      if (tid < nv) {
        u32x4 x[W];
        if (!keep_own) own = ld16(a.in + 8u * (size_t)tid);
#pragma unroll
        for (int src = 0; src < W; ++src)
          x[src] = (src == a.rank) ? own : bload16<CP_SYS>(rs[src], tid * 16u);
        st16(a.out + 8u * (size_t)tid, sum_bf16x8<W>(x));
      }
    } else {
      // Past the last-level cache (nt_peer, set by oneshot_shape) the peer
      // loads stream nontemporally; after the acquire fence above they see
      // the peers' data as the system-coherent ones do.
      if (a.nt_peer) {
        for (uint32_t v = tid; v < nv; v += nthr) {
          u32x4 x[W];
#pragma unroll
          for (int src = 0; src < W; ++src)
            x[src] = (src == a.rank) ? ld16(a.in + 8u * (size_t)v) : bload16<CP_NT>(rs[src], v * 16u);
          st16(a.out + 8u * (size_t)v, sum_bf16x8<W>(x));
        }
      } else {
        for (uint32_t v = tid; v < nv; v += nthr) {
          u32x4 x[W];
#pragma unroll
          for (int src = 0; src < W; ++src)
            x[src] = (src == a.rank) ? ld16(a.in + 8u * (size_t)v) : bload16<CP_SYS>(rs[src], v * 16u);
          st16(a.out + 8u * (size_t)v, sum_bf16x8<W>(x));
        }
      }
    }
    if (tid < tail) {
      const uint32_t i = 8u * nv + tid;
      uint16_t x[W];
#pragma unroll
      for (int src = 0; src < W; ++src) x[src] = (src == a.rank) ? a.in[i] : bload2<CP_SYS>(rs[src], i * 2u);
      a.out[i] = sum_bf16x1<W>(x);
    }
  }

  // 5. last block out: the last workgroup to count itself finished resets
  //    the finish counter and records the completed seq. Relaxed: the only reader of the counter
  //    and of seq_dev is the next kernel on the stream, which the kernel
  //    boundary orders after this one; ctl.done is progress information for
  //    the host's watchdog.
  if (threadIdx.x == 0) {
    if (finished == gridDim.x - 1u) {
      store_relaxed_agent(cnt1, 0u);
      store_relaxed_agent(seq_dev, seq);
      store_relaxed_system(&a.ctl->done, seq);
    }
  }
}

// Workgroups that copy and count arrival: half the grid once it reaches 64
// workgroups, else all of it. Each copying workgroup pays a system-scope
// release fence (they serialise per XCD) and one atomic on the shared
// arrival counter before the publish; halving them shortened the call on
// MI355X at W=8 by 4 % at n = 128 Ki, 8 % at 1 Mi and 11 % at 4 Mi, while
// below 64 workgroups the longer copy costs more than the arrivals save.
unsigned oneshot_copiers(unsigned grid) { return grid >= 64u ? grid / 2u : grid; }

unsigned oneshot_grid(uint32_t n, int block, unsigned max_grid) {
  const uint32_t nv = n >> 3;
  uint32_t g = (nv + block - 1) / block;
  if (g < 1) g = 1;
  if (g > max_grid) g = max_grid;
  return g;
}

// Workgroups of oneshot_kernel<W, ONE_PASS, BLOCK> that fit on the device at
// once: its occupancy per CU times the CU count, at most kMaxOneShotGrid + 1
// (the reducing workgroups and the poll workgroup); 0 if the occupancy query
// fails. The occupancy is queried once per variant.
template <int W, bool ONE_PASS, int BLOCK>
static unsigned coresident(int cus) {
  static const int per_cu = [] {
    int o = 0;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
               &o, reinterpret_cast<const void*>(oneshot_kernel<W, ONE_PASS, BLOCK>), BLOCK, 0) == hipSuccess
               ? o
               : 0;
  }();
  const long long cap = (long long)per_cu * cus;
  return (unsigned)(cap < kMaxOneShotGrid + 1 ? cap : kMaxOneShotGrid + 1);
}

OneShotShape oneshot_shape(uint32_t n, int W, int block, unsigned resident, bool disjoint) {
  OneShotShape sh{};
  if (resident < 2) return sh;  // no room for the poll workgroup: grid 0
  // the reducing workgroups, in resident - 1 beside the poll workgroup
  sh.grid = oneshot_grid(n, block, resident - 1);
  sh.launched = sh.grid + 1;
  sh.one_pass = (n >> 3) <= sh.grid * (uint32_t)block;
  // With out == in, every reducing workgroup copies: each thread then
  // copies a vector before it reduces (and overwrites) it. Were other
  // workgroups copying, go could come before their copy (go follows the
  // peers' flags, which a peer running ahead posts before this rank
  // publishes) and the send slot would get the output instead of the input.
  sh.ncopy = disjoint ? oneshot_copiers(sh.grid) : sh.grid;
  // Go before the publish (a peer ahead) lets the workgroups that do not
  // copy reduce while the copiers copy; past 4 vectors copied per copying
  // thread the copiers then finish alone, and the call gets slower than
  // with go after the publish (W=8, run-ahead peers, n = 16 Mi: 84.6 against
  // 75.9 us; at n = 4 Mi, 2 vectors per reducing thread, early go is 1.8 us
  // faster). So early go is allowed up to 4 vectors per copying thread.
  sh.early_go = ((n >> 3) + sh.ncopy * block - 1) / (sh.ncopy * block) <= 4u;
  // Cache policies once the peers' partials outgrow the 256 MiB last-level
  // cache: both parities' peer slots take 4 n (W - 1) bytes. From 224 MiB
  // (n (W - 1) >= 56 Mi) the copy's stores are nontemporal, from 384 MiB
  // (96 Mi) the sum's peer loads too. Below, the peer data the benchmark
  // re-reads every other call stays cached and the cached forms win.
  // Measured on MI355X, lockstep, one box, write-through copy against
  // nontemporal: W=8 36.7 -> 34.9 us at 8 Mi, 157 -> 153 at 32 Mi; W=4
  // 83.5 -> 80.7 at 32 Mi but 43.0 -> 43.4 at 16 Mi and 23.4 -> 25.3 at
  // 8 Mi; W=2 31.5 -> 33.8 at 16 Mi. Nontemporal peer loads on top: W=8
  // 73.8 -> 69.5 at 16 Mi and 152.8 -> 127.5 at 32 Mi, but 34.9 -> 36.9 at
  // 8 Mi; W=4 80.7 -> 76.7 at 32 Mi, 43.4 -> 44.5 at 16 Mi; W=2 57.3 ->
  // 58.8 at 32 Mi.
  const uint64_t peer = (uint64_t)n * (uint64_t)(W - 1);
  sh.nt_copy = peer >= (56ull << 20);
  sh.nt_peer = peer >= (96ull << 20);
  return sh;
}

template <int W, int BLOCK>
static hipError_t launch_oneshot_wb(const OneShotArgs& a, int cus, hipStream_t s) {
  // every workgroup waits on the others, so all must be resident together
  const unsigned cap = coresident<W, false, BLOCK>(cus);
  const unsigned cap1 = coresident<W, true, BLOCK>(cus);
  const unsigned resident = cap < cap1 ? cap : cap1;
  if (resident < 2) return hipErrorInvalidConfiguration;
  const uint64_t ib = (uint64_t)(uintptr_t)a.in, ob = (uint64_t)(uintptr_t)a.out, nb = 2ull * a.n;
  const OneShotShape sh = oneshot_shape(a.n, W, BLOCK, resident, ib + nb <= ob || ob + nb <= ib);
  OneShotArgs b = a;
  b.ncopy = sh.ncopy;
  b.early_go = sh.early_go ? 1u : 0u;
  b.nt_copy = sh.nt_copy ? 1u : 0u;
  b.nt_peer = sh.nt_peer ? 1u : 0u;
  if (sh.one_pass)
    hipLaunchKernelGGL((oneshot_kernel<W, true, BLOCK>), dim3(sh.launched), dim3(BLOCK), 0, s, b);
  else
    hipLaunchKernelGGL((oneshot_kernel<W, false, BLOCK>), dim3(sh.launched), dim3(BLOCK), 0, s, b);
  return hipGetLastError();
}

// Threads per one-shot workgroup: 256 while that keeps the reducing grid
// within 32 workgroups, 512 while within 64 (where half of them copy) for
// W >= 5 and within 48 for W <= 4, else 1024. Fewer workgroups mean fewer
// arrivals, go pollers and last-block-out atomics, more threads per
// workgroup a longer copy and reduction per workgroup, and that reduction
// is shorter the fewer partials it sums. Measured on MI355X, same box,
// lockstep and with peers ahead:
//  - W=8, n from 16 Ki to 768 Ki elements: at n = 128 Ki, 512 threads
//    (32 workgroups) take 8.36-8.39 us per call, 256 threads (64, 32
//    copying) 8.63-8.67 us and 1024 threads 9.04-9.07 us;
//  - below 16 Ki elements 256 threads win too: at n = 8 Ki, W=8, four
//    workgroups of 256 take 5.76-5.78 us (lockstep) and 4.22-4.24 us (peers
//    ahead), two of 512 5.90-6.01 and 4.32-4.35, one of 1024 6.37-6.40 and
//    4.83;
//  - W from 2 to 7, n from 144 Ki to 256 Ki: past 48 workgroups of 512,
//    32 of 1024 are 0.1-0.25 us faster at W <= 4 (W=2, n = 256 Ki:
//    6.50-6.57 against 6.77-6.80 us lockstep, 4.77 against 4.94-4.95 with
//    peers ahead) and slower or a tie at W >= 5 (W=7: 7.17-7.19 against
//    7.11-7.12 and 5.53-5.54 against 5.27-5.28).
int oneshot_block(uint32_t n, int W) {
  const uint32_t nv = n >> 3;
  if (nv <= 256u * 32u) return 256;
  if (nv <= 512u * (W <= 4 ? 48u : 64u)) return 512;
  return 1024;
}

template <int W>
static hipError_t launch_oneshot_w(const OneShotArgs& a, int block, int cus, hipStream_t s) {
  if (block == 0) block = oneshot_block(a.n, W);
  switch (block) {
    case 256: return launch_oneshot_wb<W, 256>(a, cus, s);
    case 512: return launch_oneshot_wb<W, 512>(a, cus, s);
    case 1024: return launch_oneshot_wb<W, 1024>(a, cus, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_oneshot(const OneShotArgs& a, int W, int block, int cus, hipStream_t s) {
  switch (W) {
    case 2: return launch_oneshot_w<2>(a, block, cus, s);
    case 3: return launch_oneshot_w<3>(a, block, cus, s);
    case 4: return launch_oneshot_w<4>(a, block, cus, s);
    case 5: return launch_oneshot_w<5>(a, block, cus, s);
    case 6: return launch_oneshot_w<6>(a, block, cus, s);
    case 7: return launch_oneshot_w<7>(a, block, cus, s);
    case 8: return launch_oneshot_w<8>(a, block, cus, s);
    default: return hipErrorInvalidValue;
  }
}

// ---- reduction alone, streaming from HBM -------------------------------------

// Workgroup b covers vectors [b * kBlock * U, (b + 1) * kBlock * U); thread t
// handles vectors base + u * kBlock, u < U, issuing all U * W loads before
// the first add. Inputs were written before the launch, so the loads are
// nontemporal (stream through, keep nothing). The stores write through the
// L2 at device scope rather than staying dirty there; for this 8:1
// read/write mix that measured 1.2 % faster than plain stores, while
// nontemporal stores were 5 % slower.
template <int W, int U>
__global__ __launch_bounds__(kBlock) void reduce_kernel(ReduceArgs a) {
  const uint32_t nv = a.n >> 3, tail = a.n & 7u;
  const uint32_t base = blockIdx.x * (uint32_t)(kBlock * U) + threadIdx.x;
  __amdgpu_buffer_rsrc_t rs[W];
#pragma unroll
  for (int src = 0; src < W; ++src)
    rs[src] = (src == a.rank) ? make_rsrc(a.in, a.n * 2u)
                              : make_rsrc(a.recv_par + (size_t)src * a.stride, slot_bytes(a.stride));
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.out, a.n * 2u);
  u32x4 x[U][W];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t v = base + u * kBlock;
#pragma unroll
    for (int src = 0; src < W; ++src) x[u][src] = bload16<CP_NT>(rs[src], v * 16u);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t v = base + u * kBlock;
    if (v < nv) bstore16<CP_DEV>(ro, v * 16u, sum_bf16x8<W>(x[u]));
  }
  if (blockIdx.x == 0 && threadIdx.x < tail) {
    const uint32_t i = 8u * nv + threadIdx.x;
    uint16_t y[W];
#pragma unroll
    for (int src = 0; src < W; ++src) y[src] = bload2<CP_NT>(rs[src], i * 2u);
    a.out[i] = sum_bf16x1<W>(y);
  }
}

constexpr int kReduceU = 2;

template <int W>
static hipError_t launch_reduce_w(const ReduceArgs& a, hipStream_t s) {
  const uint32_t nv = a.n >> 3;
  uint32_t grid = (nv + kBlock * kReduceU - 1) / (kBlock * kReduceU);
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((reduce_kernel<W, kReduceU>), dim3(grid), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_reduce(const ReduceArgs& a, int W, hipStream_t s) {
  switch (W) {
    case 2: return launch_reduce_w<2>(a, s);
    case 3: return launch_reduce_w<3>(a, s);
    case 4: return launch_reduce_w<4>(a, s);
    case 5: return launch_reduce_w<5>(a, s);
    case 6: return launch_reduce_w<6>(a, s);
    case 7: return launch_reduce_w<7>(a, s);
    case 8: return launch_reduce_w<8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// ---- the rounding alone ------------------------------------------------------

__global__ __launch_bounds__(kBlock) void round_test_kernel(const uint32_t* in, uint16_t* out, size_t n) {
  const size_t stride = (size_t)gridDim.x * kBlock;
  for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride)
    out[i] = (uint16_t)(round_bf16_hi(__uint_as_float(in[i])) >> 16);
}

hipError_t launch_round_test(const uint32_t* in, uint16_t* out, size_t n, hipStream_t s) {
  size_t grid = (n + kBlock - 1) / kBlock;
  if (grid > 8192) grid = 8192;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(round_test_kernel, dim3((unsigned)grid), dim3(kBlock), 0, s, in, out, n);
  return hipGetLastError();
}

}  // namespace arx
