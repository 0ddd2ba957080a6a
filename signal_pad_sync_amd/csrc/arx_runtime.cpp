// arx_runtime.cpp — host side of libarx: state, the proxy thread that posts
// the virtual peers' flags, argument checks and the C ABI declared in arx.h
// and arx_test.h.
//
// Page "arx.cu": arx_prepare / arx_connect allocate and zero the pinned and
// device state and start the proxy; arx_allreduce checks its arguments and
// launches the kernel on the caller's stream; proxy_loop watches the
// published seq, posts the seqs one after another and reports stalls.
#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <exception>
#include <mutex>
#include <memory>
#include <thread>

#include "arx.h"
#include "arx_test.h"
#include "arx_internal.h"
#include "arx_sync.h"
#include "arx_proxy.h"

namespace {

using arx::Ctl;

static_assert(ARX_PROXY_LOCKSTEP == arx::PROXY_LOCKSTEP && ARX_PROXY_RUNAHEAD == arx::PROXY_RUNAHEAD &&
                  ARX_PROXY_MANUAL == arx::PROXY_MANUAL && ARX_PROXY_STRESS == arx::PROXY_STRESS,
              "proxy mode numbering");

struct State {
  bool inited = false;
  int world = 0, rank = 0, device = 0, cus = 0;
  size_t max_n = 0, stride = 0;
  uint16_t* send = nullptr;   // device [2][stride]
  uint16_t* recv = nullptr;   // device [2][W][stride]
  uint32_t* pads = nullptr;   // device [W][ARX_MAX_PAD_BLOCKS][W]
  arx::Semaphore* sems = nullptr;  // device [W][ARX_MAX_PAD_BLOCKS]
  uint32_t* epochs = nullptr;      // device [W][ARX_MAX_PAD_BLOCKS]
  uint16_t* symm = nullptr;        // device [W][stride]: the virtual ranks' symmetric buffers
  uint32_t* words = nullptr;  // device [WORDS_TOTAL]
  Ctl* ctl = nullptr;         // pinned, host address
  uint64_t* flags = nullptr;  // pinned, host address [8]
  Ctl* ctl_dev = nullptr;     // the same memory, device address
  uint64_t* flags_dev = nullptr;
  uint64_t clock_khz = 100000;
  uint64_t timeout_us = 2000000;
  std::unique_ptr<arx::Proxy> core;  // flag posting and the stall watchdog
  std::thread proxy;
  std::atomic<bool> proxy_err{false};
  std::atomic<bool> inject_copy_failure{false};  // test aid: the next stress copy fails
  std::atomic<bool> stop{false};
  const uint16_t* stress_pool = nullptr;  // device [sets][W][max_n], caller-owned
  int stress_sets = 0;
  hipStream_t stress_stream = nullptr;    // the proxy's own copy stream

  // A process that never called arx_finalize still must not end with a
  // joinable thread (that aborts): stop and join the proxy, CPU-side only.
  ~State() {
    if (proxy.joinable()) {
      stop.store(true);
      proxy.join();
    }
  }
};

State S;
char g_detail[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof g_detail, fmt, ap);
  va_end(ap);
  return code;
}

#define HIPCHK(call)                                                                    \
  do {                                                                                  \
    hipError_t e_ = (call);                                                             \
    if (e_ != hipSuccess) return fail(ARX_EHIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

inline uint64_t load_acquire(const uint64_t* p) { return __atomic_load_n(p, __ATOMIC_ACQUIRE); }
inline void store_release(uint64_t* p, uint64_t v) { __atomic_store_n(p, v, __ATOMIC_RELEASE); }

// Proxy thread (page "arx.cu", proxy_loop): arx::Proxy posts seqs one by one,
// none skipped, up to the target the mode allows, and runs the stall
// watchdog.
void proxy_main() {
  if (!S.core->run(S.stop)) {
    fprintf(stderr, "arx rank %d: proxy failed to post seq %llu\n", S.rank,
            (unsigned long long)(S.core->posted() + 1));
    S.proxy_err.store(true);
  }
}

int check_ready() {
  if (!S.inited) return fail(ARX_ESTATE, "arx is not initialised");
  if (S.proxy_err.load()) return fail(ARX_EPROXY, "arx proxy thread failed earlier");
  const uint64_t err = load_acquire(&S.ctl->err);
  if (err != arx::ERR_NONE)
    return fail(ARX_ETIMEOUT, "a device wait timed out earlier (kind %llu, seq %llu); finalize and init again",
                (unsigned long long)err, (unsigned long long)load_acquire(&S.ctl->err_seq));
  return ARX_OK;
}

uint64_t timeout_ticks() { return S.timeout_us * S.clock_khz / 1000u; }

// The peers' data for seq s, written before its flag (ARX_PROXY_STRESS).
bool stress_copy(uint64_t s) {
  if (S.inject_copy_failure.exchange(false)) return false;
  if (!S.stress_pool || !S.stress_stream) return false;
  const int par = (int)(s & 1);
  const uint16_t* set = S.stress_pool + (size_t)(s % (uint64_t)S.stress_sets) * S.world * S.max_n;
  // As the page's proxy sends: the size the GPU published with seq s
  // (ctl.bytes[s & 1], stored before the release of ctl.seq), not the slot.
  const uint64_t bytes = load_acquire(&S.ctl->bytes[par]);
  const size_t nb = bytes < S.max_n * sizeof(uint16_t) ? (size_t)bytes : S.max_n * sizeof(uint16_t);
  for (int src = 0; src < S.world && nb > 0; ++src) {
    if (src == S.rank) continue;
    if (hipMemcpyAsync(S.recv + ((size_t)par * S.world + src) * S.stride, set + (size_t)src * S.max_n, nb,
                       hipMemcpyDeviceToDevice, S.stress_stream) != hipSuccess)
      return false;
  }
  return hipStreamSynchronize(S.stress_stream) == hipSuccess;
}

void free_all() {
  if (S.send) (void)hipFree(S.send);
  if (S.recv) (void)hipFree(S.recv);
  if (S.pads) (void)hipFree(S.pads);
  if (S.sems) (void)hipFree(S.sems);
  if (S.epochs) (void)hipFree(S.epochs);
  if (S.symm) (void)hipFree(S.symm);
  S.symm = nullptr;
  S.sems = nullptr;
  S.epochs = nullptr;
  if (S.words) (void)hipFree(S.words);
  if (S.stress_stream) (void)hipStreamDestroy(S.stress_stream);
  S.stress_stream = nullptr;
  S.stress_pool = nullptr;
  S.stress_sets = 0;
  if (S.ctl) (void)hipHostFree(S.ctl);
  if (S.flags) (void)hipHostFree(S.flags);
  S.send = S.recv = nullptr;
  S.pads = S.words = nullptr;
  S.ctl = S.ctl_dev = nullptr;
  S.flags = S.flags_dev = nullptr;
}

int init_impl(int world, size_t max_n, int rank) {
  if (S.inited) return fail(ARX_ESTATE, "arx is already initialised in this process");
  if (world < 2 || world > ARX_MAX_WORLD) return fail(ARX_EINVAL, "world %d not in [2, %d]", world, ARX_MAX_WORLD);
  if (rank < 0 || rank >= world) return fail(ARX_EINVAL, "rank %d not in [0, %d)", rank, world);
  if (max_n < 1 || max_n > ARX_MAX_N)
    return fail(ARX_EINVAL, "max_n %zu not in [1, %zu]", max_n, (size_t)ARX_MAX_N);
  S.world = world;
  S.rank = rank;
  S.max_n = max_n;
  S.stride = (max_n + 127) & ~(size_t)127;
  HIPCHK(hipGetDevice(&S.device));
  int khz = 0;
  HIPCHK(hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, S.device));
  S.clock_khz = khz > 0 ? (uint64_t)khz : 100000;
  HIPCHK(hipDeviceGetAttribute(&S.cus, hipDeviceAttributeMultiprocessorCount, S.device));

  const size_t send_b = 2 * S.stride * sizeof(uint16_t);
  const size_t recv_b = 2 * (size_t)world * S.stride * sizeof(uint16_t);
  const size_t pads_b = (size_t)world * ARX_MAX_PAD_BLOCKS * world * sizeof(uint32_t);
  const size_t words_b = arx::WORDS_TOTAL * sizeof(uint32_t);
  const size_t sems_b = (size_t)world * ARX_MAX_PAD_BLOCKS * sizeof(arx::Semaphore);
  const size_t epochs_b = (size_t)world * ARX_MAX_PAD_BLOCKS * sizeof(uint32_t);
  const size_t symm_b = (size_t)world * S.stride * sizeof(uint16_t);
  int rc = ARX_OK;
  hipError_t e;
  if ((e = hipMalloc(&S.send, send_b)) != hipSuccess || (e = hipMalloc(&S.recv, recv_b)) != hipSuccess ||
      (e = hipMalloc(&S.pads, pads_b)) != hipSuccess || (e = hipMalloc(&S.words, words_b)) != hipSuccess ||
      (e = hipMalloc(&S.sems, sems_b)) != hipSuccess || (e = hipMalloc(&S.epochs, epochs_b)) != hipSuccess ||
      (e = hipMalloc(&S.symm, symm_b)) != hipSuccess) {
    rc = fail(ARX_ENOMEM, "device allocation of %zu bytes failed: %s",
              send_b + recv_b + pads_b + words_b + sems_b + epochs_b + symm_b, hipGetErrorString(e));
  } else if ((e = hipHostMalloc((void**)&S.ctl, 4096, hipHostMallocCoherent | hipHostMallocMapped)) !=
                 hipSuccess ||
             (e = hipHostMalloc((void**)&S.flags, 4096, hipHostMallocCoherent | hipHostMallocMapped)) !=
                 hipSuccess) {
    rc = fail(ARX_ENOMEM, "pinned allocation failed: %s", hipGetErrorString(e));
  } else if ((e = hipMemset(S.send, 0, send_b)) != hipSuccess || (e = hipMemset(S.recv, 0, recv_b)) != hipSuccess ||
             (e = hipMemset(S.pads, 0, pads_b)) != hipSuccess ||
             (e = hipMemset(S.words, 0, words_b)) != hipSuccess || (e = hipMemset(S.sems, 0, sems_b)) != hipSuccess ||
             (e = hipMemset(S.epochs, 0, epochs_b)) != hipSuccess ||
             (e = hipHostGetDevicePointer((void**)&S.ctl_dev, S.ctl, 0)) != hipSuccess ||
             (e = hipHostGetDevicePointer((void**)&S.flags_dev, S.flags, 0)) != hipSuccess ||
             (e = hipDeviceSynchronize()) != hipSuccess) {
    rc = fail(ARX_EHIP, "initialising device state failed: %s", hipGetErrorString(e));
  }
  if (rc != ARX_OK) {
    free_all();
    return rc;
  }
  memset((void*)S.ctl, 0, 4096);
  memset((void*)S.flags, 0, 4096);
  S.proxy_err.store(false);
  S.inject_copy_failure.store(false);
  S.stop.store(false);
  S.timeout_us = 2000000;
  // no C++ exception may leave the C ABI
  try {
    S.core.reset(new arx::Proxy(&S.ctl->seq, &S.ctl->done, S.flags, S.world, S.rank));
    S.core->before_post = stress_copy;
    S.proxy = std::thread(proxy_main);
  } catch (const std::exception& ex) {
    S.core.reset();
    free_all();
    return fail(ARX_ENOMEM, "starting the proxy thread failed: %s", ex.what());
  }
  S.inited = true;
  return ARX_OK;
}

// [a, a + na) and [b, b + nb) share a byte.
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na > 0 && nb > 0 && x < y + nb && y < x + na;
}

int check_ptrs(const void* in, const void* out, size_t n) {
  if (n > S.max_n) return fail(ARX_EINVAL, "n %zu exceeds max_n %zu", n, S.max_n);
  if (n > 0 && (in == nullptr || out == nullptr)) return fail(ARX_EINVAL, "null in or out");
  if (((uintptr_t)in & 15u) || ((uintptr_t)out & 15u)) return fail(ARX_EINVAL, "in and out must be 16-byte aligned");
  if (in != out && overlap(in, 2 * n, out, 2 * n))
    return fail(ARX_EINVAL, "in and out overlap without being the same buffer");
  return ARX_OK;
}

// The tag buffers of a barrier launch: both given or neither, and only with
// one workgroup per rank and block.
int check_tags(const uint32_t* tags, const uint32_t* seen, bool lanes) {
  if ((tags == nullptr) != (seen == nullptr)) return fail(ARX_EINVAL, "tags and seen go together");
  if (tags && lanes) return fail(ARX_EINVAL, "tags need one workgroup per rank and block (no ARX_BARRIER_LANES)");
  return ARX_OK;
}

// A launch of world * nblocks workgroups that wait on each other must fit on
// the device at once.
int check_groups(int nblocks, bool counter) {
  const long long cap = arx::barrier_groups_cap(counter, S.cus);
  if ((long long)S.world * nblocks > cap)
    return fail(ARX_EINVAL, "%d workgroups (W %d x nblocks %d) exceed the %lld the device holds at once",
                S.world * nblocks, S.world, nblocks, cap);
  return ARX_OK;
}

}  // namespace

namespace arx {
int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof g_detail, fmt, ap);
  va_end(ap);
  return code;
}
}  // namespace arx

extern "C" {

int arx_init(int world, size_t max_n) { return init_impl(world, max_n, 0); }

int arx_init_rank(int world, size_t max_n, int rank) { return init_impl(world, max_n, rank); }

int arx_finalize(void) {
  if (!S.inited) return fail(ARX_ESTATE, "arx is not initialised");
  // let in-flight calls finish while the proxy still posts their flags
  const hipError_t e = hipDeviceSynchronize();
  S.stop.store(true, std::memory_order_release);
  store_release(&S.ctl->stop, 1);
  if (S.proxy.joinable()) S.proxy.join();
  S.core.reset();
  free_all();
  S.inited = false;
  S.world = S.rank = 0;
  S.max_n = S.stride = 0;
  if (e != hipSuccess) return fail(ARX_EHIP, "hipDeviceSynchronize: %s", hipGetErrorString(e));
  return ARX_OK;
}

int arx_publish(uint64_t seq) {
  if (!S.inited) return fail(ARX_ESTATE, "arx is not initialised");
  if (!S.core->publish(seq))
    return fail(ARX_EORDER, "arx_publish(%llu) after %llu: seqs are posted in order", (unsigned long long)seq,
                (unsigned long long)S.core->posted());
  return ARX_OK;
}

int arx_allreduce(const void* in, void* out, size_t n, hipStream_t stream) {
  int rc = check_ready();
  if (rc != ARX_OK) return rc;
  if ((rc = check_ptrs(in, out, n)) != ARX_OK) return rc;
  arx::OneShotArgs a{};
  a.in = (const uint16_t*)in;
  a.out = (uint16_t*)out;
  a.send = S.send;
  a.recv = S.recv;
  a.stride = S.stride;
  a.flags = S.flags_dev;
  a.ctl = S.ctl_dev;
  a.words = S.words;
  a.n = (uint32_t)n;
  a.rank = S.rank;
  a.timeout = timeout_ticks();
  HIPCHK(arx::launch_oneshot(a, S.world, 0, S.cus, stream));
  return ARX_OK;
}

int arx_reduce(const void* in, void* out, size_t n, int par, hipStream_t stream) {
  int rc = check_ready();
  if (rc != ARX_OK) return rc;
  if (par != 0 && par != 1) return fail(ARX_EINVAL, "par %d not in {0, 1}", par);
  if ((rc = check_ptrs(in, out, n)) != ARX_OK) return rc;
  if (n == 0) return ARX_OK;
  arx::ReduceArgs a;
  a.in = (const uint16_t*)in;
  a.out = (uint16_t*)out;
  a.recv_par = S.recv + (size_t)par * S.world * S.stride;
  a.stride = S.stride;
  a.n = (uint32_t)n;
  a.rank = S.rank;
  HIPCHK(arx::launch_reduce(a, S.world, stream));
  return ARX_OK;
}

int arx_barrier_blockwise(int nblocks, int sem, int rounds, int flags, uint32_t* tags, uint32_t* seen,
                          hipStream_t stream) {
  int rc = check_ready();
  if (rc != ARX_OK) return rc;
  if (nblocks < 1 || nblocks > ARX_MAX_PAD_BLOCKS)
    return fail(ARX_EINVAL, "nblocks %d not in [1, %d]", nblocks, ARX_MAX_PAD_BLOCKS);
  if (sem != ARX_SEM_RELAXED && sem != ARX_SEM_ACQ_REL) return fail(ARX_EINVAL, "sem %d unknown", sem);
  if (rounds < 1 || rounds > 64) return fail(ARX_EINVAL, "rounds %d not in [1, 64]", rounds);
  if (flags & ~ARX_BARRIER_LANES) return fail(ARX_EINVAL, "barrier flags %#x unknown", flags);
  const bool lanes = (flags & ARX_BARRIER_LANES) != 0;
  if ((rc = check_tags(tags, seen, lanes)) != ARX_OK) return rc;
  if (!lanes && (rc = check_groups(nblocks, false)) != ARX_OK) return rc;
  arx::BarrierArgs a;
  for (int i = 0; i < 8; ++i)
    a.pad[i] = i < S.world ? S.pads + (size_t)i * ARX_MAX_PAD_BLOCKS * S.world : nullptr;
  a.world = S.world;
  a.acq_rel = sem == ARX_SEM_ACQ_REL;
  a.rounds = rounds;
  a.nblocks = nblocks;
  a.tags = tags;
  a.seen = seen;
  a.timeout = timeout_ticks();
  a.ctl = S.ctl_dev;
  HIPCHK(arx::launch_barrier(a, lanes, stream));
  return ARX_OK;
}

int arx_counter_barrier(int nblocks, int rounds, int flags, uint32_t* epochs_seen, uint32_t* tags, uint32_t* seen,
                        hipStream_t stream) {
  int rc = check_ready();
  if (rc != ARX_OK) return rc;
  if (nblocks < 1 || nblocks > ARX_MAX_PAD_BLOCKS)
    return fail(ARX_EINVAL, "nblocks %d not in [1, %d]", nblocks, ARX_MAX_PAD_BLOCKS);
  if (rounds < 0 || rounds > 64) return fail(ARX_EINVAL, "rounds %d not in [0, 64]", rounds);
  if (flags & ~(ARX_BARRIER_LANES | ARX_BARRIER_SPLIT)) return fail(ARX_EINVAL, "barrier flags %#x unknown", flags);
  const bool lanes = (flags & ARX_BARRIER_LANES) != 0;
  if ((rc = check_tags(tags, seen, lanes)) != ARX_OK) return rc;
  if (!lanes && (rc = check_groups(nblocks, true)) != ARX_OK) return rc;
  arx::CounterArgs a;
  for (int i = 0; i < 8; ++i) {
    a.sem[i] = i < S.world ? S.sems + (size_t)i * ARX_MAX_PAD_BLOCKS : nullptr;
    a.epochs[i] = i < S.world ? S.epochs + (size_t)i * ARX_MAX_PAD_BLOCKS : nullptr;
  }
  a.seen = epochs_seen;
  a.tags = tags;
  a.tag_seen = seen;
  a.world = S.world;
  a.rounds = rounds;
  a.nblocks = nblocks;
  a.split = (flags & ARX_BARRIER_SPLIT) != 0;
  a.timeout = timeout_ticks();
  a.ctl = S.ctl_dev;
  HIPCHK(arx::launch_counter_barrier(a, lanes, stream));
  return ARX_OK;
}

int arx_symm_allreduce(const void* inputs, void* outputs, size_t n, size_t ld, int iters, hipStream_t stream) {
  int rc = check_ready();
  if (rc != ARX_OK) return rc;
  if (n > S.max_n) return fail(ARX_EINVAL, "n %zu exceeds max_n %zu", n, S.max_n);
  if (ld < n || (ld & 7u)) return fail(ARX_EINVAL, "ld %zu must be >= n and a multiple of 8", ld);
  if (iters < 1 || iters > 65536) return fail(ARX_EINVAL, "iters %d not in [1, 65536]", iters);
  if (n > 0 && (inputs == nullptr || outputs == nullptr)) return fail(ARX_EINVAL, "null inputs or outputs");
  if (((uintptr_t)inputs & 15u) || ((uintptr_t)outputs & 15u))
    return fail(ARX_EINVAL, "inputs and outputs must be 16-byte aligned");
  const size_t extent = (size_t)iters * S.world * ld * sizeof(uint16_t);
  if (inputs != outputs && overlap(inputs, extent, outputs, extent))
    return fail(ARX_EINVAL, "inputs and outputs overlap without being the same buffer");
  arx::SymmArgs a;
  a.inputs = (const uint16_t*)inputs;
  a.outputs = (uint16_t*)outputs;
  a.symm = S.symm;
  a.stride = S.stride;
  a.ld = ld;
  a.n = (uint32_t)n;
  a.iters = iters;
  a.world = S.world;
  a.blocks = arx::symm_blocks(a.n, S.world, S.cus);
  for (int i = 0; i < 8; ++i)
    a.pad[i] = i < S.world ? S.pads + (size_t)i * ARX_MAX_PAD_BLOCKS * S.world : nullptr;
  a.timeout = timeout_ticks();
  a.ctl = S.ctl_dev;
  a.status = nullptr;
  HIPCHK(arx::launch_symm_allreduce(a, stream));
  return ARX_OK;
}

int arx_barrier_max_blocks(void) {
  if (!S.inited) return fail(ARX_ESTATE, "arx is not initialised");
  const long long a = arx::barrier_groups_cap(false, S.cus), b = arx::barrier_groups_cap(true, S.cus);
  const long long most = (a < b ? a : b) / S.world;
  return (int)(most < ARX_MAX_PAD_BLOCKS ? most : ARX_MAX_PAD_BLOCKS);
}

const uint32_t* arx_sem_ptr(int rank) {
  if (!S.inited || rank < 0 || rank >= S.world) return nullptr;
  return reinterpret_cast<const uint32_t*>(S.sems + (size_t)rank * ARX_MAX_PAD_BLOCKS);
}

const uint32_t* arx_epoch_ptr(int rank) {
  if (!S.inited || rank < 0 || rank >= S.world) return nullptr;
  return S.epochs + (size_t)rank * ARX_MAX_PAD_BLOCKS;
}

void* arx_recv_ptr(int par, int src) {
  if (!S.inited || (par != 0 && par != 1) || src < 0 || src >= S.world) return nullptr;
  return S.recv + ((size_t)par * S.world + src) * S.stride;
}

void* arx_send_ptr(int par) {
  if (!S.inited || (par != 0 && par != 1)) return nullptr;
  return S.send + (size_t)par * S.stride;
}

uint32_t* arx_pad_ptr(int rank) {
  if (!S.inited || rank < 0 || rank >= S.world) return nullptr;
  return S.pads + (size_t)rank * ARX_MAX_PAD_BLOCKS * S.world;
}

int arx_set_proxy_mode(int mode) {
  if (!S.inited) return fail(ARX_ESTATE, "arx is not initialised");
  if (mode != ARX_PROXY_LOCKSTEP && mode != ARX_PROXY_RUNAHEAD && mode != ARX_PROXY_MANUAL &&
      mode != ARX_PROXY_STRESS)
    return fail(ARX_EINVAL, "proxy mode %d unknown", mode);
  if (mode == ARX_PROXY_STRESS && !S.stress_pool)
    return fail(ARX_EINVAL, "stress mode needs arx_set_stress_source first");
  S.core->mode.store(mode);
  return ARX_OK;
}

int arx_set_stress_source(const void* pool, int sets) {
  if (!S.inited) return fail(ARX_ESTATE, "arx is not initialised");
  if (S.core->mode.load() == ARX_PROXY_STRESS) return fail(ARX_ESTATE, "leave stress mode before changing its source");
  const bool clear = pool == nullptr || sets == 0;
  if (!clear && sets < 0) return fail(ARX_EINVAL, "sets %d < 0", sets);
  if (!clear && !S.stress_stream) HIPCHK(hipStreamCreateWithFlags(&S.stress_stream, hipStreamNonBlocking));
  // under the proxy's lock: a stress post that read the mode before it
  // left stress mode has finished with the old source
  S.core->locked([&] {
    S.stress_pool = clear ? nullptr : (const uint16_t*)pool;
    S.stress_sets = clear ? 0 : sets;
  });
  return ARX_OK;
}

int arx_set_timeout_us(uint64_t us) {
  if (!S.inited) return fail(ARX_ESTATE, "arx is not initialised");
  if (us < 1 || us > 60000000ull) return fail(ARX_EINVAL, "timeout %llu us not in [1, 60000000]",
                                              (unsigned long long)us);
  S.timeout_us = us;
  return ARX_OK;
}

int arx_status(uint64_t* published, uint64_t* posted, uint64_t* done) {
  if (!S.inited) return fail(ARX_ESTATE, "arx is not initialised");
  if (published) *published = load_acquire(&S.ctl->seq);
  if (posted) *posted = S.core->posted();
  if (done) *done = load_acquire(&S.ctl->done);
  return ARX_OK;
}

int arx_debug_state(uint64_t* words, int nwords) {
  if (!S.inited) return fail(ARX_ESTATE, "arx is not initialised");
  if (words == nullptr || nwords < 0) return fail(ARX_EINVAL, "bad output array");
  HIPCHK(hipDeviceSynchronize());
  uint32_t dw[arx::WORDS_TOTAL];
  HIPCHK(hipMemcpy(dw, S.words, sizeof dw, hipMemcpyDeviceToHost));
  uint64_t all[12 + ARX_MAX_WORLD];
  all[0] = dw[arx::WORD_SEQ] | (uint64_t)dw[arx::WORD_SEQ + 1] << 32;
  all[1] = dw[arx::WORD_CNT0];
  all[2] = dw[arx::WORD_CNT1];
  // go (replica 0): 2 * seq of the last call past its flag wait, + 1 if aborted
  const uint64_t go = dw[arx::WORD_GO] | (uint64_t)dw[arx::WORD_GO + 1] << 32;
  all[3] = (go >> 1) & 0xFFFFFFFFull;
  all[4] = (go & 1u) ? go >> 1 : 0u;
  all[5] = load_acquire(&S.ctl->seq);
  all[6] = load_acquire(&S.ctl->bytes[0]);
  all[7] = load_acquire(&S.ctl->bytes[1]);
  all[8] = load_acquire(&S.ctl->done);
  all[9] = load_acquire(&S.ctl->err);
  all[10] = load_acquire(&S.ctl->err_seq);
  all[11] = S.core->posted();
  for (int i = 0; i < S.world; ++i) all[12 + i] = load_acquire(&S.flags[i]);
  const int total = 12 + S.world;
  const int m = nwords < total ? nwords : total;
  for (int i = 0; i < m; ++i) words[i] = all[i];
  return m;
}

int arx_debug_set_seq(uint64_t seq) {
  if (!S.inited) return fail(ARX_ESTATE, "arx is not initialised");
  const int mode = S.core->mode.load();
  if (mode != ARX_PROXY_LOCKSTEP && mode != ARX_PROXY_MANUAL)
    return fail(ARX_ESTATE, "set the seq in lockstep or manual mode");
  HIPCHK(hipDeviceSynchronize());
  HIPCHK(hipMemcpy(S.words + arx::WORD_SEQ, &seq, sizeof seq, hipMemcpyHostToDevice));
  const uint64_t go = seq << 1;
  for (int k = 0; k < arx::kGoReplicas; ++k)
    HIPCHK(hipMemcpy(S.words + arx::WORD_GO + 64 * k, &go, sizeof go, hipMemcpyHostToDevice));
  HIPCHK(hipMemcpy(S.words + arx::WORD_PUBLISHED, &seq, sizeof seq, hipMemcpyHostToDevice));
  // The proxy first: were ctl.seq stored before its posted seq, the proxy
  // thread could see the jump and post every seq up to it, one by one.
  S.core->reset(seq);
  store_release(&S.ctl->done, seq);
  store_release(&S.ctl->seq, seq);
  return ARX_OK;
}

int arx_debug_fail_proxy(void) {
  if (!S.inited) return fail(ARX_ESTATE, "arx is not initialised");
  S.inject_copy_failure.store(true);
  return ARX_OK;
}

int arx_test_round_bf16(const void* in, void* out, size_t n, hipStream_t stream) {
  if (n > 0xFFFFFFFFull) return fail(ARX_EINVAL, "n %zu too large", n);
  if (n > 0 && (in == nullptr || out == nullptr)) return fail(ARX_EINVAL, "null in or out");
  if (n == 0) return ARX_OK;
  HIPCHK(arx::launch_round_test((const uint32_t*)in, (uint16_t*)out, n, stream));
  return ARX_OK;
}

int arx_test_oneshot_shape(size_t n, int world, int block, unsigned resident, int in_place, int* out, int nout) {
  if (n > ARX_MAX_N) return fail(ARX_EINVAL, "n %zu above ARX_MAX_N", n);
  if (world < 2 || world > 8) return fail(ARX_EINVAL, "world %d not in [2, 8]", world);
  if (block != 0 && block != 256 && block != 512 && block != 1024) return fail(ARX_EINVAL, "block %d", block);
  if (resident < 2) return fail(ARX_EINVAL, "resident %u: the poll workgroup and a reducing one need 2", resident);
  if (out == nullptr || nout < 8) return fail(ARX_EINVAL, "out needs 8 entries");
  const int b = block ? block : arx::oneshot_block((uint32_t)n, world);
  const unsigned cap = resident < arx::kMaxOneShotGrid + 1u ? resident : arx::kMaxOneShotGrid + 1u;
  const arx::OneShotShape sh = arx::oneshot_shape((uint32_t)n, world, b, cap, in_place == 0);
  out[0] = b;
  out[1] = (int)sh.grid;
  out[2] = (int)sh.launched;
  out[3] = (int)sh.ncopy;
  out[4] = sh.one_pass ? 1 : 0;
  out[5] = sh.early_go ? 1 : 0;
  out[6] = sh.nt_copy ? 1 : 0;
  out[7] = sh.nt_peer ? 1 : 0;
  return ARX_OK;
}

const char* arx_strerror(int err) {
  static char buf[640];
  const char* base;
  switch (err) {
    case ARX_OK: return "ok";
    case ARX_EINVAL: base = "invalid argument"; break;
    case ARX_ESTATE: base = "wrong library state"; break;
    case ARX_ENOMEM: base = "out of memory"; break;
    case ARX_EHIP: base = "HIP error"; break;
    case ARX_EPROXY: base = "proxy thread failed"; break;
    case ARX_EORDER: base = "seq published out of order"; break;
    case ARX_ETIMEOUT: base = "device wait timed out"; break;
    default: return "unknown error";
  }
  if (g_detail[0]) snprintf(buf, sizeof buf, "%s: %s", base, g_detail);
  else snprintf(buf, sizeof buf, "%s", base);
  return buf;
}

size_t arx_max_n(void) { return S.inited ? S.max_n : 0; }
int arx_world(void) { return S.inited ? S.world : 0; }
int arx_rank(void) { return S.inited ? S.rank : 0; }

}  // extern "C"
