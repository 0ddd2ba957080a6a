// arx_internal.h — layouts and launchers shared by the kernels and the host
// runtime of libarx (not part of the public C ABI).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace arx {

struct Semaphore;

// Control block in pinned, coherent host memory (page "arx.cu": struct Ctl).
// Line 0 is written by the GPU when it publishes and read by the proxy;
// line 1 is written by the GPU when a call finishes or a wait times out;
// line 2 is host-only.
struct alignas(64) Ctl {
  uint64_t seq;       // last seq this GPU published
  uint64_t bytes[2];  // call size in bytes, one slot per parity of seq
  uint64_t pad0[5];
  uint64_t done;      // last seq whose reduction finished
  uint64_t err;       // first device-side error kind (ERR_*), 0 if none
  uint64_t err_seq;   // seq of that error
  uint64_t pad1[5];
  uint64_t stop;      // asks the proxy thread to return
  uint64_t pad2[7];
};
static_assert(sizeof(Ctl) == 192, "Ctl layout");

enum : uint64_t {
  ERR_NONE = 0,
  ERR_FLAG_TIMEOUT = 1,     // the flag wait gave up waiting for a peer flag
  ERR_GO_TIMEOUT = 2,       // a workgroup gave up waiting for go
  ERR_BARRIER_TIMEOUT = 3,  // a signal-pad CAS wait gave up
  ERR_COUNTER_TIMEOUT = 4,  // a counter-barrier wait gave up
  ERR_SYMM_TIMEOUT = 5,     // a barrier wait of the symmetric-buffer exchange gave up
};

// Device words (u32), each on its own 256-byte line of one allocation.
enum : int {
  WORD_SEQ = 0,      // last completed seq (u64: words 0 and 1)
  WORD_CNT0 = 64,    // arrivals: copying workgroups past the copy, and the poll workgroup
  WORD_CNT1 = 128,   // workgroups finished (finish counter)
  WORD_GO = 192,     // go (u64): 2 * seq of the call whose peers' partials are all in place, + 1 if that call
                     // is aborted; kGoReplicas copies, WORD_GO + 64 * k for replica k
  WORD_PUBLISHED = 704,  // seq (u64) of the last call whose seq was published to the proxy: a hint
                         // that tells the flag wait when to read the peers' flags again
  WORD_BYTES_SHADOW = 768,  // ctl.bytes[0] and ctl.bytes[1] as last stored (u64 at words 768 and 770)
  WORDS_TOTAL = 1024,
};
constexpr int kGoReplicas = 8;
static_assert(WORD_GO + 64 * kGoReplicas <= WORD_PUBLISHED, "go replicas fit below the published word");
static_assert(WORD_PUBLISHED + 64 <= WORD_BYTES_SHADOW, "the published word has a line of its own");
static_assert(WORD_BYTES_SHADOW + 64 <= WORDS_TOTAL, "the size shadow fits in the word block");

constexpr int kBlock = 256;       // threads per workgroup of the reduction kernels
constexpr int kMaxOneShotGrid = 256;  // reducing workgroups of the one-shot kernel, at most

struct OneShotArgs {
  const uint16_t* in;
  uint16_t* out;
  uint16_t* send;          // send slot 0; slot 1 at + stride
  const uint16_t* recv;    // [2][W][stride]
  uint64_t stride;         // elements per slot
  const uint64_t* flags;   // pinned [W]
  Ctl* ctl;                // pinned
  uint32_t* words;         // device
  uint32_t n;
  int rank;
  uint64_t timeout;        // wall-clock ticks per wait
  uint32_t ncopy;          // reducing workgroups that copy and count arrival (set by the launcher)
  uint32_t early_go;       // 1: go may precede this rank's publish (set by the launcher)
  uint32_t nt_copy;        // 1: the copy's grid-stride stores are nontemporal (set by the launcher)
  uint32_t nt_peer;        // 1: the grid-stride sum's peer loads are nontemporal (set by the launcher)
};

struct ReduceArgs {
  const uint16_t* in;
  uint16_t* out;
  const uint16_t* recv_par;  // recv slots of the chosen parity: [W][stride]
  uint64_t stride;
  uint32_t n;
  int rank;
};

struct BarrierArgs {
  uint32_t* pad[8];
  int world;
  int acq_rel;
  int rounds;
  int nblocks;
  uint32_t* tags;      // [W][rounds][nblocks] barrier tags written (or null)
  uint32_t* seen;      // [W][rounds][nblocks][W] tags read back after each round (or null)
  uint64_t timeout;
  Ctl* ctl;
};

struct CounterArgs {
  Semaphore* sem[8];   // rank r's semaphores, one per block id
  uint32_t* epochs[8]; // rank r's epochs, one per block id
  uint32_t* seen;      // [W][nblocks]: the epoch each rank's block read (for checks), or null
  uint32_t* tags;      // [W][rounds][nblocks] barrier tags written before each end stage (or null)
  uint32_t* tag_seen;  // [W][rounds][nblocks][W] tags read back after each end stage (or null)
  int world;
  int rounds;
  int nblocks;
  int split;           // separate start- and end-stage semaphores
  uint64_t timeout;
  Ctl* ctl;
};

struct SymmArgs {
  const uint16_t* inputs;  // [iters][W][ld]: rank v's partial for iteration k at (k * W + v) * ld
  uint16_t* outputs;       // [iters][W][ld]: rank v's result for iteration k
  uint16_t* symm;          // [W][stride]: rank v's symmetric buffer at v * stride
  uint64_t stride;
  uint64_t ld;
  uint32_t n;
  int iters;
  int blocks;              // workgroups per rank
  int world;
  uint32_t* pad[8];
  uint64_t timeout;
  Ctl* ctl;                // pinned control block for a timeout report, or null
  uint32_t* status;        // device word set to 1 on a timeout, or null
};

// Launchers (defined in arx_reduce.hip and arx_sync.hip). W in [2, 8]. block: threads per
// one-shot workgroup (256, 512 or 1024), or 0 to choose by n and W. cus: compute
// units of the device; kernels whose workgroups wait on each other keep
// their grid within what is resident at once.
hipError_t launch_oneshot(const OneShotArgs& a, int W, int block, int cus, hipStream_t stream);
int oneshot_block(uint32_t n, int W);
hipError_t launch_reduce(const ReduceArgs& a, int W, hipStream_t stream);
// The barrier launchers: lanes = true puts block b of every rank in one wave
// (nblocks workgroups), false gives rank v's block b a workgroup of its own
// (world * nblocks workgroups, which must all be resident at once:
// barrier_groups_cap gives the most the device holds, 0 if unknown).
hipError_t launch_barrier(const BarrierArgs& a, bool lanes, hipStream_t stream);
hipError_t launch_counter_barrier(const CounterArgs& a, bool lanes, hipStream_t stream);
long long barrier_groups_cap(bool counter, int cus);
hipError_t launch_symm_allreduce(const SymmArgs& a, hipStream_t stream);
int symm_blocks(uint32_t n, int world, int cus);
hipError_t launch_round_test(const uint32_t* in, uint16_t* out, size_t n, hipStream_t stream);

// Records the detail of an error for arx_strerror and returns `code`
// (defined in arx_runtime.cpp).
int set_error(int code, const char* fmt, ...);

// Reducing workgroups the one-shot kernel uses for n elements with `block`
// threads per workgroup, at most max_grid (all its workgroups must be
// resident at once, since they wait on each other; a grid of more than one
// adds the poll workgroup).
unsigned oneshot_grid(uint32_t n, int block, unsigned max_grid);
// Workgroups of a one-shot grid that copy the partial and count arrival.
unsigned oneshot_copiers(unsigned grid);

// Launch shape of one one-shot call with `block` threads per workgroup, at
// most `resident` workgroups resident at once, and `in` and `out` apart or
// not (the host-side rules of the launcher, also exported as a test aid).
struct OneShotShape {
  unsigned grid;      // reducing workgroups
  unsigned launched;  // workgroups launched: grid, plus the poll workgroup
  unsigned ncopy;     // reducing workgroups that copy and count arrival
  bool one_pass;      // a reducing thread for every 16-byte vector
  bool early_go;      // go may precede this rank's publish
  bool nt_copy;       // the copy's grid-stride stores are nontemporal
  bool nt_peer;       // the grid-stride sum's peer loads are nontemporal
};
OneShotShape oneshot_shape(uint32_t n, int W, int block, unsigned resident, bool disjoint);

}  // namespace arx
