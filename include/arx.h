/*
 * arx.h — C ABI of libarx: the one-shot W-way bf16 reduction gated by a
 * seq/parity flag protocol, and the blockwise signal-pad barrier, on one
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (page "arx.cu", protocol comment and arx_kernel): this GPU
 * is rank `rank` of a group of W ranks. A call with sequence number
 * seq = previous + 1 and parity par = seq & 1
 *   1. copies the caller's bf16 partial `in` into the send slot send[par],
 *   2. publishes seq (a host proxy thread sees it and posts the peers' flags),
 *   3. waits until the flag of every other rank has reached seq,
 *   4. writes out[i] = bf16(sum over src = 0..W-1, in that order, of the
 *      binary32 value of partial src at i), where partial `rank` is `in` and
 *      partial src != rank is recv[par][src]; the sum is accumulated in
 *      binary32 and rounded once to bf16, round to nearest, ties to even,
 *      every NaN result written as 0x7FC0, subnormals kept,
 *   5. resets its own counters, so calls can be captured in a hipGraph.
 * Every rank running the same calls gets the same bits.
 *
 * On one GPU the W - 1 peers are virtual: their partials already sit in the
 * recv slots of this library (the caller fills them through arx_recv_ptr),
 * and their flags are posted into pinned host memory by the library's proxy
 * thread (or by the caller in manual mode). Nothing crosses GPUs.
 *
 * Conventions for every call below:
 *   - return value: ARX_OK (0) or a negative ARX_E* code; the library never
 *     exits the process; arx_strerror() gives the message of the last error.
 *   - device pointers are HIP device addresses; host pointers are ordinary
 *     process memory. The caller owns `in`, `out` and the stream; the library
 *     owns every slot, flag, counter, pad and its proxy thread.
 *   - the library keeps one instance per process and is not thread-safe:
 *     issue all calls from one thread, in order on one stream (seq is a
 *     running counter kept on the device).
 */
#ifndef ARX_H
#define ARX_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Error codes. */
#define ARX_OK 0
#define ARX_EINVAL (-1)   /* bad argument: world, rank, n, alignment, null pointer */
#define ARX_ESTATE (-2)   /* not initialised, or initialised twice */
#define ARX_ENOMEM (-3)   /* device or pinned allocation failed */
#define ARX_EHIP (-4)     /* a HIP runtime call failed (message kept for arx_strerror) */
#define ARX_EPROXY (-5)   /* the proxy thread failed earlier (latched) */
#define ARX_EORDER (-6)   /* arx_publish called with a seq that is not last + 1 */
#define ARX_ETIMEOUT (-7) /* a kernel's bounded wait ran out (latched until finalize) */

/* Limits. */
#define ARX_MAX_WORLD 8          /* page "arx.cu": kMaxWorld; page "common.cuh": kMaxNumGPU */
#define ARX_MAX_PAD_BLOCKS 1024  /* workgroups per barrier launch */
#define ARX_MAX_N ((size_t)1 << 30) /* elements per partial */
#define ARX_NOALLOC_MAX_N ((size_t)1 << 20) /* elements per partial of arx_symm_allreduce_noalloc */

/* Proxy modes: when the virtual peers post the flag of seq s. */
#define ARX_PROXY_LOCKSTEP 0 /* once this rank has published s (peers exactly as fast) */
#define ARX_PROXY_RUNAHEAD 1 /* once this rank has published s - 1 (the earliest a peer can) */
#define ARX_PROXY_MANUAL 2   /* never; the caller calls arx_publish */
#define ARX_PROXY_STRESS 3   /* lockstep, and before posting s the proxy writes the peers' data for s
                                into recv[s & 1] from the source set by arx_set_stress_source */

/* Barrier memory semantics (page "triton_barrier.py", blockwise_barrier). */
#define ARX_SEM_RELAXED 0 /* relaxed system-scope CAS on both sides */
#define ARX_SEM_ACQ_REL 1 /* release CAS to signal, acquire CAS to consume */

/* Barrier launch flags. By default rank v's block b is a workgroup of its
 * own: W * nblocks workgroups, the W with block id b wait on each other. */
#define ARX_BARRIER_LANES 1 /* the named lane-group variant: workgroup b is one wave whose lanes
                               [v*W, v*W + W) play rank v, so no workgroup waits on another */
#define ARX_BARRIER_SPLIT 2 /* counter barrier only: separate start- and end-stage semaphores */

/*
 * Barrier tags. A tagged barrier launch checks what each round makes
 * visible: before round r, rank v's workgroup for block b writes the tag
 *     tag(v, b, r) = 0x80000000 | r << 16 | b << 4 | v
 * with a plain store into tags[(v * rounds + r) * nblocks + b]; after the
 * round its thread p < W reads rank p's tag for the same block and round
 * with a plain load into seen[((v * rounds + r) * nblocks + b) * W + p].
 * Every round has slots of its own. With ARX_SEM_ACQ_REL the barrier makes
 * the peers' tags visible, so seen holds tag(p, b, r) everywhere; with
 * ARX_SEM_RELAXED a slot may still read as its earlier contents. The caller
 * zero-fills both buffers before the launch.
 */

/*
 * arx_init — allocate and zero all state, start the proxy thread.
 * Page "arx.cu": arx_prepare (world range check, pinned flag and control
 * blocks, zeroed) and arx_connect (device seq/counter/go words zeroed, proxy
 * thread started). This GPU is rank 0.
 *   world: W in [2, 8].  max_n: largest n any later call may use, in bf16
 *   elements, 1 <= max_n <= ARX_MAX_N.
 * The proxy thread busy-polls the published seq (one host core) from here
 * until arx_finalize, as the page's proxy_loop does; its poll latency is
 * part of every call's flag wait.
 * Allocates on the current HIP device: send slots [2][max_n], recv slots
 * [2][W][max_n] and symmetric buffers [W][max_n] bf16 in device memory, W
 * signal pads u32[ARX_MAX_PAD_BLOCKS][W], W x ARX_MAX_PAD_BLOCKS semaphores
 * and W x ARX_MAX_PAD_BLOCKS epochs, the device words (seq, two counters,
 * the go word in 8 replicas, the published seq, a copy of the two call
 * sizes last stored), and in pinned coherent
 * host memory the control block and flags[W] (u64). Errors: ARX_EINVAL,
 * ARX_ESTATE (already initialised), ARX_ENOMEM, ARX_EHIP.
 */
int arx_init(int world, size_t max_n);

/* arx_init with an explicit rank in [0, world): this GPU's partial then takes
 * position `rank` in the sum and the proxy posts flags for every other rank. */
int arx_init_rank(int world, size_t max_n, int rank);

/* Stop the proxy thread (page "arx.cu": the stop word of struct Ctl), wait
 * for the device, free everything. Allowed only when initialised; a later
 * arx_init starts afresh with seq 0. */
int arx_finalize(void);

/*
 * arx_publish — the virtual peers publish seq: store-release flags[src] = seq
 * for every src != rank into pinned memory. seq must be exactly the last
 * posted seq + 1 (page "arx.cu", proxy_loop: seqs are posted one by one with
 * none left out, since a skipped seq would let a peer accept a later flag
 * over stale data);
 * otherwise ARX_EORDER and nothing is written. Called by the proxy thread in
 * the lockstep and run-ahead modes, by the caller in manual mode.
 */
int arx_publish(uint64_t seq);

/*
 * arx_allreduce — one call of the one-shot path (page "arx.cu": arx_kernel,
 * arx_allreduce). Launches one kernel on `stream`, asynchronously; the call
 * is hipGraph-capturable (each replay is the next seq).
 *   in:  device bf16 [n], this rank's partial, 16-byte aligned.
 *   out: device bf16 [n], 16-byte aligned; either `in` itself (in place)
 *        or a range that does not overlap it (a partial overlap is
 *        ARX_EINVAL). out[i >= n] is never written.
 *   n:   0 <= n <= max_n, any value (n % 8 != 0 allowed); n == 0 still runs
 *        the protocol and advances seq.
 * Errors (nothing launched): ARX_ESTATE, ARX_EINVAL, ARX_EPROXY (proxy failed
 * earlier), ARX_ETIMEOUT (an earlier call's wait timed out), ARX_EHIP.
 * If this call's own flag wait times out on the device, out is left
 * untouched, seq still advances and the error is latched for the next call.
 * The kernel's workgroups wait on each other, so its grid never exceeds
 * what the device holds at once (occupancy per CU times the CU count: at
 * most 256 workgroups that reduce and one that waits for the flags); past
 * one vector per thread, threads loop.
 */
int arx_allreduce(const void* in, void* out, size_t n, hipStream_t stream);

/*
 * arx_reduce — the reduction step alone, no copy, publish or wait: out[i] =
 * rank-ordered sum of `in` (at position rank) and recv[par][src] (src !=
 * rank), as in arx_allreduce. par in {0, 1}. Same pointer and n rules as
 * arx_allreduce; does not touch seq, counters or flags.
 */
int arx_reduce(const void* in, void* out, size_t n, int par, hipStream_t stream);

/*
 * arx_barrier_blockwise — the blockwise signal-pad barrier (page
 * "triton_barrier.py": blockwise_barrier, send_signal, wait_signal) for the
 * W virtual ranks on block ids 0..nblocks-1, `rounds` consecutive times.
 * Each rank's part on block b runs the device function barrier_blockwise of
 * arx_device.h on the library's pads (lane s < W CASes slot (b, v) of rank
 * s's pad from 0 to 1, then slot (b, s) of its own pad from 1 to 0). The
 * pads start zero-filled and are zero-filled again after every barrier, so
 * the launch is hipGraph-capturable with no host reset.
 *   Default launch: W * nblocks workgroups of one wave; workgroup g plays
 *   rank g % W's block g / W, so the W workgroups of a block id are
 *   consecutive and run on different XCDs. They wait on each other, so
 *   W * nblocks must not exceed what the device holds at once (the kernel's
 *   occupancy per CU times the CU count), else ARX_EINVAL. With acq_rel each
 *   round follows the page's usage pattern 1 (workgroup barrier, barrier,
 *   workgroup barrier), with relaxed pattern 0.
 *   flags & ARX_BARRIER_LANES: nblocks workgroups of one wave, lanes
 *   [v*W, v*W + W) of workgroup b playing rank v; every signal precedes
 *   every consume in one instruction stream and no workgroup waits on
 *   another (it measures the atomics and fences alone).
 *   nblocks: 1..ARX_MAX_PAD_BLOCKS.  sem: ARX_SEM_RELAXED or ARX_SEM_ACQ_REL.
 *   rounds: 1..64.  tags, seen: device u32 [W][rounds][nblocks] and
 *   [W][rounds][nblocks][W] for the tag check described above, both NULL
 *   for none; default launch only.
 * Errors: ARX_ESTATE, ARX_EINVAL, ARX_ETIMEOUT (latched), ARX_EHIP.
 */
int arx_barrier_blockwise(int nblocks, int sem, int rounds, int flags, uint32_t* tags, uint32_t* seen,
                          hipStream_t stream);

/*
 * arx_counter_barrier — the counter barrier and per-block epochs of page
 * "common.cuh" (Semaphore, PullController::sync, PushController) for the W
 * virtual ranks on block ids 0..nblocks-1. Each rank's block records its
 * epoch in epochs_seen[v * nblocks + b] (if epochs_seen is not NULL), runs
 * `rounds` rounds of a start stage (every rank adds 1 to block b's flag of
 * every rank, the owner waits) and a fenced end stage (release adds, the
 * owner's wait then an acquire), then flips its epoch between 0 and 1.
 *   Page design (default): one flag per rank and block; the start stage
 *   waits for flag - base >= W, the end stage for >= 2W and then advances
 *   the base by 2W. Flags only grow: after R rounds in total every flag and
 *   base of the blocks used is 2 * W * R. At W >= 3 over two or more rounds
 *   an add from a rank a stage ahead (an unfenced start-stage add) can stand
 *   in for a slow rank's end-stage add, so a rank can leave an end stage
 *   without its acquire pairing with that slow rank's release.
 *   flags & ARX_BARRIER_SPLIT (a repair, not the page's design): start
 *   stages count on the semaphore's flag and base, end stages on its
 *   end-stage pair; each stage waits for W and advances its base by W, so
 *   every end stage pairs with every rank's release. After R rounds both
 *   pairs are W * R.
 *   Launch layouts as for arx_barrier_blockwise (default one workgroup per
 *   rank and block, or ARX_BARRIER_LANES); the tag check writes each tag
 *   between the start and the end stage and reads the peers' after the end
 *   stage.
 *   nblocks: 1..ARX_MAX_PAD_BLOCKS.  rounds: 0..64.  epochs_seen: device u32
 *   [W][nblocks] or NULL.  tags, seen: as for arx_barrier_blockwise.
 * Errors: ARX_ESTATE, ARX_EINVAL, ARX_ETIMEOUT (latched), ARX_EHIP.
 */
int arx_counter_barrier(int nblocks, int rounds, int flags, uint32_t* epochs_seen, uint32_t* tags, uint32_t* seen,
                        hipStream_t stream);

/*
 * arx_symm_allreduce — an all-reduce among the W virtual ranks of this GPU
 * through symmetric buffers, fenced by the blockwise barrier's usage
 * patterns (page "triton_barrier.py", blockwise_barrier docstring): one
 * kernel of W * G workgroups (G per rank: about two 16-byte vectors per
 * thread, at most 64, and all W * G resident at once); at its start
 * pattern 0; then for each of `iters` iterations every rank writes its
 * partial into its own symmetric buffer, passes pattern 1 (acq_rel, which
 * publishes the write to the matching blocks), reads its slice of every
 * rank's buffer, writes the rank-ordered sum (the same reduction as
 * arx_allreduce), and passes pattern 2 (relaxed, so the next iteration's
 * write cannot overwrite a slice a peer still reads).
 *   inputs:  device bf16 [iters][W][ld]; rank v's partial for iteration k
 *            starts at element (k * W + v) * ld.
 *   outputs: device bf16 [iters][W][ld], same layout; every rank's result.
 *   n <= max_n; ld >= n and a multiple of 8; both pointers 16-byte aligned;
 *   iters in [1, 65536]; outputs == inputs (in place) or not overlapping it. Uses the signal pads (block ids 0..G-1) and the
 *   library's symmetric buffers [W][max_n], allocated by arx_init.
 * Errors: ARX_ESTATE, ARX_EINVAL, ARX_ETIMEOUT (latched), ARX_EHIP.
 */
int arx_symm_allreduce(const void* inputs, void* outputs, size_t n, size_t ld, int iters, hipStream_t stream);

/* The largest nblocks the default launch (one workgroup per rank and block)
 * of arx_barrier_blockwise and arx_counter_barrier accepts at this W: what
 * the device holds at once divided by W, at most ARX_MAX_PAD_BLOCKS (0 if the
 * occupancy query failed). The lane-group variant accepts
 * ARX_MAX_PAD_BLOCKS. Errors: ARX_ESTATE. */
int arx_barrier_max_blocks(void);

/*
 * arx_symm_allreduce_noalloc — arx_symm_allreduce for callers that cannot
 * allocate device memory: code under hipGraph capture, tight serving loops,
 * harnesses that forbid allocation. Same kernel, same results, but needs no
 * arx_init and allocates nothing: the W symmetric buffers and the signal
 * pads live in one fixed array in device memory that the library's code
 * object holds on every GPU it is loaded on, until the process ends
 * (ARX_MAX_WORLD x ARX_NOALLOC_MAX_N bf16 plus 16 KiB of pads: about
 * 16 MiB per GPU). Each call first zero-fills the pads it uses (one small
 * kernel; a completed exchange leaves them zero, one that timed out may
 * not), then runs the exchange, both on `stream`.
 *   world: W in [2, 8].  inputs, outputs, ld, iters: as arx_symm_allreduce.
 *   n <= ARX_NOALLOC_MAX_N.  status: device u32, 4-byte aligned, or NULL;
 *   set to 1 if a barrier wait timed out (2 s), when that call's outputs are
 *   incomplete; never cleared by the library.
 * Every call on one GPU uses the same array, which keeps the last call's
 * contents: calls that overlap on one GPU (concurrent streams, threads)
 * race and must be ordered by the caller.
 * Errors (nothing launched): ARX_EINVAL (arguments, n beyond the limit),
 * ARX_EHIP.
 */
int arx_symm_allreduce_noalloc(int world, const void* inputs, void* outputs, size_t n, size_t ld, int iters,
                               uint32_t* status, hipStream_t stream);

/* Device address of rank `rank`'s semaphores: ARX_MAX_PAD_BLOCKS entries of
 * 32 u32 (128 bytes): flag at [0] and base at [1], the split design's
 * end-stage flag at [16] and base at [17]; NULL if not initialised or rank
 * out of range. */
const uint32_t* arx_sem_ptr(int rank);

/* Device address of rank `rank`'s per-block epochs, u32
 * [ARX_MAX_PAD_BLOCKS]; NULL if not initialised or rank out of range. */
const uint32_t* arx_epoch_ptr(int rank);

/* Device address of recv slot [par][src] (max_n bf16), where the caller puts
 * peer src's partial for parity par; NULL if not initialised or out of range
 * (par not in {0,1}, src not in [0, W)). The slot at src == rank is unused. */
void* arx_recv_ptr(int par, int src);

/* Device address of send slot [par] (max_n bf16); NULL as above. */
void* arx_send_ptr(int par);

/* Device address of virtual rank `rank`'s signal pad, u32[ARX_MAX_PAD_BLOCKS][W]
 * (block b, slot s at b * W + s); NULL as above. */
uint32_t* arx_pad_ptr(int rank);

/* Choose when the proxy posts flags (ARX_PROXY_*). Change it only while no
 * call is in flight. */
int arx_set_proxy_mode(int mode);

/*
 * arx_set_stress_source — the data the proxy writes in ARX_PROXY_STRESS
 * mode, standing for peers whose partials arrive with their flags (page
 * "arx.cu", protocol comment: the peer writes recv[seq & 1][rank], then the
 * flag, on one ordered channel). Before posting seq s the proxy copies
 * pool[s % sets][src] into recv[s & 1][src] for every src != rank on a
 * stream of its own, waits for the copies, then posts the flags.
 *   pool: device bf16 [sets][W][max_n], owned by the caller, kept alive and
 *   unchanged while the mode is in use; sets >= 1. NULL / 0 clears it.
 * Refused (ARX_ESTATE) while the stress mode is on; once the mode has been
 * left, the call waits for a copy still in progress, and no copy reads the
 * old source afterwards.
 * Errors: ARX_ESTATE, ARX_EINVAL, ARX_EHIP. A copy failure during the mode
 * latches ARX_EPROXY.
 */
int arx_set_stress_source(const void* pool, int sets);

/* Bound of every device-side wait, in microseconds (default 2000000, i.e.
 * 2 s; 1 us .. 60 s). Applies to calls launched after it. */
int arx_set_timeout_us(uint64_t us);

/* Watchdog view (page "arx.cu": the STALL report of proxy_loop): last seq
 * published by this GPU, last seq posted for the peers, last seq whose
 * reduction finished. Any pointer may be NULL. */
int arx_status(uint64_t* published, uint64_t* posted, uint64_t* done);

/* Message for an error code; for the last failing call, the message includes
 * its detail (a HIP error string, the offending argument). */
const char* arx_strerror(int err);

/* max_n given to arx_init (0 if not initialised); page "arx.cu": arx_max_bytes. */
size_t arx_max_n(void);

/* W and this GPU's rank (0 if not initialised). */
int arx_world(void);
int arx_rank(void);

#ifdef __cplusplus
}
#endif

#endif /* ARX_H */
