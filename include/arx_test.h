/*
 * arx_test.h — test aids of libarx, exported beside the C ABI of arx.h but
 * not part of the one-shot path: they read or set the protocol's state,
 * force a proxy failure, and run the reduction's rounding alone, so that
 * tests can check every protocol word, reach sequence numbers past 2^32,
 * exercise the failure latch and compare the rounding exhaustively.
 * Conventions (return codes, pointers, one instance per process) as in
 * arx.h.
 */
#ifndef ARX_TEST_H
#define ARX_TEST_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * arx_debug_state — copy every protocol word, synchronously (waits for the
 * device), into words[0..nwords): [0] seq_dev, [1] arrival counter,
 * [2] finish counter, [3] go, [4] abort, [5] ctl.seq, [6] ctl.bytes[0],
 * [7] ctl.bytes[1], [8] ctl.done, [9] ctl.err, [10] ctl.err_seq,
 * [11] posted, [12 .. 12+W) flags[src]. seq_dev, ctl.seq, ctl.done, posted
 * and the flags are 64-bit sequence numbers. [3] and [4] are read from the
 * device's go word, which holds the seq of the last call that passed its
 * flag wait and whether that call was aborted: [3] is the low 32 bits of
 * that seq, [4] the seq if the call was aborted (its flag wait timed out and
 * it summed nothing), else 0. Returns the number of words written.
 */
int arx_debug_state(uint64_t* words, int nwords);

/* Test aid: set the protocol's state as if `seq` calls had completed
 * (the device's seq, go and published words, ctl.seq, ctl.done, the proxy's
 * posted seq and every peer flag), so tests can reach large sequence
 * numbers. Waits for the device; allowed in the lockstep and manual modes
 * only, with no call in flight. Errors: ARX_ESTATE, ARX_EHIP. */
int arx_debug_set_seq(uint64_t seq);

/* Test aid: the proxy's next post in ARX_PROXY_STRESS mode fails, as a
 * failed copy of the peers' data would. The proxy thread then stops and the
 * failure is latched: the next arx_allreduce (or any call that launches)
 * returns ARX_EPROXY until arx_finalize, as the page's proxy error latch
 * makes the next all-reduce throw. A call already in flight never gets its
 * flags and ends through its bounded wait. Errors: ARX_ESTATE. */
int arx_debug_fail_proxy(void);

/* The binary32 -> bf16 rounding of the reduction alone (for exhaustive
 * checks): out[i] = the bf16 pattern the reduction writes for the binary32
 * pattern in[i]. in: device u32 [n], out: device u16 [n]; n <= 2^32 - 1. */
int arx_test_round_bf16(const void* in, void* out, size_t n, hipStream_t stream);

/* The launch shape arx_allreduce uses for n elements at `world` partials
 * (host-side rules only; no device is touched): out[0] threads per
 * workgroup (block = 0: the library's choice for n and world, else 256,
 * 512 or 1024), out[1] reducing
 * workgroups, out[2] workgroups launched (out[1], plus the workgroup that
 * waits for the flags), out[3] reducing workgroups that copy
 * the partial and count arrival, out[4] 1 if every vector has a thread of
 * its own, out[5] 1 if go may come before this rank's publish, out[6] 1 if
 * the copy's stores are nontemporal (else write-through), out[7] 1 if the
 * sum's peer loads are nontemporal (else system-coherent). resident:
 * workgroups the device holds at once (the library caps it at 257, the
 * most its grids use); in_place: out == in. Errors: ARX_EINVAL (n above
 * ARX_MAX_N, world outside [2, 8], another block, resident below 2, out
 * NULL or nout < 8). */
int arx_test_oneshot_shape(size_t n, int world, int block, unsigned resident, int in_place, int* out, int nout);

#ifdef __cplusplus
}
#endif

#endif /* ARX_TEST_H */
