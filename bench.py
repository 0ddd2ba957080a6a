"""Benchmark of the one-shot W-way bf16 reduction on one MI355X.

Workload (the headline): W = 8 partials of bf16 [32, 4096] (n = 131072,
256 KiB each), values N(0,1)*0.1, K consecutive one-shot calls on one
stream with parity alternating and the virtual peers' flags posted by the
library's host proxy thread into pinned memory (lockstep). One step = one
call: copy into the send slot, publish, flag wait, go broadcast, W-way
reduction, last-block-out. Inputs are resident in HBM before timing.

value = algorithmic bytes per call / time per call, with the algorithmic
bytes (W + 3) * 2n = 2,883,584 B (copy read + write, W reads, one write).
The same run also measures the reduction alone on W = 8, bf16 [8192, 8192]
(128 MiB per partial), the run-ahead proxy mode, the blockwise barrier, and
the CPU oracle on a bounded sample of the headline workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "one-shot reduce GB/s (% of HBM peak) + µs/call at W=8, 256 KB bf16"


KERNEL_SOURCES = ("arx_reduce.hip", "arx_kernel_util.h", "arx_prims.h", "arx_internal.h")


def kernel_source_hash(csrc=os.path.join(ROOT, "signal_pad_sync_amd", "csrc")):
    """sha256 over the sources of the reduction kernels, in a fixed order."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(key, path=os.path.join(ROOT, "profiles", "hbm_traffic.json"), csrc=None):
    """HBM bytes per launch recorded from the rocprofv3 counter runs
    summarised in profiles/hbm_traffic_pmc.md (FETCH_SIZE scaled by what a
    plain copy of known size reads on it, plus WRITE_SIZE; or, under the
    keys ending in _by_request_size, the read and write request counts by
    size), or None when the kernel sources have changed since those counters
    were taken."""
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    current = kernel_source_hash(csrc) if csrc else kernel_source_hash()
    return rec.get(key) if rec.get("kernel_source_sha256") == current else None


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--reduce-reps", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--only", default="", help="comma list of phases: copy,oneshot,runahead,floor,graph,reduce,barrier,symm; "
                    "copy1g (a 1 GiB copy, for the byte counters) and configs (every workload, oracle "
                    "included) run only when named")
    return ap.parse_args()


# A spin kernel this long (GPU clock cycles, tens of ms) holds the stream
# while the host enqueues the timed launches, so the events time the GPU
# running them back to back, not the host issuing them.
GATE_CYCLES = 200_000_000


def timed(fn, steps, stream, gate=False, warmup=0):
    """Event time of `steps` calls of fn on `stream`, in microseconds, after
    `warmup` untimed calls. With gate, a spin kernel ahead of the warm-up
    calls keeps the GPU busy while the host enqueues every call (for
    launches shorter than the host's enqueue cost); the warm-up calls then
    run on the GPU right before the timed ones, with no idle time between."""
    import torch
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    if gate and hasattr(torch.cuda, "_sleep"):   # without it the timing is merely ungated
        torch.cuda._sleep(GATE_CYCLES)
    for _ in range(warmup):
        fn()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e3  # microseconds


def bench_oneshot(args, mode, graph=False):
    """K one-shot calls at W=8, n=131072; returns microseconds per call."""
    import numpy as np
    import torch
    from signal_pad_sync_amd import arx
    from signal_pad_sync_amd import workloads as WL

    W, n = 8, 131072
    arx.init(W, n)
    try:
        arx.set_proxy_mode(mode)
        for par in (0, 1):
            parts = WL.recv_partials(2, par, n)
            for src in range(1, W):
                arx.recv_view(par, src, n).copy_(torch.from_numpy(parts[src].view(np.int16)).cuda().view(torch.bfloat16))
        x = torch.from_numpy(WL.own_partial(2, 1, n).view(np.int16)).cuda().view(torch.bfloat16)
        out = torch.empty_like(x)
        stream = torch.cuda.current_stream()
        if graph:
            per = 100
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(per):
                    arx.allreduce(x, out, n)
            fn, reps = g.replay, max(1, args.steps // per)
        else:
            # the timed loop calls the C entry point directly with its
            # arguments prepared once, so Python adds as little as possible
            per = 1
            call, xp, op, sh = arx.lib.arx_allreduce, x.data_ptr(), out.data_ptr(), stream.cuda_stream
            rcs = []
            fn, reps = (lambda: rcs.append(call(xp, op, n, sh))), args.steps
        if graph:
            for _ in range(max(1, args.warmup // per)):
                fn()
            us = timed(fn, reps, stream)
        else:
            fn()                       # the first call's one-time host set-up, outside the gate
            torch.cuda.synchronize()
            us = timed(fn, reps, stream, gate=True, warmup=max(1, args.warmup))
        calls = reps * per
        if not graph:
            assert not any(rcs), f"arx_allreduce failed: {set(rcs)}"
        st = arx.debug_state()
        assert st["ctl_err"] == 0 and st["cnt0"] == 0 and st["cnt1"] == 0, st
    finally:
        torch.cuda.synchronize()
        arx.finalize()
    return us / calls, calls


def bench_launch_floor(args):
    """The smallest kernel of the library back to back: the reduction alone
    at W=8 on one vector (n = 8), K launches through the C entry point with
    its arguments prepared once; returns microseconds per launch. It is what
    one dependent launch costs on this stream, the reference for the
    one-shot call's latency."""
    import torch
    from signal_pad_sync_amd import arx

    W, n = 8, 8
    arx.init(W, 1024)
    try:
        x = torch.zeros(n, device="cuda", dtype=torch.bfloat16)
        out = torch.empty_like(x)
        stream = torch.cuda.current_stream()
        call, xp, op, sh = arx.lib.arx_reduce, x.data_ptr(), out.data_ptr(), stream.cuda_stream
        rcs = []
        fn = lambda: rcs.append(call(xp, op, n, 0, sh))
        fn()
        torch.cuda.synchronize()
        us = timed(fn, args.steps, stream, gate=True, warmup=max(1, args.warmup)) / args.steps
        assert not any(rcs), f"arx_reduce failed: {set(rcs)}"
    finally:
        torch.cuda.synchronize()
        arx.finalize()
    return us


def bench_reduce(args):
    """Reduction alone at W=8, n = 8192*8192; returns microseconds per call."""
    import torch
    from signal_pad_sync_amd import arx

    W, n = 8, 8192 * 8192
    arx.init(W, n)
    try:
        g = torch.Generator(device="cuda")
        g.manual_seed(4000)
        for par in (0, 1):
            for src in range(1, W):
                v = arx.recv_view(par, src, n)
                v.copy_(torch.randn(n, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16))
        x = torch.randn(n, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        out = torch.empty_like(x)
        stream = torch.cuda.current_stream()
        k = [0]

        def step():
            arx.reduce(x, out, k[0] & 1, n)
            k[0] += 1

        for _ in range(3):
            step()
        samples = [timed(step, 1, stream) for _ in range(args.reduce_reps)]
        us_total = timed(step, args.reduce_reps, stream)
        # the same launches one by one, each after a read of 512 MiB of
        # other data that sweeps the last-level cache (a read, so it leaves
        # no dirty lines to write back), so no launch can find warm inputs
        sa = torch.ones(256 << 20, device="cuda", dtype=torch.bfloat16)
        scrubbed = []
        for _ in range(args.reduce_reps):
            sa.sum()
            scrubbed.append(timed(step, 1, stream))
        del sa
    finally:
        torch.cuda.synchronize()
        arx.finalize()
    samples.sort()
    scrubbed.sort()
    return samples[len(samples) // 2], us_total / args.reduce_reps, scrubbed[len(scrubbed) // 2]


BARRIER_KINDS = {
    # name: (counter barrier?, sem or flags)
    "pad_acq_rel": (False, 1, 0),
    "pad_relaxed": (False, 0, 0),
    "pad_acq_rel_lanes": (False, 1, 1),
    "pad_relaxed_lanes": (False, 0, 1),
    "counter_page": (True, None, 0),
    "counter_split": (True, None, 2),
    "counter_page_lanes": (True, None, 1),
}


def bench_barrier(args, kind):
    """One barrier round on 256 block ids at W=8, 100 launches per hipGraph;
    returns microseconds per launch. Default launches give every virtual
    rank's block a workgroup of its own (2048 workgroups that wait on each
    other); the _lanes variants put the 8 ranks of a block in one wave (256
    workgroups, none waiting on another). counter_*: one round (start + end
    stage) of the counter barrier, page design or split stages."""
    import torch
    from signal_pad_sync_amd import arx
    counter, sem, flags = BARRIER_KINDS[kind]
    arx.init(8, 1024)
    try:
        stream = torch.cuda.current_stream()
        per = 100
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per):
                if counter:
                    arx.counter_barrier(256, 1, flags)
                else:
                    arx.barrier_blockwise(256, sem, 1, flags)
        for _ in range(3):
            g.replay()
        reps = max(1, args.steps // per)
        us = timed(g.replay, reps, stream)
        for r in range(8):
            assert int(arx.pad_view(r).abs().sum()) == 0
        assert arx.debug_state()["ctl_err"] == 0
    finally:
        torch.cuda.synchronize()
        arx.finalize()
    return us / (reps * per)


def bench_copy(args, mib=64):
    """A plain device-to-device copy of `mib` MiB: the known-size kernel that
    scales the HBM byte counters. At 64 MiB source and destination fit in
    the 256 MB last-level cache (MALL), so its rate is not an HBM ceiling;
    at 1 GiB they do not, and the copy streams through HBM."""
    import torch
    n = mib << 19   # bf16 elements
    if mib <= 64:
        a = torch.randn(n, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    else:
        a = torch.empty(n, device="cuda", dtype=torch.bfloat16).fill_(1.0)
    b = torch.empty_like(a)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        b.copy_(a)
    reps = 20
    us = timed(lambda: b.copy_(a), reps, stream) / reps
    del a, b
    torch.cuda.empty_cache()
    return 2 * n * 2, us


def bench_symm(args):
    """Symmetric-buffer all-reduce among the 8 virtual ranks, n=131072, 100
    iterations in one launch; returns microseconds per iteration."""
    import torch
    from signal_pad_sync_amd import arx
    W, n, iters = 8, 131072, 100
    arx.init(W, n)
    try:
        g = torch.Generator(device="cuda")
        g.manual_seed(5000)
        inp = torch.randn(iters * W * n, generator=g, device="cuda").to(torch.bfloat16).view(iters, W, n)
        out = torch.empty_like(inp)
        stream = torch.cuda.current_stream()
        arx.symm_allreduce(inp, out, n, iters)
        us = timed(lambda: arx.symm_allreduce(inp, out, n, iters), 5, stream) / 5
        assert arx.debug_state()["ctl_err"] == 0
    finally:
        torch.cuda.synchronize()
        arx.finalize()
    return us / iters


def _oracle_times(parts, n, reps=3):
    """Median seconds of the oracle's reduction over n elements, on one
    thread and on every host core this process may use."""
    from oracle import reduce as R
    T = len(os.sched_getaffinity(0))
    out = {}
    for name, threads in (("1", 1), ("T", T)):
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            R.reduce(parts, n=n, threads=threads)
            ts.append(time.perf_counter() - t0)
        out[name] = sorted(ts)[len(ts) // 2]
    return out, T


def bench_configs(args):
    """Every workload once more, as a table: GPU time per call (or per
    launch / graph replay) and the oracle's time on 1 and T host threads."""
    import numpy as np
    import torch
    from signal_pad_sync_amd import arx
    from signal_pad_sync_amd import workloads as WL

    rows = {}
    stream = torch.cuda.current_stream()

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)

    def fill(recv, W, rank=0):
        for par in (0, 1):
            for src in range(W):
                if src != rank:
                    arx.recv_view(par, src, recv[par][src].size).copy_(dev(recv[par][src]))

    # workloads 1, 2 and 5: consecutive eager one-shot calls, lockstep proxy
    for cfg, n_buf in ((1, 8192), (2, 131072), (5, 131072)):
        w = WL.WORKLOADS[cfg]
        W, n = w["W"], w["n"]
        recv = [WL.recv_partials(cfg, par, n) for par in (0, 1)]
        arx.init(W, n_buf)
        try:
            fill(recv, W)
            x = torch.zeros(n_buf, dtype=torch.bfloat16, device="cuda")
            x[:n].copy_(dev(recv[1][0]))
            out = torch.empty_like(x)
            call, xp, op, sh = arx.lib.arx_allreduce, x.data_ptr(), out.data_ptr(), stream.cuda_stream
            for _ in range(20):
                call(xp, op, n, sh)
            us = timed(lambda: call(xp, op, n, sh), args.steps, stream) / args.steps
            assert arx.debug_state()["ctl_err"] == 0
        finally:
            torch.cuda.synchronize()
            arx.finalize()
        cpu, T = _oracle_times(recv[1], n)
        rows[f"workload{cfg}"] = {"W": W, "n": n, "gpu_us_per_call": round(us, 3),
                                  "gpu_GBps": round((W + 3) * 2 * n / us / 1e3, 1),
                                  "oracle_ms_1thread": round(cpu["1"] * 1e3, 3),
                                  "oracle_ms_Tthreads": round(cpu["T"] * 1e3, 3), "T": T}
    # workload 3: one-shot call + 256-workgroup barrier in one hipGraph, per n
    W = 4
    for n in WL.WORKLOADS[3]["ns"]:
        recv = [WL.recv_partials(3, par, n) for par in (0, 1)]
        arx.init(W, n)
        try:
            fill(recv, W)
            x = dev(WL.own_partial(3, 1, n))
            out = torch.empty_like(x)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(10):
                    arx.allreduce(x, out, n)
                    arx.barrier_blockwise(256, arx.SEM_ACQ_REL, 1)
            for _ in range(3):
                g.replay()
            reps = max(1, args.steps // 10)
            us = timed(g.replay, reps, stream) / (reps * 10)
            assert arx.debug_state()["ctl_err"] == 0
        finally:
            torch.cuda.synchronize()
            arx.finalize()
        cpu, T = _oracle_times(recv[1], n)
        rows[f"workload3_n{n}"] = {"W": W, "n": n, "gpu_us_per_call_and_barrier": round(us, 3),
                                   "oracle_ms_1thread": round(cpu["1"] * 1e3, 4),
                                   "oracle_ms_Tthreads": round(cpu["T"] * 1e3, 4), "T": T}
    # workload 4: the oracle on the full size (the GPU figure is the reduce phase)
    n = 8192 * 8192
    parts = WL.recv_partials(4, 0, n)
    cpu, T = _oracle_times(parts, n, reps=1)
    rows["workload4"] = {"W": 8, "n": n, "oracle_ms_1thread": round(cpu["1"] * 1e3, 1),
                         "oracle_ms_Tthreads": round(cpu["T"] * 1e3, 1), "T": T,
                         "oracle_GBps_Tthreads": round(9 * 2 * n / cpu["T"] / 1e9, 2)}
    return rows


def cpu_baseline(seconds, threads=1):
    """The oracle's one-shot model (sequential protocol + C reduction, the
    reduction on `threads` host threads) on the headline workload, for
    about `seconds` of wall time; returns (calls, seconds)."""
    from oracle import protocol as P
    from signal_pad_sync_amd import workloads as WL

    W, n = 8, 131072
    recv = [WL.recv_partials(2, par, n) for par in (0, 1)]
    x = WL.own_partial(2, 1, n)
    t0 = time.perf_counter()
    P.sequential_model([(x, n)] * 10, recv, W, threads=threads)
    per = (time.perf_counter() - t0) / 10
    calls = max(10, int(seconds / per))
    t0 = time.perf_counter()
    P.sequential_model([(x, n)] * calls, recv, W, threads=threads)
    dt = time.perf_counter() - t0
    return calls, dt


def cpu_leg(seconds):
    """cpu_baseline of the JSON line: the oracle on every host core this
    process may use (T threads, stated), with the one-core figure beside it."""
    W, n = 8, 131072
    bytes_call = (W + 3) * 2 * n
    T = len(os.sched_getaffinity(0))
    out = None
    for threads in (T, 1):
        calls, dt = cpu_baseline(seconds / 2, threads)
        leg = {"value": round(bytes_call * calls / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "sample": f"{calls} one-shot calls of the headline workload (W=8, n=131072): the sequential protocol "
                         f"model with the C reduction on {threads} thread(s), contiguous index ranges",
               "us_per_call": round(dt / calls * 1e6, 1)}
        log(f"  {leg['us_per_call']} us/call on {threads} thread(s)")
        if out is None:
            out = leg
        else:
            out["one_core"] = leg
    return out


def make_line(args, us_call, cpu, extra):
    """The one JSON line: the headline workload's throughput, its roofline
    and the CPU oracle's rate."""
    W, n = 8, 131072
    bytes_call = (W + 3) * 2 * n
    value = bytes_call / us_call / 1e3 if us_call else None
    # launches run back to back, so the event time of the timed region over
    # the number of launches is the kernel's average launch duration
    achieved = value
    return {
        "metric": METRIC, "value": round(value, 2) if value else None, "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us_call / 1e3, 6) if us_call else None,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "one-shot reduce, W=8, bf16 [32,4096] per partial (n=131072), consecutive calls, "
                               "parity alternating, lockstep host-proxy flags in pinned memory",
                   "W": W, "n": n, "io_dtype": "bf16", "accumulate": "f32"},
        "us_per_call": round(us_call, 3) if us_call else None,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2) if achieved else None, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 5) if achieved else None,
                     "traffic": recorded_traffic("oneshot_kernel_w8_n131072_bytes"),
                     "traffic_by_request_size": recorded_traffic("oneshot_kernel_w8_n131072_bytes_by_request_size"),
                     "kernel": "oneshot_kernel<8,true,512>", "bytes_per_launch": bytes_call,
                     "event_us_per_launch": round(us_call, 3) if us_call else None},
        "cpu_baseline": cpu,
        "extra": extra,
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the one-shot reduction; the virtual peers live on the "
              "same GPU, so --gpus must be 1 (there is no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch
    from signal_pad_sync_amd import arx

    torch.cuda.set_device(0)
    only = set(filter(None, args.only.split(",")))
    want = lambda p: not only or p in only
    W, n = 8, 131072
    bytes_call = (W + 3) * 2 * n
    extra = {}

    us_call = None
    if want("copy"):
        log("plain device copy, 64 MiB")
        cb, cus = bench_copy(args)
        extra["copy_64MiB"] = {"bytes_per_call": cb, "us": round(cus, 2), "GBps": round(cb / cus / 1e3, 1)}
        log(f"  {cus:.1f} us, {cb / cus / 1e3:.0f} GB/s (read + write)")
    if only and "copy1g" in only:
        log("plain device copy, 1 GiB (beyond the last-level cache)")
        cb, cus = bench_copy(args, 1024)
        extra["copy_1GiB"] = {"bytes_per_call": cb, "us": round(cus, 2), "GBps": round(cb / cus / 1e3, 1)}
        log(f"  {cus:.1f} us, {cb / cus / 1e3:.0f} GB/s (read + write)")
    if want("oneshot"):
        log("one-shot, lockstep proxy")
        us_call, calls = bench_oneshot(args, arx.PROXY_LOCKSTEP)
        log(f"  {us_call:.2f} us/call over {calls} calls")
    if want("runahead"):
        log("one-shot, run-ahead proxy")
        us_ra, _ = bench_oneshot(args, arx.PROXY_RUNAHEAD)
        extra["runahead_us_per_call"] = round(us_ra, 3)
        log(f"  {us_ra:.2f} us/call")
    if want("floor"):
        log("launch floor: the reduction alone on one vector, back to back")
        extra["launch_floor_us"] = round(bench_launch_floor(args), 3)
        log(f"  {extra['launch_floor_us']:.2f} us/launch")
    if want("graph"):
        log("one-shot, lockstep proxy, 100 calls per hipGraph")
        us_g, _ = bench_oneshot(args, arx.PROXY_LOCKSTEP, graph=True)
        extra["graph_us_per_call"] = round(us_g, 3)
        log(f"  {us_g:.2f} us/call")
    if want("reduce"):
        log("reduction alone, W=8, bf16 [8192, 8192]")
        med, mean, med_scrub = bench_reduce(args)
        rb = (8 + 1) * 2 * 8192 * 8192
        extra["reduce_128MiB"] = {
            "workload": "W=8, bf16 [8192,8192] per partial, reduction alone",
            "bytes_per_call": rb, "us_median_single": round(med, 2),
            "us_median_single_after_cache_sweep": round(med_scrub, 2), "us_mean_back_to_back": round(mean, 2),
            "GBps": round(rb / mean / 1e3, 1), "frac_of_hbm_peak": round(rb / mean / 1e3 / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic("reduce_kernel_w8_n67108864_bytes"),
            "traffic_by_request_size": recorded_traffic("reduce_kernel_w8_n67108864_bytes_by_request_size")}
        log(f"  {mean:.1f} us per launch back to back ({med:.1f} us median timed one by one), "
            f"{rb / mean / 1e3:.0f} GB/s")
    if want("barrier"):
        for kind in BARRIER_KINDS:
            log(f"barrier {kind}, 256 block ids, W=8, 100 launches per hipGraph")
            us_b = bench_barrier(args, kind)
            extra[f"barrier_w8_256blk_{kind}_us"] = round(us_b, 3)
            log(f"  {us_b:.3f} us/launch")

    if args.only and "configs" in only:
        log("every workload: GPU time and oracle time on 1 and T threads")
        extra["configs"] = bench_configs(args)
        for k, v in extra["configs"].items():
            log(f"  {k}: {v}")
    if want("symm"):
        log("symmetric-buffer all-reduce among 8 virtual ranks, n=131072, 100 iterations per launch")
        us_s = bench_symm(args)
        extra["symm_w8_n131072_us_per_iteration"] = round(us_s, 3)
        log(f"  {us_s:.2f} us per iteration")

    cpu = None
    if not args.skip_cpu:
        log(f"oracle on the CPU, ~{args.cpu_seconds} s")
        cpu = cpu_leg(args.cpu_seconds)

    line = make_line(args, us_call, cpu, extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
