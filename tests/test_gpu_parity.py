"""GPU parity: the HIP path through the C ABI against the oracle, bit-exact.

Every output element is compared with the oracle's (0 ulp, NaN patterns
included), elements past n are checked untouched, and every protocol word is
read back and compared with the oracle's sequential protocol model.
"""
import time

import numpy as np
import pytest
import torch

from oracle import protocol as P
from oracle import reduce as R
from signal_pad_sync_amd import arx
from signal_pad_sync_amd import workloads as WL
from tests.gpu_util import fill_recv, library, note, sentinel, to_dev, to_host

pytestmark = pytest.mark.gpu


def assert_bits(got, want, what):
    if not np.array_equal(got, want):
        bad = np.flatnonzero(got != want)
        i = int(bad[0])
        raise AssertionError(f"{what}: {bad.size} elements differ, first at {i}: "
                             f"got {hex(int(got[i]))} want {hex(int(want[i]))}")


def check_state(st: P.ProtocolState, rank: int, wait_posted: int = None):
    """Compares every protocol word with the model's prediction."""
    if wait_posted is not None:       # the proxy posts asynchronously in run-ahead mode
        t0 = time.time()
        while arx.status()[1] < wait_posted and time.time() - t0 < 5:
            time.sleep(0.001)
    d = arx.debug_state()
    assert d["ctl_err"] == 0, d
    assert d["cnt0"] == 0 and d["cnt1"] == 0, d
    assert d["seq_dev"] == st.seq_dev and d["go"] == st.go, d
    assert d["ctl_seq"] == st.ctl_seq and d["ctl_done"] == st.ctl_done, d
    assert [d["ctl_bytes0"], d["ctl_bytes1"]] == st.ctl_bytes, d
    assert d["posted"] == st.posted, d
    assert d["flags"] == st.flags, (d["flags"], st.flags)


def test_round_bf16_exhaustive():
    """The device rounding equals the oracle's on all 2^32 binary32 patterns."""
    chunk = 1 << 26
    base = torch.arange(chunk, dtype=torch.int32, device="cuda")
    out = torch.empty(chunk, dtype=torch.int16, device="cuda")
    for k in range((1 << 32) // chunk):
        start = k * chunk
        if k % 16 == 0:
            note(f"round_bf16 chunk {k}")
        inp = base + (start if start < (1 << 31) else start - (1 << 32))
        arx.test_round_bf16(inp, out)
        got = out.cpu().numpy().view(np.uint16)
        want = R.round_bf16(np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32))
        assert_bits(got, want, f"rounding chunk at {hex(start)}")


def test_workload1_single_call():
    """W=2, [2, 4096], N(0,1); one call, seq 1, parity 1."""
    W, n = 2, 8192
    recv = [WL.recv_partials(1, par, n) for par in (0, 1)]
    x = recv[1][0]
    with library(W, n):
        fill_recv(recv, 0)
        inp, out = to_dev(x), sentinel(n + 64)
        note("workload 1 allreduce")
        arx.allreduce(inp, out, n)
        torch.cuda.synchronize()
        got = to_host(out)
        st, outs = P.sequential_model([(x, n)], recv, W)
        assert_bits(got[:n], outs[0], "workload 1")
        assert np.all(got[n:] == 0xDEAD)
        check_state(st, 0)
        assert_bits(to_host(arx.send_view(1, n)), x, "send slot 1")


@pytest.mark.parametrize("mode,K", [(arx.PROXY_LOCKSTEP, 1000), (arx.PROXY_RUNAHEAD, 300)])
def test_workload2_consecutive_calls(mode, K):
    """W=8, [32, 4096], N(0,1)*0.1; K consecutive calls with a fresh partial
    each, parity alternating, flags posted by the proxy thread."""
    W, n = 8, 131072
    recv = [WL.recv_partials(2, par, n) for par in (0, 1)]
    ins = np.stack([WL.own_partial(2, k, n) for k in range(1, K + 1)])
    with library(W, n, mode=mode):
        fill_recv(recv, 0)
        din = to_dev(ins.reshape(-1)).view(K, n)
        dout = torch.empty_like(din)
        note(f"workload 2: {K} calls, mode {mode}")
        for k in range(K):
            arx.allreduce(din[k], dout[k], n)
        torch.cuda.synchronize()
        got = to_host(dout).reshape(K, n)
        st, outs = P.sequential_model([(ins[k], n) for k in range(K)], recv, W,
                                      mode=P.RUNAHEAD if mode == arx.PROXY_RUNAHEAD else P.LOCKSTEP)
        for k in range(K):
            assert_bits(got[k], outs[k], f"workload 2 call {k + 1}")
        check_state(st, 0, wait_posted=st.posted)
        assert_bits(to_host(arx.send_view(K & 1, n)), ins[K - 1], "send slot of the last call")
        assert_bits(to_host(arx.send_view((K - 1) & 1, n)), ins[K - 2], "send slot of the call before")


@pytest.mark.parametrize("n", WL.WORKLOADS[3]["ns"])
def test_workload3_graph_with_barrier(n):
    """W=4, uniform[-1,1]; the one-shot call and the blockwise barrier on 256
    block ids (one workgroup per virtual rank and block: 1024 workgroups that
    wait on each other, acq_rel, with the tag check) captured in one hipGraph,
    replayed with eager calls between the replays; every replay matches the
    oracle, reads every peer's tag and leaves every pad zero."""
    W, nblocks = 4, 256
    recv = [WL.recv_partials(3, par, n) for par in (0, 1)]
    x = WL.own_partial(3, 1, n)
    y = WL.own_partial(3, 2, n)
    want_tags = P.barrier_tags_written(W, nblocks, 1)
    want_seen = P.barrier_tags_seen(W, nblocks, 1)
    with library(W, n):
        fill_recv(recv, 0)
        inp, out = to_dev(x), sentinel(n + 16)
        inp2, out2 = to_dev(y), sentinel(n + 16)
        tags = torch.zeros(W * nblocks, dtype=torch.int32, device="cuda")
        seen = torch.zeros(W * nblocks * W, dtype=torch.int32, device="cuda")
        g = torch.cuda.CUDAGraph()
        note(f"workload 3 n={n}: capture")
        with torch.cuda.graph(g):
            arx.allreduce(inp, out, n)
            arx.barrier_blockwise(nblocks, arx.SEM_ACQ_REL, 1, 0, tags, seen)
        st = None
        for rep in range(6):
            tags.zero_()
            seen.zero_()
            note(f"workload 3 n={n}: replay {rep}")
            g.replay()
            torch.cuda.synchronize()
            st, outs = P.sequential_model([(x, n)], recv, W, state=st)
            got = to_host(out)
            assert_bits(got[:n], outs[0], f"replay {rep}")
            assert np.all(got[n:] == 0xDEAD)
            for r in range(W):
                assert int(arx.pad_view(r).abs().sum()) == 0, f"pad {r} not zero after replay {rep}"
            assert np.array_equal(tags.cpu().numpy().view(np.uint32).reshape(W, 1, nblocks), want_tags)
            assert np.array_equal(seen.cpu().numpy().view(np.uint32).reshape(W, 1, nblocks, W), want_seen), \
                f"tags seen after replay {rep}"
            check_state(st, 0)
            if rep in (1, 2):             # eager work between replays
                arx.allreduce(inp2, out2, n)
                torch.cuda.synchronize()
                st, outs = P.sequential_model([(y, n)], recv, W, state=st)
                assert_bits(to_host(out2)[:n], outs[0], f"eager call after replay {rep}")


def test_workload4_reduce_full_size():
    """W=8, [8192, 8192] (128 MiB per partial), N(0,1); reduction alone."""
    W, n = 8, 8192 * 8192
    note("workload 4: generating inputs")
    parts = WL.recv_partials(4, 0, n)
    with library(W, n):
        fill_recv([parts, None], 0)
        inp = to_dev(parts[0])
        out = torch.empty_like(inp)
        note("workload 4: reduce")
        arx.reduce(inp, out, 0, n)
        torch.cuda.synchronize()
        got = to_host(out)
        assert_bits(got, R.reduce(parts, threads=16), "workload 4")


def test_workload5_adversarial():
    """W=8, [32, 4096] buffers, n = 131071, adversarial values: one-shot call
    and the reduction alone, both bit-exact, out[131071] untouched."""
    W, n, buf = 8, 131071, 131072
    recv = [WL.recv_partials(5, par, n) for par in (0, 1)]
    x = recv[1][0]
    with library(W, buf):
        fill_recv(recv, 0)
        inp, out = to_dev(x, pad_to=buf), sentinel(buf)
        note("workload 5 allreduce")
        arx.allreduce(inp, out, n)
        torch.cuda.synchronize()
        st, outs = P.sequential_model([(x, n)], recv, W, max_n=buf)
        got = to_host(out)
        assert_bits(got[:n], outs[0], "workload 5 one-shot")
        assert got[n] == 0xDEAD
        check_state(st, 0)
        out2 = sentinel(buf)
        note("workload 5 reduce")
        arx.reduce(inp, out2, 0, n)
        torch.cuda.synchronize()
        got2 = to_host(out2)
        assert_bits(got2[:n], R.reduce([x] + recv[0][1:], n=n), "workload 5 reduce only")
        assert got2[n] == 0xDEAD


@pytest.mark.parametrize("W,rank", [(3, 1), (5, 4), (6, 5), (7, 0), (8, 3)])
def test_sizes_tails_and_rank(W, rank):
    """Any n (tails of 1..7, partial workgroups, n = 0), this GPU at rank r,
    one call after another; includes n past one pass of the co-resident grid."""
    max_n = (1 << 20) + 64
    sizes = [0, 1, 7, 8, 9, 15, 17, 255, 256, 257, 1000, 2047, 2049, 65539, 524288, 524289, 1 << 20]
    rng = np.random.default_rng(7 + W)
    recv = [[WL.uniform(9000 + 10 * par + s, max_n) for s in range(W)] for par in (0, 1)]
    with library(W, max_n, rank=rank):
        fill_recv(recv, rank)
        st = None
        for n in sizes:
            x = WL.uniform(int(rng.integers(1 << 30)), max(n, 1))[:n]
            inp, out = to_dev(x, pad_to=max_n), sentinel(max_n)
            note(f"W={W} rank={rank} n={n}")
            arx.allreduce(inp, out, n)
            torch.cuda.synchronize()
            st, outs = P.sequential_model([(x, n)], recv, W, rank=rank, max_n=max_n, state=st)
            got = to_host(out)
            assert_bits(got[:n], outs[0], f"W={W} rank={rank} n={n}")
            assert np.all(got[n:] == 0xDEAD), n
        check_state(st, rank)


def test_reduce_only_empty():
    """The reduction alone at n = 0 launches nothing and writes nothing."""
    with library(3, 1024):
        inp, out = to_dev(np.ones(16, np.uint16)), sentinel(16)
        note("reduce n=0")
        arx.reduce(inp, out, 1, 0)
        torch.cuda.synchronize()
        assert np.all(to_host(out) == 0xDEAD)
        assert arx.debug_state()["seq_dev"] == 0


def test_grid_stride_path():
    """n beyond one vector per thread of the largest co-resident grid
    (256 reducing workgroups x 1024 threads x 8 elements = 2 Mi), so each
    thread loops over several vectors; ragged tail included."""
    W, rank = 3, 2
    max_n = (1 << 22) + 64
    recv = [[WL.normal(7000 + 10 * par + s, max_n) for s in range(W)] for par in (0, 1)]
    with library(W, max_n, rank=rank):
        fill_recv(recv, rank)
        st = None
        for n in ((1 << 21) + 8, (1 << 22) + 5):
            x = WL.normal(7100 + n, n)
            inp, out = to_dev(x, pad_to=max_n), sentinel(max_n)
            note(f"grid-stride W={W} n={n}")
            arx.allreduce(inp, out, n)
            torch.cuda.synchronize()
            st, outs = P.sequential_model([(x, n)], recv, W, rank=rank, max_n=max_n, state=st)
            got = to_host(out)
            assert_bits(got[:n], outs[0], f"grid-stride n={n}")
            assert np.all(got[n:] == 0xDEAD)
        check_state(st, rank)


@pytest.mark.parametrize("mode", [arx.PROXY_LOCKSTEP, arx.PROXY_RUNAHEAD])
@pytest.mark.parametrize("n", [100003, 131072, (1 << 20) + 7])
def test_in_place(mode, n):
    """in and out may be the same buffer, at grids with and without the
    copy split, also in run-ahead mode (go may then come before this rank's
    publish): every output is the oracle's, and the send slot of each call
    holds that call's input, not its output."""
    W, K = 4, 4
    recv = [WL.recv_partials(3, par, n, W) for par in (0, 1)]
    xs = [WL.own_partial(3, 7 + k, n) for k in range(K)]
    with library(W, n + 5, mode=mode):
        fill_recv(recv, 0)
        st = None
        for k in range(K):
            buf = to_dev(xs[k], pad_to=n + 5)
            note(f"in-place allreduce n={n} mode={mode} call {k + 1}")
            arx.allreduce(buf, buf, n)
            torch.cuda.synchronize()
            st, outs = P.sequential_model([(xs[k], n)], recv, W, max_n=n + 5, state=st,
                                          mode=P.RUNAHEAD if mode == arx.PROXY_RUNAHEAD else P.LOCKSTEP)
            assert_bits(to_host(buf)[:n], outs[0], f"in place, call {k + 1}")
            assert_bits(to_host(arx.send_view((k + 1) & 1, n)), xs[k], f"send slot of call {k + 1}")


@pytest.mark.parametrize("W,n", [(2, 196608), (2, 196616), (4, 262144), (5, 262144), (5, 196616)])
def test_block_size_by_world(W, n):
    """The block size depends on W past 48 workgroups of 512 threads: at
    W <= 4, 1024 threads from n = 196616 on (25 to 32 workgroups, all
    copying), at W >= 5 still 512 (49 to 64 workgroups, half copying from
    64 on). Three calls each, rank 1, alternating parity, against the oracle,
    with the send slot and every protocol word checked."""
    K, rank = 3, 1
    want_block = 1024 if (W <= 4 and (n >> 3) > 512 * 48) else 512
    assert arx.test_oneshot_shape(n, W)["block"] == want_block
    recv = [WL.recv_partials(4, par, n, W) for par in (0, 1)]
    xs = [WL.own_partial(4, 21 + k, n) for k in range(K)]
    with library(W, n, rank=rank):
        fill_recv(recv, rank)
        st = None
        out = sentinel(n)
        for k in range(K):
            note(f"block by world, W={W} n={n} block={want_block} call {k + 1}")
            arx.allreduce(to_dev(xs[k]), out, n)
            torch.cuda.synchronize()
            st, outs = P.sequential_model([(xs[k], n)], recv, W, rank=rank, max_n=n, state=st)
            assert_bits(to_host(out), outs[0], f"W={W} n={n}, call {k + 1}")
            assert_bits(to_host(arx.send_view((k + 1) & 1, n)), xs[k], f"send slot of call {k + 1}")
        check_state(st, rank)


@pytest.mark.parametrize("mode", [arx.PROXY_LOCKSTEP, arx.PROXY_RUNAHEAD])
def test_go_after_publish_past_4_vectors(mode):
    """n = 8 Mi + 3 at W = 4 with in and out apart: 256 reducing workgroups
    of 1024 threads, 128 of them copying, 8 vectors per copying thread, so
    the poll workgroup holds go until this rank's publish even when the
    peers' flags are already there (run-ahead). Every output is the
    oracle's, the send slot holds each call's input, and every protocol
    word is the model's."""
    W, K, n = 4, 3, (1 << 23) + 3
    recv = [WL.recv_partials(3, par, n, W) for par in (0, 1)]
    xs = [WL.own_partial(3, 11 + k, n) for k in range(K)]
    pmode = P.RUNAHEAD if mode == arx.PROXY_RUNAHEAD else P.LOCKSTEP
    with library(W, n + 5, mode=mode):
        fill_recv(recv, 0)
        st = None
        out = sentinel(n + 5)
        for k in range(K):
            inp = to_dev(xs[k], pad_to=n + 5)
            note(f"go after publish, n={n} mode={mode} call {k + 1}")
            arx.allreduce(inp, out, n)
            torch.cuda.synchronize()
            st, outs = P.sequential_model([(xs[k], n)], recv, W, max_n=n + 5, state=st, mode=pmode)
            got = to_host(out)
            assert_bits(got[:n], outs[0], f"n={n}, call {k + 1}")
            assert np.all(got[n:] == 0xDEAD)
            assert_bits(to_host(arx.send_view((k + 1) & 1, n)), xs[k], f"send slot of call {k + 1}")
        check_state(st, 0, wait_posted=st.posted)


@pytest.mark.parametrize("n", [1000, 131072])
def test_manual_publish_and_order(n):
    """Manual mode: the kernel waits until the caller publishes; a publish
    out of order is refused and writes nothing. The poll workgroup has read
    the flags once, seen this rank's publish and is polling again when the
    caller publishes, 5 ms later; one reducing workgroup and a tail at
    n = 1000, 32 at n = 131072."""
    W = 4
    recv = [WL.recv_partials(3, par, n, W) for par in (0, 1)]
    x = WL.own_partial(3, 9, n)
    with library(W, n, mode=arx.PROXY_MANUAL):
        fill_recv(recv, 0)
        inp, out = to_dev(x), sentinel(n)
        note(f"manual publish n={n}")
        arx.allreduce(inp, out, n)
        with pytest.raises(arx.ArxError) as e:
            arx.publish(2)
        assert e.value.code == arx.EORDER
        time.sleep(0.005)
        assert arx.status()[0] == 1             # this rank has published seq 1
        arx.publish(1)
        torch.cuda.synchronize()
        st, outs = P.sequential_model([(x, n)], recv, W, mode=P.MANUAL,
                                      state=P.ProtocolState(W=W, rank=0, flags=[0, 1, 1, 1], posted=1))
        assert_bits(to_host(out), outs[0], "manual")
        check_state(st, 0)


@pytest.mark.parametrize("W,n", [(2, 4096), (8, 131072), (4, 4194305)])
def test_flag_timeout_is_latched(W, n):
    """No flag ever comes (manual mode, never published): the bounded wait
    runs out, the output stays untouched, counters still reset, seq advances,
    and the next call reports the timeout. Two reducing workgroups
    (n = 4096), 32 all copying, and a grid-stride grid with half of them
    copying: the reducing workgroups learn of the abort from the go
    word."""
    with library(W, n, mode=arx.PROXY_MANUAL, timeout_us=20000):
        inp, out = to_dev(np.ones(n, np.uint16)), sentinel(n)
        note(f"forced flag timeout (20 ms), W={W} n={n}")
        arx.allreduce(inp, out, n)
        torch.cuda.synchronize()
        assert np.all(to_host(out) == 0xDEAD)
        d = arx.debug_state()
        assert d["ctl_err"] == 1 and d["ctl_err_seq"] == 1 and d["abort"] == 1
        assert d["cnt0"] == 0 and d["cnt1"] == 0 and d["seq_dev"] == 1 and d["ctl_done"] == 1
        with pytest.raises(arx.ArxError) as e:
            arx.allreduce(inp, out, n)
        assert e.value.code == arx.ETIMEOUT


def test_argument_errors():
    """Bad arguments are refused before anything is launched, among them an
    in / out (or inputs / outputs) overlap other than the same buffer: a
    thread's output store could otherwise overwrite a vector another thread
    has not yet read."""
    with library(2, 1024):
        t = torch.zeros(2048, dtype=torch.bfloat16, device="cuda")
        sym = torch.zeros(2 * 2 * 64 + 8, dtype=torch.bfloat16, device="cuda")
        for call in (lambda: arx.allreduce(t, t, 1025), lambda: arx.allreduce(t[1:], t, 8),
                     lambda: arx.reduce(t, t, 2, 8), lambda: arx.barrier_blockwise(1025),
                     lambda: arx.barrier_blockwise(4, 7), lambda: arx.set_proxy_mode(5),
                     lambda: arx.set_timeout_us(0),
                     lambda: arx.allreduce(t[8:], t, 64), lambda: arx.allreduce(t, t[8:], 64),
                     lambda: arx.allreduce(t[:1024], t[8:], 9),
                     lambda: arx.reduce(t[8:], t, 0, 64), lambda: arx.reduce(t, t[1000:], 1, 1001),
                     lambda: arx.symm_allreduce(sym[8:].view(2, 2, 64), sym[:256].view(2, 2, 64), 64, 2)):
            with pytest.raises(arx.ArxError) as e:
                call()
            assert e.value.code == arx.EINVAL
        with pytest.raises(arx.ArxError) as e:
            arx.init(2, 16)
        assert e.value.code == arx.ESTATE
        # edges that touch but do not overlap, and exact aliasing, are accepted
        arx.allreduce(t[:64], t[64:128], 64)
        arx.reduce(t[:64], t[:64], 0, 64)
        arx.symm_allreduce(sym[:256].view(2, 2, 64), sym[:256].view(2, 2, 64), 64, 2)
        torch.cuda.synchronize()
        d = arx.debug_state()
        assert d["seq_dev"] == 1 and d["ctl_err"] == 0, d        # only the accepted one-shot ran


def test_binding_checks_tensor_extents():
    """The binding passes only addresses to the library, so it checks that
    every tensor is a contiguous GPU tensor of the right element size that
    holds the elements the call touches, before anything is launched."""
    with library(2, 1024):
        t = torch.zeros(2048, dtype=torch.bfloat16, device="cuda")
        short = torch.zeros(100, dtype=torch.bfloat16, device="cuda")
        f32 = torch.zeros(2048, dtype=torch.float32, device="cuda")
        host = torch.zeros(2048, dtype=torch.bfloat16)
        symm_in = torch.zeros(2, 2, 512, dtype=torch.bfloat16, device="cuda")
        for call in (lambda: arx.allreduce(t, short, 200), lambda: arx.allreduce(short, t, 101),
                     lambda: arx.allreduce(f32, t, 8), lambda: arx.allreduce(host, t, 8),
                     lambda: arx.allreduce(t[::2], t, 8), lambda: arx.reduce(t, short, 0, 200),
                     lambda: arx.counter_barrier(8, 1, 0, torch.zeros(4, dtype=torch.int32, device="cuda")),
                     lambda: arx.symm_allreduce(symm_in, symm_in, 512, 3),
                     lambda: arx.recv_view(0, 1, 1025), lambda: arx.send_view(1, 0)):
            with pytest.raises(arx.ArxError) as e:
                call()
            assert e.value.code == arx.EINVAL
        torch.cuda.synchronize()
        d = arx.debug_state()
        assert d["seq_dev"] == 0 and d["ctl_err"] == 0, d        # nothing was launched


@pytest.mark.parametrize("W", [2, 3, 4, 5, 6, 7])
def test_reduce_only_every_world(W):
    """The reduction alone at every W below 8, with this GPU at the last rank
    and ragged tails, both parities."""
    rank = W - 1
    max_n = 300007
    recv = [[WL.uniform(15000 + 10 * par + s, max_n) for s in range(W)] for par in (0, 1)]
    with library(W, max_n, rank=rank):
        fill_recv(recv, rank)
        for n in (1, 9, 2048 + 3, 300007):
            for par in (0, 1):
                x = WL.uniform(16000 + n + par, n)
                inp, out = to_dev(x, pad_to=max_n + 1), sentinel(max_n + 1)
                note(f"reduce-only W={W} n={n} par={par}")
                arx.reduce(inp, out, par, n)
                torch.cuda.synchronize()
                parts = [x if s == rank else recv[par][s] for s in range(W)]
                got = to_host(out)
                assert_bits(got[:n], R.reduce(parts, n=n), f"reduce-only W={W} n={n} par={par}")
                assert np.all(got[n:] == 0xDEAD)


@pytest.mark.parametrize("mode", [arx.PROXY_LOCKSTEP, arx.PROXY_RUNAHEAD])
def test_seq_crosses_32_bits(mode):
    """Sequence numbers past 2^32: the device seq, the go word (2 * seq +
    abort) and the published word are 64-bit like the flags, parity keeps
    alternating, every call bit-exact."""
    W, n, start = 4, 8192 + 3, (1 << 32) - 3
    recv = [WL.recv_partials(3, par, n, W) for par in (0, 1)]
    xs = [WL.uniform(18000 + k, n) for k in range(8)]
    with library(W, n):
        fill_recv(recv, 0)
        arx.debug_set_seq(start)
        arx.set_proxy_mode(mode)
        st = P.ProtocolState(W=W, rank=0, seq_dev=start, go=start & 0xFFFFFFFF, ctl_seq=start, ctl_done=start,
                             flags=[0] + [start] * (W - 1), posted=start)
        for k, x in enumerate(xs):
            inp, out = to_dev(x, pad_to=n + 5), sentinel(n + 5)
            note(f"seq {start + k + 1}, mode {mode}")
            arx.allreduce(inp, out, n)
            torch.cuda.synchronize()
            st, outs = P.sequential_model([(x, n)], recv, W, mode=P.RUNAHEAD if mode == arx.PROXY_RUNAHEAD else
                                          P.LOCKSTEP, max_n=n, state=st)
            assert_bits(to_host(out)[:n], outs[0], f"seq {start + k + 1}")
        check_state(st, 0, wait_posted=st.posted)
        assert st.seq_dev == start + len(xs) > (1 << 32)
