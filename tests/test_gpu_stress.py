"""GPU: peer data written by another agent just before each flag.

Page "arx.cu", protocol comment: a peer writes its partial into
recv[seq & 1][rank] and then the flag, on one ordered channel, and the GPU
sums once every flag has reached seq. In stress mode the library's proxy
plays those peers: before posting seq s it copies a different data set into
recv[s & 1] on its own stream. The slot of the same parity was last read two
calls earlier, so a stale cached line would give a wrong sum. Every output is
compared bit-exact with the oracle.
"""
import numpy as np
import pytest
import torch

from oracle import reduce as R
from signal_pad_sync_amd import arx
from signal_pad_sync_amd import workloads as WL
from tests.gpu_util import library, note, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("W,n,sets,K", [(8, 131072, 5, 200), (4, 262147, 3, 64), (2, 1000, 7, 100),
                                        (8, (8 << 20) + 3, 2, 4), (4, (32 << 20) + 5, 2, 4)])
def test_fresh_peer_data_every_seq(W, n, sets, K):
    """The proxy writes the peers' data for each seq just before its flag,
    from a pool of `sets` data sets, so every call sums data no earlier call
    saw. The two large cases run the copy's nontemporal stores (8 Mi + 3 at
    W = 8) and the sum's nontemporal peer loads as well (32 Mi + 5 at
    W = 4), which must see each seq's fresh data like the system-coherent
    loads."""
    pool = np.stack([np.stack([WL.normal(8000 + 10 * k + src, n) for src in range(W)]) for k in range(sets)])
    npad = (n + 7) & ~7                               # rows start 16-byte aligned
    ins = np.zeros((K, npad), np.uint16)
    for k in range(K):
        ins[k, :n] = WL.normal(9000 + k + 1, n)
    with library(W, n):
        dpool = to_dev(pool.reshape(-1)).view(sets, W, n)
        arx.set_stress_source(dpool, sets)
        arx.set_proxy_mode(arx.PROXY_STRESS)
        din = to_dev(ins.reshape(-1)).view(K, npad)
        dout = torch.empty_like(din)
        note(f"stress W={W} n={n} sets={sets}: {K} calls")
        for k in range(K):
            arx.allreduce(din[k], dout[k], n)
        torch.cuda.synchronize()
        arx.set_proxy_mode(arx.PROXY_LOCKSTEP)
        got = to_host(dout).reshape(K, npad)[:, :n]
        d = arx.debug_state()
        assert d["ctl_err"] == 0 and d["seq_dev"] == K and d["posted"] == K, d
    for k in range(K):
        seq = k + 1
        parts = [ins[k, :n]] + [pool[seq % sets][src] for src in range(1, W)]
        want = R.reduce(parts, n=n)
        if not np.array_equal(got[k], want):
            bad = np.flatnonzero(got[k] != want)
            raise AssertionError(f"call {seq}: {bad.size} elements differ, first at {bad[0]}")


@pytest.mark.parametrize("W", [4, 8])
def test_call_size_changes(W):
    """The proxy copies as many bytes as the GPU published with each seq
    (ctl.bytes[seq & 1]), so a size left stale in its slot would leave the
    tail of the peers' data from an older set and give a wrong sum. The
    sizes repeat and change per parity: kept as they are, grown and shrunk,
    over grids of 2 to 30 reducing workgroups."""
    ns = [9000, 9000, 20003, 20003, 9000, 50000, 50000, 50000, 20003, 9000, 9000, 4096, 4096, 60001, 9000]
    sets, K, max_n = 5, len(ns), 60008
    pool = np.stack([np.stack([WL.normal(8500 + 10 * k + src, max_n) for src in range(W)]) for k in range(sets)])
    ins = [WL.normal(9500 + k + 1, n) for k, n in enumerate(ns)]
    with library(W, max_n):
        dpool = to_dev(pool.reshape(-1)).view(sets, W, max_n)
        arx.set_stress_source(dpool, sets)
        arx.set_proxy_mode(arx.PROXY_STRESS)
        outs = []
        for k, n in enumerate(ns):
            note(f"stress W={W} call {k + 1}: n={n}")
            out = torch.empty(max_n, dtype=torch.bfloat16, device="cuda")
            arx.allreduce(to_dev(ins[k], pad_to=max_n), out, n)
            outs.append(out)
        torch.cuda.synchronize()
        arx.set_proxy_mode(arx.PROXY_LOCKSTEP)
        d = arx.debug_state()
        assert d["ctl_err"] == 0 and d["seq_dev"] == K and d["posted"] == K, d
        last = {p: 2 * ns[max(k for k in range(K) if (k + 1) % 2 == p)] for p in (0, 1)}
        assert [d["ctl_bytes0"], d["ctl_bytes1"]] == [last[0], last[1]], d
        got = [to_host(o) for o in outs]
    for k, n in enumerate(ns):
        seq = k + 1
        parts = [ins[k]] + [pool[seq % sets][src][:n] for src in range(1, W)]
        want = R.reduce(parts, n=n)
        if not np.array_equal(got[k][:n], want):
            bad = np.flatnonzero(got[k][:n] != want)
            raise AssertionError(f"call {seq} (n={n}): {bad.size} elements differ, first at {bad[0]}")


def test_stress_source_rules():
    with library(2, 64):
        with pytest.raises(arx.ArxError) as e:
            arx.set_proxy_mode(arx.PROXY_STRESS)       # no source yet
        assert e.value.code == arx.EINVAL
        pool = torch.zeros(2 * 2 * 64, dtype=torch.bfloat16, device="cuda")
        with pytest.raises(arx.ArxError) as e:
            arx.set_stress_source(pool, 3)             # 3 sets do not fit in the pool
        assert e.value.code == arx.EINVAL
        arx.set_stress_source(pool, 2)
        arx.set_proxy_mode(arx.PROXY_STRESS)
        with pytest.raises(arx.ArxError) as e:
            arx.set_stress_source(pool, 1)             # not while in use
        assert e.value.code == arx.ESTATE
        arx.set_proxy_mode(arx.PROXY_LOCKSTEP)
        arx.set_stress_source(None, 0)


@pytest.mark.parametrize("n", [1000, 131072])
def test_proxy_failure_is_latched(n):
    """Page "arx.cu": a failed proxy post latches an error, and the next
    all-reduce refuses to run. Forced from the host: the proxy's next
    peer-data copy reports failure; the call in flight never gets its flags
    and ends through its 20 ms flag wait, writing nothing (one reducing
    workgroup and a tail at n = 1000, 32 at n = 131072)."""
    W = 2
    with library(W, n, timeout_us=20000):
        pool = torch.zeros(W * n, dtype=torch.bfloat16, device="cuda")
        arx.set_stress_source(pool, 1)
        arx.set_proxy_mode(arx.PROXY_STRESS)
        inp, out = to_dev(WL.normal(8800, n)), to_dev(np.full(n, 0xDEAD, np.uint16))
        arx.debug_fail_proxy()
        note(f"proxy failure n={n}: one call whose flags never come")
        arx.allreduce(inp, out, n)
        torch.cuda.synchronize()
        assert np.all(to_host(out) == 0xDEAD)
        with pytest.raises(arx.ArxError) as e:
            arx.allreduce(inp, out, n)
        assert e.value.code == arx.EPROXY
        d = arx.debug_state()
        assert d["seq_dev"] == 1 and d["posted"] == 0 and d["ctl_err"] != 0, d


def test_watchdog_reports_a_dead_peer(capfd):
    """Page "arx.cu", proxy_loop: a rank whose published work has not
    finished for 2 s prints one STALL line with what it published, posted
    and finished and each peer's flag. Forced from the host: manual mode
    and no publish, so the call waits for flags that never come, bounded at
    3 s; the report must appear while it waits."""
    import time
    W, n = 3, 1024
    with library(W, n, mode=arx.PROXY_MANUAL, timeout_us=3_000_000):
        inp, out = to_dev(WL.normal(8900, n)), to_dev(np.full(n, 0xDEAD, np.uint16))
        note("watchdog: one call whose peers never publish, 3 s bound")
        arx.allreduce(inp, out, n)
        time.sleep(2.5)
        published, posted, done = arx.status()
        assert (published, posted, done) == (1, 0, 0), (published, posted, done)
        torch.cuda.synchronize()                     # the 3 s flag wait ends the call
        err = capfd.readouterr().err
        assert "STALL: published 1 posted 0 done 0" in err, err
        assert err.count("STALL") == 1, err
        assert np.all(to_host(out) == 0xDEAD)
        assert arx.debug_state()["ctl_err"] != 0
