"""GPU: one library instance driven through a seeded random sequence of
every entry point — one-shot calls (out of place and in place, sizes from 0
to max_n with ragged tails), the reduction alone, the blockwise barrier in
both semantics, the counter barrier and the symmetric-buffer exchange —
each result checked bit-exact against the oracle as it comes. The calls
share the library's state: the seq and parity running through the one-shot
calls, and the signal pads that both the barrier and the symmetric exchange
use and must leave zero. At the end every protocol word is compared with
the sequential model."""
import numpy as np
import pytest
import torch

from oracle import protocol as P
from oracle import reduce as R
from signal_pad_sync_amd import arx
from signal_pad_sync_amd import workloads as WL
from tests.gpu_util import fill_recv, library, note, sentinel, to_dev, to_host

pytestmark = pytest.mark.gpu

OPS = ["oneshot", "oneshot_in_place", "reduce", "barrier", "counter", "symm"]
SIZES = [0, 1, 7, 8, 13, 1000, 4096, 65531, 131072, 131073, 262144, 300007]


def same(got, want, what):
    if not np.array_equal(got, want):
        i = int(np.flatnonzero(got != want)[0])
        raise AssertionError(f"{what}: first difference at {i}: got {hex(int(got[i]))} want {hex(int(want[i]))}")


@pytest.mark.parametrize("W,rank,seed", [(8, 0, 1), (5, 2, 2), (3, 1, 3)])
def test_mixed_call_sequence(W, rank, seed):
    rng = np.random.default_rng(40000 + seed)
    max_n = 300007
    recv = [[WL.uniform(41000 + 100 * seed + 10 * par + s, max_n) for s in range(W)] for par in (0, 1)]
    rounds_done = np.zeros(arx.MAX_PAD_BLOCKS, np.int64)
    launches = np.zeros(arx.MAX_PAD_BLOCKS, np.int64)
    split = None                      # the counter barrier's design, fixed by its first launch
    with library(W, max_n, rank=rank):
        fill_recv(recv, rank)
        st = None
        ran = {op: 0 for op in OPS}
        for step in range(200):
            op = OPS[int(rng.integers(len(OPS)))]
            ran[op] += 1
            n = int(SIZES[int(rng.integers(len(SIZES)))])
            note(f"mixed W={W} rank={rank} step {step}: {op} n={n}")
            if op in ("oneshot", "oneshot_in_place"):
                x = WL.uniform(int(rng.integers(1 << 30)), max(n, 1))[:n]
                if op == "oneshot":
                    inp, out = to_dev(x, pad_to=max_n), sentinel(max_n)
                else:
                    xs = np.full(max_n, 0xDEAD, np.uint16)
                    xs[:n] = x
                    inp = out = to_dev(xs)
                arx.allreduce(inp, out, n)
                torch.cuda.synchronize()
                st, outs = P.sequential_model([(x, n)], recv, W, rank=rank, max_n=max_n, state=st)
                got = to_host(out)
                same(got[:n], outs[0], f"step {step} {op} n={n}")
                assert np.all(got[n:] == 0xDEAD), f"step {step}: written past n"
                same(to_host(arx.send_view(st.seq_dev & 1, max_n))[:n], x, f"step {step}: send slot")
            elif op == "reduce":
                par = int(rng.integers(2))
                x = WL.uniform(int(rng.integers(1 << 30)), max(n, 1))[:n]
                inp, out = to_dev(x, pad_to=max_n), sentinel(max_n)
                arx.reduce(inp, out, par, n)
                torch.cuda.synchronize()
                parts = [x if s == rank else recv[par][s][:n] for s in range(W)]
                got = to_host(out)
                same(got[:n], R.reduce(parts, n=n) if n else got[:0], f"step {step} reduce n={n} par={par}")
                assert np.all(got[n:] == 0xDEAD)
            elif op == "barrier":
                lanes = bool(rng.integers(2))
                most = arx.MAX_PAD_BLOCKS if lanes else arx.barrier_max_blocks()
                nblocks = int(rng.integers(1, most + 1))
                sem = int(rng.integers(2))
                arx.barrier_blockwise(nblocks, sem, int(rng.integers(1, 5)), arx.BARRIER_LANES if lanes else 0)
                torch.cuda.synchronize()
            elif op == "counter":
                lanes = bool(rng.integers(2))
                if split is None:
                    split = bool(rng.integers(2))
                most = arx.MAX_PAD_BLOCKS if lanes else arx.barrier_max_blocks()
                nblocks = int(rng.integers(1, most + 1))
                rounds = int(rng.integers(0, 4))
                arx.counter_barrier(nblocks, rounds, (arx.BARRIER_LANES if lanes else 0) |
                                    (arx.BARRIER_SPLIT if split else 0))
                torch.cuda.synchronize()
                rounds_done[:nblocks] += rounds
                launches[:nblocks] += 1
                per = W if split else 2 * W
                for r in range(W):
                    sem_r = arx.sem_view(r).cpu().numpy()
                    assert np.array_equal(sem_r[:, 0], per * rounds_done), f"step {step}: flags of rank {r}"
                    assert np.array_equal(sem_r[:, 1], per * rounds_done), f"step {step}: bases of rank {r}"
                    assert np.array_equal(arx.epoch_view(r).cpu().numpy(), launches % 2)
            else:
                iters = int(rng.integers(1, 4))
                ld = max(8, (n + 7) & ~7)
                data = np.zeros((iters, W, ld), np.uint16)
                for k in range(iters):
                    for v in range(W):
                        data[k, v, :n] = WL.uniform(int(rng.integers(1 << 30)), max(n, 1))[:n]
                din = to_dev(data.reshape(-1)).view(iters, W, ld)
                dout = to_dev(np.full(iters * W * ld, 0xDEAD, np.uint16)).view(iters, W, ld)
                arx.symm_allreduce(din, dout, n, iters)
                torch.cuda.synchronize()
                got = to_host(dout).reshape(iters, W, ld)
                for k in range(iters):
                    want = R.reduce([data[k, v, :n] for v in range(W)], n=n) if n else got[k, 0, :0]
                    for v in range(W):
                        same(got[k, v, :n], want, f"step {step} symm n={n} iteration {k} rank {v}")
                        assert np.all(got[k, v, n:] == 0xDEAD)
            if op in ("barrier", "symm"):
                for r in range(W):
                    assert int(arx.pad_view(r).abs().sum()) == 0, f"step {step}: pad {r} not zero after {op}"
            assert arx.debug_state()["ctl_err"] == 0, f"step {step}: {op}"
        assert all(ran.values()), ran
        if st is not None:
            d = arx.debug_state()
            assert d["seq_dev"] == st.seq_dev and d["ctl_seq"] == st.ctl_seq and d["ctl_done"] == st.ctl_done, d
            assert d["cnt0"] == 0 and d["cnt1"] == 0 and d["go"] == st.go, d
            assert d["flags"] == st.flags, (d["flags"], st.flags)
