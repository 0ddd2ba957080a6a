"""GPU: seeded random one-shot calls across the parameter space — W from 2
to 8, this GPU at a random rank, lockstep or run-ahead proxy, n from 0 to
max_n (up to 2 Mi elements, so every grid shape: one reducing workgroup,
several, the copy split and the grid-stride loop), in place or not, on uniformly
random bf16 bit patterns (Inf and NaN included). Every output is compared
bit-exact with the oracle, the elements past n must keep their sentinel,
and the send slot must hold the call's input."""
import numpy as np
import pytest
import torch

from oracle import protocol as P
from signal_pad_sync_amd import arx
from signal_pad_sync_amd import workloads as WL
from tests.gpu_util import library, note, to_dev, to_host

pytestmark = pytest.mark.gpu

SENTINEL = 0xDEAD


@pytest.mark.parametrize("seed", list(range(1, 13)))
def test_random_oneshot_calls(seed):
    rng = np.random.default_rng(50000 + seed)
    for inst in range(4):
        W = int(rng.integers(2, 9))
        rank = int(rng.integers(W))
        mode = (arx.PROXY_LOCKSTEP, arx.PROXY_RUNAHEAD)[int(rng.integers(2))]
        max_n = int(rng.integers(1, 1 << 21))
        recv = [[WL.bits(int(rng.integers(1 << 30)), max_n) for _ in range(W)] for _ in (0, 1)]
        with library(W, max_n, rank=rank, mode=mode):
            for par in (0, 1):
                for s in range(W):
                    if s != rank:
                        arx.recv_view(par, s, max_n).copy_(to_dev(recv[par][s]))
            torch.cuda.synchronize()
            st = None
            for call in range(25):
                n = int(rng.integers(0, max_n + 1)) if rng.random() < 0.5 else int(min(max_n, rng.integers(0, 9000)))
                x = WL.bits(int(rng.integers(1 << 30)), max(n, 1))[:n]
                in_place = bool(rng.random() < 0.3)
                buf = np.full(max_n + 8, SENTINEL, np.uint16)
                buf[:n] = x
                d_in = to_dev(buf)
                d_out = d_in if in_place else to_dev(np.full(max_n + 8, SENTINEL, np.uint16))
                note(f"random seed={seed} W={W} rank={rank} mode={mode} n={n} in_place={in_place}")
                arx.allreduce(d_in, d_out, n)
                torch.cuda.synchronize()
                st, outs = P.sequential_model([(x, n)], recv, W, rank=rank, max_n=max_n, state=st,
                                              mode=P.RUNAHEAD if mode == arx.PROXY_RUNAHEAD else P.LOCKSTEP)
                got = to_host(d_out)
                case = f"seed {seed} W={W} rank={rank} mode={mode} n={n} in_place={in_place} call {call}"
                if not np.array_equal(got[:n], outs[0]):
                    i = int(np.flatnonzero(got[:n] != outs[0])[0])
                    raise AssertionError(f"{case}: first difference at {i}: got {hex(int(got[i]))} "
                                         f"want {hex(int(outs[0][i]))}")
                assert np.all(got[n:] == SENTINEL), f"{case}: written past n"
                assert np.array_equal(to_host(arx.send_view(st.seq_dev & 1, max_n))[:n], x), f"{case}: send slot"
            assert arx.debug_state()["ctl_err"] == 0
