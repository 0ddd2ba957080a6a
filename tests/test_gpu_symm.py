"""GPU: all-reduce among the virtual ranks through symmetric buffers, fenced
by the blockwise barrier's usage patterns (page "triton_barrier.py",
blockwise_barrier docstring: pattern 0 at kernel start, pattern 1 after each
write, pattern 2 after each read). Every iteration's result of every rank is
compared bit-exact with the oracle's rank-ordered sum; the pads must be zero
after every launch."""
import numpy as np
import pytest
import torch

from oracle import reduce as R
from signal_pad_sync_amd import arx
from signal_pad_sync_amd import workloads as WL
from tests.gpu_util import library, note, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("W,n,iters", [(2, 1000, 5), (4, 131071, 6), (8, 131072, 8), (8, 8, 3), (3, 262147, 4),
                                       (5, 65536 * 3 + 5, 3)])
def test_symm_allreduce(W, n, iters):
    ld = (n + 7) & ~7
    rng_seed = 12000 + 100 * W + iters
    with library(W, ld):
        for launch in range(2):
            data = np.zeros((iters, W, ld), np.uint16)
            if W == 8 and n == 131072:                    # the adversarial mix on one case
                for k in range(iters):
                    parts = WL.adversarial(rng_seed + 10 * k + launch, W, n)
                    for v in range(W):
                        data[k, v, :n] = parts[v]
            else:
                for k in range(iters):
                    for v in range(W):
                        data[k, v, :n] = WL.normal(rng_seed + 1000 * launch + 10 * k + v, n)
            din = to_dev(data.reshape(-1)).view(iters, W, ld)
            dout = to_dev(np.full(iters * W * ld, 0xDEAD, np.uint16)).view(iters, W, ld)
            note(f"symm W={W} n={n} iters={iters} launch {launch}")
            arx.symm_allreduce(din, dout, n, iters)
            torch.cuda.synchronize()
            got = to_host(dout).reshape(iters, W, ld)
            for k in range(iters):
                want = R.reduce([data[k, v, :n] for v in range(W)], n=n)
                for v in range(W):
                    if not np.array_equal(got[k, v, :n], want):
                        bad = np.flatnonzero(got[k, v, :n] != want)
                        raise AssertionError(f"launch {launch} iteration {k} rank {v}: {bad.size} differ, "
                                             f"first at {bad[0]}")
                    assert np.all(got[k, v, n:] == 0xDEAD)
            for r in range(W):
                assert int(arx.pad_view(r).abs().sum()) == 0, f"pad {r} not zero"
            assert arx.debug_state()["ctl_err"] == 0


def test_symm_empty():
    """n = 0: the kernel still runs its barrier patterns (pads zero after),
    writes nothing and raises no error."""
    W, iters, ld = 4, 3, 8
    with library(W, 64):
        din = to_dev(np.ones(iters * W * ld, np.uint16)).view(iters, W, ld)
        dout = to_dev(np.full(iters * W * ld, 0xDEAD, np.uint16)).view(iters, W, ld)
        note("symm n=0")
        arx.symm_allreduce(din, dout, 0, iters)
        torch.cuda.synchronize()
        assert np.all(to_host(dout) == 0xDEAD)
        for r in range(W):
            assert int(arx.pad_view(r).abs().sum()) == 0
        assert arx.debug_state()["ctl_err"] == 0


def test_symm_argument_errors():
    with library(2, 1024):
        t = torch.zeros(2 * 2 * 1024, dtype=torch.bfloat16, device="cuda").view(2, 2, 1024)
        for call in (lambda: arx.lib.arx_symm_allreduce(t.data_ptr(), t.data_ptr(), 1025, 1032, 2, None),
                     lambda: arx.lib.arx_symm_allreduce(t.data_ptr(), t.data_ptr(), 1000, 1004, 2, None),
                     lambda: arx.lib.arx_symm_allreduce(t.data_ptr(), t.data_ptr(), 1000, 1024, 0, None),
                     lambda: arx.lib.arx_symm_allreduce(t.data_ptr() + 2, t.data_ptr(), 8, 8, 1, None)):
            assert call() == arx.EINVAL


def test_symm_graph_replays():
    """The symmetric all-reduce captured in a hipGraph and replayed, with the
    inputs changed between replays by eager copies: every replay matches the
    oracle and leaves the pads zero."""
    W, n, iters = 4, 4096 + 5, 3
    ld = (n + 7) & ~7
    with library(W, ld):
        din = torch.zeros(iters * W * ld, dtype=torch.bfloat16, device="cuda").view(iters, W, ld)
        dout = torch.zeros_like(din)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            arx.symm_allreduce(din, dout, n, iters)
        for rep in range(4):
            data = np.zeros((iters, W, ld), np.uint16)
            for k in range(iters):
                for v in range(W):
                    data[k, v, :n] = WL.normal(17000 + 100 * rep + 10 * k + v, n)
            din.copy_(to_dev(data.reshape(-1)).view(iters, W, ld))
            note(f"symm graph replay {rep}")
            g.replay()
            torch.cuda.synchronize()
            got = to_host(dout).reshape(iters, W, ld)
            for k in range(iters):
                want = R.reduce([data[k, v, :n] for v in range(W)], n=n)
                for v in range(W):
                    assert np.array_equal(got[k, v, :n], want), (rep, k, v)
            for r in range(W):
                assert int(arx.pad_view(r).abs().sum()) == 0
