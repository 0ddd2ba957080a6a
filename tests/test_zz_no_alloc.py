"""GPU: arx_symm_allreduce_noalloc, the symmetric exchange for callers that
cannot allocate, called through the C ABI with no library instance, against
the allocating arx_symm_allreduce on the same inputs: bit-exact over the
whole output buffers (elements past n untouched), on two calls in a row with
the second smaller than the first; then captured in a hipGraph and replayed
with eager calls between the replays."""
import numpy as np
import pytest
import torch

from signal_pad_sync_amd import arx
from tests.gpu_util import library, note, to_dev, to_host

pytestmark = pytest.mark.gpu


def rand_bits(seed, shape):
    """Seeded bf16 patterns from the finite, moderately sized range (so sums
    stay finite and both entry points are compared on ordinary values)."""
    rng = np.random.default_rng(seed)
    sign = rng.integers(0, 2, size=shape, dtype=np.uint16) << 15
    exp = rng.integers(110, 135, size=shape, dtype=np.uint16) << 7
    man = rng.integers(0, 128, size=shape, dtype=np.uint16)
    return (sign | exp | man).astype(np.uint16)


def noalloc(W, din, dout, n, iters, status):
    stream = torch.cuda.current_stream().cuda_stream
    rc = arx.lib.arx_symm_allreduce_noalloc(W, din.data_ptr(), dout.data_ptr(), n, din.shape[-1], iters,
                                            status.data_ptr(), stream)
    assert rc == 0, arx.lib.arx_strerror(rc).decode()


def reference(W, data, n, iters, max_n):
    """The allocating entry point's outputs for the same inputs."""
    ld = data.shape[-1]
    with library(W, max_n):
        din = to_dev(data.reshape(-1)).view(iters, W, ld)
        dout = to_dev(np.full(iters * W * ld, 0xDEAD, np.uint16)).view(iters, W, ld)
        arx.symm_allreduce(din, dout, n, iters)
        torch.cuda.synchronize()
        return to_host(dout).reshape(iters, W, ld)


@pytest.mark.parametrize("W", [8, 3])
def test_noalloc_matches_the_allocating_entry_point(W):
    assert arx.world() == 0                    # no library instance
    cases = [(arx.NOALLOC_MAX_N, 2, 0), (200003, 3, 16)]   # (n, iters, ld - n rounded); the second smaller
    runs = []
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for k, (n, iters, extra) in enumerate(cases):
        ld = ((n + 7) & ~7) + extra
        data = rand_bits(50000 + 10 * W + k, (iters, W, ld))
        din = to_dev(data.reshape(-1)).view(iters, W, ld)
        dout = to_dev(np.full(iters * W * ld, 0xDEAD, np.uint16)).view(iters, W, ld)
        note(f"noalloc W={W} n={n} iters={iters} ld={ld}")
        noalloc(W, din, dout, n, iters, status)
        runs.append((n, iters, data, dout))
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert arx.world() == 0
    for n, iters, data, dout in runs:
        got = to_host(dout).reshape(data.shape)
        note(f"reference W={W} n={n}")
        want = reference(W, data, n, iters, arx.NOALLOC_MAX_N)
        if not np.array_equal(got, want):
            i = int(np.flatnonzero(got.reshape(-1) != want.reshape(-1))[0])
            raise AssertionError(f"W={W} n={n}: first difference at flat index {i}: "
                                 f"got {hex(int(got.reshape(-1)[i]))} want {hex(int(want.reshape(-1)[i]))}")
        assert np.all(got[..., n:] == 0xDEAD)


def test_noalloc_graph_replays():
    """Captured in a hipGraph (the allocation-free call is what capture
    needs), replayed three times with eager calls of other sizes between the
    replays: every replay equals the allocating entry point's result."""
    W, n, iters = 4, 65536 + 3, 2
    ld = (n + 7) & ~7
    data = rand_bits(51000, (iters, W, ld))
    other = rand_bits(51001, (1, W, 4096))
    want = reference(W, data, n, iters, n)
    din = to_dev(data.reshape(-1)).view(iters, W, ld)
    dout = to_dev(np.full(iters * W * ld, 0xDEAD, np.uint16)).view(iters, W, ld)
    oin = to_dev(other.reshape(-1)).view(1, W, 4096)
    oout = torch.empty_like(oin)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    note("noalloc graph capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        noalloc(W, din, dout, n, iters, status)
    for rep in range(3):
        dout.view(torch.int16).fill_(-8531)     # 0xDEAD
        note(f"noalloc graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(dout).reshape(iters, W, ld), want), f"replay {rep}"
        noalloc(W, oin, oout, 4095, 1, status)    # eager work between replays
        torch.cuda.synchronize()
    assert int(status.item()) == 0
