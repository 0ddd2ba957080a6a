"""GPU: the library at its largest size, max_n = 2^30 bf16 elements (2 GiB
per partial), where the kernels' 32-bit byte offsets reach 2^31. W=2 keeps
the slots at 16 GiB. Every pattern class (subnormals, +-0, +-Inf, NaNs)
appears in the random bit inputs. The oracle computes sampled outputs one
by one: the first and last 4096 elements and 2^18 random positions, each
bit-exact; the elements past n must keep their sentinel."""
import numpy as np
import pytest
import torch

from oracle import reduce as R
from signal_pad_sync_amd import arx
from signal_pad_sync_amd import workloads as WL
from tests.gpu_util import fill_recv, library, note, to_dev, to_host

pytestmark = pytest.mark.gpu

SENTINEL = 0xDEAD


def device_sentinel(n):
    return torch.full((n,), SENTINEL - 0x10000, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def sample(n, seed):
    rng = np.random.default_rng(seed)
    idx = np.concatenate([np.arange(min(n, 4096)), rng.integers(0, n, 1 << 18), np.arange(max(0, n - 4096), n)])
    return np.unique(idx)


def gather(t, idx):
    return to_host(t.view(torch.int16)[torch.from_numpy(idx).to("cuda")].view(torch.bfloat16))


def assert_sampled(got, want, idx, what):
    if not np.array_equal(got, want):
        bad = np.flatnonzero(got != want)
        i = int(bad[0])
        raise AssertionError(f"{what}: {bad.size} sampled elements differ, first at {int(idx[i])}: "
                             f"got {hex(int(got[i]))} want {hex(int(want[i]))}")


@pytest.mark.skipif(not torch.cuda.is_available() or torch.cuda.get_device_properties(0).total_memory < (64 << 30),
                    reason="needs about 40 GiB of device memory")
def test_maximum_size():
    W, max_n = 2, arx.MAX_N
    note("limits: generating 2 x 2^30 random bf16 patterns")
    x = WL.bits(31001, max_n)
    peer = WL.bits(31002, max_n)
    with library(W, max_n):
        fill_recv([None, [None, peer]], 0)        # the first call has seq 1, parity 1
        inp = to_dev(x)

        n = max_n - 3                             # ragged: 3 elements short of the limit
        out = device_sentinel(max_n)
        note(f"limits: one-shot n={n}")
        arx.allreduce(inp, out, n)
        torch.cuda.synchronize()
        idx = sample(n, 31003)
        assert_sampled(gather(out, idx), R.reduce([x[idx], peer[idx]]), idx, "one-shot at n = 2^30 - 3")
        assert np.all(to_host(out[n:]) == SENTINEL), "one-shot wrote past n"
        assert_sampled(gather(arx.send_view(1, max_n), idx), x[idx], idx, "send slot copy")
        d = arx.debug_state()
        assert d["ctl_err"] == 0 and d["seq_dev"] == 1 and d["ctl_bytes1"] == 2 * n, d
        del out

        out = device_sentinel(max_n)
        note(f"limits: reduce-only n={max_n}")
        arx.reduce(inp, out, 1, max_n)
        torch.cuda.synchronize()
        idx = sample(max_n, 31004)
        assert_sampled(gather(out, idx), R.reduce([x[idx], peer[idx]]), idx, "reduce at n = 2^30")
        del out

        n = max_n - 5
        din = torch.stack([inp, to_dev(peer)]).view(1, W, max_n)
        dout = device_sentinel(W * max_n).view(1, W, max_n)
        note(f"limits: symmetric-buffer all-reduce n={n}")
        arx.symm_allreduce(din, dout, n, 1)
        torch.cuda.synchronize()
        idx = sample(n, 31005)
        want = R.reduce([x[idx], peer[idx]])
        for v in range(W):
            assert_sampled(gather(dout[0, v], idx), want, idx, f"symmetric all-reduce, rank {v}")
            assert np.all(to_host(dout[0, v, n:]) == SENTINEL), f"rank {v} wrote past n"
        for r in range(W):
            assert int(arx.pad_view(r).abs().sum()) == 0
        assert arx.debug_state()["ctl_err"] == 0
