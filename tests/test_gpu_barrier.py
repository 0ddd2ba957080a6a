"""GPU: the barriers with every virtual rank's block as a workgroup of its
own, so the W workgroups of one block id really wait on each other (page
"triton_barrier.py": blockwise_barrier synchronises the blocks with matching
block id across ranks, and its barrier test runs many blocks on every rank;
page "common.cuh": PullController::sync). Each launch carries the tag check
of the library's barrier-tag format: before a round every rank's block
writes its tag, after the round it reads every rank's tag for the same
block and round. The expected tags and the values read back come from the
oracle's barrier model; pads must be zero afterwards, and the counter
barrier's flags, bases and epochs must follow its closed form.

The public device-side barrier (include/arx_device.h) is checked from a
caller's kernel in a separate library built against include/ alone."""
import ctypes
import os

import numpy as np
import pytest
import torch

from oracle import protocol as P
from signal_pad_sync_amd import arx
from tests.gpu_util import library, note

pytestmark = pytest.mark.gpu

DEVAPI = os.path.join(os.path.dirname(os.path.abspath(__file__)), "devapi", "libdevapi_user.so")


def zeros_u32(*shape):
    return torch.zeros(shape, dtype=torch.int32, device="cuda")


def host_u32(t):
    return t.cpu().numpy().view(np.uint32)


def check_tags(tags, seen, W, nblocks, rounds, exact: bool, what: str):
    """tags must hold every rank's own tags; seen must equal the oracle's
    prediction everywhere (exact) or hold, in every slot, either it or the
    zero the slot started with (relaxed visibility). Returns the fraction of
    slots of seen that equal the prediction."""
    assert np.array_equal(host_u32(tags).reshape(W, rounds, nblocks), P.barrier_tags_written(W, nblocks, rounds)), \
        f"{what}: tag rows"
    want = P.barrier_tags_seen(W, nblocks, rounds)
    got = host_u32(seen).reshape(W, rounds, nblocks, W)
    hit = got == want
    if exact:
        if not hit.all():
            v, r, b, p = (int(x[0]) for x in np.nonzero(~hit))
            raise AssertionError(f"{what}: rank {v} block {b} round {r} read {hex(int(got[v, r, b, p]))} for rank {p}, "
                                 f"want {hex(int(want[v, r, b, p]))} ({int((~hit).sum())} slots differ)")
    else:
        assert np.all(hit | (got == 0)), f"{what}: a slot read neither the tag nor its initial zero"
    return float(hit.mean())


def pads_zero(W):
    return all(int(arx.pad_view(r).abs().sum()) == 0 for r in range(W))


@pytest.mark.parametrize("W", [2, 4, 8])
def test_pad_barrier_across_workgroups(W):
    """W * nblocks workgroups, both semantics, up to 64 rounds: acq_rel makes
    every peer's tag visible after every round, relaxed reads a tag or the
    slot's initial zero; pads zero after every launch."""
    with library(W, 1024):
        most = arx.barrier_max_blocks()
        note(f"W={W}: at most {most} blocks per rank at once")
        assert most >= 256
        for sem in (arx.SEM_ACQ_REL, arx.SEM_RELAXED):
            for nblocks, rounds in [(1, 1), (256, 8), (256, 16), (most, 2), (32, 64), (7, 9)]:
                tags, seen = zeros_u32(W, rounds, nblocks), zeros_u32(W, rounds, nblocks, W)
                note(f"pad barrier W={W} sem={sem} nblocks={nblocks} rounds={rounds}")
                arx.barrier_blockwise(nblocks, sem, rounds, 0, tags, seen)
                torch.cuda.synchronize()
                assert arx.debug_state()["ctl_err"] == 0
                assert pads_zero(W)
                frac = check_tags(tags, seen, W, nblocks, rounds, sem == arx.SEM_ACQ_REL,
                                  f"W={W} sem={sem} nblocks={nblocks} rounds={rounds}")
                note(f"  tags seen: {frac:.4f}")
            # and untagged, as the benchmark and workload 3 launch it
            arx.barrier_blockwise(256, sem, 4)
            torch.cuda.synchronize()
            assert arx.debug_state()["ctl_err"] == 0 and pads_zero(W)


@pytest.mark.parametrize("W", [2, 4, 8])
def test_pad_barrier_lane_groups_leave_pads_zero(W):
    """The named lane-group variant: pads zero again after every launch, both
    semantics, many workgroups, repeated rounds."""
    with library(W, 1024):
        for sem in (arx.SEM_RELAXED, arx.SEM_ACQ_REL):
            for nblocks, rounds in [(1, 1), (32, 1), (256, 1), (256, 8), (1024, 2), (1024, 64)]:
                note(f"lane-group barrier W={W} sem={sem} nblocks={nblocks} rounds={rounds}")
                arx.barrier_blockwise(nblocks, sem, rounds, arx.BARRIER_LANES)
                torch.cuda.synchronize()
                assert pads_zero(W)
                assert arx.debug_state()["ctl_err"] == 0


def check_semaphores(W, rounds_done, split, what):
    """Page design: flag = base = 2 W R after R rounds; split design: both
    the start pair and the end pair are W R."""
    for r in range(W):
        sem = arx.sem_view(r).cpu().numpy()
        if split:
            for col in (0, 1, 16, 17):
                assert np.array_equal(sem[:, col], W * rounds_done), f"{what}: rank {r} column {col}"
        else:
            assert np.array_equal(sem[:, 0], 2 * W * rounds_done), f"{what}: flags of rank {r}"
            assert np.array_equal(sem[:, 1], 2 * W * rounds_done), f"{what}: bases of rank {r}"
            assert not sem[:, 16:18].any(), f"{what}: end-stage pair used by the page design"


@pytest.mark.parametrize("W", [2, 3, 4, 8])
@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("lanes", [False, True])
def test_counter_barrier_flags_bases_epochs(W, split, lanes):
    """Page "common.cuh": over seven launches, flags and bases follow the
    closed form, every rank's epoch per block flips at each launch and each
    launch saw the parity of the launches before it. With one workgroup per
    rank and block, the tag check: exact for the split design (every end
    stage pairs with every rank's release) and at W = 2; for the page's
    single-semaphore design at W >= 3, whose end stage can lack that pairing
    (the oracle's model shows how), every slot holds the tag or its initial
    zero."""
    flags = (arx.BARRIER_SPLIT if split else 0) | (arx.BARRIER_LANES if lanes else 0)
    with library(W, 1024):
        rounds_done = np.zeros(arx.MAX_PAD_BLOCKS, np.int64)
        launches = np.zeros(arx.MAX_PAD_BLOCKS, np.int64)
        most = arx.MAX_PAD_BLOCKS if lanes else arx.barrier_max_blocks()
        for nblocks, rounds in [(1, 1), (256, 1), (256, 3), (most, 2), (256, 0), (64, 64), (7, 5)]:
            what = f"counter W={W} split={split} lanes={lanes} nblocks={nblocks} rounds={rounds}"
            note(what)
            eseen = torch.full((W, nblocks), -1, dtype=torch.int32, device="cuda")
            tagged = not lanes and rounds > 0
            tags = zeros_u32(W, rounds, nblocks) if tagged else None
            seen = zeros_u32(W, rounds, nblocks, W) if tagged else None
            arx.counter_barrier(nblocks, rounds, flags, eseen, tags, seen)
            torch.cuda.synchronize()
            assert arx.debug_state()["ctl_err"] == 0
            got = eseen.cpu().numpy()
            for r in range(W):
                assert np.array_equal(got[r], launches[:nblocks] % 2), f"{what}: epochs seen by rank {r}"
            rounds_done[:nblocks] += rounds
            launches[:nblocks] += 1
            check_semaphores(W, rounds_done, split, what)
            for r in range(W):
                assert np.array_equal(arx.epoch_view(r).cpu().numpy(), launches % 2), f"{what}: epochs of rank {r}"
            if tagged:
                frac = check_tags(tags, seen, W, nblocks, rounds, split or W == 2, what)
                note(f"  tags seen: {frac:.4f}")


@pytest.mark.parametrize("split", [False, True])
def test_counter_barrier_graph_replays(split):
    """The counter barrier captured in a hipGraph, replayed with eager launches
    between replays: flags and bases keep following the closed form."""
    W = 4
    flags = arx.BARRIER_SPLIT if split else 0
    with library(W, 1024):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            arx.counter_barrier(256, 2, flags)
        done = np.zeros(arx.MAX_PAD_BLOCKS, np.int64)
        for rep in range(5):
            note(f"counter barrier graph replay {rep} split={split}")
            g.replay()
            done[:256] += 2
            if rep % 2:
                arx.counter_barrier(256, 1, flags)
                done[:256] += 1
            torch.cuda.synchronize()
            check_semaphores(W, done, split, f"replay {rep}")
            assert arx.debug_state()["ctl_err"] == 0


def test_barrier_argument_errors():
    """Tag buffers go together and need the default launch; unknown flags,
    and a grid beyond what the device holds at once, are refused before
    anything is launched."""
    W = 4
    with library(W, 1024):
        t = zeros_u32(W, 1, 8)
        s = zeros_u32(W, 1, 8, W)
        for call in (lambda: arx.lib.arx_barrier_blockwise(8, 1, 1, 0, t.data_ptr(), None, None),
                     lambda: arx.lib.arx_barrier_blockwise(8, 1, 1, 0, None, s.data_ptr(), None),
                     lambda: arx.lib.arx_barrier_blockwise(8, 1, 1, arx.BARRIER_LANES, t.data_ptr(), s.data_ptr(),
                                                           None),
                     lambda: arx.lib.arx_barrier_blockwise(8, 1, 1, arx.BARRIER_SPLIT, None, None, None),
                     lambda: arx.lib.arx_barrier_blockwise(8, 1, 1, 4, None, None, None),
                     lambda: arx.lib.arx_counter_barrier(8, 1, 4, None, None, None, None),
                     lambda: arx.lib.arx_counter_barrier(8, 1, arx.BARRIER_LANES, None, t.data_ptr(), s.data_ptr(),
                                                         None)):
            assert call() == arx.EINVAL
        most = arx.barrier_max_blocks()
        if most < arx.MAX_PAD_BLOCKS:
            assert arx.lib.arx_barrier_blockwise(most + 1, 1, 1, 0, None, None, None) == arx.EINVAL
            assert arx.lib.arx_counter_barrier(most + 1, 1, 0, None, None, None, None) == arx.EINVAL
        torch.cuda.synchronize()
        assert not t.any() and not s.any()
        assert pads_zero(W)


def _devapi():
    lib = ctypes.CDLL(DEVAPI)
    lib.devapi_barrier.restype = ctypes.c_int
    lib.devapi_barrier.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                   ctypes.c_void_p]
    return lib


@pytest.mark.parametrize("W", [2, 5, 8])
def test_public_device_barrier_from_a_callers_kernel(W):
    """A kernel built against include/arx_device.h alone calls
    barrier_blockwise(arx_pad_t, block_id) on pads of its own: acq_rel makes
    every peer's tag visible after every round (relaxed: tag or initial
    zero), the pads end zero, no wait times out."""
    assert os.path.exists(DEVAPI), "build tests/devapi first (__graft_entry__.build())"
    lib = _devapi()
    stream = torch.cuda.current_stream().cuda_stream
    for sem in (arx.SEM_ACQ_REL, arx.SEM_RELAXED):
        for nblocks, rounds in [(1, 3), (256, 8), (64, 32)]:
            pads = zeros_u32(W, nblocks * W)
            ptrs = (ctypes.c_void_p * W)(*[pads[r].data_ptr() for r in range(W)])
            tags, seen = zeros_u32(W, rounds, nblocks), zeros_u32(W, rounds, nblocks, W)
            status = zeros_u32(1)
            note(f"public barrier W={W} sem={sem} nblocks={nblocks} rounds={rounds}")
            rc = lib.devapi_barrier(ptrs, W, nblocks, sem, rounds, tags.data_ptr(), seen.data_ptr(),
                                    status.data_ptr(), 0, stream)
            assert rc == 0
            torch.cuda.synchronize()
            assert int(status.item()) == 0
            assert int(pads.abs().sum()) == 0
            frac = check_tags(tags, seen, W, nblocks, rounds, sem == arx.SEM_ACQ_REL,
                              f"public barrier W={W} sem={sem} nblocks={nblocks}")
            note(f"  tags seen: {frac:.4f}")
