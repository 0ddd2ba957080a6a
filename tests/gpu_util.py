"""Helpers for the GPU tests: moving bf16 bit patterns between numpy and
device tensors, filling the library's recv slots, and a context that
initialises / finalises the library."""
import contextlib
import sys

import numpy as np
import torch

from signal_pad_sync_amd import arx


def note(msg):
    """Names the case before a GPU step (flushed, so it survives a crash)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray, pad_to: int = None) -> torch.Tensor:
    """uint16 bf16 patterns -> bf16 device tensor (optionally zero-padded)."""
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    if pad_to is not None and pad_to > a.size:
        a = np.concatenate([a, np.zeros(pad_to - a.size, np.uint16)])
    return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def sentinel(n: int, value: int = 0xDEAD) -> torch.Tensor:
    return to_dev(np.full(n, value, dtype=np.uint16))


def fill_recv(parts_by_par, rank: int):
    """parts_by_par[par][src] (uint16 arrays) -> recv slot [par][src], src != rank."""
    for par, parts in enumerate(parts_by_par):
        if parts is None:
            continue
        for src, p in enumerate(parts):
            if src == rank or p is None:
                continue
            view = arx.recv_view(par, src, p.size)
            view.copy_(to_dev(p))
    torch.cuda.synchronize()


@contextlib.contextmanager
def library(world: int, max_n: int, rank: int = 0, mode: int = arx.PROXY_LOCKSTEP, timeout_us: int = None):
    note(f"init world={world} max_n={max_n} rank={rank} mode={mode}")
    arx.init(world, max_n, rank)
    try:
        arx.set_proxy_mode(mode)
        if timeout_us is not None:
            arx.set_timeout_us(timeout_us)
        yield
    finally:
        torch.cuda.synchronize()
        arx.finalize()
