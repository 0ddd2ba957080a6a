"""The Python binding's own checks (CPU only). The library sees addresses
only, so the binding checks each tensor's device, element size, layout and
extent before a call; a stand-in object with a tensor's attributes drives
every branch without a GPU, and no call below reaches the device."""
import os
import subprocess
import sys

import pytest

from signal_pad_sync_amd import arx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


class FakeTensor:
    def __init__(self, numel, itemsize=2, cuda=True, contiguous=True, shape=None):
        self._numel, self._itemsize, self.is_cuda, self._contig = numel, itemsize, cuda, contiguous
        self.shape = shape or (numel,)
        self.dtype = f"{itemsize}-byte"

    def numel(self):
        return self._numel

    def element_size(self):
        return self._itemsize

    def is_contiguous(self):
        return self._contig

    def data_ptr(self):
        return 0x10000


@pytest.mark.parametrize("t,n,itemsize,why", [
    (None, 1, 2, "is None"),
    (FakeTensor(100, cuda=False), 8, 2, "GPU tensor"),
    (FakeTensor(100, itemsize=4), 8, 2, "2-byte elements"),
    (FakeTensor(100, contiguous=False), 8, 2, "contiguous"),
    (FakeTensor(100), 101, 2, "fewer than 101"),
    (FakeTensor(7, itemsize=2), 8, 4, "4-byte elements"),
])
def test_buf_rejects(t, n, itemsize, why):
    with pytest.raises(arx.ArxError) as e:
        arx._buf(t, n, "x", itemsize)
    assert e.value.code == arx.EINVAL and why in str(e.value)


def test_buf_accepts():
    assert arx._buf(FakeTensor(100), 100, "x") == 0x10000
    assert arx._buf(FakeTensor(8, itemsize=4), 8, "x", 4) == 0x10000
    assert arx._buf(None, 0, "x") is None          # n = 0 needs no buffer


def test_calls_check_before_the_library():
    """A short buffer is refused by the binding (EINVAL), not passed on: the
    uninitialised library would have answered ESTATE."""
    assert arx.world() == 0
    with pytest.raises(arx.ArxError) as e:
        arx.allreduce(FakeTensor(1000), FakeTensor(999), 1000, stream=0)
    assert e.value.code == arx.EINVAL
    with pytest.raises(arx.ArxError) as e:
        arx.reduce(FakeTensor(10), FakeTensor(1000), 0, 1000, stream=0)
    assert e.value.code == arx.EINVAL
    with pytest.raises(arx.ArxError) as e:
        arx.counter_barrier(16, 1, epochs_seen=FakeTensor(16, itemsize=2), stream=0)
    assert e.value.code == arx.EINVAL
    with pytest.raises(arx.ArxError) as e:
        arx.barrier_blockwise(16, arx.SEM_ACQ_REL, 1, tags=FakeTensor(64, itemsize=4), stream=0)
    assert e.value.code == arx.EINVAL and "go together" in str(e.value)
    with pytest.raises(arx.ArxError) as e:        # extents fine: the library itself refuses
        arx.allreduce(FakeTensor(1000), FakeTensor(1000), 1000, stream=0)
    assert e.value.code == arx.ESTATE


def test_one_hip_runtime_per_process():
    """Importing the binding first (before torch) must still leave a single
    HIP runtime and a single HSA runtime mapped: torch's, which is the one
    that owns the tensors and streams the library is handed."""
    code = ("from signal_pad_sync_amd import arx\n"
            "import torch\n"
            "libs = {ln.split()[-1] for ln in open('/proc/self/maps') if 'libamdhip64' in ln or 'libhsa-runtime64' in ln}\n"
            "print(sorted(libs))\n"
            "assert sum('libamdhip64' in x for x in libs) == 1, libs\n"
            "assert sum('libhsa-runtime64' in x for x in libs) == 1, libs\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr


def test_missing_library_fails_loudly(tmp_path):
    """There is no fallback path: without libarx.so the binding refuses to
    load."""
    with pytest.raises(ImportError, match="libarx.so not found"):
        arx.load(str(tmp_path / "libarx.so"))
