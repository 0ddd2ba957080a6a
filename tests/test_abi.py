"""The C ABI library loads and exports exactly what include/arx.h declares,
and its host-side argument checks work without a GPU (CPU only: none of
these calls reaches the device)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "arx.h")
LIB = os.path.join(ROOT, "signal_pad_sync_amd", "libarx.so")


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(arx_\w+)\s*\(", src, flags=re.M)))


def exported():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], check=True, capture_output=True, text=True).stdout
    return sorted({ln.split()[-1] for ln in out.splitlines() if " T " in ln and ln.split()[-1].startswith("arx_")})


def test_header_declares_the_boundary():
    names = declared()
    for must in ("arx_init", "arx_publish", "arx_allreduce", "arx_barrier_blockwise", "arx_reduce"):
        assert must in names
    assert len(names) >= 15


def test_library_exports_every_declared_symbol_and_no_other():
    assert os.path.exists(LIB), "build libarx.so first (__graft_entry__.build())"
    assert exported() == declared()


def test_binding_covers_every_symbol():
    from signal_pad_sync_amd import arx
    assert sorted(n for n, _, _ in arx.SIGNATURES) == declared()


def test_library_has_gfx950_code_object():
    out = subprocess.run(["readelf", "-S", LIB], check=True, capture_output=True, text=True).stdout
    assert ".hip_fatbin" in out
    assert b"amdgcn-amd-amdhsa--gfx950" in open(LIB, "rb").read()


@pytest.fixture(scope="module")
def L():
    from signal_pad_sync_amd import arx
    return arx.lib


def test_host_checks_before_init(L):
    from signal_pad_sync_amd import arx
    assert L.arx_max_n() == 0 and L.arx_world() == 0 and L.arx_rank() == 0
    assert L.arx_publish(1) == arx.ESTATE
    assert L.arx_allreduce(None, None, 0, None) == arx.ESTATE
    assert L.arx_reduce(None, None, 0, 0, None) == arx.ESTATE
    assert L.arx_barrier_blockwise(1, 1, 1, None) == arx.ESTATE
    assert L.arx_set_proxy_mode(0) == arx.ESTATE
    assert L.arx_set_timeout_us(10) == arx.ESTATE
    assert L.arx_finalize() == arx.ESTATE
    assert L.arx_status(None, None, None) == arx.ESTATE
    assert L.arx_recv_ptr(0, 0) is None and L.arx_send_ptr(0) is None and L.arx_pad_ptr(0) is None
    assert b"not initialised" in L.arx_strerror(arx.ESTATE)


def test_init_argument_checks_need_no_gpu(L):
    from signal_pad_sync_amd import arx
    for world, max_n, rank in [(1, 16, 0), (9, 16, 0), (0, 16, 0), (2, 0, 0), (2, (1 << 30) + 1, 0),
                               (4, 16, 4), (4, 16, -1)]:
        assert L.arx_init_rank(world, max_n, rank) == arx.EINVAL, (world, max_n, rank)
    assert L.arx_world() == 0


def test_round_test_entry_with_nothing_to_do(L):
    assert L.arx_test_round_bf16(None, None, 0, None) == 0
    assert L.arx_test_round_bf16(None, None, 5, None) == -1


def test_strerror_codes(L):
    for code in range(-7, 1):
        assert L.arx_strerror(code)
    assert L.arx_strerror(-99) == b"unknown error"
