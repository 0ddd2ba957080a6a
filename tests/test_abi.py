"""The C ABI library loads and exports exactly what include/arx.h and
include/arx_test.h declare, the public device header compiles on its own in
a caller's code, and the library's host-side argument checks work without a
GPU (CPU only: none of these calls reaches the device)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("arx.h", "arx_test.h")]
DEVICE_HEADER = os.path.join(ROOT, "include", "arx_device.h")
DEVAPI_LIB = os.path.join(ROOT, "tests", "devapi", "libdevapi_user.so")
LIB = os.path.join(ROOT, "signal_pad_sync_amd", "libarx.so")


def declared(headers=HEADERS):
    names = set()
    for h in headers:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^[A-Za-z_][\w \*]*?\b(arx_\w+)\s*\(", src, flags=re.M))
    return sorted(names)


def exported():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], check=True, capture_output=True, text=True).stdout
    return sorted({ln.split()[-1] for ln in out.splitlines() if " T " in ln and ln.split()[-1].startswith("arx_")})


def test_header_declares_the_boundary():
    names = declared(HEADERS[:1])
    for must in ("arx_init", "arx_publish", "arx_allreduce", "arx_barrier_blockwise", "arx_reduce"):
        assert must in names
    assert len(names) >= 15
    aids = declared(HEADERS[1:])
    assert aids == ["arx_debug_fail_proxy", "arx_debug_set_seq", "arx_debug_state", "arx_test_oneshot_shape",
                    "arx_test_round_bf16"]
    assert not set(aids) & set(names)


def test_device_header_declares_the_barrier():
    """include/arx_device.h: arx_pad_t {ptr[8], rank, W, sem, timeout} and
    barrier_blockwise(arx_pad_t, uint32_t block_id), header-only."""
    src = open(DEVICE_HEADER).read()
    assert re.search(r"typedef struct arx_pad \{[^}]*uint32_t\* ptr\[8\];[^}]*int rank;[^}]*int W;[^}]*int sem;"
                     r"[^}]*uint64_t timeout;[^}]*\} arx_pad_t;", src, flags=re.S)
    assert re.search(r"__device__ __forceinline__ bool barrier_blockwise\(arx_pad_t pad, uint32_t block_id\)", src)


def test_device_header_builds_alone(tmp_path):
    """A caller's kernel that includes arx_device.h and nothing else of the
    library compiles for gfx950 (device code only, no GPU needed)."""
    src = tmp_path / "user.hip"
    src.write_text('#include "arx_device.h"\n'
                   '__global__ void k(arx_pad_t p, int* ok) { ok[threadIdx.x] = barrier_blockwise(p, blockIdx.x); }\n')
    r = subprocess.run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "--cuda-device-only", "-c", "-O3",
                        "-I", os.path.join(ROOT, "include"), str(src), "-o", str(tmp_path / "user.o")],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr


def test_devapi_test_library_uses_only_the_public_header():
    """The test library of the public device barrier includes arx_device.h
    and no private header, and exports its one entry point."""
    src = open(os.path.join(ROOT, "tests", "devapi", "devapi_user.hip")).read()
    assert re.findall(r'#include "([^"]+)"', src) == ["arx_device.h"]
    assert os.path.exists(DEVAPI_LIB), "build it first (__graft_entry__.build())"
    out = subprocess.run(["nm", "-D", "--defined-only", DEVAPI_LIB], check=True, capture_output=True,
                         text=True).stdout
    assert "devapi_barrier" in out


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
    assert L.arx_barrier_blockwise(1, 1, 1, 0, None, None, None) == arx.ESTATE
    assert L.arx_counter_barrier(1, 1, 0, None, None, None, None) == arx.ESTATE
    assert L.arx_barrier_max_blocks() == arx.ESTATE
    assert L.arx_epoch_ptr(0) is None and L.arx_sem_ptr(0) is None
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


def test_noalloc_argument_checks_need_no_gpu(L):
    """arx_symm_allreduce_noalloc refuses bad arguments before any HIP call:
    world, n beyond ARX_NOALLOC_MAX_N, ld, iters, alignment, overlap."""
    from signal_pad_sync_amd import arx
    big = arx.NOALLOC_MAX_N
    base = 1 << 20
    for args in [(1, base, base + 4096, 8, 8, 1, None), (9, base, base + 4096, 8, 8, 1, None),
                 (2, base, base + (1 << 24), big + 1, big + 8, 1, None),
                 (2, base, base + 4096, 16, 8, 1, None), (2, base, base + 4096, 9, 12, 1, None),
                 (2, base, base + 4096, 8, 8, 0, None), (2, base, base + 4096, 8, 8, 65537, None),
                 (2, None, base, 8, 8, 1, None), (2, base + 8, base + 4096, 8, 8, 1, None),
                 (2, base, base + 4096, 8, 8, 1, base + 8192 + 2),
                 (2, base, base + 16, 8, 8, 1, None)]:
        assert L.arx_symm_allreduce_noalloc(*args, None) == arx.EINVAL, args
