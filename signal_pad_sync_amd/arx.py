"""ctypes binding of libarx.so (C ABI in include/arx.h, test aids in
include/arx_test.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels. torch provides device memory and streams; tensors are passed as
``data_ptr()`` and streams as ``torch.cuda.current_stream().cuda_stream``.
Importing this module raises if libarx.so is missing: there is no fallback.
"""
import atexit
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libarx.so")

OK, EINVAL, ESTATE, ENOMEM, EHIP, EPROXY, EORDER, ETIMEOUT = 0, -1, -2, -3, -4, -5, -6, -7
PROXY_LOCKSTEP, PROXY_RUNAHEAD, PROXY_MANUAL, PROXY_STRESS = 0, 1, 2, 3
SEM_RELAXED, SEM_ACQ_REL = 0, 1
BARRIER_LANES, BARRIER_SPLIT = 1, 2
MAX_WORLD, MAX_PAD_BLOCKS, MAX_N = 8, 1024, 1 << 30
NOALLOC_MAX_N = 1 << 20

# names of arx_debug_state's words, in order
STATE_WORDS = ["seq_dev", "cnt0", "cnt1", "go", "abort", "ctl_seq", "ctl_bytes0", "ctl_bytes1",
               "ctl_done", "ctl_err", "ctl_err_seq", "posted"]

_c = ctypes
_u64p = _c.POINTER(_c.c_uint64)

# (name, restype, argtypes) for every entry point of arx.h and arx_test.h
SIGNATURES = [
    ("arx_init", _c.c_int, [_c.c_int, _c.c_size_t]),
    ("arx_init_rank", _c.c_int, [_c.c_int, _c.c_size_t, _c.c_int]),
    ("arx_finalize", _c.c_int, []),
    ("arx_publish", _c.c_int, [_c.c_uint64]),
    ("arx_allreduce", _c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    ("arx_reduce", _c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_int, _c.c_void_p]),
    ("arx_barrier_blockwise", _c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_void_p, _c.c_void_p,
                                         _c.c_void_p]),
    ("arx_counter_barrier", _c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                       _c.c_void_p]),
    ("arx_symm_allreduce", _c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_size_t, _c.c_int, _c.c_void_p]),
    ("arx_symm_allreduce_noalloc", _c.c_int, [_c.c_int, _c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_size_t, _c.c_int,
                                              _c.c_void_p, _c.c_void_p]),
    ("arx_barrier_max_blocks", _c.c_int, []),
    ("arx_sem_ptr", _c.c_void_p, [_c.c_int]),
    ("arx_epoch_ptr", _c.c_void_p, [_c.c_int]),
    ("arx_recv_ptr", _c.c_void_p, [_c.c_int, _c.c_int]),
    ("arx_send_ptr", _c.c_void_p, [_c.c_int]),
    ("arx_pad_ptr", _c.c_void_p, [_c.c_int]),
    ("arx_set_proxy_mode", _c.c_int, [_c.c_int]),
    ("arx_set_stress_source", _c.c_int, [_c.c_void_p, _c.c_int]),
    ("arx_set_timeout_us", _c.c_int, [_c.c_uint64]),
    ("arx_status", _c.c_int, [_u64p, _u64p, _u64p]),
    ("arx_debug_state", _c.c_int, [_u64p, _c.c_int]),
    ("arx_debug_set_seq", _c.c_int, [_c.c_uint64]),
    ("arx_debug_fail_proxy", _c.c_int, []),
    ("arx_test_round_bf16", _c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    ("arx_test_oneshot_shape", _c.c_int, [_c.c_size_t, _c.c_int, _c.c_int, _c.c_uint, _c.c_int,
                                          _c.POINTER(_c.c_int), _c.c_int]),
    ("arx_strerror", _c.c_char_p, [_c.c_int]),
    ("arx_max_n", _c.c_size_t, []),
    ("arx_world", _c.c_int, []),
    ("arx_rank", _c.c_int, []),
]


class ArxError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"arx error {code}: {msg}")
        self.code = code


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"libarx.so not found at {path}; build it with signal_pad_sync_amd/build.py")
    # One HIP runtime per process: torch's. The library receives torch's
    # device pointers and streams, which only that runtime knows. Loaded
    # first, libarx.so would bring in the system's runtime, and torch would
    # then load its own copy beside it (torch's libraries name the runtime
    # by another file name), and one of the two would see no device. torch
    # loaded first, libarx.so binds to its runtime by soname.
    import torch  # noqa: F401
    L = ctypes.CDLL(path)
    for name, res, args in SIGNATURES:
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


lib = load()


@atexit.register
def _finalize_at_exit():
    if lib.arx_world() != 0:
        lib.arx_finalize()


def _check(rc):
    if rc < 0:
        raise ArxError(rc, lib.arx_strerror(rc).decode())
    return rc


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _buf(t, n: int, what: str, itemsize: int = 2):
    """Device address of tensor t, after checking that it is a contiguous GPU
    tensor of itemsize-byte elements holding at least n of them (the library
    sees only the address, so it cannot check the extent itself)."""
    if t is None:
        if n > 0:
            raise ArxError(EINVAL, f"{what} is None")
        return None
    if not getattr(t, "is_cuda", False):
        raise ArxError(EINVAL, f"{what} must be a GPU tensor")
    if t.element_size() != itemsize:
        raise ArxError(EINVAL, f"{what} must have {itemsize}-byte elements, not {t.dtype}")
    if not t.is_contiguous():
        raise ArxError(EINVAL, f"{what} must be contiguous")
    if t.numel() < n:
        raise ArxError(EINVAL, f"{what} holds {t.numel()} elements, fewer than {n}")
    return t.data_ptr()


def init(world: int, max_n: int, rank: int = 0):
    _check(lib.arx_init_rank(world, max_n, rank))


def finalize():
    _check(lib.arx_finalize())


def publish(seq: int):
    _check(lib.arx_publish(seq))


def allreduce(inp, out, n: int = None, stream=None):
    """One one-shot call: out[:n] = rank-ordered sum; inp/out bf16 tensors."""
    if n is None:
        n = inp.numel()
    _check(lib.arx_allreduce(_buf(inp, n, "inp"), _buf(out, n, "out"), n, _stream(stream)))


def reduce(inp, out, par: int, n: int = None, stream=None):
    if n is None:
        n = inp.numel()
    _check(lib.arx_reduce(_buf(inp, n, "inp"), _buf(out, n, "out"), n, par, _stream(stream)))


def _tag_bufs(tags, seen, rounds: int, nblocks: int):
    """Addresses of a tag check's buffers: tags u32 [W, rounds, nblocks] and
    seen u32 [W, rounds, nblocks, W], both given or neither."""
    if tags is None and seen is None:
        return None, None
    if tags is None or seen is None:
        raise ArxError(EINVAL, "tags and seen go together")
    W = world()
    return _buf(tags, W * rounds * nblocks, "tags", 4), _buf(seen, W * rounds * nblocks * W, "seen", 4)


def barrier_blockwise(nblocks: int, sem: int = SEM_ACQ_REL, rounds: int = 1, flags: int = 0, tags=None, seen=None,
                      stream=None):
    """W * nblocks workgroups (or nblocks with flags=BARRIER_LANES) pass the
    blockwise barrier `rounds` times; tags / seen: int32 device tensors for
    the tag check (arx.h, barrier tags)."""
    tp, sp = _tag_bufs(tags, seen, rounds, nblocks)
    _check(lib.arx_barrier_blockwise(nblocks, sem, rounds, flags, tp, sp, _stream(stream)))


def counter_barrier(nblocks: int, rounds: int = 1, flags: int = 0, epochs_seen=None, tags=None, seen=None,
                    stream=None):
    """epochs_seen: optional int32 device tensor [W, nblocks] receiving each
    rank's block's epoch; tags / seen as for barrier_blockwise."""
    ptr = None if epochs_seen is None else _buf(epochs_seen, world() * nblocks, "epochs_seen", 4)
    tp, sp = _tag_bufs(tags, seen, rounds, nblocks)
    _check(lib.arx_counter_barrier(nblocks, rounds, flags, ptr, tp, sp, _stream(stream)))


def symm_allreduce_noalloc(world_size: int, inputs, outputs, n: int, iters: int, status=None, stream=None):
    """The symmetric exchange with no allocation and no library instance:
    inputs / outputs bf16 device tensors [iters, W, ld]; status: optional
    int32 device tensor of one element, set to 1 on a timeout."""
    ld = inputs.shape[-1]
    if tuple(outputs.shape[-1:]) != (ld,):
        raise ArxError(EINVAL, "inputs and outputs must have the same last dimension")
    need = iters * world_size * ld
    sp = None if status is None else _buf(status, 1, "status", 4)
    _check(lib.arx_symm_allreduce_noalloc(world_size, _buf(inputs, need, "inputs"), _buf(outputs, need, "outputs"),
                                          n, ld, iters, sp, _stream(stream)))


def barrier_max_blocks() -> int:
    """Largest nblocks of a barrier launch with one workgroup per rank and block."""
    return _check(lib.arx_barrier_max_blocks())


def symm_allreduce(inputs, outputs, n: int, iters: int, stream=None):
    """inputs / outputs: bf16 device tensors [iters, W, ld] (ld >= n, ld % 8 == 0)."""
    ld = inputs.shape[-1]
    if tuple(outputs.shape[-1:]) != (ld,):
        raise ArxError(EINVAL, "inputs and outputs must have the same last dimension")
    need = iters * world() * ld
    _check(lib.arx_symm_allreduce(_buf(inputs, need, "inputs"), _buf(outputs, need, "outputs"), n, ld, iters,
                                  _stream(stream)))


def sem_view(rank: int):
    """int32 tensor viewing rank `rank`'s semaphores, shape [MAX_PAD_BLOCKS, 32]
    (flag in column 0, base in column 1; the split design's end-stage flag in
    column 16, its base in column 17)."""
    return _view(lib.arx_sem_ptr(rank), MAX_PAD_BLOCKS * 32, "<i4", None).view(MAX_PAD_BLOCKS, 32)


def epoch_view(rank: int):
    """int32 tensor viewing rank `rank`'s per-block epochs, shape [MAX_PAD_BLOCKS]."""
    return _view(lib.arx_epoch_ptr(rank), MAX_PAD_BLOCKS, "<i4", None)


def set_proxy_mode(mode: int):
    _check(lib.arx_set_proxy_mode(mode))


def set_stress_source(pool, sets: int):
    """pool: bf16 device tensor [sets, W, max_n] (kept alive by the caller);
    None (or sets 0) clears the source."""
    ptr = None if pool is None or sets == 0 else _buf(pool, max(sets, 0) * world() * max_n(), "pool")
    _check(lib.arx_set_stress_source(ptr, sets))


def set_timeout_us(us: int):
    _check(lib.arx_set_timeout_us(us))


def status():
    a, b, c = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
    _check(lib.arx_status(ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


def debug_state() -> dict:
    buf = (ctypes.c_uint64 * 32)()
    m = _check(lib.arx_debug_state(buf, 32))
    d = {name: buf[i] for i, name in enumerate(STATE_WORDS)}
    d["flags"] = [buf[i] for i in range(len(STATE_WORDS), m)]
    return d


def debug_set_seq(seq: int):
    _check(lib.arx_debug_set_seq(seq))


def debug_fail_proxy():
    _check(lib.arx_debug_fail_proxy())


def max_n() -> int:
    return lib.arx_max_n()


def world() -> int:
    return lib.arx_world()


def test_round_bf16(inp_u32, out_u16, stream=None):
    n = inp_u32.numel()
    _check(lib.arx_test_round_bf16(_buf(inp_u32, n, "inp_u32", 4), _buf(out_u16, n, "out_u16"), n,
                                   _stream(stream)))


def test_oneshot_shape(n, world=8, block=0, resident=257, in_place=False) -> dict:
    out = (_c.c_int * 8)()
    _check(lib.arx_test_oneshot_shape(n, world, block, resident, 1 if in_place else 0, out, 8))
    return dict(zip(("block", "grid", "launched", "ncopy", "one_pass", "early_go", "nt_copy", "nt_peer"), list(out)))


class _DevArray:
    """__cuda_array_interface__ view of library-owned device memory."""

    def __init__(self, ptr, n, typestr):
        self.__cuda_array_interface__ = {"shape": (n,), "typestr": typestr, "data": (ptr, False),
                                         "version": 2, "strides": None}


def _view(ptr, n, typestr, dtype):
    import torch
    if not ptr:
        raise ArxError(EINVAL, "null slot (library not initialised or index out of range)")
    t = torch.as_tensor(_DevArray(ptr, n, typestr), device="cuda")
    return t.view(dtype) if dtype is not None else t


def _slot_len(n):
    m = max_n()
    if n is None:
        return m
    if not 0 < n <= m:
        raise ArxError(EINVAL, f"a slot view holds 1 to max_n = {m} elements, not {n}")
    return n


def recv_view(par: int, src: int, n: int = None):
    """bf16 tensor viewing recv slot [par][src] (library memory, no copy)."""
    import torch
    return _view(lib.arx_recv_ptr(par, src), _slot_len(n), "<i2", torch.bfloat16)


def send_view(par: int, n: int = None):
    import torch
    return _view(lib.arx_send_ptr(par), _slot_len(n), "<i2", torch.bfloat16)


def pad_view(rank: int):
    """int32 tensor viewing virtual rank `rank`'s pad, shape [MAX_PAD_BLOCKS, W]."""
    W = world()
    return _view(lib.arx_pad_ptr(rank), MAX_PAD_BLOCKS * W, "<i4", None).view(MAX_PAD_BLOCKS, W)
