"""The one-shot launch shape on the CPU (the library's host-side rules,
through arx_test_oneshot_shape; no device is touched): the block size for
n and the number of partials W, 256 threads up to 32 reducing workgroups,
512 up to 64 (48 at W <= 4), else 1024; at most 256 reducing workgroups (at least one) and the workgroup that waits
for the flags besides; half of them copy from 64 on unless out == in; go
may precede the publish only while a copying thread copies at most 4
vectors."""
import pytest

from signal_pad_sync_amd import arx

# (n, resident, in_place) at W = 8 -> block, reducing grid, launched, copiers, one pass, early go
CASES = [
    ((0, 257, False), (256, 1, 2, 1, 1, 1)),
    ((8, 257, False), (256, 1, 2, 1, 1, 1)),
    ((1000, 257, False), (256, 1, 2, 1, 1, 1)),          # 125 vectors and a tail
    ((4096, 257, False), (256, 2, 3, 2, 1, 1)),
    ((8192, 257, False), (256, 4, 5, 4, 1, 1)),
    ((8200, 257, False), (256, 5, 6, 5, 1, 1)),          # 1025 vectors
    ((65536, 257, False), (256, 32, 33, 32, 1, 1)),
    ((65544, 257, False), (512, 17, 18, 17, 1, 1)),
    ((131072, 257, False), (512, 32, 33, 32, 1, 1)),     # the headline: 32 of 512 and the poll workgroup
    ((262144, 257, False), (512, 64, 65, 32, 1, 1)),     # 64 from here on: half copy
    ((262144, 257, True), (512, 64, 65, 64, 1, 1)),      # in place: every one copies
    ((2097152, 257, False), (1024, 256, 257, 128, 1, 1)),
    (((1 << 22) + 5, 257, False), (1024, 256, 257, 128, 0, 1)),   # 4 vectors per copying thread
    ((1 << 23, 257, False), (1024, 256, 257, 128, 0, 0)),         # 8: go after the publish
    ((1 << 23, 257, True), (1024, 256, 257, 256, 0, 1)),          # in place, 4 per copying thread
    ((1 << 30, 257, False), (1024, 256, 257, 128, 0, 0)),
    ((131072, 32, False), (512, 31, 32, 31, 0, 1)),      # 32 resident (a partition of 32 CUs)
    ((131072, 2, False), (512, 1, 2, 1, 0, 0)),          # room for the poll workgroup and one more
    ((131072, 100000, False), (512, 32, 33, 32, 1, 1)),  # resident capped at 257
]


# (n, W) -> the same; 512 threads end at 48 workgroups for W <= 4
CASES_W = [
    ((196608, 2), (512, 48, 49, 48, 1, 1)),
    ((196616, 2), (1024, 25, 26, 25, 1, 1)),         # one vector past 48 x 512
    ((196616, 4), (1024, 25, 26, 25, 1, 1)),
    ((196616, 5), (512, 49, 50, 49, 1, 1)),
    ((262144, 3), (1024, 32, 33, 32, 1, 1)),
    ((262144, 5), (512, 64, 65, 32, 1, 1)),
    ((131072, 2), (512, 32, 33, 32, 1, 1)),
    ((8192, 2), (256, 4, 5, 4, 1, 1)),
    ((1 << 20, 2), (1024, 128, 129, 64, 1, 1)),
]

FIELDS = ("block", "grid", "launched", "ncopy", "one_pass", "early_go")


@pytest.mark.parametrize("args,want", CASES)
def test_oneshot_shape(args, want):
    n, resident, in_place = args
    got = arx.test_oneshot_shape(n, 8, 0, resident, in_place)
    assert tuple(got[k] for k in FIELDS) == want, got


@pytest.mark.parametrize("args,want", CASES_W)
def test_oneshot_shape_by_world(args, want):
    n, W = args
    got = arx.test_oneshot_shape(n, W)
    assert tuple(got[k] for k in FIELDS) == want, got


def test_oneshot_shape_forced_block():
    assert arx.test_oneshot_shape(131072, 8, 1024)["grid"] == 16
    assert arx.test_oneshot_shape(131072, 8, 256)["grid"] == 64
    assert arx.test_oneshot_shape(131072, 8, 256)["ncopy"] == 32


@pytest.mark.parametrize("n,W,block,resident", [((1 << 30) + 1, 8, 0, 257), (64, 8, 128, 257), (64, 8, 0, 0),
                                                (64, 8, 0, 1), (64, 1, 0, 257), (64, 9, 0, 257)])
def test_oneshot_shape_refuses(n, W, block, resident):
    with pytest.raises(arx.ArxError) as e:
        arx.test_oneshot_shape(n, W, block, resident)
    assert e.value.code == arx.EINVAL


@pytest.mark.parametrize("n,W,copy,peer", [
    (1 << 20, 8, 0, 0), ((8 << 20) - 1, 8, 0, 0), (8 << 20, 8, 1, 0), (12 << 20, 8, 1, 0),
    (14 << 20, 8, 1, 1), (1 << 30, 8, 1, 1),
    (16 << 20, 4, 0, 0), ((56 << 20) // 3 + 1, 4, 1, 0), (32 << 20, 4, 1, 1),
    (32 << 20, 2, 0, 0), (56 << 20, 2, 1, 0), (96 << 20, 2, 1, 1)])
def test_oneshot_cache_policies_past_the_last_level_cache(n, W, copy, peer):
    """The copy's stores turn nontemporal once both parities' peer slots
    take 224 MiB (n (W - 1) >= 56 Mi), the peer loads once they take
    384 MiB (n (W - 1) >= 96 Mi); the grid loops there at every block
    size, where the policies apply."""
    want_copy = int(n * (W - 1) >= 56 << 20)
    want_peer = int(n * (W - 1) >= 96 << 20)
    assert (want_copy, want_peer) == (copy, peer)
    for block in (0, 256, 1024):
        got = arx.test_oneshot_shape(n, W, block)
        assert (got["nt_copy"], got["nt_peer"]) == (want_copy, want_peer), (n, W, block, got)
        if want_copy:
            assert got["one_pass"] == 0, got
