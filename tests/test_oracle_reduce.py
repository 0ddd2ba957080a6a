"""Pins for the oracle's rank-ordered reduction (CPU only).

Page "arx.cu", arx_kernel: the W bf16 partials are widened, added in rank
order in binary32 and rounded once to bf16. The oracle is pinned against
hand-worked cases, closed forms (one-hot partials, W identical partials),
an exact rational emulation of binary32 addition, and an independent numpy
float32 loop on the full workloads.
"""
import numpy as np
import pytest
import torch

from oracle import reduce as R
from signal_pad_sync_amd import workloads as WL
from tests import ieee_ref as ref
from tests.conftest import read_golden


def _parse_golden():
    cases = []
    for ln in read_golden("reduce_cases.txt"):
        lhs, rest = ln.split("->", 1)
        want = int(rest.split(";")[0].strip(), 16)
        parts = [int(x, 16) for x in lhs.strip().split(",")]
        cases.append((parts, want, ln))
    return cases


def test_golden_reduce_cases():
    for parts, want, ln in _parse_golden():
        arrs = [np.array([p], dtype=np.uint16) for p in parts]
        got = int(R.reduce(arrs)[0])
        assert got == want, (ln, hex(got))
        # the exact emulation agrees with the hand-worked value too
        assert ref.reduce_exact([parts])[0] == want, ln


def test_one_hot_reproduces_inputs():
    """Only partial k(i) is nonzero at each i -> out == x_k bit-exact
    (x + 0 == x for every non-NaN x; NaN -> 0x7FC0)."""
    rng = np.random.default_rng(11)
    for W in range(1, 9):
        n = 5000
        x = rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16)
        k = rng.integers(0, W, n)
        zero = np.where(rng.random((W, n)) < 0.5, 0x8000, 0).astype(np.uint16)
        parts = [np.where(k == w, x, zero[w]).astype(np.uint16) for w in range(W)]
        got = R.reduce(parts)
        is_nan = ((x >> 7) & 0xFF == 0xFF) & ((x & 0x7F) != 0)
        want = np.where(is_nan, 0x7FC0, x)
        # a column of nothing but -0 with x = -0 sums to -0, with x = +0 to +0:
        # x itself either way, so the rule holds everywhere
        assert np.array_equal(got, want), W


def test_identical_partials_give_rounded_multiple():
    """W identical partials -> bf16(W * x): k * x is exact in binary32 for a
    bf16 x and k <= 8 (at most 11 significand bits), so the only rounding is
    the final one, computed here from the definition."""
    rng = np.random.default_rng(12)
    xs = rng.integers(0, 1 << 16, 3000, dtype=np.uint32).astype(np.uint16)
    xs = np.concatenate([xs, np.array([0x0000, 0x8000, 0x0001, 0x807F, 0x7F7F, 0x7F00, 0x3F81, 0x3F80],
                                      dtype=np.uint16)])
    for W in (2, 3, 4, 5, 7, 8):
        got = R.reduce([xs] * W)
        for x, g in zip(xs.tolist(), got.tolist()):
            kind, sign, mag = ref.decode(x, 16)
            if kind == "num":
                # partial sums k*x, k < W, stay below the binary32 overflow
                # threshold unless k*x itself is past it
                partial = [ref.round_to(k * mag, ref.F32_P) for k in range(1, W + 1)]
                if any(p is None for p in partial):
                    want = ref.encode(sign, None, 16)
                else:
                    want = ref.bf16_of_value("num", sign, W * mag)
            else:
                want = ref.bf16_of_value(kind, sign, mag)
            assert g == want, (W, hex(x), hex(g), hex(want))


def test_exact_emulation_random_columns():
    """Random columns mixing large, small, subnormal, zero and special values:
    the oracle equals the rational emulation of rank-ordered binary32 adds."""
    rng = np.random.default_rng(13)
    cols = []
    for W in (2, 3, 4, 8):
        parts = WL.adversarial(99 + W, W, 400)
        for i in range(400):
            cols.append([int(parts[w][i]) for w in range(W)])
        raw = rng.integers(0, 1 << 16, (300, W), dtype=np.uint32)
        cols += [[int(v) for v in row] for row in raw]
    for col in cols:
        want = ref.reduce_exact([col])[0]
        got = int(R.reduce([np.array([v], np.uint16) for v in col])[0])
        assert got == want, ([hex(v) for v in col], hex(got), hex(want))


def _numpy_loop(parts, n):
    """Independent statement of the sum: numpy float32 adds in rank order,
    torch's float32 -> bfloat16 rounding, NaN canonicalised."""
    acc = np.full(n, -0.0, dtype=np.float32)
    for p in parts:
        acc = acc + (p[:n].astype(np.uint32) << 16).view(np.float32)
    out = torch.from_numpy(acc).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    out[np.isnan(acc)] = 0x7FC0
    return out


@pytest.mark.parametrize("cfg", [1, 2, 5])
def test_matches_numpy_float32_loop_on_workloads(cfg):
    w = WL.WORKLOADS[cfg]
    n = w["n"]
    for par in (0, 1):
        parts = WL.recv_partials(cfg, par, n)
        with np.errstate(invalid="ignore", over="ignore"):
            want = _numpy_loop(parts, n)
        got = R.reduce(parts, n=n)
        assert np.array_equal(got, want), cfg


def test_workload3_sizes_match_numpy_loop():
    for n in WL.WORKLOADS[3]["ns"]:
        parts = WL.recv_partials(3, 1, n)
        assert np.array_equal(R.reduce(parts, n=n), _numpy_loop(parts, n))


def test_tail_and_untouched():
    """Any n; elements at or past n keep their previous contents."""
    W = 8
    parts = WL.recv_partials(5, 1, 131072)
    full = R.reduce(parts, n=131072)
    for n in (0, 1, 7, 8, 9, 15, 16, 17, 1000, 131071):
        out = np.full(131072, 0xDEAD, dtype=np.uint16)
        R.reduce(parts, n=n, out=out)
        assert np.array_equal(out[:n], full[:n]), n
        assert np.all(out[n:] == 0xDEAD), n


def test_thread_count_does_not_change_bits():
    parts = WL.recv_partials(2, 0, 131072)
    one = R.reduce(parts)
    for t in (2, 3, 8, 17):
        assert np.array_equal(R.reduce(parts, threads=t), one)


def test_within_one_bf16_ulp_of_exact_sum():
    """Sanity on well-conditioned data: the rank-ordered binary32 sum rounded
    once is within one bf16 ulp of the exact sum rounded once."""
    parts = WL.recv_partials(1, 1, 8192)
    got = R.reduce(parts)
    exact = sum((p.astype(np.uint32) << 16).view(np.float32).astype(np.float64) for p in parts)
    g = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    # one bf16 ulp at |exact|: 2^(floor(log2|x|) - 7)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(exact), 1e-30))) - 7)
    assert np.all(np.abs(g - exact) <= ulp)


def test_rank_order_is_observable():
    """Summing in another order changes bits on workload 5 (so a GPU that sums
    out of rank order cannot pass a bit-exact comparison)."""
    parts = WL.recv_partials(5, 0, 131071)
    fwd = R.reduce(parts)
    rev = R.reduce(parts[::-1])
    assert np.count_nonzero(fwd != rev) > 100
