"""Pins for the oracle's bf16 conversions (CPU only).

The oracle's binary32 -> bf16 rounding is checked three independent ways:
hand-worked cases from the IEEE definition (tests/golden), the exact
definition computed with rationals on structured and random patterns, and an
exhaustive sweep of all 2^32 patterns against torch's CPU float32 -> bfloat16
conversion (a library routine) on every non-NaN input.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from oracle import reduce as R
from tests import ieee_ref as ref
from tests.conftest import read_golden


def test_golden_round_cases():
    rows = [ln.split()[:2] for ln in read_golden("bf16_round_cases.txt")]
    f = np.array([int(a, 16) for a, _ in rows], dtype=np.uint32)
    want = np.array([int(b, 16) for _, b in rows], dtype=np.uint16)
    got = R.round_bf16(f)
    bad = [(hex(a), hex(b), hex(c)) for a, b, c in zip(f, want, got) if b != c]
    assert not bad, bad


def _structured_patterns():
    """Every exponent x sign x fraction endings around the tie points."""
    tails = [0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000]
    heads = [0x00, 0x01, 0x02, 0x3F, 0x40, 0x7E, 0x7F]   # the 7 kept fraction bits
    pats = []
    for sign in (0, 1):
        for exp in range(0, 256):
            for h in heads:
                for t in tails:
                    pats.append((sign << 31) | (exp << 23) | (h << 16) | t)
    return np.array(pats, dtype=np.uint32)


def test_round_matches_definition_structured():
    pats = _structured_patterns()
    got = R.round_bf16(pats)
    for p, g in zip(pats.tolist(), got.tolist()):
        want = ref.bf16_of_value(*ref.decode(p, 32))
        assert g == want, (hex(p), hex(g), hex(want))


def test_round_matches_definition_random():
    rng = np.random.default_rng(7)
    pats = rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32)
    got = R.round_bf16(pats)
    for p, g in zip(pats.tolist(), got.tolist()):
        assert g == ref.bf16_of_value(*ref.decode(p, 32)), hex(p)


@pytest.mark.slow
def _check_round_chunk(start, chunk):
    pats = np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32)
    got = R.round_bf16(pats)
    exp_field = (pats >> 23) & 0xFF
    is_nan = (exp_field == 0xFF) & ((pats & 0x7FFFFF) != 0)
    if not np.all(got[is_nan] == 0x7FC0):
        return f"a NaN in the chunk at {hex(start)} did not give 0x7FC0"
    t = torch.from_numpy(pats.view(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ok = is_nan | (got == t)
    if not ok.all():
        i = int(np.flatnonzero(~ok)[0])
        return f"{hex(int(pats[i]))}: oracle {hex(int(got[i]))} torch {hex(int(t[i]))}"
    return None


def test_round_exhaustive_against_torch():
    """All 2^32 binary32 patterns: non-NaN inputs agree with torch's CPU
    float32 -> bfloat16 (round to nearest even); every NaN gives 0x7FC0.
    Chunks run on a few threads (numpy, the oracle's C and torch release
    the interpreter lock)."""
    chunk = 1 << 24
    workers = max(1, min(8, (os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        for err in pool.map(lambda st: _check_round_chunk(st, chunk), range(0, 1 << 32, chunk)):
            assert err is None, err


def test_widen_exhaustive_against_definition_and_torch():
    h = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    w = R.widen_bf16(h)
    # torch's bf16 -> float32 is exact too; compare patterns on non-NaN
    t = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).to(torch.float32).view(torch.int32).numpy().view(np.uint32)
    is_nan = ((h >> 7) & 0xFF == 0xFF) & ((h & 0x7F) != 0)
    assert np.all((w == t) | is_nan)
    # the value of every widened pattern equals the bf16 value by definition
    for hv, wv in zip(h.tolist()[::7], w.tolist()[::7]):
        a = ref.decode(hv, 16)
        b = ref.decode(wv, 32)
        assert a[0] == b[0] and a[1] == b[1] and a[2] == b[2], hex(hv)
    # NaN stays NaN, with sign and payload carried in the upper half
    assert np.all(((w[is_nan] >> 23) & 0xFF) == 0xFF)
    assert np.all((w[is_nan] & 0x7FFFFF) != 0)
