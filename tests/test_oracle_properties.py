"""Property-based pins of the oracle's reduction (CPU only, hypothesis).

For random partial counts W in 1..8 and random bf16 columns, drawn with
extra weight on the values where a sum goes wrong first (±0, subnormals,
±Inf, NaN, the largest finite value, values one apart in the last place),
the oracle must equal the exact rational emulation of rank-ordered binary32
additions followed by one round-to-nearest-even to bf16 (tests/ieee_ref.py,
written from the IEEE 754 definitions). Failures shrink to a minimal column.
"""
import numpy as np
from hypothesis import given, settings, strategies as st

from oracle import reduce as R
from tests import ieee_ref as ref

SPECIAL = [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x807F, 0x0080, 0x8080, 0x7F7F, 0xFF7F, 0x7F80, 0xFF80,
           0x7FC0, 0xFFC0, 0x7F81, 0xFF81, 0x3F80, 0xBF80, 0x3F81, 0xBF81, 0x4000, 0x3B80, 0x3C00, 0x4380, 0xC380]

bf16 = st.one_of(st.sampled_from(SPECIAL), st.integers(0, 0xFFFF),
                 st.integers(0x3000, 0x5000),                      # ordinary magnitudes near 1
                 st.integers(0x0001, 0x00FF).map(lambda v: v | (0x8000 if v & 1 else 0)))


@settings(max_examples=3000, deadline=None)
@given(st.lists(bf16, min_size=1, max_size=8))
def test_oracle_equals_rational_emulation(col):
    got = int(R.reduce([np.array([v], np.uint16) for v in col])[0])
    assert got == ref.reduce_exact([col])[0], [hex(v) for v in col]


@settings(max_examples=300, deadline=None)
@given(st.integers(2, 8), st.lists(bf16, min_size=1, max_size=64))
def test_permuting_zeros_in_does_not_change_nonzero_sums(W, xs):
    """Adding partials of +0 anywhere after the first changes nothing unless
    the column sums to -0 (then +0 wins): x + (+0) = x for every x != -0."""
    xs = np.array(xs, np.uint16)
    base = R.reduce([xs])
    parts = [xs] + [np.zeros_like(xs)] * (W - 1)
    got = R.reduce(parts)
    want = np.where(base == 0x8000, 0x0000, base)
    assert np.array_equal(got, want)
