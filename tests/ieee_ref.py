"""Definition-level IEEE 754 helpers used to pin the oracle.

Written from the standard's definitions (binary32 and bf16 as sign, biased
exponent and fraction; roundTiesToEven as "nearest representable value, the
one with an even last significand bit on a tie"), with exact rational
arithmetic. Deliberately slow and unrelated to the oracle's bit tricks.
"""
import math
import struct
from fractions import Fraction

# binary32: 24 significand bits, exponent range of normals [-126, 127]
# bf16:      8 significand bits, same exponent range
F32_P, BF16_P = 24, 8
EMIN = -126
EMAX = 127


def decode(bits: int, width: int):
    """bits of a binary32 (width 32) or bf16 (width 16) pattern -> ('nan'|'inf'|'num', sign, Fraction)."""
    frac_bits = 23 if width == 32 else 7
    sign = (bits >> (width - 1)) & 1
    exp = (bits >> frac_bits) & 0xFF
    frac = bits & ((1 << frac_bits) - 1)
    if exp == 0xFF:
        return ("nan" if frac else "inf", sign, None)
    if exp == 0:
        mag = Fraction(frac, 1 << frac_bits) * Fraction(2) ** EMIN
    else:
        mag = (1 + Fraction(frac, 1 << frac_bits)) * Fraction(2) ** (exp - 127)
    return ("num", sign, mag)


def round_to(mag: Fraction, p: int):
    """Rounds a non-negative rational to p significand bits, ties to even,
    with gradual underflow below 2^EMIN. Returns the rounded Fraction, or
    None on overflow (magnitude at or past 2^(EMAX+1) after rounding)."""
    if mag == 0:
        return Fraction(0)
    e = math.floor(math.log2(mag.numerator) - math.log2(mag.denominator))
    # fix possible off-by-one of the float log2
    while Fraction(2) ** e > mag:
        e -= 1
    while Fraction(2) ** (e + 1) <= mag:
        e += 1
    e = max(e, EMIN)
    q = Fraction(2) ** (e - (p - 1))      # spacing of representable values here
    m = mag / q
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    r = lo * q
    if r >= Fraction(2) ** (EMAX + 1):
        return None
    return r


def encode(sign: int, mag, width: int) -> int:
    """sign and exactly representable magnitude (or None for Inf) -> pattern."""
    frac_bits = 23 if width == 32 else 7
    top = 1 << (width - 1)
    if mag is None:
        return (top if sign else 0) | (0xFF << frac_bits)
    if mag == 0:
        return top if sign else 0
    if mag < Fraction(2) ** EMIN:
        frac = mag / (Fraction(2) ** EMIN) * (1 << frac_bits)
        assert frac.denominator == 1
        return (top if sign else 0) | int(frac)
    e = EMIN
    while Fraction(2) ** (e + 1) <= mag:
        e += 1
    frac = (mag / Fraction(2) ** e - 1) * (1 << frac_bits)
    assert frac.denominator == 1, "magnitude not representable"
    return (top if sign else 0) | ((e + 127) << frac_bits) | int(frac)


def bf16_of_value(kind: str, sign: int, mag) -> int:
    """The bf16 result of rounding an exact value once (NaN -> 0x7FC0)."""
    if kind == "nan":
        return 0x7FC0
    if kind == "inf":
        return encode(sign, None, 16)
    return encode(sign, round_to(mag, BF16_P), 16)


def f32_add(a, b):
    """IEEE binary32 addition of two decoded values, round to nearest even.
    Values are (kind, sign, Fraction) triples as from decode()."""
    ka, sa, ma = a
    kb, sb, mb = b
    if ka == "nan" or kb == "nan":
        return ("nan", 0, None)
    if ka == "inf" and kb == "inf":
        return ("inf", sa, None) if sa == sb else ("nan", 0, None)
    if ka == "inf":
        return a
    if kb == "inf":
        return b
    va = -ma if sa else ma
    vb = -mb if sb else mb
    s = va + vb
    if s == 0:
        # exact zero sum: -0 only when both addends are -0 (round to nearest)
        return ("num", 1 if (sa and sb and ma == 0 and mb == 0) else 0, Fraction(0))
    sign = 1 if s < 0 else 0
    r = round_to(abs(s), F32_P)
    if r is None:
        return ("inf", sign, None)
    return ("num", sign, r)


def reduce_exact(columns):
    """Rank-ordered binary32 sum of bf16 patterns, rounded once to bf16,
    computed from the definitions. columns: list of per-element lists of W
    bf16 patterns. Accumulator starts at -0."""
    out = []
    for col in columns:
        acc = ("num", 1, Fraction(0))
        for h in col:
            acc = f32_add(acc, decode(int(h), 16))
        out.append(bf16_of_value(*acc))
    return out


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]
