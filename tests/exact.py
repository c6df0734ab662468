"""Exact rational arithmetic used to pin the oracle from outside.

These helpers take a different route from the oracle on purpose: Python
integers and ``fractions.Fraction`` instead of numpy float32 and table
searches, so that a slip in the oracle does not repeat here.
"""
import bisect
import math
import struct
from fractions import Fraction


def f32_bits(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


def f32_from_bits(u):
    return struct.unpack("<f", struct.pack("<I", u))[0]


def _round_binary(q, p, emin):
    """Nearest binary floating-point value with p significand bits and
    minimum normal exponent emin, ties to even (subnormals handled, no
    overflow), as a Python float (sign of zero aside)."""
    q = Fraction(q)
    if q == 0:
        return 0.0
    neg = q < 0
    a = -q if neg else q
    # e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - (p - 1))
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = float(fl * quantum)
    return -v if neg else v


def rn32(q):
    """Round a rational to the nearest binary32 value, ties to even.

    Returns a Python float holding the binary32 value (sign of zero aside).
    Handles subnormals; assumes no overflow.
    """
    return _round_binary(q, 24, -126)


def rn64(q):
    """Round a rational to the nearest binary64 value, ties to even."""
    return _round_binary(q, 53, -1022)


# E4M3 magnitudes built from the bit fields, as exact integers in units of 2^-9.
def _e4m3_mag_units(code):
    e, m = (code >> 3) & 0xF, code & 7
    if e == 0:
        return m                      # m * 2^-9
    # (8 + m) * 2^(e-10) in units of 2^-9 = (8+m) * 2^(e-1)
    return (8 + m) << (e - 1)


_MAG_UNITS = [_e4m3_mag_units(c) for c in range(127)]   # strictly increasing


def e4m3_value_exact(code):
    """Fraction value of a finite E4M3 code (None for NaN codes)."""
    if code & 0x7F == 0x7F:
        return None
    v = Fraction(_MAG_UNITS[code & 0x7F], 512)
    return -v if code & 0x80 else v


def e4m3_encode_exact(v, neg_zero=False):
    """Nearest E4M3 code of a rational magnitude, ties to the even code.

    Brute force over the integer magnitude list; saturates above 448.
    ``neg_zero`` carries the sign of a zero value.
    """
    v = Fraction(v)
    neg = v < 0 or (v == 0 and neg_zero)
    a = abs(v) * 512                      # in units of 2^-9
    if a >= _MAG_UNITS[126]:
        code = 126
    else:
        hi = bisect.bisect_left(_MAG_UNITS, a)      # first >= a
        if _MAG_UNITS[hi] == a:
            code = hi
        else:
            lo = hi - 1
            d_lo, d_hi = a - _MAG_UNITS[lo], _MAG_UNITS[hi] - a
            if d_lo < d_hi:
                code = lo
            elif d_hi < d_lo:
                code = hi
            else:
                code = lo if lo % 2 == 0 else hi
    return code | (0x80 if neg else 0)


def quantize_tile_exact(values):
    """One tile by exact arithmetic: (codes list, scale float).

    amax / 448 and x / s are each rounded once to binary32 (``rn32``); the
    guard replaces s by 1 when s is not above rn32(1e-10).
    """
    vals = [float(v) for v in values]
    amax = max(abs(v) for v in vals)
    s = rn32(Fraction(amax) / 448)
    guard = rn32(Fraction(1e-10))
    if not s > guard:
        s = 1.0
    codes = []
    for x in vals:
        q = rn32(Fraction(x) / Fraction(s))
        codes.append(e4m3_encode_exact(q, neg_zero=math.copysign(1.0, x) < 0))
    return codes, s


# E5M2 magnitudes from the bit fields, as exact integers in units of 2^-16:
# E=0 -> M; E=1..30 -> (4 + M) * 2^(E-1).
def _e5m2_mag_units(code):
    e, m = (code >> 2) & 0x1F, code & 3
    if e == 0:
        return m
    return (4 + m) << (e - 1)


_E5M2_UNITS = [_e5m2_mag_units(c) for c in range(124)]   # finite codes 0..0x7B


def e5m2_value_exact(code):
    """Fraction value of a finite E5M2 code (None for infinities and NaN)."""
    if (code >> 2) & 0x1F == 31:
        return None
    v = Fraction(_E5M2_UNITS[code & 0x7F], 1 << 16)
    return -v if code & 0x80 else v


def e5m2_encode_exact(v, neg_zero=False):
    """Nearest E5M2 code of a rational, ties to the even code, saturating at 57344."""
    v = Fraction(v)
    neg = v < 0 or (v == 0 and neg_zero)
    a = abs(v) * (1 << 16)
    if a >= _E5M2_UNITS[123]:
        code = 123
    else:
        hi = bisect.bisect_left(_E5M2_UNITS, a)
        if _E5M2_UNITS[hi] == a:
            code = hi
        else:
            lo = hi - 1
            d_lo, d_hi = a - _E5M2_UNITS[lo], _E5M2_UNITS[hi] - a
            code = lo if d_lo < d_hi else hi if d_hi < d_lo else (lo if lo % 2 == 0 else hi)
    return code | (0x80 if neg else 0)


def tensor_quantize_exact(values, fmt_max, encode_exact, margin=0.0, amax=None):
    """Per-tensor scaling by exact arithmetic, each step rounded once.

    The scale takes the page's Python-float (binary64) steps:
    d = rn64(rn64(amax * rn64(1 + margin)) / fmt_max); s = 1 if d < 1e-6
    (the binary64 literal), else s = rn32(d).  Codes: encode(rn32(x / s)).
    `margin` is the binary64 value passed; `amax` overrides the tensor's own
    (delayed scaling).
    """
    vals = [float(v) for v in values]
    if amax is None:
        amax = max(abs(v) for v in vals)
    widen = rn64(1 + Fraction(float(margin)))
    d = rn64(Fraction(rn64(Fraction(amax) * Fraction(widen))) / fmt_max)
    s = 1.0 if Fraction(d) < Fraction(1e-6) else rn32(Fraction(d))
    codes = [encode_exact(rn32(Fraction(x) / Fraction(s)), neg_zero=math.copysign(1.0, x) < 0)
             for x in vals]
    return codes, s
