"""E5M2 (OCP "E5M2") codec, written from the format's definition.

Test infrastructure only (see the package docstring).

Source passages: the German HolySheep article names E5M2 (5 exponent and 2
mantissa bits) beside E4M3 and says that the usual hybrid recipe handles
activations in E4M3 and gradients in E5M2; the French HolySheep article
lists weight gradients as "FP8_E5M2" for the same reason (dynamic range);
codingmall (sv) "Unified E4M3 Format" says DeepSeek-V3 drops that hybrid and
uses E4M3 everywhere.  E5M2 is therefore the prior-art gradient format here.

The format (``float8_e5m2``): 1 sign bit S, 5 exponent bits E, 2 mantissa
bits M, bias 15.  E == 0 encodes the subnormals M * 2^-16; E in 1..30
encodes (1 + M/4) * 2^(E-15); E == 31 is infinity (M == 0) or NaN.  The
largest finite magnitude is (1 + 3/4) * 2^15 = 57344 (code 0x7B).

Readings (the same as for E4M3, listed in the design notes):
* round to nearest, ties to the even code;
* finite magnitudes above 57344, and infinities, saturate to 57344;
* the sign of zero is kept; NaN keeps its sign and maps to S.11111.11.
"""
import numpy as np

E5M2_MAX = 57344.0


def e5m2_decode(codes):
    """Value of each 8-bit code as float64 (inf for S.11111.00, NaN above)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    neg = ((c >> 7) & 1) == 1
    e = (c >> 2) & 0x1F
    m = c & 0x3
    sub = m.astype(np.float64) * 2.0 ** -16
    norm = (1.0 + m.astype(np.float64) / 4.0) * np.exp2((e - 15).astype(np.float64))
    mag = np.where(e == 0, sub, norm)
    mag = np.where((e == 31) & (m == 0), np.inf, mag)
    mag = np.where((e == 31) & (m != 0), np.nan, mag)
    return np.copysign(mag, np.where(neg, -1.0, 1.0))


def e5m2_magnitudes():
    """The 124 finite non-negative magnitudes, indexed by their code 0..123."""
    return e5m2_decode(np.arange(124, dtype=np.uint8))


def e5m2_encode(v):
    """Round float32 values to E5M2 codes: nearest magnitude, ties to even code."""
    v = np.asarray(v, dtype=np.float32)
    shape = v.shape
    v = v.reshape(-1)
    a = np.abs(v).astype(np.float64)
    sign = np.signbit(v).astype(np.uint8) << 7
    mags = e5m2_magnitudes()
    a_clip = np.where(np.isnan(a), 0.0, np.minimum(a, E5M2_MAX))
    hi = np.clip(np.searchsorted(mags, a_clip, side="left"), 0, 123)
    lo = np.clip(hi - 1, 0, 123)
    mid = (mags[lo] + mags[hi]) / 2.0
    even = np.where(lo % 2 == 0, lo, hi)
    code = np.where(a_clip < mid, lo, np.where(a_clip > mid, hi, even))
    code = np.where(a_clip == mags[hi], hi, code)
    code = np.where(a > E5M2_MAX, 123, code)            # saturate, infinities included
    code = np.where(np.isnan(a), 127, code)
    return (code.astype(np.uint8) | sign).astype(np.uint8).reshape(shape)


def e5m2_half_ulp(v):
    """Half the E5M2 spacing at |v|: 2^(e-2)/2 for normals, 2^-17 below 2^-14."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.where(np.exp2(e) > a, e - 1, e)
    e = np.where(np.exp2(e + 1) <= a, e + 1, e)
    e = np.where(a > 0, np.maximum(e, -14.0), -14.0)
    return np.exp2(e - 2.0) / 2.0
