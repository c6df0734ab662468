"""E4M3 (OCP "E4M3FN") codec, written from the format's definition.

Test infrastructure only (see the package docstring).

Source passages:
* HolySheep (zh), section 2.2: the quantizer casts to ``torch.float8_e4m3fn``
  and takes 448 as the largest E4M3 value; its overflow troubleshooting
  section gives the representable range as (-448, 448).
* codingmall (sv), "Unified E4M3 Format": E4M3 is used for every GEMM operand,
  forward and backward.
* The German HolySheep article describes E4M3 as 4 exponent and 3 mantissa
  bits.

The format (``float8_e4m3fn``): 1 sign bit S, 4 exponent bits E, 3 mantissa
bits M, exponent bias 7, no infinities.  E == 0 encodes the subnormals
M * 2^-9; E in 1..15 encodes (1 + M/8) * 2^(E-7), except that E == 15 with
M == 7 is NaN.  The largest finite magnitude is (1 + 6/8) * 2^8 = 448 (code
0x7E).

Readings where the pages leave a step open (each is also listed in the design
notes of the repository):
* rounding is to nearest with ties to the even code, which is what the cast
  in section 2.2 does;
* magnitudes above 448 saturate to 448 instead of raising the overflow error
  that the troubleshooting section shows (the quantizer never produces them
  except through that rounding edge, and saturation keeps the cast total);
* the sign of zero is kept (negative values that round to zero give 0x80);
* NaN keeps its sign and maps to S.1111.111.
"""
import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Value of each 8-bit code as float64 (NaN for S.1111.111).

    Closed form of the format: subnormal M*2^-9 for E == 0, otherwise
    (1 + M/8) * 2^(E-7).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    neg = ((c >> 7) & 1) == 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = m.astype(np.float64) * 2.0 ** -9
    norm = (1.0 + m.astype(np.float64) / 8.0) * np.exp2((e - 7).astype(np.float64))
    mag = np.where(e == 0, sub, norm)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.copysign(mag, np.where(neg, -1.0, 1.0))   # keeps the sign of NaN too


def e4m3_magnitudes():
    """The 127 finite non-negative magnitudes, indexed by their code 0..126."""
    return e4m3_decode(np.arange(127, dtype=np.uint8))


def e4m3_encode(v):
    """Round float32 values to E4M3 codes: nearest magnitude, ties to even code.

    ``v`` is taken as exact binary32 values (every float32 is exact in
    float64).  The sign of ``v`` (including -0.0) becomes the sign bit; NaN
    gives S.1111.111; any magnitude above 448, infinity included, saturates
    to 448.  Otherwise the magnitude goes to the nearer of the two codes that
    bracket it, and a value exactly halfway between two codes goes to the
    even code.
    """
    v = np.asarray(v, dtype=np.float32)
    shape = v.shape
    v = v.reshape(-1)                  # elementwise; one flat pass is much faster in numpy
    a = np.abs(v).astype(np.float64)
    sign = np.signbit(v).astype(np.uint8) << 7
    mags = e4m3_magnitudes()
    # hi = first code whose magnitude is >= a; lo = the one below it.
    a_clip = np.where(np.isnan(a), 0.0, np.minimum(a, E4M3_MAX))
    hi = np.searchsorted(mags, a_clip, side="left")
    hi = np.clip(hi, 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    mid = (mags[lo] + mags[hi]) / 2.0          # exact: dyadic with few bits
    even = np.where(lo % 2 == 0, lo, hi)
    code = np.where(a_clip < mid, lo, np.where(a_clip > mid, hi, even))
    code = np.where(a_clip == mags[hi], hi, code)   # exact hits (incl. 0)
    code = np.where(a > E4M3_MAX, 126, code)          # saturate, incl. inf
    code = np.where(np.isnan(a), 127, code)           # NaN keeps its sign
    return (code.astype(np.uint8) | sign).astype(np.uint8).reshape(shape)


def e4m3_half_ulp(v):
    """Half the E4M3 spacing at |v| (float64): the largest rounding error.

    Normals with exponent e (2^e <= |v| < 2^(e+1), e >= -6) have spacing
    2^(e-3); below 2^-6 the spacing is the subnormal step 2^-9.
    """
    a = np.abs(np.asarray(v, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    # log2 of an exact float is exact at powers of two; guard the floor anyway
    e = np.where(np.exp2(e) > a, e - 1, e)
    e = np.where(np.exp2(e + 1) <= a, e + 1, e)
    e = np.where(a > 0, np.maximum(e, -6.0), -6.0)   # zero sits in the subnormal step
    return np.exp2(e - 3.0) / 2.0
