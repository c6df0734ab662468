"""Host check of the quantizers' division-free tile scale for bf16 inputs
(csrc/quant.hip, scale_recip_bf16): amax * fl32(1/7) with one Markstein
correction step, then the exact division by 64, must give the IEEE float32
value of amax / 448 for every bf16 amax whose scale passes the 1e-10 guard,
and a value at or below the guard for every smaller amax (so the guard picks
1 either way).  Exact rational arithmetic stands in for the hardware FMA.
No GPU is needed; the GPU side is covered by the exhaustive bf16 codec sweep."""
from fractions import Fraction

import numpy as np

GUARD = np.float32(1e-10)


def rn32(q):
    """Round a Fraction to the nearest binary32, ties to even (finite range)."""
    if q == 0:
        return np.float32(0.0)
    f = np.float32(float(q))          # within one ulp of the correct result
    best = None
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        key = (abs(Fraction(float(c)) - q), int(np.array(c, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def kernel_scale(x, c7):
    """The kernel's steps: q0 = x*c7, q1 = fma(fma(-q0, 7, x), c7, q0), q1/64."""
    xf = Fraction(float(x))
    q0 = np.float32(x * c7)
    t = rn32(-Fraction(float(q0)) * 7 + xf)
    q1 = rn32(Fraction(float(t)) * Fraction(float(c7)) + Fraction(float(q0)))
    return np.float32(q1 * np.float32(0.015625))


def test_fl32_one_seventh():
    c7 = np.float32(float.fromhex('0x1.24924ap-3'))
    assert c7 == rn32(Fraction(1, 7))


def test_division_free_scale_matches_ieee_for_every_bf16_amax():
    c7 = np.float32(float.fromhex('0x1.24924ap-3'))
    above = below = 0
    for hi in range(0x0001, 0x7F80):            # every positive finite bf16
        x = np.array(hi << 16, dtype=np.uint32).view(np.float32)
        ref = rn32(Fraction(float(x)) / 448)
        got = kernel_scale(x, c7)
        if ref > GUARD:
            assert got == ref, (float(x), float(ref), float(got))
            above += 1
        else:
            assert not (got > GUARD), (float(x), float(ref), float(got))
            below += 1
    assert above == 19519 and above + below == 0x7F7F


def test_uncorrected_product_is_caught():
    """Negative control: amax * fl32(1/448) alone misses fl32(amax/448) for
    many bf16 amax, so the check above has the power to see a missing step."""
    c = np.float32(1.0) / np.float32(448.0)
    misses = 0
    for hi in range(0x3000, 0x4000):
        x = np.array(hi << 16, dtype=np.uint32).view(np.float32)
        if np.float32(x * c) != rn32(Fraction(float(x)) / 448):
            misses += 1
    assert misses > 100
