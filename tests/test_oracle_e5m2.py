"""Pins of the oracle's E5M2 codec: the format's bit fields, the fact that an
E5M2 code is the top byte of an IEEE half, exact rational rounding, and
torch's own float8_e5m2 cast."""
import numpy as np
import pytest

from oracle import e5m2_decode, e5m2_encode, e5m2_magnitudes, e5m2_half_ulp
import exact


def test_decode_closed_form_points():
    d = e5m2_decode(np.arange(256, dtype=np.uint8))
    assert d[0x7B] == 57344.0 and d[0xFB] == -57344.0
    assert d[0x04] == 2.0 ** -14 and d[0x01] == 2.0 ** -16 and d[0x03] == 3 * 2.0 ** -16
    assert d[0x3C] == 1.0 and d[0x00] == 0.0 and np.signbit(d[0x80])
    assert d[0x7C] == np.inf and d[0xFC] == -np.inf
    assert all(np.isnan(d[c]) for c in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF))
    for c in range(256):
        ref = exact.e5m2_value_exact(c)
        if ref is not None:
            assert d[c] == float(ref)


def test_code_is_the_top_byte_of_a_half():
    """E5M2 has the exponent bias and field widths of IEEE binary16 with the
    mantissa cut to 2 bits, so code c decodes to the half with bits c << 8."""
    codes = np.arange(256, dtype=np.uint16)
    halves = (codes << 8).astype(np.uint16).view(np.float16).astype(np.float64)
    d = e5m2_decode(codes.astype(np.uint8))
    both_nan = np.isnan(d) & np.isnan(halves)
    assert np.array_equal(d[~both_nan], halves[~both_nan])
    assert np.array_equal(np.isnan(d), np.isnan(halves))


def test_magnitudes_and_round_trip():
    m = e5m2_magnitudes()
    assert m.shape == (124,) and np.all(np.diff(m) > 0) and m[-1] == 57344.0
    finite = np.array([c for c in range(256) if (c >> 2) & 0x1F != 31], np.uint8)
    assert np.array_equal(e5m2_encode(e5m2_decode(finite).astype(np.float32)), finite)
    # infinities saturate; NaN keeps its sign as S.11111.11
    assert e5m2_encode(np.float32([np.inf, -np.inf, np.nan, -np.nan])).tolist() == [0x7B, 0xFB, 0x7F, 0xFF]


def test_all_bf16_patterns_brute_force():
    v = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)
    v = v[np.isfinite(v)]
    got = e5m2_encode(v)
    for x, c in zip(v.tolist(), got.tolist()):
        assert c == exact.e5m2_encode_exact(x, neg_zero=np.signbit(np.float32(x))), (x, hex(c))


def test_midpoints_and_neighbours():
    m = e5m2_magnitudes()
    for lo in range(123):
        mid = np.float32((m[lo] + m[lo + 1]) / 2)
        assert float(mid) == (m[lo] + m[lo + 1]) / 2
        even = lo if lo % 2 == 0 else lo + 1
        got = e5m2_encode(np.array([mid, np.nextafter(mid, np.float32(0)),
                                    np.nextafter(mid, np.float32(np.inf)), -mid], np.float32))
        assert got.tolist() == [even, lo, lo + 1, even | 0x80]


def test_matches_torch_cast_in_range():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    v = np.concatenate([
        (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32),
        rng.standard_normal(1_000_000).astype(np.float32) * np.float32(3000),
        (rng.random(500_000).astype(np.float32) - np.float32(0.5)) * np.float32(2 ** -12),
    ])
    v = v[np.isfinite(v) & (np.abs(v) <= 57344)]
    theirs = torch.from_numpy(v).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(e5m2_encode(v), theirs)


def test_half_ulp():
    v = np.array([1.0, 1.9, 2.0, 57344.0, 2.0 ** -14, 2.0 ** -15, 0.0])
    assert e5m2_half_ulp(v).tolist() == [2.0 ** -3, 2.0 ** -3, 2.0 ** -2, 2.0 ** 12,
                                         2.0 ** -17, 2.0 ** -17, 2.0 ** -17]
    rng = np.random.default_rng(4)
    x = rng.uniform(-57344, 57344, 100_000).astype(np.float32)
    assert np.all(np.abs(e5m2_decode(e5m2_encode(x)) - x) <= e5m2_half_ulp(x))
