"""Pins of the oracle's E4M3 codec against the format definition and an
independent library cast (torch's CPU float8_e4m3fn)."""
import os

import numpy as np
import pytest

from oracle import e4m3_decode, e4m3_encode, e4m3_half_ulp, e4m3_magnitudes
import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_values.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        val, code = line.split()[:2]
        rows.append((float.fromhex(val), int(code, 16)))
    return rows


def test_golden_values():
    rows = _golden()
    assert len(rows) >= 18
    v = np.array([r[0] for r in rows], dtype=np.float32)
    want = np.array([r[1] for r in rows], dtype=np.uint8)
    got = e4m3_encode(v)
    assert [hex(c) for c in got] == [hex(c) for c in want]


def test_decode_closed_form_points():
    d = e4m3_decode(np.arange(256, dtype=np.uint8))
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0
    assert d[0x08] == 2.0 ** -6 and d[0x01] == 2.0 ** -9 and d[0x07] == 7 * 2.0 ** -9
    assert d[0x38] == 1.0 and d[0x00] == 0.0 and np.signbit(d[0x80])
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    assert np.sum(np.isfinite(d)) == 254
    # every finite code against the bit-field integer construction
    for c in range(256):
        ref = exact.e4m3_value_exact(c)
        if ref is None:
            assert np.isnan(d[c])
        else:
            assert d[c] == float(ref)


def test_magnitudes_strictly_increasing():
    m = e4m3_magnitudes()
    assert m.shape == (127,) and np.all(np.diff(m) > 0) and m[-1] == 448.0


def test_round_trip_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    back = e4m3_encode(e4m3_decode(codes).astype(np.float32))
    assert np.array_equal(back, codes)


def _all_bf16_values():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    return bits.view(np.float32)


def test_all_bf16_patterns_brute_force():
    v = _all_bf16_values()
    v = v[np.isfinite(v)]
    got = e4m3_encode(v)
    for x, c in zip(v.tolist(), got.tolist()):
        want = exact.e4m3_encode_exact(x, neg_zero=np.signbit(np.float32(x)))
        assert c == want, (x, hex(c), hex(want))


def test_midpoints_and_neighbours():
    m = e4m3_magnitudes()
    for lo in range(126):
        mid = np.float32((m[lo] + m[lo + 1]) / 2)
        assert float(mid) == (m[lo] + m[lo + 1]) / 2          # exact in binary32
        even = lo if lo % 2 == 0 else lo + 1
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(np.inf))
        got = e4m3_encode(np.array([mid, below, above, -mid], dtype=np.float32))
        assert got.tolist() == [even, lo, lo + 1, even | 0x80]


def test_special_values():
    v = np.array([np.nan, -np.nan, np.inf, -np.inf, 0.0, -0.0, 448.0, 449.0,
                  463.999, 464.0, 1e30, 2.0 ** -149, -(2.0 ** -149)], dtype=np.float32)
    got = e4m3_encode(v)
    assert got.tolist() == [0x7F, 0xFF, 0x7E, 0xFE, 0x00, 0x80, 0x7E, 0x7E,
                            0x7E, 0x7E, 0x7E, 0x00, 0x80]


def test_matches_torch_cast_in_range():
    torch = pytest.importorskip("torch")
    v = _all_bf16_values()
    rng = np.random.default_rng(1)
    r = rng.standard_normal(2_000_000).astype(np.float32) * np.float32(64)
    r2 = (rng.random(1_000_000).astype(np.float32) - np.float32(0.5)) * np.float32(2 ** -5)
    v = np.concatenate([v, r, r2])
    v = v[np.isfinite(v) & (np.abs(v) <= 448)]
    ours = e4m3_encode(v)
    theirs = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_half_ulp_bound_and_monotone():
    rng = np.random.default_rng(2)
    v = np.concatenate([
        rng.uniform(-448, 448, 200_000),
        rng.uniform(-2 ** -5, 2 ** -5, 200_000),
    ]).astype(np.float32)
    d = e4m3_decode(e4m3_encode(v))
    err = np.abs(d - v.astype(np.float64))
    assert np.all(err <= e4m3_half_ulp(v))
    a = np.sort(np.abs(v))
    codes = e4m3_encode(a).astype(np.int64)
    assert np.all(np.diff(codes) >= 0)


def test_half_ulp_closed_form():
    v = np.array([1.0, 1.9, 2.0, 448.0, 2.0 ** -6, 2.0 ** -7, 0.0])
    assert e4m3_half_ulp(v).tolist() == [2.0 ** -4, 2.0 ** -4, 2.0 ** -3, 2.0 ** 4,
                                         2.0 ** -10, 2.0 ** -10, 2.0 ** -10]
