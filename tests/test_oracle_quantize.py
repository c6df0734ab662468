"""Pins of the oracle quantizers: exact rational brute force, closed forms and
invariants that the tile-scaling definition fixes."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import (SCALE_GUARD, tile_scale, quant_1x128, quant_128x1_t, quant_128x128,
                    dequant_1x128, dequant_128x128, e4m3_decode, e4m3_half_ulp)
from fp8_block_scaled_05_amd import synth
import exact


def test_guard_constant():
    assert exact.f32_bits(float(SCALE_GUARD)) == 0x2EDBE6FF
    assert float(SCALE_GUARD) == exact.rn32(Fraction(1e-10))


def test_scale_exact_for_every_bf16_amax():
    bits = np.arange(0, 0x7F80, dtype=np.uint32) << 16           # +0 .. max finite
    amax = bits.view(np.float32)
    got = tile_scale(amax)
    guard = exact.rn32(Fraction(1e-10))
    for a, s in zip(amax.tolist(), got.tolist()):
        want = exact.rn32(Fraction(a) / 448)
        if not want > guard:
            want = 1.0
        assert s == want, (a, s, want)


def test_float32_division_is_correctly_rounded():
    rng = np.random.default_rng(3)
    x = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(
        rng.standard_normal(20000).astype(np.float32) * np.float32(3)))
    s = tile_scale(np.abs(rng.standard_normal(20000)).astype(np.float32) * np.float32(7))
    q = x / s
    for xi, si, qi in zip(x.tolist(), s.tolist(), q.tolist()):
        assert qi == exact.rn32(Fraction(xi) / Fraction(si))


def _bf16_tiles(rng, rows, cols, scale=1.0, outliers=0.0):
    x = rng.standard_normal((rows, cols)).astype(np.float32) * np.float32(scale)
    if outliers:
        idx = rng.choice(x.size, int(outliers * x.size), replace=False)
        x.reshape(-1)[idx] *= np.float32(100)
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))


def test_1x128_brute_force_exact():
    rng = np.random.default_rng(4)
    x = _bf16_tiles(rng, 3, 256, outliers=0.02)
    x[2, :128] *= np.float32(2.0 ** -120)      # tiny tile: amax/448 under the guard
    x[2, 128:] *= np.float32(2.0 ** 100)       # huge tile
    x[1, 5] = -0.0
    codes, s = quant_1x128(x)
    for r in range(3):
        for t in range(2):
            want_codes, want_s = exact.quantize_tile_exact(x[r, t * 128:(t + 1) * 128])
            assert s[r, t] == want_s
            assert codes[r, t * 128:(t + 1) * 128].tolist() == want_codes
    assert s[2, 0] == 1.0


def test_max_element_maps_to_448():
    rng = np.random.default_rng(5)
    x = _bf16_tiles(rng, 64, 512, outliers=0.01)
    codes, s = quant_1x128(x)
    tiles = x.reshape(64, 4, 128)
    arg = np.abs(tiles).argmax(axis=2)
    top = np.take_along_axis(codes.reshape(64, 4, 128), arg[:, :, None], axis=2)[..., 0]
    sign = np.signbit(np.take_along_axis(tiles, arg[:, :, None], axis=2)[..., 0])
    assert np.all(top == np.where(sign, 0xFE, 0x7E))


def test_dequant_error_within_half_ulp():
    rng = np.random.default_rng(6)
    x = _bf16_tiles(rng, 32, 1024, outliers=0.01)
    codes, s = quant_1x128(x)
    v = (x.reshape(32, 8, 128) / s[:, :, None]).reshape(32, 1024)
    err = np.abs(e4m3_decode(codes) - v.astype(np.float64))
    assert np.all(err <= e4m3_half_ulp(v))
    back = dequant_1x128(codes, s)
    assert np.all(np.abs(back - x) <= np.repeat(s.astype(np.float64), 128, axis=1)
                  * e4m3_half_ulp(v) * (1 + 2.0 ** -20))


def test_sign_symmetry_and_power_of_two_covariance():
    rng = np.random.default_rng(7)
    x = _bf16_tiles(rng, 16, 384)
    c, s = quant_1x128(x)
    cn, sn = quant_1x128(-x)
    assert np.array_equal(sn, s) and np.array_equal(cn, c ^ 0x80)
    for j in (-7, 3, 20):
        c2, s2 = quant_1x128(x * np.float32(2.0 ** j))
        assert np.array_equal(c2, c)
        assert np.array_equal(s2, s * np.float32(2.0 ** j))


def test_permutation_and_tile_independence():
    rng = np.random.default_rng(8)
    x = _bf16_tiles(rng, 4, 512)
    c, s = quant_1x128(x)
    perm = rng.permutation(128)
    xp = x.copy()
    xp[:, 128:256] = x[:, 128:256][:, perm]
    cp, sp = quant_1x128(xp)
    assert np.array_equal(sp, s)
    assert np.array_equal(cp[:, 128:256], c[:, 128:256][:, perm])
    xs = x.copy()
    xs[1, 300] = np.float32(1e6)              # spike in row 1, tile 2
    cs, ss = quant_1x128(xs)
    changed = ss != s
    assert changed[1, 2] and changed.sum() == 1
    mask = np.ones_like(c, dtype=bool)
    mask[1, 256:384] = False
    assert np.array_equal(cs[mask], c[mask])


def test_zero_and_guard_tiles():
    x = np.zeros((2, 256), dtype=np.float32)
    x[0, 128:] = -0.0
    x[1, :128] = np.float32(4.0e-8)           # amax/448 < 1e-10 -> s = 1
    x[1, 128:] = np.float32(5.0e-8)           # amax/448 > 1e-10 -> real scale
    c, s = quant_1x128(x)
    assert s[0].tolist() == [1.0, 1.0]
    assert np.all(c[0, :128] == 0x00) and np.all(c[0, 128:] == 0x80)
    assert s[1, 0] == 1.0 and np.all(c[1, :128] == 0x00)
    assert s[1, 1] == exact.rn32(Fraction(float(np.float32(5.0e-8))) / 448)
    assert np.all(c[1, 128:] == 0x7E)


def test_128x1_t_brute_force():
    rng = np.random.default_rng(9)
    x = _bf16_tiles(rng, 256, 6, outliers=0.02)
    codes_t, s = quant_128x1_t(x)
    assert codes_t.shape == (6, 256) and s.shape == (6, 2)
    for col in range(6):
        for t in range(2):
            want_codes, want_s = exact.quantize_tile_exact(x[t * 128:(t + 1) * 128, col])
            assert s[col, t] == want_s
            assert codes_t[col, t * 128:(t + 1) * 128].tolist() == want_codes


def test_128x128_brute_force_and_block_independence():
    rng = np.random.default_rng(10)
    w = _bf16_tiles(rng, 256, 384, scale=0.02)
    w[:128, 128:256] *= np.float32(37.0)
    codes, s = quant_128x128(w)
    assert codes.shape == (256, 384) and s.shape == (2, 3)
    for bi in range(2):
        for bj in range(3):
            blk = w[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
            want_codes, want_s = exact.quantize_tile_exact(blk.reshape(-1))
            assert s[bi, bj] == want_s
            assert codes[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128].reshape(-1).tolist() \
                == want_codes
    w2 = w.copy()
    w2[128:, :128] *= np.float32(2.0 ** 5)
    c2, s2 = quant_128x128(w2)
    assert np.array_equal(c2, codes)
    diff = s2 != s
    assert diff[1, 0] and diff.sum() == 1 and s2[1, 0] == s[1, 0] * 32
    back = dequant_128x128(codes, s)
    assert np.max(np.abs(back - w)) <= np.max(s) * 16      # half ulp at 448 is 16


def test_shapes_rejected():
    with pytest.raises(ValueError):
        quant_1x128(np.zeros((2, 100), np.float32))
    with pytest.raises(ValueError):
        quant_128x1_t(np.zeros((100, 2), np.float32))
    with pytest.raises(ValueError):
        quant_128x128(np.zeros((128, 100), np.float32))
    with pytest.raises(ValueError):
        quant_1x128(np.full((1, 128), np.inf, np.float32))
