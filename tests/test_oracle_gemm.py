"""Pins of the oracle GEMM: exact rational brute force, closed forms that catch
transposed operands or mis-routed scales, and the tolerance's attainability."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import (blockscaled_gemm_ref, grouped_gemm_ref, blockscaled_gemm_fp32_model,
                    gemm_tolerance_ok, quant_1x128, quant_128x128, quant_128x1_t)
from oracle.gemm import bf16_half_ulp
from fp8_block_scaled_05_amd import synth
import exact

ONE = 0x38   # E4M3 code of 1.0


def _rand_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3C        # no NaN codes
    return c


def _exact_gemm(a, sa, b, sb, kind):
    m, k = a.shape
    n = b.shape[0]
    out = np.empty((m, n), dtype=object)
    av = [[exact.e4m3_value_exact(int(c)) for c in row] for row in a]
    bv = [[exact.e4m3_value_exact(int(c)) for c in row] for row in b]
    for i in range(m):
        for j in range(n):
            tot = Fraction(0)
            for kb in range(k // 128):
                p = sum(av[i][t] * bv[j][t] for t in range(kb * 128, (kb + 1) * 128))
                sbv = sb[j // 128, kb] if kind == "block128" else sb[j, kb]
                tot += Fraction(float(sa[i, kb])) * Fraction(float(sbv)) * p
            out[i, j] = tot
    return out


@pytest.mark.parametrize("kind", ["block128", "row"])
def test_brute_force_rational(kind):
    rng = np.random.default_rng(11)
    m, n, k = 3, 130 if kind == "row" else 128, 256
    a = _rand_codes(rng, (m, k))
    b = _rand_codes(rng, (n, k))
    sa = (rng.random((m, 2)) * 3 + 0.01).astype(np.float32)
    sb_shape = (1, 2) if kind == "block128" else (n, 2)
    sb = (rng.random(sb_shape) * 3 + 0.01).astype(np.float32)
    cols = [0, 1, 77, 127] + ([128, 129] if kind == "row" else [])
    y, bound = blockscaled_gemm_ref(a, sa, b, sb, kind)
    ex = _exact_gemm(a, sa, b[cols] if kind == "row" else b, sb[cols] if kind == "row" else sb,
                     kind)
    for ci, j in enumerate(cols):
        for i in range(m):
            e = ex[i, ci] if kind == "row" else ex[i, j]
            assert abs(Fraction(y[i, j]) - e) <= Fraction(bound[i, j]) * Fraction(1, 2 ** 45)


def test_selection_closed_form_catches_transpose():
    rng = np.random.default_rng(12)
    m, n, k = 64, 256, 512
    perm = rng.permutation(k)[:m]
    a = np.zeros((m, k), np.uint8)
    a[np.arange(m), perm] = ONE                      # row m picks k = perm[m]
    b = _rand_codes(rng, (n, k))
    sa = np.ones((m, k // 128), np.float32)
    sb = np.ones((n // 128, k // 128), np.float32)
    y, _ = blockscaled_gemm_ref(a, sa, b, sb)
    from oracle import e4m3_decode
    assert np.array_equal(y, e4m3_decode(b[:, perm]).T)


def test_scale_routing_closed_form():
    m, n, k = 8, 256, 512
    kbs = k // 128
    a = np.zeros((m, k), np.uint8)
    for i in range(m):
        for kb in range(kbs):
            a[i, kb * 128 + (i + kb) % 128] = ONE
    b = np.zeros((n, k), np.uint8)
    b[:, :] = ONE
    sa = np.array([[2.0 ** (i + 3 * kb) for kb in range(kbs)] for i in range(m)], np.float32)
    sb = np.array([[2.0 ** (-(7 * nb) - 11 * kb) for kb in range(kbs)] for nb in range(2)],
                  np.float32)
    y, _ = blockscaled_gemm_ref(a, sa, b, sb)
    want = np.array([[sum(2.0 ** (i + 3 * kb) * 2.0 ** (-(7 * (j // 128)) - 11 * kb)
                          for kb in range(kbs)) for j in range(n)] for i in range(m)])
    assert np.array_equal(y, want)
    # ROW scales: every column its own factor
    sbr = np.array([[2.0 ** (-(j % 5) - kb) for kb in range(kbs)] for j in range(n)], np.float32)
    yr, _ = blockscaled_gemm_ref(a, sa, b, sbr, "row")
    want_r = np.array([[sum(2.0 ** (i + 3 * kb) * 2.0 ** (-(j % 5) - kb) for kb in range(kbs))
                        for j in range(n)] for i in range(m)])
    assert np.array_equal(yr, want_r)


def test_all_ones():
    k = 1024
    a = np.full((4, k), ONE, np.uint8)
    b = np.full((128, k), ONE, np.uint8)
    y, bound = blockscaled_gemm_ref(a, np.full((4, 8), 2.0, np.float32), b,
                                    np.full((1, 8), 0.5, np.float32))
    assert np.all(y == k) and np.all(bound == k)


def _quantized_problem(seed, m, n, k):
    rng = np.random.default_rng(seed)
    x = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(
        rng.standard_normal((m, k)).astype(np.float32)))
    w = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(
        rng.standard_normal((n, k)).astype(np.float32) * np.float32(0.02)))
    a, sa = quant_1x128(x)
    b, sb = quant_128x128(w)
    return x, w, a, sa, b, sb


def test_fp32_model_within_tolerance_and_dropped_block_fails():
    x, w, a, sa, b, sb = _quantized_problem(13, 96, 256, 1024)
    y, bound = blockscaled_gemm_ref(a, sa, b, sb)
    y32 = blockscaled_gemm_fp32_model(a, sa, b, sb)
    assert np.all(gemm_tolerance_ok(y32, y, bound))
    # quantization error vs the unquantized product stays at the E4M3 level
    assert np.max(np.abs(y - x.astype(np.float64) @ w.T.astype(np.float64))) < 0.05 * np.max(bound)
    # a mistake the tolerance must catch: one K block's contribution dropped
    sa_bad = sa.copy()
    sa_bad[:, 3] = 0
    y_bad = blockscaled_gemm_fp32_model(a, sa_bad, b, sb)
    assert not np.all(gemm_tolerance_ok(y_bad, y, bound))
    # and a transposed-scale mistake
    sb_bad = sb.copy()
    sb_bad[:, [0, 1]] = sb_bad[:, [1, 0]]
    if not np.array_equal(sb_bad, sb):
        y_bad2 = blockscaled_gemm_fp32_model(a, sa, b, sb_bad)
        assert not np.all(gemm_tolerance_ok(y_bad2, y, bound))


def test_bf16_tolerance_term():
    assert bf16_half_ulp(np.array([1.0, 3.0, 2.0 ** 20])).tolist() == \
        [2.0 ** -8, 2.0 ** -7, 2.0 ** 12]
    y = np.array([1.0])
    assert gemm_tolerance_ok(y, np.array([1.0 + 2.0 ** -9]), np.array([0.0]), "bf16")[0]
    assert not gemm_tolerance_ok(y, np.array([1.0 + 2.0 ** -9]), np.array([0.0]), "f32")[0]


def test_wgrad_row_scales_match_dequantized_product():
    rng = np.random.default_rng(14)
    t, h, f = 256, 128, 256
    x = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(rng.standard_normal((t, h)).astype(np.float32)))
    dy = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(
        rng.standard_normal((t, f)).astype(np.float32) * np.float32(1e-3)))
    xt, sxt = quant_128x1_t(x)        # [h, t], [h, t/128]
    dyt, sdyt = quant_128x1_t(dy)     # [f, t], [f, t/128]
    y, bound = blockscaled_gemm_ref(xt, sxt, dyt, sdyt, "row")
    from oracle import e4m3_decode
    deq_x = e4m3_decode(xt) * np.repeat(sxt.astype(np.float64), 128, axis=1)
    deq_dy = e4m3_decode(dyt) * np.repeat(sdyt.astype(np.float64), 128, axis=1)
    assert np.allclose(y, deq_x @ deq_dy.T, rtol=0, atol=1e-12 * np.max(bound))


def test_grouped_equals_per_group_dense():
    rng = np.random.default_rng(15)
    g, n, k = 4, 128, 256
    counts = np.array([5, 0, 130, 1])
    off = np.concatenate([[0], np.cumsum(counts)])
    a = _rand_codes(rng, (off[-1], k))
    sa = rng.random((off[-1], 2)).astype(np.float32) + np.float32(0.1)
    b = _rand_codes(rng, (g, n, k))
    sb = rng.random((g, 1, 2)).astype(np.float32) + np.float32(0.1)
    y, bound = grouped_gemm_ref(off, a, sa, b, sb)
    for e in range(g):
        lo, hi = off[e], off[e + 1]
        if hi > lo:
            ye, be = blockscaled_gemm_ref(a[lo:hi], sa[lo:hi], b[e], sb[e])
            assert np.array_equal(y[lo:hi], ye) and np.array_equal(bound[lo:hi], be)
    y1, _ = grouped_gemm_ref(np.array([0, off[-1]]), a, sa, b[:1], sb[:1])
    yd, _ = blockscaled_gemm_ref(a, sa, b[0], sb[0])
    assert np.array_equal(y1, yd)
    with pytest.raises(ValueError):
        grouped_gemm_ref(np.array([0, 3, 2, 136, 136]), a, sa, b, sb)
