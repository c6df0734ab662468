"""Pins of the per-tensor (prior-art) quantizers: exact rational arithmetic,
closed forms and the delayed-scaling history semantics."""
import numpy as np

import oracle
from oracle import e4m3_encode, e5m2_encode
import exact


def test_scale_closed_forms():
    assert oracle.tensor_scale(np.float32(448.0)) == np.float32(1.0)
    assert oracle.tensor_scale(np.float32(57344.0), "e5m2") == np.float32(1.0)
    assert oracle.tensor_scale(np.float32(0.0)) == np.float32(1.0)                 # guard
    assert oracle.tensor_scale(np.float32(448e-6 * 0.99)) == np.float32(1.0)       # s < 1e-6
    assert oracle.tensor_scale(np.float32(896.0), margin=0.0) == np.float32(2.0)
    # margin 0.15: fl32(1.15) and one rounding per step
    s = oracle.tensor_scale(np.float32(448.0), margin=0.15)
    assert s == np.float32(np.float32(448.0) * np.float32(1.15)) / np.float32(448.0)


def test_current_scaling_matches_exact_arithmetic():
    rng = np.random.default_rng(60)
    for fmt, fmax, enc in (("e4m3", 448, exact.e4m3_encode_exact), ("e5m2", 57344, exact.e5m2_encode_exact)):
        for margin in (0.0, 0.15):
            x = (rng.standard_normal(700) * np.exp2(rng.uniform(-8, 8))).astype(np.float32)
            x[:5] = [0.0, -0.0, 1e-30, -3.5, 2.0 ** -130]
            codes, s, amax = oracle.quant_tensor_current(x, fmt, margin)
            want_codes, want_s = exact.tensor_quantize_exact(x, fmax, enc, margin)
            assert float(s) == want_s and amax == np.abs(x).max()
            assert codes.tolist() == want_codes


def test_current_scaling_max_element_and_error():
    rng = np.random.default_rng(61)
    x = rng.standard_normal((64, 96)).astype(np.float32) * np.float32(7.0)
    codes, s, amax = oracle.quant_tensor_current(x)
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert codes[i] & 0x7F == 0x7E                                # margin 0: amax -> 448
    err = np.abs(oracle.e4m3_decode(codes) * float(s) - x)
    assert np.all(err <= oracle.e4m3_half_ulp(x / float(s)) * float(s) * (1 + 2 ** -20))
    codes2, _, _ = oracle.quant_tensor_current(x, margin=0.25)     # the margin leaves headroom
    assert np.abs(oracle.e4m3_decode(codes2)).max() <= 448 / 1.25 * (1 + 2 ** -4)


def test_delayed_scaling_history_and_saturation():
    rng = np.random.default_rng(62)
    x = rng.standard_normal(512).astype(np.float32)
    amax = np.float32(np.abs(x).max())
    hist = np.zeros(8, np.float32)
    hist[:3] = [amax, amax / 2, amax / 4]
    codes, s, a, new = oracle.quant_tensor_delayed(x, hist)
    c_now, s_now, _ = oracle.quant_tensor_current(x)
    assert s == s_now and np.array_equal(codes, c_now)             # history max == current amax
    assert a == amax and new.tolist() == [amax, amax, amax / 2, amax / 4, 0, 0, 0, 0]
    # stale, too small history: the largest values saturate at +-448
    codes, s, _, _ = oracle.quant_tensor_delayed(x, np.float32([amax / 8] + [0] * 7))
    assert s == oracle.tensor_scale(amax / 8)
    big = np.abs(x) / float(s) > 464
    assert big.any() and np.all(codes[big] & 0x7F == 0x7E)
    want, _ = exact.tensor_quantize_exact(x, 448, exact.e4m3_encode_exact, amax=float(amax / 8))
    assert codes.tolist() == want
    # an empty history gives the guard scale 1
    _, s, _, _ = oracle.quant_tensor_delayed(x, np.zeros(1024, np.float32))
    assert s == np.float32(1.0)


def test_e5m2_delayed_uses_its_own_maximum():
    x = np.float32([1000.0, -2.0, 0.5])
    codes, s, _, _ = oracle.quant_tensor_delayed(x, np.float32([1000.0]), "e5m2")
    assert s == np.float32(1000.0) / np.float32(57344.0)
    assert codes[0] == 0x7B and np.array_equal(codes, e5m2_encode(x / s))
    assert not np.array_equal(codes, e4m3_encode(x / s))
