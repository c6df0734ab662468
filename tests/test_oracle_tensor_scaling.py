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
    # margin 1 doubles the amax exactly: 448 * 2 / 448 = 2
    assert oracle.tensor_scale(np.float32(448.0), margin=1.0) == np.float32(2.0)
    # margin 0: one float32 rounding of amax / 448 (rounding the binary64
    # quotient again to float32 cannot change it)
    for a in (1.0, 3.0, 1e-3, 7.5e5):
        assert oracle.tensor_scale(np.float32(a)) == exact.rn32(exact.Fraction(float(np.float32(a))) / 448)


def test_scale_follows_binary64_steps():
    """The scale takes the page's Python-float steps and one final float32
    rounding.  A chain of float32 operations would differ in the last bit for
    a good share of amax values at margins 0.1 / 0.15, so these values tell the
    two readings apart."""
    rng = np.random.default_rng(64)
    amaxes = (rng.standard_normal(3000) * np.exp2(rng.uniform(-20, 20, 3000))).astype(np.float32)
    differ = 0
    for margin in (0.1, 0.15):
        for a in np.abs(amaxes):
            got = oracle.tensor_scale(a, margin=margin)
            _, want = exact.tensor_quantize_exact([float(a)], 448, exact.e4m3_encode_exact, margin)
            assert float(got) == want, (a, margin)
            f32_chain = np.float32(np.float32(a * np.float32(np.float32(1) + np.float32(margin))) / np.float32(448))
            differ += int(f32_chain != got)
    assert differ > 0.1 * 2 * len(amaxes)


def test_current_scaling_against_torch_cpu_cast():
    """SafeFP8Quantizer's steps done with torch on the CPU for a float32
    tensor: amax through .item(), the scale on Python floats, the quotient in
    float32 and torch's E4M3 cast.  Its codes and scale equal the oracle's."""
    import torch
    rng = np.random.default_rng(65)
    for margin in (0.1, 0.15, 0.0):
        x = (rng.standard_normal((48, 40)) * np.exp2(rng.uniform(-6, 6))).astype(np.float32)
        t = torch.from_numpy(x)
        amax = torch.abs(t).max().item()
        scale = amax * (1 + margin) / 448.0
        if scale < 1e-6:
            scale = 1.0
        want = (t / scale).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        codes, s, a = oracle.quant_tensor_current(x, "e4m3", margin)
        assert a == np.float32(amax)
        assert s == np.float32(scale)
        assert np.array_equal(codes, want)


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
