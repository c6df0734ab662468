"""Pins of the oracle's dequantization and bf16 rounding against routes that
share nothing with them: float32 multiplication, torch's own bf16 cast, and
values fixed by the formats."""
import numpy as np
import pytest

import oracle
from oracle import e4m3_decode


def _scales(rng, n):
    s = np.exp2(rng.uniform(-40, 40, n)).astype(np.float32) * rng.uniform(1, 2, n).astype(np.float32)
    return np.concatenate([s, np.float32([1.0, 448 ** -1, 1e-10, 2.0 ** -126, 3.0e38 / 448])])


def test_dequant_f32_is_one_float32_multiply():
    """fl32(dec * s) equals the IEEE float32 product of the float32 code value
    and s, for all 256 codes and scales across the float32 range."""
    rng = np.random.default_rng(20)
    s = _scales(rng, 400)
    codes = np.tile(np.arange(256, dtype=np.uint8), (len(s), 1))            # [n, 256] = 2 tiles of 128
    scales = np.repeat(s[:, None], 2, axis=1)
    got = oracle.dequant_f32(codes, scales, "1x128")
    want = e4m3_decode(codes).astype(np.float32) * scales.repeat(128, axis=1)  # float32 * float32
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2 * len(s)                                            # 0x7F and 0xFF
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def test_dequant_layouts_brute_force():
    rng = np.random.default_rng(21)
    codes = rng.integers(0, 256, (256, 384), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x11
    s_row = rng.uniform(0.1, 3, (256, 3)).astype(np.float32)
    s_blk = rng.uniform(0.1, 3, (2, 3)).astype(np.float32)
    y_row = oracle.dequant_f32(codes, s_row, "1x128")
    y_blk = oracle.dequant_f32(codes, s_blk, "128x128")
    for (r, c) in [(0, 0), (5, 127), (5, 128), (200, 383), (255, 256), (128, 129)]:
        v = float(e4m3_decode(codes[r, c]))
        assert y_row[r, c] == np.float32(v * float(s_row[r, c // 128]))
        assert y_blk[r, c] == np.float32(v * float(s_blk[r // 128, c // 128]))
    with pytest.raises(ValueError):
        oracle.dequant_f32(codes, s_row, "128x1")


def test_bf16_rne_fixed_values():
    f = oracle.f32_to_bf16_rne
    vals = np.float32([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -0.0, 0.0,
                       3.3895314e38, 3.4e38, 2.0 ** -133, -(2.0 ** -126)])
    want = [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0x8000, 0x0000, 0x7F7F, 0x7F80, 0x0001, 0x8080]
    assert f(vals).tolist() == want
    n = f(np.float32([np.nan, -np.nan]))
    assert all((b & 0x7F80) == 0x7F80 and (b & 0x7F) for b in n.tolist())


def test_bf16_rne_matches_torch_cast():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(22)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(1e3),
        np.exp2(rng.uniform(-140, 127, 100000)).astype(np.float32),
        # exact ties: a bf16 value plus half its spacing
        (rng.integers(0, 0x7F00, 50000).astype(np.uint32) << 16 | 0x8000).view(np.float32),
    ])
    x = x[np.isfinite(x)]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16_rne(x), want)


def test_dequant_bf16_is_rounded_f32():
    rng = np.random.default_rng(23)
    codes = rng.integers(0, 0x7E, (128, 256), dtype=np.uint8)
    s = rng.uniform(0.5, 2, (1, 2)).astype(np.float32)
    y32 = oracle.dequant_f32(codes, s, "128x128")
    assert np.array_equal(oracle.dequant_bf16(codes, s, "128x128"), oracle.f32_to_bf16_rne(y32))
