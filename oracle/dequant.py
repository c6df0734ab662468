"""Dequantization of E4M3 codes with their tile scales, as float32 or bf16.

Test infrastructure only (see the package docstring).

HolySheep (zh), section 2.2, ``FP8BlockQuantizer.dequantize``: the codes are
taken back to float32 and multiplied by the stored per-tile scale.  So the
result is fl32(dec(code) * s): the product of a code value (at most 4
significant bits) and a float32 scale (24 bits) is exact in float64, and
rounding it to float32 once is the float32 multiply.  A bf16 result rounds
that float32 to the nearest bf16, ties to the even one (the usual cast).

Readings: the tile layouts are those of the quantizer (1x128 along the rows,
128x128 blocks); a NaN code gives NaN.
"""
import numpy as np

from .quantize import dequant_1x128, dequant_128x128


def dequant_f32(codes, scales, tiling="1x128"):
    """fl32(dec(code) * s) for every code, as float32 [rows, cols]."""
    if tiling == "1x128":
        exact = dequant_1x128(codes, scales)
    elif tiling == "128x128":
        exact = dequant_128x128(codes, scales)
    else:
        raise ValueError(f"unknown tiling {tiling!r}")
    return exact.astype(np.float32)         # one round-to-nearest-even of the exact product


def f32_to_bf16_rne(x):
    """bf16 bit patterns (uint16) nearest to float32 values, ties to even.

    bf16 keeps the top 16 bits of a float32.  Rounding adds half of the
    dropped 16-bit unit, minus one when the kept part is even, so that exact
    halves go to the even pattern; a carry out of the significand bumps the
    exponent, which is the correct rounding (up to infinity past the largest
    finite value).  NaN stays a (quiet) NaN with its sign.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep_odd = (u >> 16) & 1
    r = ((u + 0x7FFF + keep_odd) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    r = np.where(nan, ((u >> 16).astype(np.uint16) | np.uint16(0x0040)), r)
    return r.astype(np.uint16)


def dequant_bf16(codes, scales, tiling="1x128"):
    """bf16 bits of fl32(dec(code) * s), rounded to nearest even."""
    return f32_to_bf16_rne(dequant_f32(codes, scales, tiling))
