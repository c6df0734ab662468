"""Block-scaled FP8 GEMM with FP32 promotion per 128-deep K block: plain CPU reference.

Test infrastructure only (see the package docstring).

codingmall (sv), "Ökad ackumuleringsprecision": the FP8 GEMM's partial results
are promoted into FP32 at fixed intervals.  With activation tiles of 1x128 and
weight blocks of 128x128 ("Finkornig kvantisering") the scales are constant
over each 128-deep K interval, so the interval is 128 and the promoted value is

    Y[m, n] = sum_kb  sa[m, kb] * sb[., kb] * P_kb[m, n],
    P_kb[m, n] = sum_{k in block kb} dec(a[m, k]) * dec(b[n, k]),

where dec() is the E4M3 value of a code, sa are the A tiles' scales
([M, K/128]) and sb the B scales: one per 128x128 block ([N/128, K/128],
"block128") or, for the weight-gradient GEMM whose B operand is itself
128x1-quantized along K, one per row and K block ([N, K/128], "row").

The reference evaluates this definition in float64.  Each product of two
E4M3 values is an integer times 2^-18 below 2^18, so a 128-term block
partial stays below 2^43 * 2^-18 and is exact in float64 whatever order the
BLAS library sums it in; sa*sb (two float32) is exact too.  Only the final
multiply and the K/128-term sum round, at ~2^-53.

Tolerance (the one the build is held to): |y - Y| <= 2e-5 * S per element,
with S[m, n] = sum_k |a_k * b_k| over the dequantized operands, plus half a
bf16 ulp of y when the output is bf16.  The linear error bound of an fp32
evaluation with one rounding per block partial, one per scale product, one
per promotion and one per accumulation is (128 + K/128 + 2) * 2^-24, below
1.2e-5 for every K here.
"""
import numpy as np

from .e4m3 import e4m3_decode

TOL_REL = 2e-5


def _sb_per_col(b_scale, n, kind):
    """B scales expanded to one row per output column: [N, K/128] float64."""
    sb = np.asarray(b_scale, dtype=np.float64)
    if kind == "block128":
        return np.repeat(sb, 128, axis=0)[:n]
    if kind == "row":
        return sb
    raise ValueError("b_kind must be 'block128' or 'row'")


def blockscaled_gemm_ref(a_codes, a_scale, b_codes, b_scale, b_kind="block128"):
    """Y = dequant(A) . dequant(B)^T promoted per 128-K block, in float64.

    a_codes: uint8 [M, K]; a_scale: float32 [M, K/128];
    b_codes: uint8 [N, K]; b_scale: [N/128, K/128] (block128) or [N, K/128] (row).
    Returns (Y float64 [M, N], S float64 [M, N]) where S is the sum of
    |a_k * b_k| that scales the tolerance.
    """
    a = e4m3_decode(a_codes)
    b = e4m3_decode(b_codes)
    m, k = a.shape
    n = b.shape[0]
    if k % 128 or b.shape[1] != k:
        raise ValueError("K must match and be a multiple of 128")
    sa = np.asarray(a_scale, dtype=np.float64)
    sb = _sb_per_col(b_scale, n, b_kind)
    y = np.zeros((m, n))
    bound = np.zeros((m, n))
    for kb in range(k // 128):
        blk = slice(kb * 128, (kb + 1) * 128)
        p = a[:, blk] @ b[:, blk].T                       # exact block partial
        pabs = np.abs(a[:, blk]) @ np.abs(b[:, blk]).T
        sc = sa[:, kb][:, None] * sb[:, kb][None, :]      # exact in float64
        y += sc * p
        bound += np.abs(sc) * pabs
    return y, bound


def grouped_gemm_ref(offsets, a_codes, a_scale, b_codes, b_scale):
    """Per-group GEMM over contiguous row ranges (mixture-of-experts layout).

    The HolySheep (zh) MoE module loops over experts and multiplies each
    expert's tokens by that expert's weight; here group g owns rows
    [offsets[g], offsets[g+1]) of A and has its own B (block128 scales).
    b_codes: [G, N, K]; b_scale: [G, N/128, K/128].  Returns (Y, S) for all
    M_total rows; an empty group contributes no rows.
    """
    off = np.asarray(offsets, dtype=np.int64)
    g_count = b_codes.shape[0]
    m_total = a_codes.shape[0]
    n = b_codes.shape[1]
    if off.shape != (g_count + 1,) or off[0] != 0 or off[-1] != m_total \
            or np.any(np.diff(off) < 0):
        raise ValueError("offsets must be a nondecreasing prefix sum of length G+1")
    y = np.zeros((m_total, n))
    bound = np.zeros((m_total, n))
    for g in range(g_count):
        lo, hi = off[g], off[g + 1]
        if hi == lo:
            continue
        y[lo:hi], bound[lo:hi] = blockscaled_gemm_ref(
            a_codes[lo:hi], a_scale[lo:hi], b_codes[g], b_scale[g], "block128")
    return y, bound


def blockscaled_gemm_fp32_model(a_codes, a_scale, b_codes, b_scale, b_kind="block128"):
    """The same promotion carried out step by step in float32.

    p = fl32(P_kb); c = fl32(sa * sb); acc = fl32(acc + fl32(p * c)).  This is
    one valid float32 evaluation of the method; the tests use it to show the
    tolerance is attainable by an fp32 accumulator.
    """
    a = e4m3_decode(a_codes)
    b = e4m3_decode(b_codes)
    m, k = a.shape
    n = b.shape[0]
    sa = np.asarray(a_scale, dtype=np.float32)
    sb = _sb_per_col(b_scale, n, b_kind).astype(np.float32)
    acc = np.zeros((m, n), dtype=np.float32)
    for kb in range(k // 128):
        blk = slice(kb * 128, (kb + 1) * 128)
        p = (a[:, blk] @ b[:, blk].T).astype(np.float32)
        c = sa[:, kb][:, None] * sb[:, kb][None, :]
        acc = acc + p * c
    return acc


def bf16_half_ulp(y):
    """Half the bf16 spacing at |y| (float64); normal spacing 2^(e-7)."""
    a = np.abs(np.asarray(y, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 2.0 ** -126)))
    e = np.maximum(e, -126.0)
    return np.exp2(e - 7.0) / 2.0


def gemm_tolerance_ok(y, y_ref, bound, out_dtype="f32"):
    """Elementwise pass mask of |y - Y| <= 2e-5 * S (+ half bf16 ulp of y)."""
    y = np.asarray(y, dtype=np.float64)
    tol = TOL_REL * np.asarray(bound, dtype=np.float64)
    if out_dtype == "bf16":
        tol = tol + bf16_half_ulp(y)
    return np.abs(y - y_ref) <= tol
