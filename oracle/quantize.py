"""Fine-grained online quantization to E4M3 with one FP32 scale per tile.

Test infrastructure only (see the package docstring).

What is computed, per tile T (a 1x128 row segment, a 128x1 column segment or
a 128x128 block), in the order of HolySheep (zh) section 2.2,
``FP8BlockQuantizer.quantize``:

1. take the tile's values as float32 (a bf16 input widens exactly);
2. amax = the largest |x| in the tile;
3. s = amax / 448 in float32; when s is not above float32(1e-10) the tile
   gets s = 1 instead (the page's divide-by-zero guard);
4. v = x / s in float32 for every element;
5. code = E4M3 rounding of v (``e4m3.e4m3_encode``);
6. the stored scale is s itself, so dequantization multiplies
   (``dequantize`` in the same section).

Tile shapes follow codingmall (sv) "Finkornig kvantisering": activations in
1x128 tiles along the contiguous (K) dimension, weights in 128x128 blocks;
"Online-kvantisering": each scale comes from its own tile's current values,
with no history.  The 128x1 tiling (128 consecutive rows of one column) is
the same rule applied to the transpose; the weight-gradient GEMM needs it
because its contraction runs over tokens, and "Unified E4M3 Format" puts the
backward GEMMs in E4M3 too.

Readings where the pages leave a step open:
* all arithmetic is float32 (the page's docstring calls the scale FP32; its
  literal code would divide a bf16 tensor in bf16, which the docstring rules
  out);
* tile size 128, not the 32 the page's class defaults to;
* a partial tail tile is rejected instead of dropped;
* inputs are finite.
"""
import numpy as np

from .e4m3 import e4m3_encode, e4m3_decode

E4M3_MAX_F32 = np.float32(448.0)
SCALE_GUARD = np.float32(1e-10)   # float32(1e-10) == 0x2EDBE6FF


def tile_scale(amax):
    """FP32 dequantizing scale of tiles with the given float32 amax values.

    s = fl32(amax / 448); s := 1 when not (s > fl32(1e-10)).
    """
    amax = np.asarray(amax, dtype=np.float32)
    s = amax / E4M3_MAX_F32                      # IEEE binary32 division
    return np.where(s > SCALE_GUARD, s, np.float32(1.0)).astype(np.float32)


def _check(x):
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("oracle quantizer takes finite inputs only")
    return x


def quant_1x128(x):
    """1x128 tiles along each row.  x: [M, K] with K % 128 == 0.

    Returns (codes uint8 [M, K], scales float32 [M, K // 128]).
    """
    x = _check(x)
    m, k = x.shape
    if k % 128:
        raise ValueError("K must be a multiple of 128")
    tiles = x.reshape(m, k // 128, 128)
    amax = np.abs(tiles).max(axis=2)
    s = tile_scale(amax)
    v = tiles / s[:, :, None]                     # float32 / float32
    codes = e4m3_encode(v).reshape(m, k)
    return codes, s


def quant_128x1_t(x):
    """128x1 tiles: 128 consecutive rows of one column.  x: [R, C], R % 128 == 0.

    The codes come out transposed, so the tiled (token) dimension is the
    contiguous one: returns (codes uint8 [C, R] = codes of x^T,
    scales float32 [C, R // 128]).  A 128x1 tile of x is a 1x128 tile of x^T.
    """
    x = _check(x)
    r, c = x.shape
    if r % 128:
        raise ValueError("rows must be a multiple of 128")
    return quant_1x128(np.ascontiguousarray(x.T))


def quant_128x128(w):
    """128x128 blocks.  w: [N, K], both multiples of 128.

    Returns (codes uint8 [N, K], scales float32 [N // 128, K // 128]).  The
    transposed operand for the data-gradient GEMM is codes.T with scales.T:
    a block's scale does not depend on the orientation.
    """
    w = _check(w)
    n, k = w.shape
    if n % 128 or k % 128:
        raise ValueError("both dimensions must be multiples of 128")
    blocks = w.reshape(n // 128, 128, k // 128, 128)
    amax = np.abs(blocks).max(axis=(1, 3))
    s = tile_scale(amax)
    v = blocks / s[:, None, :, None]
    codes = e4m3_encode(v).reshape(n, k)
    return codes, s


def dequant_1x128(codes, scales):
    """code value times its tile's scale (float64), for 1x128 tiles.

    HolySheep (zh) section 2.2, ``dequantize``: multiply each code by the
    stored scale.
    """
    m, k = codes.shape
    vals = e4m3_decode(codes).reshape(m, k // 128, 128)
    return (vals * np.asarray(scales, np.float64)[:, :, None]).reshape(m, k)


def dequant_128x128(codes, scales):
    """code value times its block's scale (float64), for 128x128 blocks."""
    n, k = codes.shape
    vals = e4m3_decode(codes).reshape(n // 128, 128, k // 128, 128)
    s = np.asarray(scales, np.float64)[:, None, :, None]
    return (vals * s).reshape(n, k)
