"""Per-tensor FP8 scaling: the prior-art baselines the fine-grained method is
compared with.

Test infrastructure only (see the package docstring).

* Current scaling with a margin, HolySheep (zh) troubleshooting entry
  "错误 1: FP8 精度溢出", class ``SafeFP8Quantizer.safe_quantize``: one amax
  over the whole tensor, widened by (1 + margin); scale = that / 448; a scale
  below 1e-6 is replaced by 1; codes = cast of tensor / scale.
* Delayed scaling, HolySheep (zh) ``FP8Config`` (``amax_history_len`` 1024,
  ``margin`` 0.0, on Transformer Engine): the page gives only these settings.
  Reading: the scale of this call comes from the largest amax in the history
  of earlier calls, with the same margin, division and guard as above; the
  codes saturate (a stale scale can be too small); afterwards this tensor's
  amax enters the history at the front and the oldest entry drops out.
* Formats: E4M3 (max 448) for activations and weights; E5M2 (max 57344) for
  gradients in the hybrid recipe (``e5m2``).

Precision reading.  The page computes the scale on Python floats: ``.item()``
turns the tensor's amax into a binary64 value (exactly), and (1 + margin), the
widened amax, the division by 448.0 and the ``scale < 1e-6`` test are binary64
operations.  The oracle does the same and rounds the result once to float32,
the precision in which the scale is stored and in which x / s is taken (one
float32 division, as the fine-grained quantizer takes it).
"""
import numpy as np

from .e4m3 import e4m3_encode
from .e5m2 import e5m2_encode

FORMATS = {"e4m3": (448.0, e4m3_encode), "e5m2": (57344.0, e5m2_encode)}
TENSOR_GUARD = 1e-6          # the page's "scale too small" threshold, a Python float


def _finite(x):
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("per-tensor quantizers take finite inputs only")
    return x


def tensor_scale(amax, fmt="e4m3", margin=0.0):
    """SafeFP8Quantizer's scale: d = amax * (1 + margin) / fmt_max on Python
    floats (binary64, the page's order of operations); 1.0 if d < 1e-6; then
    rounded once to float32."""
    fmax, _ = FORMATS[fmt]
    dynamic_amax = float(amax) * (1.0 + float(margin))
    d = dynamic_amax / fmax
    if d < TENSOR_GUARD:
        return np.float32(1.0)
    return np.float32(d)


def quant_tensor_current(x, fmt="e4m3", margin=0.0):
    """Current per-tensor scaling.  Returns (codes uint8, scale, amax)."""
    x = _finite(x)
    amax = np.float32(np.abs(x).max()) if x.size else np.float32(0.0)
    s = tensor_scale(amax, fmt, margin)
    _, enc = FORMATS[fmt]
    return enc(x / s), s, amax


def quant_tensor_delayed(x, history, fmt="e4m3", margin=0.0):
    """Delayed per-tensor scaling.  Returns (codes, scale, amax, new history)."""
    x = _finite(x)
    history = np.asarray(history, dtype=np.float32)
    s = tensor_scale(history.max(), fmt, margin)
    _, enc = FORMATS[fmt]
    with np.errstate(over="ignore"):        # a stale scale may overflow x / s to inf,
        codes = enc(x / s)                  # which the encoder saturates to the format maximum
    amax = np.float32(np.abs(x).max()) if x.size else np.float32(0.0)
    new_history = np.concatenate([[amax], history[:-1]]).astype(np.float32)
    return codes, s, amax, new_history
