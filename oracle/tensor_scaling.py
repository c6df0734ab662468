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

Precision reading: everything in float32, as for the fine-grained quantizer:
amax, (1 + margin), the widened amax, the division by the format maximum and
x / s are each one float32 operation.
"""
import numpy as np

from .e4m3 import e4m3_encode
from .e5m2 import e5m2_encode

FORMATS = {"e4m3": (np.float32(448.0), e4m3_encode), "e5m2": (np.float32(57344.0), e5m2_encode)}
TENSOR_GUARD = np.float32(1e-6)


def _finite(x):
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("per-tensor quantizers take finite inputs only")
    return x


def tensor_scale(amax, fmt="e4m3", margin=0.0):
    """s = fl32(fl32(amax * fl32(1 + margin)) / fmt_max); s := 1 if s < fl32(1e-6)."""
    fmax, _ = FORMATS[fmt]
    widen = np.float32(1.0) + np.float32(margin)
    s = np.float32(np.float32(amax) * widen) / fmax
    return np.float32(1.0) if s < TENSOR_GUARD else np.float32(s)


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
    codes = enc(x / s)                      # the encoder saturates at the format maximum
    amax = np.float32(np.abs(x).max()) if x.size else np.float32(0.0)
    new_history = np.concatenate([[amax], history[:-1]]).astype(np.float32)
    return codes, s, amax, new_history
