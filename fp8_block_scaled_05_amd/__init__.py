"""fp8_block_scaled_05_amd: fine-grained FP8 block-scaled quantization and GEMM for MI355X.

A thin binding over the C ABI of ``libfp8bs.so`` (declared in
``include/fp8bs.h``).  Every function here only marshals arguments: it checks
tensor devices/dtypes/strides, allocates outputs with PyTorch when the caller
does not pass them, and calls the library entry point of the same name on
PyTorch's current HIP stream.  All quantization and GEMM work runs in the
library's gfx950 kernels; there is no fallback.  If the library is missing
the first call raises.

The method follows the codingmall.com knowledge-base article on the role of
FP8 precision in DeepSeek-V3 training (sections "Finkornig kvantisering",
"Online-kvantisering", "Ökad ackumuleringsprecision", "Unified E4M3 Format")
and the HolySheep AI (zh) FP8 mixed-precision article, section 2.2
(FP8BlockQuantizer).
"""
import ctypes
import os
import re

__all__ = [
    "fp8_quant_act_1x128", "fp8_quant_act_dual", "fp8_quant_w_128x128", "fp8_quant_batch",
    "fp8_dequant", "fp8_quant_tensor",
    "fp8_blockscaled_gemm", "fp8_blockscaled_gemm_fp8mma", "fp8_blockscaled_gemm_quant",
    "fp8_blockscaled_grouped_gemm", "last_error", "version", "lib", "lib_path",
    "Fp8bsError", "STATUS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libfp8bs.so"

STATUS = {0: "OK", 1: "INVALID_ARG", 2: "SHAPE", 3: "ALIGNMENT", 4: "UNSUPPORTED", 5: "HIP"}
BF16, F32 = 0, 1
TILE_1x128, TILE_128x1_T, TILE_128x128 = 0, 1, 2
BSCALE_BLOCK128, BSCALE_ROW = 0, 1
FMT_E4M3, FMT_E5M2 = 0, 1
_FMT = {"e4m3": FMT_E4M3, "e5m2": FMT_E5M2}


class Fp8bsError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"fp8bs {STATUS.get(status, status)}: {message}")
        self.status = status


MAX_QUANT_JOBS = 8


class QuantJob(ctypes.Structure):
    """fp8bs_quant_job of include/fp8bs.h."""
    _fields_ = [("x", ctypes.c_void_p), ("x_dtype", ctypes.c_int32), ("tiling", ctypes.c_int32),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("ld_x", ctypes.c_int64),
                ("q", ctypes.c_void_p), ("ld_q", ctypes.c_int64), ("scale", ctypes.c_void_p)]


_lib = None


def lib_path():
    return os.path.join(_PKG, _LIB_NAME)


def lib():
    """The loaded libfp8bs.so with argument types set (raises if not built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m fp8_block_scaled_05_amd.build`")
    L = ctypes.CDLL(path)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    L.fp8_quant_act_1x128.argtypes = [vp, i32, i64, i64, i64, i32, vp, i64, vp, vp]
    L.fp8_quant_w_128x128.argtypes = [vp, i32, i64, i64, i64, vp, i64, vp, vp, i64, vp]
    L.fp8_quant_act_dual.argtypes = [vp, i32, i64, i64, i64, vp, i64, vp, vp, i64, vp, vp]
    L.fp8_quant_batch.argtypes = [ctypes.POINTER(QuantJob), i32, vp]
    L.fp8_dequant.argtypes = [vp, i64, i64, i64, vp, i32, vp, i32, i64, vp]
    L.fp8_quant_tensor.argtypes = [vp, i32, i64, i64, i64, i32, ctypes.c_double, vp, i32, vp, i64,
                                   vp, vp, vp]
    L.fp8_blockscaled_gemm.argtypes = [i64, i64, i64, vp, i64, vp, vp, i64, vp, i32, vp, i32, i64, vp]
    L.fp8_blockscaled_gemm_fp8mma.argtypes = [i64, i64, i64, vp, i64, vp, vp, i64, vp, i32, vp, i32, i64, vp]
    L.fp8_blockscaled_gemm_quant.argtypes = [i64, i64, i64, vp, i64, vp, vp, i64, vp, i32, vp, i64, vp, vp]
    L.fp8_blockscaled_grouped_gemm.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, i32, vp]
    for f in ("fp8_quant_act_1x128", "fp8_quant_act_dual", "fp8_quant_w_128x128", "fp8_quant_batch",
              "fp8_dequant",
              "fp8_quant_tensor", "fp8_blockscaled_gemm", "fp8_blockscaled_gemm_fp8mma",
              "fp8_blockscaled_gemm_quant", "fp8_blockscaled_grouped_gemm"):
        getattr(L, f).restype = ctypes.c_int
    L.fp8bs_last_error.restype = ctypes.c_char_p
    L.fp8bs_last_error.argtypes = []
    L.fp8bs_version.restype = ctypes.c_char_p
    L.fp8bs_version.argtypes = []
    _lib = L
    return L


def last_error():
    return lib().fp8bs_last_error().decode()


def version():
    return lib().fp8bs_version().decode()


def header_functions():
    """Names of the functions declared in include/fp8bs.h."""
    hdr = os.path.join(os.path.dirname(_PKG), "include", "fp8bs.h")
    text = open(hdr).read()
    return re.findall(r"^\s*(?:fp8bs_status|const char\*)\s+(\w+)\s*\(", text, re.M)


def _check(status):
    if status != 0:
        raise Fp8bsError(status, last_error())


# --------------------------------------------------------------------------
# torch marshalling
def _torch():
    import torch
    return torch


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _pitch(t, name):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")
    return t.stride(0)


def _dtype_code(t, name):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"{name} must be bfloat16 or float32, got {t.dtype}")


def _on_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


def _need(t, shape, dtype, name):
    """The kernels write/read exactly `shape` through `t`: refuse anything smaller."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def fp8_quant_act_1x128(x, tiling="1x128", q=None, scale=None):
    """Online activation quantization.

    tiling "1x128": returns (q uint8 [rows, cols], scale f32 [rows, cols/128]).
    tiling "128x1_T": returns (q uint8 [cols, rows] = codes of x^T,
    scale f32 [cols, rows/128]).
    """
    torch = _torch()
    _on_gpu(x, q, scale)
    rows, cols = x.shape
    tcode = {"1x128": TILE_1x128, "128x1_T": TILE_128x1_T}[tiling]
    if q is None:
        shape = (rows, cols) if tcode == TILE_1x128 else (cols, rows)
        q = torch.empty(shape, dtype=torch.uint8, device=x.device)
    if scale is None:
        shape = (rows, cols // 128) if tcode == TILE_1x128 else (cols, rows // 128)
        scale = torch.empty(shape, dtype=torch.float32, device=x.device)
    qshape = (rows, cols) if tcode == TILE_1x128 else (cols, rows)
    sshape = (rows, cols // 128) if tcode == TILE_1x128 else (cols, rows // 128)
    _need(q, qshape, torch.uint8, "q")
    _need(scale, sshape, torch.float32, "scale")
    if not scale.is_contiguous():
        raise ValueError("scale must be contiguous")
    _check(lib().fp8_quant_act_1x128(_ptr(x), _dtype_code(x, "x"), rows, cols, _pitch(x, "x"),
                                     tcode, _ptr(q), _pitch(q, "q"), _ptr(scale), _stream()))
    return q, scale


def fp8_quant_act_dual(x, q=None, scale=None, q_t=None, scale_t=None):
    """Both activation tilings from one read of x: returns (q [rows, cols],
    scale [rows, cols/128]) of the 1x128 tiling and (q_t [cols, rows],
    scale_t [cols, rows/128]) of the 128x1 tiling written transposed."""
    torch = _torch()
    _on_gpu(x, q, scale, q_t, scale_t)
    rows, cols = x.shape
    dev = x.device
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty((rows, cols // 128), dtype=torch.float32, device=dev)
    if q_t is None:
        q_t = torch.empty((cols, rows), dtype=torch.uint8, device=dev)
    if scale_t is None:
        scale_t = torch.empty((cols, rows // 128), dtype=torch.float32, device=dev)
    _need(q, (rows, cols), torch.uint8, "q")
    _need(scale, (rows, cols // 128), torch.float32, "scale")
    _need(q_t, (cols, rows), torch.uint8, "q_t")
    _need(scale_t, (cols, rows // 128), torch.float32, "scale_t")
    for t, nm in ((scale, "scale"), (scale_t, "scale_t")):
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    _check(lib().fp8_quant_act_dual(_ptr(x), _dtype_code(x, "x"), rows, cols, _pitch(x, "x"),
                                    _ptr(q), _pitch(q, "q"), _ptr(scale), _ptr(q_t),
                                    _pitch(q_t, "q_t"), _ptr(scale_t), _stream()))
    return q, scale, q_t, scale_t


def fp8_quant_w_128x128(w, transpose=False, q=None, scale=None, q_t=None):
    """128x128 block quantization.  Returns (q [rows, cols], scale
    [rows/128, cols/128], q_t, scale_t): with transpose=True q_t holds the same
    codes transposed [cols, rows] and scale_t is scale.t() (a view: a block's
    scale does not depend on its orientation); otherwise both are None."""
    torch = _torch()
    _on_gpu(w, q, scale, q_t)
    rows, cols = w.shape
    dev = w.device
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty((rows // 128, cols // 128), dtype=torch.float32, device=dev)
    if transpose and q_t is None:
        q_t = torch.empty((cols, rows), dtype=torch.uint8, device=dev)
    _need(q, (rows, cols), torch.uint8, "q")
    _need(scale, (rows // 128, cols // 128), torch.float32, "scale")
    if q_t is not None:
        _need(q_t, (cols, rows), torch.uint8, "q_t")
    if not scale.is_contiguous():
        raise ValueError("scale must be contiguous")
    ld_qt = _pitch(q_t, "q_t") if q_t is not None else 0
    _check(lib().fp8_quant_w_128x128(_ptr(w), _dtype_code(w, "w"), rows, cols, _pitch(w, "w"),
                                     _ptr(q), _pitch(q, "q"), _ptr(scale), _ptr(q_t), ld_qt,
                                     _stream()))
    return q, scale, q_t, (scale.t() if q_t is not None else None)


def fp8_quant_batch(jobs, outs=None):
    """Several quantizations in one launch.  jobs: list of (x, tiling) with
    tiling "1x128" (activations) or "128x128" (weights); outs: optional list
    of (q, scale) per job.  Returns [(q, scale), ...], bit-identical to
    fp8_quant_act_1x128 / fp8_quant_w_128x128 on each job."""
    torch = _torch()
    if len(jobs) > MAX_QUANT_JOBS:
        raise ValueError(f"at most {MAX_QUANT_JOBS} jobs per call")
    arr = (QuantJob * max(1, len(jobs)))()
    res = []
    for i, (x, tiling) in enumerate(jobs):
        _on_gpu(x)
        rows, cols = x.shape
        tcode = {"1x128": TILE_1x128, "128x128": TILE_128x128}[tiling]
        sshape = (rows, cols // 128) if tcode == TILE_1x128 else (rows // 128, cols // 128)
        q, sc = outs[i] if outs is not None else (None, None)
        if q is None:
            q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
        if sc is None:
            sc = torch.empty(sshape, dtype=torch.float32, device=x.device)
        _on_gpu(q, sc)
        _need(q, (rows, cols), torch.uint8, "q")
        _need(sc, sshape, torch.float32, "scale")
        if not sc.is_contiguous():
            raise ValueError("scale must be contiguous")
        arr[i] = QuantJob(x.data_ptr(), _dtype_code(x, "x"), tcode, rows, cols, _pitch(x, "x"),
                          q.data_ptr(), _pitch(q, "q"), sc.data_ptr())
        res.append((q, sc))
    _check(lib().fp8_quant_batch(arr, len(jobs), _stream()))
    return res


def fp8_dequant(q, scale, tiling="1x128", out_dtype=None, y=None):
    """y = fl32(e4m3(q) * scale of its tile) (bf16: that float32 rounded to
    nearest even).  tiling "1x128": scale [rows, cols/128]; "128x128":
    scale [rows/128, cols/128]."""
    torch = _torch()
    _on_gpu(q, scale, y)
    rows, cols = q.shape
    if out_dtype is None:
        out_dtype = torch.float32 if y is None else y.dtype
    if y is None:
        y = torch.empty((rows, cols), dtype=out_dtype, device=q.device)
    tcode = {"1x128": TILE_1x128, "128x128": TILE_128x128}[tiling]
    sshape = (rows, cols // 128) if tcode == TILE_1x128 else (rows // 128, cols // 128)
    _need(q, (rows, cols), torch.uint8, "q")
    _need(scale, sshape, torch.float32, "scale")
    _need(y, (rows, cols), y.dtype, "y")
    if not scale.is_contiguous():
        raise ValueError("scale must be contiguous")
    _check(lib().fp8_dequant(_ptr(q), rows, cols, _pitch(q, "q"), _ptr(scale), tcode, _ptr(y),
                             _dtype_code(y, "y"), _pitch(y, "y"), _stream()))
    return y


def fp8_quant_tensor(x, fmt="e4m3", margin=0.0, history=None, q=None, scale=None, amax=None):
    """Per-tensor quantization (the prior-art baselines).  history None:
    current scaling from max|x|; history (float32 [L] on the GPU): delayed
    scaling from max(history), which is then updated in place.
    Returns (q uint8 like x, scale f32 [1], amax f32 [1])."""
    torch = _torch()
    _on_gpu(x, history, q, scale, amax)
    rows, cols = x.shape
    dev = x.device
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty((1,), dtype=torch.float32, device=dev)
    if amax is None:
        amax = torch.empty((1,), dtype=torch.float32, device=dev)
    _need(q, (rows, cols), torch.uint8, "q")
    _need(scale, (1,), torch.float32, "scale")
    _need(amax, (1,), torch.float32, "amax")
    hl = 0
    if history is not None:
        if history.dtype != torch.float32 or history.dim() != 1 or not history.is_contiguous():
            raise ValueError("history must be a contiguous float32 vector")
        hl = history.numel()
    _check(lib().fp8_quant_tensor(_ptr(x), _dtype_code(x, "x"), rows, cols, _pitch(x, "x"),
                                  _FMT[fmt], float(margin), _ptr(history), hl, _ptr(q),
                                  _pitch(q, "q"), _ptr(scale), _ptr(amax), _stream()))
    return q, scale, amax


def _dense_gemm(entry, a, a_scale, b, b_scale, b_kind, out_dtype, y):
    torch = _torch()
    _on_gpu(a, a_scale, b, b_scale, y)
    m, k = a.shape
    n = b.shape[0]
    if out_dtype is None:
        out_dtype = torch.float32 if y is None else y.dtype
    if y is None:
        y = torch.empty((m, n), dtype=out_dtype, device=a.device)
    kind = {"block128": BSCALE_BLOCK128, "row": BSCALE_ROW}[b_kind]
    if b.shape[1] != k:
        raise ValueError(f"a is [M, {k}] but b is {tuple(b.shape)}")
    _need(a, (m, k), torch.uint8, "a")
    _need(b, (n, k), torch.uint8, "b")
    _need(a_scale, (m, k // 128), torch.float32, "a_scale")
    _need(b_scale, (n // 128 if kind == BSCALE_BLOCK128 else n, k // 128), torch.float32,
          "b_scale")
    _need(y, (m, n), y.dtype, "y")
    for t, nm in ((a_scale, "a_scale"), (b_scale, "b_scale")):
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    _check(getattr(lib(), entry)(m, n, k, _ptr(a), _pitch(a, "a"), _ptr(a_scale), _ptr(b),
                                 _pitch(b, "b"), _ptr(b_scale), kind, _ptr(y),
                                 _dtype_code(y, "y"), _pitch(y, "y"), _stream()))
    return y


def fp8_blockscaled_gemm(a, a_scale, b, b_scale, b_kind="block128", out_dtype=None, y=None):
    """y[M, N] = dequant(a) . dequant(b)^T with FP32 promotion per 128-K block
    (each block's exact products summed in FP32)."""
    return _dense_gemm("fp8_blockscaled_gemm", a, a_scale, b, b_scale, b_kind, out_dtype, y)


def fp8_blockscaled_gemm_fp8mma(a, a_scale, b, b_scale, b_kind="block128", out_dtype=None, y=None):
    """The same product on the FP8 matrix instructions (faster; their
    ~14-bit accumulation inside each group of 8 K is outside the accuracy
    contract of fp8_blockscaled_gemm)."""
    return _dense_gemm("fp8_blockscaled_gemm_fp8mma", a, a_scale, b, b_scale, b_kind, out_dtype, y)


def fp8_blockscaled_gemm_quant(a, a_scale, b, b_scale, b_kind="block128", yq=None, y_scale=None):
    """The GEMM with its float32 output quantized in 1x128 tiles by the GEMM's
    epilogue.  Returns (yq uint8 [M, N], y_scale f32 [M, N/128])."""
    torch = _torch()
    _on_gpu(a, a_scale, b, b_scale, yq, y_scale)
    m, k = a.shape
    n = b.shape[0]
    if yq is None:
        yq = torch.empty((m, n), dtype=torch.uint8, device=a.device)
    if y_scale is None:
        y_scale = torch.empty((m, n // 128), dtype=torch.float32, device=a.device)
    kind = {"block128": BSCALE_BLOCK128, "row": BSCALE_ROW}[b_kind]
    if b.shape[1] != k:
        raise ValueError(f"a is [M, {k}] but b is {tuple(b.shape)}")
    _need(a, (m, k), torch.uint8, "a")
    _need(b, (n, k), torch.uint8, "b")
    _need(a_scale, (m, k // 128), torch.float32, "a_scale")
    _need(b_scale, (n // 128 if kind == BSCALE_BLOCK128 else n, k // 128), torch.float32,
          "b_scale")
    _need(yq, (m, n), torch.uint8, "yq")
    _need(y_scale, (m, n // 128), torch.float32, "y_scale")
    for t, nm in ((a_scale, "a_scale"), (b_scale, "b_scale"), (y_scale, "y_scale")):
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    _check(lib().fp8_blockscaled_gemm_quant(m, n, k, _ptr(a), _pitch(a, "a"), _ptr(a_scale),
                                            _ptr(b), _pitch(b, "b"), _ptr(b_scale), kind,
                                            _ptr(yq), _pitch(yq, "yq"), _ptr(y_scale),
                                            _stream()))
    return yq, y_scale


def fp8_blockscaled_grouped_gemm(offsets, a, a_scale, b, b_scale, out_dtype=None, y=None):
    """Per-group GEMM: group g owns rows [offsets[g], offsets[g+1]) of a and y,
    multiplied by b[g] ([G, N, K] codes, [G, N/128, K/128] scales)."""
    torch = _torch()
    _on_gpu(offsets, a, a_scale, b, b_scale, y)
    m, k = a.shape
    g, n, _ = b.shape
    if out_dtype is None:
        out_dtype = torch.float32 if y is None else y.dtype
    if y is None:
        y = torch.empty((m, n), dtype=out_dtype, device=a.device)
    for t, nm in ((a, "a"), (a_scale, "a_scale"), (b, "b"), (b_scale, "b_scale"), (y, "y"),
                  (offsets, "offsets")):
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    if offsets.dtype != torch.int32 or offsets.numel() != g + 1:
        raise ValueError("offsets must be int32 [G+1]")
    _need(a, (m, k), torch.uint8, "a")
    _need(b, (g, n, k), torch.uint8, "b")
    _need(a_scale, (m, k // 128), torch.float32, "a_scale")
    _need(b_scale, (g, n // 128, k // 128), torch.float32, "b_scale")
    _need(y, (m, n), y.dtype, "y")
    _check(lib().fp8_blockscaled_grouped_gemm(m, n, k, g, _ptr(offsets), _ptr(a), _ptr(a_scale),
                                              _ptr(b), _ptr(b_scale), _ptr(y),
                                              _dtype_code(y, "y"), _stream()))
    return y
