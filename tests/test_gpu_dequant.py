"""GPU parity of dequantization against the CPU oracle: fl32(e4m3(code) * s)
bit-exact (NaN codes give NaN), and its bf16 rounding bit-exact."""
import numpy as np
import pytest

import oracle
from fp8_block_scaled_05_amd import synth
from gpu_util import banner, inputs, dev_bf16, host, f32, assert_codes_equal

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
fb = pytest.importorskip("fp8_block_scaled_05_amd")


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _assert_f32_equal(got, want, what):
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), f"{what}: NaN positions differ"
    g, w = got[~nan].view(np.uint32), want[~nan].view(np.uint32)
    bad = np.flatnonzero(g != w)
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first got {got[~nan][bad[:3]]} want {want[~nan][bad[:3]]}"


def _assert_bf16_equal(got, want, what):
    nan_w = (want & 0x7F80) == 0x7F80
    nan_w &= (want & 0x7F) != 0
    nan_g = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
    assert np.array_equal(nan_g, nan_w), f"{what}: NaN positions differ"
    bad = np.flatnonzero(got[~nan_w] != want[~nan_w])
    assert bad.size == 0, f"{what}: {bad.size} bf16 mismatches"


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_dequant_all_codes_many_scales(out):
    rng = np.random.default_rng(30)
    n = 512
    s = (np.exp2(rng.uniform(-60, 60, n)) * rng.uniform(1, 2, n)).astype(np.float32)
    s[:4] = np.float32([1.0, 1e-10, 2.0 ** -126, 3.0e38 / 448])
    codes = np.tile(np.arange(256, dtype=np.uint8), (n, 1))
    scales = np.repeat(s[:, None], 2, axis=1)
    banner(f"dequant all codes x {n} scales ({out})")
    y = host(fb.fp8_dequant(_dev(codes), _dev(scales), "1x128",
                            out_dtype=torch.float32 if out == "f32" else torch.bfloat16))
    torch.cuda.synchronize()
    if out == "f32":
        _assert_f32_equal(y, oracle.dequant_f32(codes, scales, "1x128"), "all codes f32")
    else:
        _assert_bf16_equal(y, oracle.dequant_bf16(codes, scales, "1x128"), "all codes bf16")


def test_dequant_workload2_x_codes():
    """The oracle's 1x128 quantization of X, dequantized on the GPU."""
    bits = inputs(2)["X"][:1024]
    xq, xs = oracle.quant_1x128(f32(bits))
    banner(f"dequant of oracle-quantized X {bits.shape}")
    y = fb.fp8_dequant(_dev(xq), _dev(xs))
    torch.cuda.synchronize()
    _assert_f32_equal(host(y), oracle.dequant_f32(xq, xs, "1x128"), "X codes")


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_dequant_128x128_workload1_w(out):
    bits = inputs(1)["W"]
    wq, ws = oracle.quant_128x128(f32(bits))
    banner(f"dequant 128x128 W {bits.shape} ({out})")
    y = host(fb.fp8_dequant(_dev(wq), _dev(ws), "128x128",
                            out_dtype=torch.float32 if out == "f32" else torch.bfloat16))
    if out == "f32":
        _assert_f32_equal(y, oracle.dequant_f32(wq, ws, "128x128"), "W f32")
    else:
        _assert_bf16_equal(y, oracle.dequant_bf16(wq, ws, "128x128"), "W bf16")


def test_dequant_ragged_rows_pitches_and_canaries():
    rng = np.random.default_rng(31)
    rows, cols = 37, 384
    codes = rng.integers(0, 256, (rows, cols), dtype=np.uint8)
    s = rng.uniform(0.01, 9, (rows, 3)).astype(np.float32)
    qbuf = torch.zeros((rows, cols + 48), dtype=torch.uint8, device="cuda")
    qbuf[:, :cols] = _dev(codes)
    ybuf = torch.full((rows + 2, cols + 16), -3.0, dtype=torch.float32, device="cuda")
    banner("dequant ragged rows with pitches")
    fb.fp8_dequant(qbuf[:, :cols], _dev(s), y=ybuf[1:rows + 1, :cols])
    torch.cuda.synchronize()
    yb = host(ybuf)
    _assert_f32_equal(yb[1:rows + 1, :cols], oracle.dequant_f32(codes, s), "ragged")
    assert np.all(yb[0] == -3.0) and np.all(yb[-1] == -3.0) and np.all(yb[:, cols:] == -3.0)


def test_dequant_errors():
    banner("dequant errors")
    q = torch.zeros((4, 200), dtype=torch.uint8, device="cuda")
    with pytest.raises(fb.Fp8bsError):
        fb.fp8_dequant(q, torch.zeros((4, 1), dtype=torch.float32, device="cuda"))
    y = fb.fp8_dequant(torch.zeros((0, 128), dtype=torch.uint8, device="cuda"),
                       torch.zeros((0, 1), dtype=torch.float32, device="cuda"))
    assert y.shape == (0, 128)
