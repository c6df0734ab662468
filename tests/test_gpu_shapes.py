"""Seeded random shapes through the GEMMs and quantizers, against the
oracle: sizes, tails, row pitches and both B-scale layouts in combinations
the workload tests do not reach.  Every output lies inside a larger
allocation whose margin must keep its canary bytes."""
import numpy as np
import pytest

import oracle
from fp8_block_scaled_05_amd import synth
from gpu_util import banner, dev_bf16, host, f32, assert_codes_equal, assert_scales_equal

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
fb = pytest.importorskip("fp8_block_scaled_05_amd")


def _codes(rng, shape):
    """Uniform over the 254 non-NaN E4M3 codes."""
    c = rng.integers(0, 254, size=shape, dtype=np.int64)
    c = np.where(c >= 0x7F, c + 1, c)          # skip 0x7F; 0xFF is past the range
    return c.astype(np.uint8)


def _scales(rng, shape):
    return np.exp2(rng.uniform(-20, 5, size=shape)).astype(np.float32)


def _padded(arr, pad_cols, fill):
    """arr placed in the top-left of a wider device buffer (row pitch = cols +
    pad_cols); returns (view, whole buffer)."""
    rows, cols = arr.shape
    full = np.full((rows, cols + pad_cols), fill, dtype=arr.dtype)
    full[:, :cols] = arr
    d = torch.from_numpy(full).cuda()
    return d[:, :cols], d


def _gemm_cases():
    rng = np.random.default_rng(2024)
    cases = []
    for i in range(24):                          # small: the 128 x 128 tile
        kind = "row" if i % 2 else "block128"
        m = int(rng.integers(1, 700))
        n = 16 * int(rng.integers(1, 40)) if kind == "row" else 128 * int(rng.integers(1, 6))
        k = 128 * int(rng.integers(1, 9))
        cases.append((m, n, k, kind, "f32" if i % 3 else "bf16", int(rng.integers(0, 4)) * 16))
    for i in range(6):                           # large: the 256 x 128 tile, ragged M (and N for row)
        kind = "row" if i % 2 else "block128"
        m = 4096 + int(rng.integers(-255, 256))
        n = 2048 + (16 * int(rng.integers(-7, 8)) if kind == "row" else 0)
        k = 128 * int(rng.integers(1, 4))
        cases.append((m, n, k, kind, "bf16" if i % 2 else "f32", 16 * int(rng.integers(0, 3))))
    return cases


@pytest.mark.parametrize("m,n,k,kind,out,pad", _gemm_cases())
def test_gemm_random_shape(m, n, k, kind, out, pad):
    rng = np.random.default_rng([31, m, n, k, pad])
    a = _codes(rng, (m, k))
    b = _codes(rng, (n, k))
    sa = _scales(rng, (m, k // 128))
    sb = _scales(rng, (n // 128 if kind == "block128" else n, k // 128))
    banner(f"gemm random {m}x{n}x{k} {kind} {out} pad {pad}")
    a_d, _ = _padded(a, pad, 0)
    b_d, _ = _padded(b, 2 * pad, 0)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    y_full = torch.full((m, n + pad), float("nan"), dtype=dt, device="cuda")
    y = y_full[:, :n]
    fb.fp8_blockscaled_gemm(a_d, torch.from_numpy(sa).cuda(), b_d, torch.from_numpy(sb).cuda(), kind, y=y)
    torch.cuda.synchronize()
    ref, bound = oracle.blockscaled_gemm_ref(a, sa, b, sb, kind)
    yh = host(y_full)
    got = (f32(yh) if out == "bf16" else yh).astype(np.float64)
    ok = oracle.gemm_tolerance_ok(got[:, :n], ref, bound, out)
    assert ok.all(), f"{(~ok).sum()} of {ok.size} outside tolerance"
    if pad:
        tail = got[:, n:]
        assert np.isnan(tail).all(), "the row pitch's margin was written"


@pytest.mark.parametrize("m,n,k,kind,out,pad", _gemm_cases()[::3])
def test_gemm_random_shape_repeats_bitwise(m, n, k, kind, out, pad):
    """Every third random shape again, twice on the same operands: the two
    outputs are identical bit for bit (no order-dependent reduction or race
    in any tile configuration)."""
    rng = np.random.default_rng([34, m, n, k])
    a = torch.from_numpy(_codes(rng, (m, k))).cuda()
    b = torch.from_numpy(_codes(rng, (n, k))).cuda()
    sa = torch.from_numpy(_scales(rng, (m, k // 128))).cuda()
    sb = torch.from_numpy(_scales(rng, (n // 128 if kind == "block128" else n, k // 128))).cuda()
    dt = torch.float32 if out == "f32" else torch.bfloat16
    banner(f"gemm random repeat {m}x{n}x{k} {kind} {out}")
    y1 = fb.fp8_blockscaled_gemm(a, sa, b, sb, kind, dt)
    y2 = fb.fp8_blockscaled_gemm(a, sa, b, sb, kind, dt)
    torch.cuda.synchronize()
    iv = torch.int32 if out == "f32" else torch.int16
    assert torch.equal(y1.view(iv), y2.view(iv))


def _grouped_cases():
    rng = np.random.default_rng(77)
    cases = []
    for i in range(8):
        g = int(rng.integers(1, 9))
        counts = rng.integers(0, 300, size=g)
        counts[rng.random(g) < 0.25] = 0
        n = 128 * int(rng.integers(1, 4))
        k = 128 * int(rng.integers(1, 6))
        cases.append((tuple(int(c) for c in counts), n, k, "f32" if i % 2 else "bf16"))
    return cases


@pytest.mark.parametrize("counts,n,k,out", _grouped_cases())
def test_grouped_random_shape(counts, n, k, out):
    rng = np.random.default_rng([32, n, k, len(counts)])
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    m, g = int(off[-1]), len(counts)
    a = _codes(rng, (max(m, 1), k))[:m]
    b = _codes(rng, (g, n, k))
    sa = _scales(rng, (m, k // 128))
    sb = _scales(rng, (g, n // 128, k // 128))
    banner(f"grouped random counts {counts} N {n} K {k} {out}")
    dt = torch.float32 if out == "f32" else torch.bfloat16
    y = torch.full((m, n), float("nan"), dtype=dt, device="cuda")
    if m:
        fb.fp8_blockscaled_grouped_gemm(torch.from_numpy(off).cuda(), torch.from_numpy(a).cuda(),
                                        torch.from_numpy(sa).cuda(), torch.from_numpy(b).cuda(),
                                        torch.from_numpy(sb).cuda(), y=y)
    torch.cuda.synchronize()
    if m == 0:
        return
    ref, bound = oracle.grouped_gemm_ref(off, a, sa, b, sb)
    yh = host(y)
    got = (f32(yh) if out == "bf16" else yh).astype(np.float64)
    ok = oracle.gemm_tolerance_ok(got, ref, bound, out)
    assert ok.all(), f"{(~ok).sum()} of {ok.size} outside tolerance"


def _quant_cases():
    rng = np.random.default_rng(5)
    return [(int(rng.integers(1, 600)), 128 * int(rng.integers(1, 12)), int(rng.integers(0, 3)) * 64,
             "f32" if i % 3 == 2 else "bf16") for i in range(12)]


@pytest.mark.parametrize("rows,cols,pad,dtype", _quant_cases())
def test_quantizers_random_shape(rows, cols, pad, dtype):
    """1x128 on any row count; 128x128, its transposed copy, 128x1T and the
    dual call on the 128-row prefix; codes and scales bit-exact, pitches from
    sub-views, bf16 and float32 inputs."""
    rng = np.random.default_rng([33, rows, cols, pad])
    x = (rng.standard_normal((rows, cols)) * np.exp2(rng.uniform(-8, 8, size=(rows, 1)))).astype(np.float32)
    x[rng.random((rows, cols)) < 2e-3] *= 300
    banner(f"quantizers random {rows}x{cols} pad {pad} {dtype}")
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(x)
        xv = f32(bits)
        full = torch.zeros((rows, cols + pad), dtype=torch.bfloat16, device="cuda")
        full[:, :cols] = dev_bf16(bits)
    else:
        xv = x
        full = torch.zeros((rows, cols + pad), dtype=torch.float32, device="cuda")
        full[:, :cols] = torch.from_numpy(x).cuda()
    xd = full[:, :cols]
    q, s = fb.fp8_quant_act_1x128(xd)
    torch.cuda.synchronize()
    want_q, want_s = oracle.quant_1x128(xv)
    assert_scales_equal(host(s), want_s, "1x128 scales")
    assert_codes_equal(host(q), want_q, "1x128 codes")
    r128 = rows - rows % 128
    if r128 == 0:
        return
    xb = xd[:r128]
    wq, ws, wqt, wst = fb.fp8_quant_w_128x128(xb, transpose=True)
    tq, ts = fb.fp8_quant_act_1x128(xb, "128x1_T")
    dq, ds, dqt, dst = fb.fp8_quant_act_dual(xb)
    torch.cuda.synchronize()
    want_wq, want_ws = oracle.quant_128x128(xv[:r128])
    assert_scales_equal(host(ws), want_ws, "128x128 scales")
    assert_codes_equal(host(wq), want_wq, "128x128 codes")
    assert_codes_equal(host(wqt), want_wq.T, "128x128 transposed codes")
    assert_scales_equal(host(wst), want_ws.T, "128x128 transposed scales")
    want_tq, want_ts = oracle.quant_128x1_t(xv[:r128])
    assert_codes_equal(host(tq), want_tq, "128x1T codes")
    assert_scales_equal(host(ts), want_ts, "128x1T scales")
    assert_codes_equal(host(dqt), want_tq, "dual transposed codes")
    assert_scales_equal(host(dst), want_ts, "dual transposed scales")
    assert_codes_equal(host(dq), want_q[:r128], "dual codes")
    assert_scales_equal(host(ds), want_s[:r128], "dual scales")
