"""Concurrent calls on separate streams.  The library keeps no state between
calls and launches only on the stream it is given, so pipelines enqueued on
two streams at once, with their kernels free to overlap, must give the same
bytes as the same calls made one after another on one stream."""
import pytest

from gpu_util import banner

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
fb = pytest.importorskip("fp8_block_scaled_05_amd")


def _bf16(shape, seed, std=1.0):
    g = torch.Generator(device="cuda").manual_seed(seed)
    x = torch.randn(shape, device="cuda", generator=g) * std
    x[torch.rand(shape, device="cuda", generator=g) < 1e-3] *= 100
    return x.to(torch.bfloat16)


def _linear(x, w):
    """Batched quantization of X (1x128) and W (128x128), then the GEMM."""
    (qa, sa), (qb, sb) = fb.fp8_quant_batch([(x, "1x128"), (w, "128x128")])
    return [qa, sa, qb, sb, fb.fp8_blockscaled_gemm(qa, sa, qb, sb, out_dtype=torch.bfloat16)]


def _backward(dy, x, w, off):
    """dY in both tilings from one read, X in 128x1 tiles, the grouped GEMM
    of dY's 1x128 codes against per-group weights, and the weight-gradient
    GEMM with per-row scales on both operands."""
    q, s, qt, st = fb.fp8_quant_act_dual(dy)
    xq, xs = fb.fp8_quant_act_1x128(x, tiling="128x1_T")
    g = off.numel() - 1
    wq, ws, _, _ = fb.fp8_quant_w_128x128(w)
    n, k = w.shape[0] // g, w.shape[1]
    yg = fb.fp8_blockscaled_grouped_gemm(off, q, s, wq.view(g, n, k), ws.view(g, n // 128, k // 128))
    dw = fb.fp8_blockscaled_gemm(xq, xs, qt, st, b_kind="row", out_dtype=torch.float32)
    return [q, s, qt, st, xq, xs, yg, dw]


def _same(a, b):
    if a.dtype in (torch.float32, torch.bfloat16):
        return torch.equal(a.view(torch.int32 if a.dtype == torch.float32 else torch.int16),
                           b.view(torch.int32 if b.dtype == torch.float32 else torch.int16))
    return torch.equal(a, b)


def test_two_streams_match_one_stream():
    m, n, k = 1024, 512, 2048                 # linear: X [m, k], W [n, k]
    t, c, g = 1024, 768, 3                    # backward: dY [t, k], X [t, c], 3 groups of W [256, k]
    x1, w1 = _bf16((m, k), 11), _bf16((n, k), 12, 0.02)
    dy, x2, w2 = _bf16((t, k), 13, 1e-3), _bf16((t, c), 14), _bf16((g * 256, k), 15, 0.02)
    off = torch.tensor([0, 300, 301, t], dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()

    banner("streams: one stream, reference")
    ref_a = _linear(x1, w1)
    ref_b = _backward(dy, x2, w2, off)
    torch.cuda.synchronize()

    banner("streams: two streams, three rounds each, interleaved")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for s in (s1, s2):
        s.wait_stream(torch.cuda.current_stream())
    got_a, got_b = [], []
    for _ in range(3):
        with torch.cuda.stream(s1):
            got_a.append(_linear(x1, w1))
        with torch.cuda.stream(s2):
            got_b.append(_backward(dy, x2, w2, off))
    torch.cuda.synchronize()
    for r in range(3):
        for i, (want, have) in enumerate(zip(ref_a, got_a[r])):
            assert _same(want, have), f"linear output {i}, round {r}"
        for i, (want, have) in enumerate(zip(ref_b, got_b[r])):
            assert _same(want, have), f"backward output {i}, round {r}"
