"""The library under HIP graph capture.  Its calls allocate nothing, never
synchronize and launch only kernels on the caller's stream (the per-tensor
path clears its amax with a one-thread kernel, not a memset), so a captured
sequence must replay exactly what the eager calls compute.  Each test
replays its graph several times with eager work and synchronization in
between, changes the captured inputs in place between replays, and checks
every replay against eager calls on the same data."""
import numpy as np
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


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                   # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_step_graph_replays_match_eager():
    """The linear step (X 1x128 and W 128x128 in one batched launch, then the
    GEMM) captured once and replayed on three different inputs."""
    m, n, k = 1024, 512, 2048
    x = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((n, k), dtype=torch.bfloat16, device="cuda")
    qa = torch.empty((m, k), dtype=torch.uint8, device="cuda")
    sa = torch.empty((m, k // 128), dtype=torch.float32, device="cuda")
    qb = torch.empty((n, k), dtype=torch.uint8, device="cuda")
    sb = torch.empty((n // 128, k // 128), dtype=torch.float32, device="cuda")
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    x.copy_(_bf16((m, k), 1))
    w.copy_(_bf16((n, k), 2, 0.02))

    def step():
        fb.fp8_quant_batch([(x, "1x128"), (w, "128x128")], outs=[(qa, sa), (qb, sb)])
        fb.fp8_blockscaled_gemm(qa, sa, qb, sb, y=y)

    banner(f"graph: batched quantize + GEMM {m}x{n}x{k}")
    g = _capture(step)
    for r in range(3):
        x.copy_(_bf16((m, k), 10 + r))
        w.copy_(_bf16((n, k), 20 + r, 0.02))
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (qa, sa, qb, sb, y)]
        # eager reference on the same inputs, into fresh buffers
        ea, esa = fb.fp8_quant_act_1x128(x)
        eb, esb, _, _ = fb.fp8_quant_w_128x128(w)
        ey = fb.fp8_blockscaled_gemm(ea, esa, eb, esb, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        for name, a, b in zip(("qa", "sa", "qb", "sb", "y"), got, (ea, esa, eb, esb, ey)):
            assert torch.equal(a, b), f"replay {r}: {name} differs from the eager call"


def test_delayed_scaling_graph_updates_history_each_replay():
    """Delayed per-tensor scaling (amax cleared by a kernel, code pass, history
    roll) captured once: each replay must advance the history exactly as an
    eager call does."""
    rows, cols = 256, 1024
    x = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    hist = torch.zeros(64, dtype=torch.float32, device="cuda")
    hist[:3] = torch.tensor([2.0, 5.0, 1.0], device="cuda")
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    sc = torch.empty((1,), dtype=torch.float32, device="cuda")
    am = torch.empty((1,), dtype=torch.float32, device="cuda")
    x.copy_(_bf16((rows, cols), 3))

    def call():
        fb.fp8_quant_tensor(x, history=hist, q=q, scale=sc, amax=am)

    banner("graph: delayed per-tensor scaling, history of 64")
    # the warm-up inside _capture advances the history once; the eager
    # reference starts from the history as the graph's first replay sees it
    g = _capture(call)
    ref_hist = hist.clone()
    for r, mult in enumerate((1.0, 8.0, 0.5, 40.0)):
        x.copy_(_bf16((rows, cols), 30 + r, mult))
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (q, sc, am, hist)]
        eq, es, ea = fb.fp8_quant_tensor(x, history=ref_hist)
        torch.cuda.synchronize()
        for name, a, b in zip(("codes", "scale", "amax", "history"), got, (eq, es, ea, ref_hist)):
            assert torch.equal(a, b), f"replay {r}: {name} differs from the eager call"


def test_grouped_gemm_graph_reads_offsets_at_replay():
    """The grouped GEMM reads its expert offsets from device memory when it
    runs, so a captured call follows offsets changed between replays."""
    groups, n, k = 4, 256, 1024
    m = 640
    a_x = _bf16((m, k), 4)
    w = _bf16((groups * n, k), 5, 0.02)
    qa, sa = fb.fp8_quant_act_1x128(a_x)
    qb, sb, _, _ = fb.fp8_quant_w_128x128(w)
    qb, sb = qb.view(groups, n, k), sb.view(groups, n // 128, k // 128)
    off = torch.tensor([0, 100, 100, 400, 640], dtype=torch.int32, device="cuda")
    y = torch.zeros((m, n), dtype=torch.float32, device="cuda")

    def call():
        fb.fp8_blockscaled_grouped_gemm(off, qa, sa, qb, sb, y=y)

    banner("graph: grouped GEMM, offsets changed between replays")
    g = _capture(call)
    tables = ([0, 100, 100, 400, 640], [0, 0, 320, 321, 640], [0, 160, 320, 480, 640])
    for r, table in enumerate(tables):
        off.copy_(torch.tensor(table, dtype=torch.int32, device="cuda"))
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        got = y.clone()
        ey = fb.fp8_blockscaled_grouped_gemm(off, qa, sa, qb, sb, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(got, ey), f"replay {r} with offsets {table}"
        assert np.isfinite(got.cpu().numpy()).all()
