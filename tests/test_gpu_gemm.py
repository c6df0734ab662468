"""GPU parity of the block-scaled GEMMs against the float64 oracle:
|y - Y| <= 2e-5 * sum|a_k b_k| per element (+ half a bf16 ulp for bf16 out),
bit-exact where every intermediate is exact in fp32, on the five workloads
(full outputs or seeded row samples) and on edge cases."""
import numpy as np
import pytest

import oracle
from fp8_block_scaled_05_amd import synth
from gpu_util import banner, inputs, dev_bf16, host, f32

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
fb = pytest.importorskip("fp8_block_scaled_05_amd")

ONE = 0x38


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _y_host(y):
    if y.dtype == torch.bfloat16:
        return f32(host(y)).astype(np.float64)
    return host(y).astype(np.float64)


def _check_tol(y, ref, bound, out, what):
    ok = oracle.gemm_tolerance_ok(y, ref, bound, out)
    if not np.all(ok):
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {ok.size} outside tolerance; first {i}: "
                             f"gpu {y[i]!r} oracle {ref[i]!r} bound {bound[i]!r}")


def _quantize_pair(xbits, wbits):
    """GPU-side operands: the library's own quantizers."""
    a, sa = fb.fp8_quant_act_1x128(dev_bf16(xbits))
    b, sb, _, _ = fb.fp8_quant_w_128x128(dev_bf16(wbits))
    return a, sa, b, sb


def _oracle_pair(xbits, wbits):
    """Oracle-side operands: the oracle's quantization of the same inputs."""
    a, sa = oracle.quant_1x128(f32(xbits))
    b, sb = oracle.quant_128x128(f32(wbits))
    return a, sa, b, sb


def _block_rows(n, count, seed):
    """`count` seeded 128-row blocks of an N-row weight, first and last included."""
    nb = n // 128
    rng = np.random.default_rng(seed)
    pick = sorted(set([0, nb - 1]) | set(rng.choice(nb, size=min(count, nb), replace=False).tolist()))
    return pick[:max(count, 2)]


def _cols_of(blocks):
    return np.concatenate([np.arange(128 * bk, 128 * bk + 128) for bk in blocks])


# ---------------------------------------------------------------- workloads
@pytest.mark.parametrize("workload,out", [(1, "f32"), (2, "f32"), (2, "bf16")])
def test_gemm_full(workload, out):
    """Whole output; both sides multiply the oracle's quantization of the inputs."""
    d = inputs(workload)
    a, sa, b, sb = _oracle_pair(d["X"], d["W"])
    banner(f"gemm workload {workload} full, out {out}")
    y = fb.fp8_blockscaled_gemm(_dev(a), _dev(sa), _dev(b), _dev(sb), "block128",
                                torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    ref, bound = oracle.blockscaled_gemm_ref(a, sa, b, sb)
    _check_tol(_y_host(y), ref, bound, out, f"workload {workload}")


def test_gemm_workload3_sampled():
    """GPU: the library's quantizers feed the GEMM.  Oracle: its own
    quantization of sampled X rows and whole 128-row blocks of W."""
    d = inputs(3)
    banner("gemm workload 3 [8192,18432,7168], sampled rows and column blocks")
    a, sa, b, sb = _quantize_pair(d["X"], d["W"])
    y = fb.fp8_blockscaled_gemm(a, sa, b, sb, "block128", torch.float32)
    torch.cuda.synchronize()
    rows = synth.sample_rows(a.shape[0], 128, seed=3, must=[0, a.shape[0] - 1])
    blocks = _block_rows(b.shape[0], 3, seed=33)
    cols = _cols_of(blocks)
    ah, sah = oracle.quant_1x128(f32(d["X"][rows]))
    bh, sbh = oracle.quant_128x128(f32(d["W"][cols]))
    ref, bound = oracle.blockscaled_gemm_ref(ah, sah, bh, sbh)
    _check_tol(_y_host(y)[rows][:, cols], ref, bound, "f32", "workload 3")


def test_grouped_workload4_sampled():
    d = inputs(4)
    off = d["offsets"]
    g, n, k = d["W"].shape
    banner(f"grouped gemm workload 4, counts {d['counts'].tolist()}")
    a, sa = fb.fp8_quant_act_1x128(dev_bf16(d["X"]))
    b, sb, _, _ = fb.fp8_quant_w_128x128(dev_bf16(d["W"].reshape(g * n, k)))
    b = b.view(g, n, k)
    sb = sb.view(g, n // 128, k // 128)
    y = fb.fp8_blockscaled_grouped_gemm(_dev(off), a, sa, b, sb, torch.bfloat16)
    torch.cuda.synchronize()
    must = [int(o) for o in off[:-1] if o < off[-1]] + [int(o) - 1 for o in off[1:] if o > 0]
    rows = synth.sample_rows(a.shape[0], 96, seed=4, must=must)
    yh = _y_host(y)
    expert = np.searchsorted(off, rows, side="right") - 1
    blocks = _block_rows(n, 2, seed=44)
    cols = _cols_of(blocks)
    for e in np.unique(expert):
        r = rows[expert == e]
        ah, sah = oracle.quant_1x128(f32(d["X"][r]))
        bh, sbh = oracle.quant_128x128(f32(d["W"][e][cols]))
        ref, bound = oracle.blockscaled_gemm_ref(ah, sah, bh, sbh)
        _check_tol(yh[r][:, cols], ref, bound, "bf16", f"expert {e}")


def test_dgrad_workload5():
    d = inputs(5)
    banner("dgrad workload 5: dY[8192,2048] x W[2048,7168] -> dX, sampled rows and columns")
    a, sa = fb.fp8_quant_act_1x128(dev_bf16(d["dY"]))
    _, _, bt, sbt = fb.fp8_quant_w_128x128(dev_bf16(d["W"]), transpose=True)
    # sbt is scale.t(), a view; the GEMM takes a dense [N/128, K/128] grid
    y = fb.fp8_blockscaled_gemm(a, sa, bt, sbt.contiguous(), "block128", torch.bfloat16)
    torch.cuda.synchronize()
    rows = synth.sample_rows(a.shape[0], 192, seed=5, must=[0, a.shape[0] - 1])
    blocks = _block_rows(bt.shape[0], 4, seed=55)           # column blocks of W = rows of W^T
    cols = _cols_of(blocks)
    ah, sah = oracle.quant_1x128(f32(d["dY"][rows]))
    wq, ws = oracle.quant_128x128(f32(d["W"][:, cols]))     # whole 128x128 blocks of W
    ref, bound = oracle.blockscaled_gemm_ref(ah, sah, np.ascontiguousarray(wq.T),
                                             np.ascontiguousarray(ws.T))
    _check_tol(_y_host(y)[rows][:, cols], ref, bound, "bf16", "dgrad")


def test_wgrad_workload5():
    d = inputs(5)
    banner("wgrad workload 5: X^T dY with 128x1 tiles along tokens -> dW fp32 [7168,2048]")
    xt, sxt = fb.fp8_quant_act_1x128(dev_bf16(d["X"]), "128x1_T")     # [7168, 8192]
    dyt, sdyt = fb.fp8_quant_act_1x128(dev_bf16(d["dY"]), "128x1_T")  # [2048, 8192]
    y = fb.fp8_blockscaled_gemm(xt, sxt, dyt, sdyt, "row", torch.float32)
    torch.cuda.synchronize()
    # sampled rows of dW, every column (each column has its own B scales)
    rows = synth.sample_rows(xt.shape[0], 128, seed=55, must=[0, xt.shape[0] - 1])
    ah, sah = oracle.quant_128x1_t(f32(d["X"][:, rows]))
    bh, sbh = oracle.quant_128x1_t(f32(d["dY"]))
    ref, bound = oracle.blockscaled_gemm_ref(ah, sah, bh, sbh, "row")
    _check_tol(_y_host(y)[rows], ref, bound, "f32", "wgrad")


# ---------------------------------------------------------------- exact cases
def _int_codes(rng, shape):
    """Codes whose values are integers with |v| <= 16 (0, +-1..16)."""
    vals = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E, 0x50, 0x51, 0x52, 0x53,
                     0x54, 0x55, 0x56, 0x57, 0x58], np.uint8)
    c = rng.choice(vals, size=shape)
    return c | (rng.integers(0, 2, size=shape, dtype=np.uint8) << 7)


@pytest.mark.parametrize("m,n,k,kind,out", [(256, 256, 7168, "block128", "f32"),
                                            (300, 384, 1024, "row", "f32"),
                                            (129, 128, 128, "block128", "f32"),
                                            (4096, 2048, 1024, "row", "f32"),   # 256 x 128 tiles
                                            (4000, 2064, 640, "row", "f32")])   # 256 x 128, ragged M and N
def test_integer_exact_is_bit_exact(m, n, k, kind, out):
    rng = np.random.default_rng([20, m, n, k])
    a = _int_codes(rng, (m, k))
    b = _int_codes(rng, (n, k))
    assert np.all(np.abs(oracle.e4m3_decode(a)) <= 16)
    sa = rng.choice(np.float32([1.0, 2.0]), size=(m, k // 128))
    sb = rng.choice(np.float32([0.5, 1.0]), size=(n // 128 if kind == "block128" else n, k // 128))
    banner(f"gemm integer-exact {m}x{n}x{k} {kind}")
    y = fb.fp8_blockscaled_gemm(_dev(a), _dev(sa), _dev(b), _dev(sb), kind, torch.float32)
    torch.cuda.synchronize()
    ref, _ = oracle.blockscaled_gemm_ref(a, sa, b, sb, kind)
    assert np.array_equal(_y_host(y), ref)


@pytest.mark.parametrize("kind", ["block128", "row"])
@pytest.mark.parametrize("k", [128, 256, 384, 512, 640, 768, 896])
def test_large_tile_integer_exact_every_tail(k, kind):
    """4096 x 2048 runs the 256 x 128 tile.  Its main loop takes three K
    blocks at a time and, with block-128 B scales, may leave the last
    block's promotion pending, so K / 128 = 1 .. 7 covers every tail and
    every pending state; with integer-valued codes and power-of-two scales
    the result is exact."""
    m, n = 4096, 2048
    rng = np.random.default_rng([25, k])
    a = _int_codes(rng, (m, k))
    b = _int_codes(rng, (n, k))
    sa = rng.choice(np.float32([1.0, 2.0]), size=(m, k // 128))
    sb = rng.choice(np.float32([0.5, 1.0]), size=(n // 128 if kind == "block128" else n, k // 128))
    banner(f"gemm integer-exact large tile {m}x{n}x{k} {kind}")
    y = fb.fp8_blockscaled_gemm(_dev(a), _dev(sa), _dev(b), _dev(sb), kind, torch.float32)
    torch.cuda.synchronize()
    rows = synth.sample_rows(m, 256, seed=k, must=[0, m - 1])
    ref, _ = oracle.blockscaled_gemm_ref(a[rows], sa[rows], b, sb, kind)
    assert np.array_equal(_y_host(y)[rows], ref)


def test_selection_closed_form():
    rng = np.random.default_rng(21)
    m, n, k = 200, 256, 1024
    perm = rng.permutation(k)[:m]
    a = np.zeros((m, k), np.uint8)
    a[np.arange(m), perm] = ONE
    b = rng.integers(0, 256, size=(n, k), dtype=np.uint8)
    b[(b & 0x7F) == 0x7F] = 0x30
    sa = np.ones((m, k // 128), np.float32)
    sb = np.ones((n // 128, k // 128), np.float32)
    banner("gemm selection closed form")
    y = fb.fp8_blockscaled_gemm(_dev(a), _dev(sa), _dev(b), _dev(sb), "block128", torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(_y_host(y), oracle.e4m3_decode(b[:, perm]).T)


def test_scale_routing_powers_of_two():
    rng = np.random.default_rng(22)
    m, n, k = 256, 384, 1024
    kbs = k // 128
    a = rng.integers(0, 256, size=(m, k), dtype=np.uint8)
    b = rng.integers(0, 256, size=(n, k), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x38
    b[(b & 0x7F) == 0x7F] = 0x38
    sa = np.float32(2.0) ** rng.integers(-20, 21, size=(m, kbs)).astype(np.float32)
    sb = np.float32(2.0) ** rng.integers(-20, 21, size=(n // 128, kbs)).astype(np.float32)
    banner("gemm scale routing 2^+-20")
    y = fb.fp8_blockscaled_gemm(_dev(a), _dev(sa), _dev(b), _dev(sb), "block128", torch.float32)
    torch.cuda.synchronize()
    ref, bound = oracle.blockscaled_gemm_ref(a, sa, b, sb)
    _check_tol(_y_host(y), ref, bound, "f32", "scale routing")


# ---------------------------------------------------------------- edges
@pytest.mark.parametrize("m,n,k,kind", [(1, 128, 128, "block128"), (5, 256, 384, "block128"),
                                        (127, 128, 256, "block128"), (129, 384, 512, "block128"),
                                        (255, 16, 256, "row"), (33, 144, 640, "row")])
def test_tails_and_pitches(m, n, k, kind):
    rng = np.random.default_rng([23, m, n, k])
    x = synth.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    ah, sah = oracle.quant_1x128(f32(x))
    a, sa = _dev(ah), _dev(sah)
    b = rng.integers(0, 256, size=(n, k), dtype=np.uint8)
    b[(b & 0x7F) == 0x7F] = 0x38
    sb = (rng.random((n // 128 if kind == "block128" else n, k // 128)) + 0.01).astype(np.float32)
    lda, ldb, ldy = k + 32, k + 16, n + 16
    abuf = torch.zeros((m, lda), dtype=torch.uint8, device="cuda")
    abuf[:, :k] = a
    bbuf = torch.zeros((n, ldb), dtype=torch.uint8, device="cuda")
    bbuf[:, :k] = _dev(b)
    ybuf = torch.full((m + 2, ldy), -3.0, dtype=torch.float32, device="cuda")
    banner(f"gemm tails {m}x{n}x{k} {kind}, pitches {lda}/{ldb}/{ldy}")
    fb.fp8_blockscaled_gemm(abuf[:, :k], sa, bbuf[:, :k], _dev(sb), kind, y=ybuf[1:m + 1, :n])
    torch.cuda.synchronize()
    yb = host(ybuf)
    ref, bound = oracle.blockscaled_gemm_ref(ah, sah, b, sb, kind)
    _check_tol(yb[1:m + 1, :n].astype(np.float64), ref, bound, "f32", "tails")
    assert np.all(yb[0] == -3.0) and np.all(yb[-1] == -3.0) and np.all(yb[:, n:] == -3.0)


def test_grouped_edges_and_single_group_equals_dense():
    rng = np.random.default_rng(24)
    n, k = 256, 512
    counts = np.array([0, 1, 130, 0, 127, 256, 0, 3])
    off = synth.offsets_from_counts(counts)
    m = int(off[-1])
    g = len(counts)
    a = rng.integers(0, 256, size=(m, k), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x38
    sa = (rng.random((m, k // 128)) + 0.1).astype(np.float32)
    b = rng.integers(0, 256, size=(g, n, k), dtype=np.uint8)
    b[(b & 0x7F) == 0x7F] = 0x38
    sb = (rng.random((g, n // 128, k // 128)) + 0.1).astype(np.float32)
    banner(f"grouped edges counts {counts.tolist()}")
    y = fb.fp8_blockscaled_grouped_gemm(_dev(off), _dev(a), _dev(sa), _dev(b), _dev(sb),
                                        torch.float32)
    torch.cuda.synchronize()
    ref, bound = oracle.grouped_gemm_ref(off, a, sa, b, sb)
    _check_tol(_y_host(y), ref, bound, "f32", "grouped")
    # one group over all rows gives the same bits as the dense kernel
    off1 = np.array([0, m], np.int32)
    y1 = fb.fp8_blockscaled_grouped_gemm(_dev(off1), _dev(a), _dev(sa), _dev(b[:1]),
                                         _dev(sb[:1]), torch.float32)
    yd = fb.fp8_blockscaled_gemm(_dev(a), _dev(sa), _dev(b[0]), _dev(sb[0]), "block128",
                                 torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y1, yd)


@pytest.mark.parametrize("off,ranges", [
    # group g reads rows [max(clamp(off[g]), end of g-1), max(clamp(off[g+1]), that)):
    # g0 [0, 200); g1 starts at 200 and ends at 100 -> empty; g2 [200, 300)
    # (900 clamped to M); g3 and g4 start at 300 -> empty.
    ([0, 200, 100, 900, -5, 300], {0: (0, 200), 2: (200, 300)}),
    # g1 = [150, 100) is empty; g2 = [100, 250) is cut to start where g0
    # ends (150); g3 is empty; g4 = [250, 300).
    ([0, 150, 100, 250, 250, 300], {0: (0, 150), 2: (150, 250), 4: (250, 300)}),
    # a table that never reaches M: rows past the last end are not written.
    ([0, 64, 128, 128, 128, 180], {0: (0, 64), 1: (64, 128), 4: (128, 180)}),
])
def test_grouped_bad_offsets_deterministic(off, ranges):
    """A decreasing, overlapping or out-of-range offset table: every group's
    rows are clamped into [0, M) and start no earlier than the previous group
    ends, so the ranges are disjoint (no two workgroups write one row), each
    written row is that group's product, and rows of no range keep their
    canary."""
    rng = np.random.default_rng(25)
    n, k, m = 128, 256, 300
    off = np.array(off, np.int32)
    a = rng.integers(0, 0x30, size=(m, k), dtype=np.uint8)
    sa = np.ones((m, 2), np.float32)
    b = rng.integers(0, 0x30, size=(5, n, k), dtype=np.uint8)
    sb = np.ones((5, 1, 2), np.float32)
    ybuf = torch.full((m + 2, n), -3.0, dtype=torch.float32, device="cuda")
    banner(f"grouped with a bad offset table {off.tolist()}")
    fb.fp8_blockscaled_grouped_gemm(_dev(off), _dev(a), _dev(sa), _dev(b), _dev(sb),
                                    y=ybuf[1:m + 1])
    torch.cuda.synchronize()
    yb = host(ybuf)
    assert np.all(yb[0] == -3.0) and np.all(yb[-1] == -3.0)
    y = yb[1:m + 1]
    written = np.zeros(m, bool)
    for g, (lo, hi) in ranges.items():
        ref, bound = oracle.blockscaled_gemm_ref(a[lo:hi], sa[lo:hi], b[g], sb[g])
        _check_tol(y[lo:hi], ref, bound, "f32", f"group {g} rows {lo}..{hi}")
        written[lo:hi] = True
    assert np.all(y[~written] == -3.0)


def _clamped_ranges(off, m):
    """The header's rule for any table: group g owns rows [P_g, P_g+1) with
    P_g the largest offset among off[0..g] clamped into [0, m]."""
    c = np.clip(np.asarray(off, np.int64), 0, m)
    p = np.maximum.accumulate(c)
    return {g: (int(p[g]), int(p[g + 1])) for g in range(len(off) - 1) if p[g + 1] > p[g]}


@pytest.mark.parametrize("kind", ["valid", "bad"])
def test_grouped_many_groups(kind):
    """More groups than one wave's 64-lane expert search covers: 150 groups
    of random sizes (a third of them empty), and an increasing table of 140
    groups with a fifth of its offsets scrambled (decreasing, negative, past
    M); every group's rows against the oracle, rows of no group keep their
    canary."""
    rng = np.random.default_rng(26 if kind == "valid" else 27)
    n, k = 128, 256
    if kind == "valid":
        counts = rng.integers(0, 12, size=150)
        counts[rng.random(150) < 0.33] = 0
        off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        m = int(off[-1])
    else:                    # an increasing table with a fifth of its entries broken
        m = 1400
        off = np.sort(rng.integers(0, m + 1, size=141))
        bad = np.nonzero(rng.random(141) < 0.2)[0]
        neg = rng.random(len(bad)) < 0.5
        off[bad[neg]] = -rng.integers(1, 40, size=int(neg.sum()))            # negative
        off[bad[~neg]] -= rng.integers(1, 30, size=int((~neg).sum()))        # below the previous one
        off[130] = m + 37                                                     # past M: the rest is empty
        off = off.astype(np.int32)
    g = len(off) - 1
    ranges = _clamped_ranges(off, m)
    a = rng.integers(0, 0x30, size=(m, k), dtype=np.uint8)
    sa = (rng.random((m, 2)) + 0.5).astype(np.float32)
    b = rng.integers(0, 0x30, size=(g, n, k), dtype=np.uint8)
    sb = (rng.random((g, 1, 2)) + 0.5).astype(np.float32)
    ybuf = torch.full((m + 2, n), -3.0, dtype=torch.float32, device="cuda")
    banner(f"grouped with {g} groups ({kind} table), M {m}")
    fb.fp8_blockscaled_grouped_gemm(_dev(off), _dev(a), _dev(sa), _dev(b), _dev(sb), y=ybuf[1:m + 1])
    torch.cuda.synchronize()
    yb = host(ybuf)
    assert np.all(yb[0] == -3.0) and np.all(yb[-1] == -3.0)
    y = yb[1:m + 1]
    written = np.zeros(m, bool)
    assert len(ranges) > 64
    for grp, (lo, hi) in ranges.items():
        ref, bound = oracle.blockscaled_gemm_ref(a[lo:hi], sa[lo:hi], b[grp], sb[grp])
        _check_tol(y[lo:hi], ref, bound, "f32", f"group {grp} rows {lo}..{hi}")
        written[lo:hi] = True
    assert np.all(y[~written] == -3.0)


def test_gemm_repeat_bitwise_identical():
    d = inputs(1)
    banner("gemm repeatability")
    a, sa, b, sb = _quantize_pair(d["X"], d["W"])
    y1 = fb.fp8_blockscaled_gemm(a, sa, b, sb)
    y2 = fb.fp8_blockscaled_gemm(a, sa, b, sb)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


@pytest.mark.parametrize("m,n,k", [(1000, 528, 1024), (4096, 2048, 1024)])
def test_gemm_row_scales_repeat_bitwise_identical(m, n, k):
    """Per-row B scales on the 128x128 tile (ragged M and N) and on the
    256x128 tile: repeated calls give the same bits."""
    banner(f"gemm repeatability, per-row B scales {m}x{n}x{k}")
    g = torch.Generator(device="cuda").manual_seed(m + n)
    x = torch.randn((m, k), device="cuda", generator=g).to(torch.bfloat16)
    w = (torch.randn((n, k), device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    a, sa = fb.fp8_quant_act_1x128(x)
    b, sb = fb.fp8_quant_act_1x128(w)
    ys = [fb.fp8_blockscaled_gemm(a, sa, b, sb, b_kind="row", out_dtype=torch.float32) for _ in range(3)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(ys[0].view(torch.int32), y.view(torch.int32))


def test_gemm_zero_m_is_noop():
    banner("gemm M=0")
    a = torch.empty((0, 256), dtype=torch.uint8, device="cuda")
    sa = torch.empty((0, 2), dtype=torch.float32, device="cuda")
    b = torch.zeros((128, 256), dtype=torch.uint8, device="cuda")
    sb = torch.ones((1, 2), dtype=torch.float32, device="cuda")
    y = fb.fp8_blockscaled_gemm(a, sa, b, sb)
    assert y.shape == (0, 128)


# ---------------------------------------------------------------- FP8-MFMA accumulation
def test_accumulation_exact_vs_fp8_group_truncation():
    """One large and seven small products in one group of 8 consecutive K:
    256*256 + 7*(2*2) = 65564 is exact in fp32.  The default path (bf16 matrix
    instructions) must return it; the FP8 matrix instructions
    (fp8_blockscaled_gemm_fp8mma) keep only bits down to 2^-13 of the group's
    largest product and return 65536, which is why the contract path does not
    use them."""
    k = 128
    a = np.zeros((1, k), np.uint8)
    b = np.zeros((16, k), np.uint8)
    a[0, 0], b[0, 0] = 0x78, 0x78          # 256 * 256
    a[0, 1:8], b[0, 1:8] = 0x40, 0x40      # 2 * 2, seven times
    sa = np.ones((1, 1), np.float32)
    sb = np.ones((16, 1), np.float32)
    banner("gemm accumulation: 2^16 + 7*4 in one K group")
    y32 = fb.fp8_blockscaled_gemm(_dev(a), _dev(sa), _dev(b), _dev(sb), "row", torch.float32)
    y8 = fb.fp8_blockscaled_gemm_fp8mma(_dev(a), _dev(sa), _dev(b), _dev(sb), "row", torch.float32)
    torch.cuda.synchronize()
    ref, _ = oracle.blockscaled_gemm_ref(a, sa, b, sb, "row")
    assert ref[0, 0] == 65564.0
    assert _y_host(y32)[0, 0] == 65564.0
    assert _y_host(y8)[0, 0] == 65536.0
    assert np.all(_y_host(y32)[0, 1:] == 0.0) and np.all(_y_host(y8)[0, 1:] == 0.0)



def _fp8_group_bound(a, sa, b, sb, kind):
    """Error allowance of the FP8-matrix-core accumulation: per group of 8
    consecutive K, up to 8 * 2^(e - 13) where 2^e <= the group's largest |product|
    (measured behaviour of the gfx950 FP8 MFMA), times |sa * sb|."""
    da, db = oracle.e4m3_decode(a), oracle.e4m3_decode(b)
    m, k = da.shape
    n = db.shape[0]
    sbn = np.repeat(sb.astype(np.float64), 128, axis=0)[:n] if kind == "block128" else sb.astype(np.float64)
    out = np.zeros((m, n))
    for g in range(k // 8):
        pa = np.abs(da[:, 8 * g:8 * g + 8])
        pb = np.abs(db[:, 8 * g:8 * g + 8])
        mx = np.max(pa[:, None, :] * pb[None, :, :], axis=2)
        with np.errstate(divide="ignore"):
            e = np.floor(np.log2(np.where(mx > 0, mx, 1.0)))
        allow = np.where(mx > 0, 8.0 * np.exp2(e - 13.0), 0.0)
        kb = (8 * g) // 128
        out += allow * np.abs(sa[:, kb].astype(np.float64))[:, None] * np.abs(sbn[:, kb])[None, :]
    return out


@pytest.mark.parametrize("m,n,k,kind", [(128, 256, 512, "block128"), (200, 128, 1024, "block128"),
                                        (64, 48, 256, "row")])
def test_fp8_mfma_mode_within_group_model(m, n, k, kind):
    d = inputs(1) if (m, k) == (128, 512) else None
    rng = np.random.default_rng([26, m, n, k])
    if d is not None:
        a, sa, b, sb = _oracle_pair(d["X"], d["W"])
    else:
        x = synth.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
        a, sa = oracle.quant_1x128(f32(x))
        b = rng.integers(0, 256, size=(n, k), dtype=np.uint8)
        b[(b & 0x7F) == 0x7F] = 0x38
        sb = (rng.random((n // 128 if kind == "block128" else n, k // 128)) + 0.01).astype(np.float32)
    banner(f"gemm fp8_mfma accumulation {m}x{n}x{k} {kind}")
    y = fb.fp8_blockscaled_gemm_fp8mma(_dev(a), _dev(sa), _dev(b), _dev(sb), kind, torch.float32)
    torch.cuda.synchronize()
    ref, bound = oracle.blockscaled_gemm_ref(a, sa, b, sb, kind)
    allow = 2e-5 * bound + _fp8_group_bound(a, sa, b, sb, kind)
    err = np.abs(_y_host(y) - ref)
    assert np.all(err <= allow), f"max err/allow {np.max(err / np.maximum(allow, 1e-300)):.3f}"
