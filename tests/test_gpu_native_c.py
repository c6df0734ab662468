"""The library from a plain C program on the GPU, with no PyTorch in the
process: tests/native_step.c allocates HIP memory, creates its own stream,
quantizes X per 1x128 tile and W per 128x128 block in one batched launch,
runs the block-scaled GEMM into float32 and writes every output to files.
Codes and scales must equal the oracle's bit for bit, Y must lie within the
GEMM tolerance."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from fp8_block_scaled_05_amd import synth
from gpu_util import banner, f32, assert_codes_equal, assert_scales_equal

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "native_step.c")
EXE = os.path.join(HERE, "native_step")


@pytest.fixture(scope="module")
def exe():
    """The caller built by build(); rebuilt here (host C, gcc) if missing or
    older than its source, the header or the library."""
    import fp8_block_scaled_05_amd as fb
    deps = [SRC, os.path.join(ROOT, "include", "fp8bs.h"), fb.lib_path()]
    if not os.path.exists(EXE) or os.path.getmtime(EXE) < max(os.path.getmtime(d) for d in deps):
        import __graft_entry__
        __graft_entry__._build_native_test()
    return EXE


def _run(exe, tmp_path, x_bits, w_bits):
    m, k = x_bits.shape
    n = w_bits.shape[0]
    xf, wf, pre = tmp_path / "x.bin", tmp_path / "w.bin", tmp_path / "out"
    np.ascontiguousarray(x_bits, dtype=np.uint16).tofile(xf)
    np.ascontiguousarray(w_bits, dtype=np.uint16).tofile(wf)
    banner(f"native C step {m}x{n}x{k}")
    r = subprocess.run([exe, str(m), str(n), str(k), str(xf), str(wf), str(pre)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    rd = lambda ext, dt, shape: np.fromfile(f"{pre}.{ext}", dtype=dt).reshape(shape)
    return (rd("qa", np.uint8, (m, k)), rd("sa", np.float32, (m, k // 128)),
            rd("qb", np.uint8, (n, k)), rd("sb", np.float32, (n // 128, k // 128)),
            rd("y", np.float32, (m, n)))


def _check(x_bits, w_bits, outs, rows=None):
    qa, sa, qb, sb, y = outs
    want_qa, want_sa = oracle.quant_1x128(f32(x_bits))
    want_qb, want_sb = oracle.quant_128x128(f32(w_bits))
    assert_scales_equal(sa, want_sa, "X 1x128 scales")
    assert_codes_equal(qa, want_qa, "X 1x128 codes")
    assert_scales_equal(sb, want_sb, "W 128x128 scales")
    assert_codes_equal(qb, want_qb, "W 128x128 codes")
    rows = np.arange(qa.shape[0]) if rows is None else rows
    ref, bound = oracle.blockscaled_gemm_ref(want_qa[rows], want_sa[rows], want_qb, want_sb)
    ok = oracle.gemm_tolerance_ok(y[rows].astype(np.float64), ref, bound, "f32")
    assert ok.all(), f"{(~ok).sum()} of {ok.size} outside tolerance"


def test_native_c_step_ragged(exe, tmp_path):
    """M = 300 (a ragged M tail), N = 256, K = 1024; every output checked."""
    rng = np.random.default_rng([41, 300])
    x = synth.normal_bf16(rng, (300, 1024), 1.0, 0.005, 50.0)
    w = synth.normal_bf16(rng, (256, 1024), 0.02)
    _check(x, w, _run(exe, tmp_path, x, w))


def test_native_c_step_workload_4096x2048x7168(exe, tmp_path):
    """The full linear-layer workload; codes and scales everywhere, Y on a
    seeded sample of rows that holds the first and the last."""
    s = synth.SHAPES[2]
    inp = synth.workload_inputs(2)
    outs = _run(exe, tmp_path, inp["X"], inp["W"])
    _check(inp["X"], inp["W"], outs, synth.sample_rows(s["M"], 256, seed=41, must=(0, s["M"] - 1)))
