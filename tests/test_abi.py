"""C-ABI boundary checks that need no GPU: the library loads, exports every
function the header declares, and rejects bad arguments synchronously with the
documented status (these paths never reach the HIP runtime)."""
import ctypes

import pytest

import fp8_block_scaled_05_amd as fb

OK, INVALID, SHAPE, ALIGN = 0, 1, 2, 3
A16 = 0x10000          # a fake, 16-byte aligned "device" address; never dereferenced
A4 = 0x10004
NULL = 0


@pytest.fixture(scope="module")
def L():
    return fb.lib()


def test_exports_every_declared_symbol(L):
    names = fb.header_functions()
    assert set(names) == {"fp8_quant_act_1x128", "fp8_quant_act_dual", "fp8_quant_w_128x128",
                          "fp8_quant_batch",
                          "fp8_dequant", "fp8_quant_tensor", "fp8_blockscaled_gemm",
                          "fp8_blockscaled_gemm_fp8mma", "fp8_blockscaled_gemm_quant",
                          "fp8_blockscaled_grouped_gemm",
                          "fp8bs_last_error", "fp8bs_version"}
    for n in names:
        assert hasattr(L, n), n
    assert "gfx950" in fb.version()


def _act(L, x=A16, dt=0, rows=4, cols=256, ldx=256, tiling=0, q=A16, ldq=256, s=A16):
    return L.fp8_quant_act_1x128(x, dt, rows, cols, ldx, tiling, q, ldq, s, None)


def test_quant_act_validation(L):
    assert _act(L, rows=0) == OK and _act(L, cols=0) == OK            # empty: no-op
    assert _act(L, rows=0, x=NULL, q=NULL, s=NULL) == OK
    assert _act(L, dt=7) == INVALID
    assert _act(L, tiling=5) == INVALID
    assert _act(L, rows=-1) == INVALID
    assert _act(L, cols=200, ldx=256) == SHAPE
    assert _act(L, tiling=1, rows=100) == SHAPE                       # 128x1 needs rows%128
    assert _act(L, x=NULL) == INVALID and _act(L, s=NULL) == INVALID
    assert "null" in fb.last_error()
    assert _act(L, ldx=128) == INVALID                                 # pitch < cols
    assert _act(L, x=A16 + 8) == ALIGN
    assert _act(L, ldx=260) == ALIGN                                   # 520 B rows
    assert _act(L, q=A16 + 4) == ALIGN
    assert _act(L, ldq=264) == ALIGN
    assert _act(L, s=A16 + 2) == ALIGN
    assert _act(L, tiling=1, rows=128, cols=8, ldx=8, ldq=136) == ALIGN  # q pitch 136 B
    assert _act(L, tiling=1, rows=128, cols=8, ldx=8, ldq=64) == INVALID  # q pitch < rows


def _w(L, w=A16, dt=0, rows=256, cols=256, ldw=256, q=A16, ldq=256, s=A16, qt=NULL, ldqt=0):
    return L.fp8_quant_w_128x128(w, dt, rows, cols, ldw, q, ldq, s, qt, ldqt, None)


def test_quant_w_validation(L):
    assert _w(L, rows=0) == OK
    assert _w(L, rows=200) == SHAPE and _w(L, cols=100) == SHAPE
    assert _w(L, dt=3) == INVALID
    assert _w(L, q=NULL) == INVALID
    assert _w(L, w=A16 + 4) == ALIGN
    assert _w(L, qt=A16, ldqt=128) == INVALID                           # ld_qt < rows
    assert _w(L, qt=A16, ldqt=264) == ALIGN
    assert _w(L, s=A16 + 1) == ALIGN


def _dual(L, x=A16, dt=0, rows=256, cols=384, ldx=384, q=A16, ldq=384, s=A16, qt=A16, ldqt=256,
          st=A16):
    return L.fp8_quant_act_dual(x, dt, rows, cols, ldx, q, ldq, s, qt, ldqt, st, None)


def test_quant_dual_validation(L):
    assert _dual(L, rows=0) == OK and _dual(L, cols=0) == OK
    assert _dual(L, rows=0, x=NULL, q=NULL, s=NULL, qt=NULL, st=NULL) == OK
    assert _dual(L, dt=2) == INVALID and _dual(L, rows=-128) == INVALID
    assert _dual(L, rows=200) == SHAPE and _dual(L, cols=100, ldx=112) == SHAPE
    for kw in ("x", "q", "s", "qt", "st"):                              # every output required
        assert _dual(L, **{kw: NULL}) == INVALID, kw
    assert _dual(L, ldx=256) == INVALID and _dual(L, ldq=256) == INVALID
    assert _dual(L, ldqt=128) == INVALID                                # ld_qt < rows
    assert _dual(L, x=A16 + 8) == ALIGN and _dual(L, q=A16 + 4) == ALIGN
    assert _dual(L, qt=A16 + 2) == ALIGN and _dual(L, ldqt=264) == ALIGN
    assert _dual(L, s=A16 + 1) == ALIGN and _dual(L, st=A4 + 2) == ALIGN
    assert _dual(L, ldx=(1 << 40) + 384) == INVALID


def _job(x=A16, dt=0, tiling=0, rows=256, cols=384, ldx=384, q=A16, ldq=384, s=A16):
    return fb.QuantJob(x, dt, tiling, rows, cols, ldx, q, ldq, s)


def _batch(L, *jobs):
    arr = (fb.QuantJob * max(1, len(jobs)))(*jobs)
    return L.fp8_quant_batch(arr, len(jobs), None)


def test_quant_batch_validation(L):
    import ctypes
    assert ctypes.sizeof(fb.QuantJob) == 64                       # the C struct's size
    assert _batch(L) == OK                                         # no jobs
    assert _batch(L, _job(rows=0), _job(cols=0, tiling=2)) == OK   # empty jobs are skipped
    assert L.fp8_quant_batch(None, 1, None) == INVALID
    assert L.fp8_quant_batch(None, -1, None) == INVALID
    assert _batch(L, *[_job()] * 9) == INVALID                     # more than 8 jobs
    assert _batch(L, _job(), _job(tiling=1)) == INVALID            # 128x1_T is not a batch tiling
    assert "job 1" in fb.last_error()
    assert _batch(L, _job(dt=5)) == INVALID
    assert _batch(L, _job(cols=200, ldx=208, ldq=208)) == SHAPE
    assert _batch(L, _job(tiling=2, rows=200)) == SHAPE            # 128x128 needs rows % 128
    assert _batch(L, _job(), _job(q=NULL)) == INVALID and "job 1" in fb.last_error()
    assert _batch(L, _job(x=A16 + 8)) == ALIGN and _batch(L, _job(s=A16 + 2)) == ALIGN
    assert _batch(L, _job(ldx=256)) == INVALID                     # pitch < cols
    assert _batch(L, _job(ldx=(1 << 40) + 384)) == INVALID
    assert _batch(L, _job(rows=-1)) == INVALID


def _deq(L, q=A16, rows=256, cols=384, ldq=384, s=A16, tiling=0, y=A16, ydt=1, ldy=384):
    return L.fp8_dequant(q, rows, cols, ldq, s, tiling, y, ydt, ldy, None)


def test_dequant_validation(L):
    assert _deq(L, rows=0) == OK and _deq(L, rows=0, q=NULL, s=NULL, y=NULL) == OK
    assert _deq(L, tiling=1) == INVALID and _deq(L, tiling=3) == INVALID
    assert "x^T" in fb.last_error() or "tiling" in fb.last_error()
    assert _deq(L, ydt=5) == INVALID and _deq(L, rows=-1) == INVALID
    assert _deq(L, cols=200, ldq=208, ldy=208) == SHAPE
    assert _deq(L, tiling=2, rows=200) == SHAPE
    assert _deq(L, q=NULL) == INVALID and _deq(L, s=NULL) == INVALID and _deq(L, y=NULL) == INVALID
    assert _deq(L, ldq=256) == INVALID and _deq(L, ldy=256) == INVALID
    assert _deq(L, q=A16 + 8) == ALIGN and _deq(L, y=A16 + 4) == ALIGN
    assert _deq(L, ldq=392) == ALIGN and _deq(L, ydt=0, ldy=388) == ALIGN   # 776 B bf16 rows
    assert _deq(L, s=A16 + 2) == ALIGN
    assert _deq(L, ldq=(1 << 40) + 384) == INVALID


def _tq(L, x=A16, dt=0, rows=4, cols=64, ldx=64, fmt=0, margin=0.0, h=NULL, hl=0, q=A16, ldq=64,
        s=A4, a=A4):
    return L.fp8_quant_tensor(x, dt, rows, cols, ldx, fmt, margin, h, hl, q, ldq, s, a, None)


def test_quant_tensor_validation(L):
    assert _tq(L, rows=0) == OK and _tq(L, rows=0, x=NULL, q=NULL, s=NULL, a=NULL) == OK
    assert _tq(L, fmt=2) == INVALID and _tq(L, dt=3) == INVALID
    assert _tq(L, margin=-0.1) == INVALID and _tq(L, margin=float("nan")) == INVALID
    assert _tq(L, margin=2e6) == INVALID
    assert _tq(L, h=A4, hl=0) == INVALID and _tq(L, h=A4, hl=5000) == INVALID
    assert _tq(L, cols=60, ldx=64, ldq=64) == SHAPE
    assert _tq(L, s=NULL) == INVALID and _tq(L, a=NULL) == INVALID and _tq(L, q=NULL) == INVALID
    assert _tq(L, ldx=56) == INVALID and _tq(L, ldq=56) == INVALID
    assert _tq(L, x=A16 + 4) == ALIGN and _tq(L, ldq=72) == ALIGN and _tq(L, ldx=68) == ALIGN
    assert _tq(L, s=A4 + 1) == ALIGN and _tq(L, h=A4 + 2, hl=8) == ALIGN
    assert _tq(L, ldx=(1 << 40) + 64) == INVALID


def _gemm(L, M=4, N=256, K=256, a=A16, lda=256, sa=A16, b=A16, ldb=256, sb=A16, kind=0, y=A16,
          ydt=1, ldy=256, entry="fp8_blockscaled_gemm"):
    return getattr(L, entry)(M, N, K, a, lda, sa, b, ldb, sb, kind, y, ydt, ldy, None)


@pytest.mark.parametrize("entry", ["fp8_blockscaled_gemm", "fp8_blockscaled_gemm_fp8mma"])
def test_gemm_validation(L, entry):
    g = lambda **kw: _gemm(L, entry=entry, **kw)   # noqa: E731
    assert g(M=0) == OK
    assert g(M=0, a=NULL, y=NULL) == OK
    assert g(K=100, lda=112, ldb=112) == SHAPE
    assert g(K=0) == SHAPE
    assert g(N=144, ldy=144) == SHAPE                                  # block128 needs N%128
    assert g(N=24, ldy=32, kind=1) == SHAPE                            # N % 16
    assert g(kind=2) == INVALID and g(ydt=9) == INVALID
    assert g(M=-3) == INVALID
    assert g(sa=NULL) == INVALID
    assert entry in fb.last_error()
    assert g(lda=128) == INVALID and g(ldy=128) == INVALID
    assert g(a=A16 + 8) == ALIGN and g(lda=264) == ALIGN
    assert g(ydt=0, ldy=260) == ALIGN                                  # bf16 pitch 520 B
    assert g(sb=A16 + 2) == ALIGN


def _gq(L, M=4, N=256, K=256, a=A16, lda=256, sa=A16, b=A16, ldb=256, sb=A16, kind=0, yq=A16,
        ldyq=256, ys=A16):
    return L.fp8_blockscaled_gemm_quant(M, N, K, a, lda, sa, b, ldb, sb, kind, yq, ldyq, ys, None)


def test_gemm_quant_validation(L):
    assert _gq(L, M=0) == OK and _gq(L, M=0, yq=NULL, ys=NULL) == OK
    assert _gq(L, N=144, ldyq=144, kind=1) == SHAPE                     # 1x128 output tiles
    assert _gq(L, K=64, lda=64, ldb=64) == SHAPE
    assert _gq(L, ys=NULL) == INVALID and _gq(L, yq=NULL) == INVALID
    assert _gq(L, kind=3) == INVALID
    assert _gq(L, ldyq=128) == INVALID
    assert _gq(L, ldyq=264) == ALIGN and _gq(L, yq=A16 + 8) == ALIGN
    assert _gq(L, ys=A16 + 2) == ALIGN
    assert _gq(L, ldyq=(1 << 40) + 256) == INVALID


def _grouped(L, M=256, N=256, K=256, G=4, off=A16, a=A16, sa=A16, b=A16, sb=A16, y=A16, ydt=0):
    return L.fp8_blockscaled_grouped_gemm(M, N, K, G, off, a, sa, b, sb, y, ydt, None)


def test_grouped_validation(L):
    assert _grouped(L, M=0) == OK
    assert _grouped(L, G=0) == INVALID and _grouped(L, G=2000) == INVALID
    assert _grouped(L, N=144) == SHAPE and _grouped(L, K=64) == SHAPE
    assert _grouped(L, off=NULL) == INVALID
    assert _grouped(L, off=A16 + 2) == ALIGN and _grouped(L, a=A16 + 4) == ALIGN
    assert _grouped(L, ydt=4) == INVALID


def test_absurd_pitches_rejected(L):
    """A 64-bit size whose upper half is garbage (as when a caller passes a
    32-bit value) must be refused before any launch."""
    big = (1 << 40) + 256
    assert _act(L, ldx=big) == INVALID and _act(L, ldq=big) == INVALID
    assert _act(L, tiling=1, rows=128, cols=8, ldx=8, ldq=big) == INVALID
    assert _w(L, ldw=big) == INVALID and _w(L, qt=A16, ldqt=big) == INVALID
    assert _gemm(L, ldy=big) == INVALID and _gemm(L, lda=big) == INVALID
    assert _gemm(L, M=(1 << 33)) == INVALID
    assert _grouped(L, M=(1 << 40)) == INVALID


def test_last_error_is_per_call_text(L):
    assert _gemm(L, K=100, lda=112, ldb=112) == SHAPE
    assert "K=100" in fb.last_error()
    assert _w(L, rows=200) == SHAPE
    assert "200" in fb.last_error()


def test_last_error_is_per_thread(L):
    """The error text is thread-local: a failing call on another thread
    between a call and its fp8bs_last_error() does not replace its text."""
    import threading
    bar = threading.Barrier(2, timeout=30)
    out = {}

    def first():
        out["a_status"] = _gemm(L, K=100, lda=112, ldb=112)
        bar.wait()          # the other thread now fails with its own text
        bar.wait()
        out["a"] = fb.last_error()

    def second():
        bar.wait()
        out["b_status"] = _w(L, rows=200)
        out["b"] = fb.last_error()
        bar.wait()

    ts = [threading.Thread(target=first), threading.Thread(target=second)]
    for t in ts:
        t.start()
    for t in ts:
        t.join(60)
    assert out["a_status"] == SHAPE and out["b_status"] == SHAPE
    assert "K=100" in out["a"] and "200" not in out["a"]
    assert "200" in out["b"] and "K=100" not in out["b"]


def test_binding_raises_typed_error():
    with pytest.raises(fb.Fp8bsError) as e:
        fb._check(2)
    assert e.value.status == 2


def test_header_is_plain_c_and_links_from_c(tmp_path):
    """fp8bs.h compiles as C99 and C++17, and a C program linked against the
    library gets the documented statuses (validation only: no GPU needed)."""
    import os
    import shutil
    import subprocess
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("gcc not found")
    here = os.path.dirname(os.path.abspath(__file__))
    inc = os.path.join(os.path.dirname(here), "include")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    flags = ["-D__HIP_PLATFORM_AMD__", "-I", inc, "-I", os.path.join(rocm, "include")]
    src = os.path.join(here, "c_abi_check.c")
    exe = str(tmp_path / "c_abi_check")
    lib_dir = os.path.dirname(fb.lib_path())
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", *flags, src, "-o", exe,
                        "-L", lib_dir, "-lfp8bs", "-Wl,-rpath," + lib_dir], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r2 = subprocess.run([shutil.which("g++") or "g++", "-std=c++17", "-Wall", "-Werror", "-fsyntax-only",
                         "-x", "c++", *flags, src], capture_output=True, text=True)
    assert r2.returncode == 0, r2.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 failure(s)" in run.stdout

