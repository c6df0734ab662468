"""Throughput of the FP8 block-scaled hot path on one MI355X.

One step = online 1x128 quantization of the activations X [4096, 7168] (bf16)
and 128x128 quantization of the weight W [2048, 7168] (bf16), in one batched
launch, then the block-scaled FP8 GEMM Y = X W^T [4096, 2048] with FP32
promotion per 128-deep K block (bf16 output by default).  Inputs are seeded synthetic tensors shaped like a
DeepSeek-V3 layer (hidden 7168), already resident in HBM; X, W and Y step
through several buffer sets so that more than 1 GiB is cycled and the 256 MB
Infinity Cache cannot serve repeated reads.

Order of work: the per-kernel figures (linear workload, then the other
workloads' shapes) come first, then W untimed steps and exactly K timed
steps, then the CPU oracle.  The seconds of GPU work before the steps let the
chip's clock settle: under sustained matrix work it goes through a transient
of tens of milliseconds after an idle period.

Prints one JSON line:
  value / ms_per_step  whole-step throughput: 2*M*N*K per step over the
                       measured step time (both quantizers included);
  roofline             the GEMM (the dominant kernel) against the 5.0 PFLOP/s
                       dense FP8 MFMA peak, from its average launch duration
                       over back-to-back launches on rotating buffers, timed
                       with HIP events on the stream the kernels run on;
  kernels              the same for every kernel of the step and the other
                       kernels of the library (quantizers as GB/s against HBM);
  workloads            the other workload shapes (dense FFN, MoE grouped,
                       dgrad/wgrad) with their GEMMs and quantizers;
  cpu_baseline         the CPU oracle timed on a bounded sample of the step
                       (and of the other workloads), with the cores it used.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

M, N, K = 4096, 2048, 7168
PEAK_FP8_TFLOPS = 5000.0        # MI355X dense FP8 MFMA
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 (= f16) MFMA, on which the exact GEMM runs
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
METRIC = "FP8 block-scaled GEMM TFLOP/s (% FP8 MFMA peak); quantize GB/s (% HBM)"

# HBM bytes per GEMM launch from two rocprofv3 --pmc runs of
# `bench.py --calib-copy` (FETCH_SIZE, then WRITE_SIZE), each scaled by what
# the same counter reads for the device copy of known size that --calib-copy
# adds; valid only for the GEMM source it was measured on (sha256 of gemm.hip).
TRAFFIC = {"gemm_sha256": "20995fa41966ad92536126e9c5510da124f793cbc723c4f80e386083acfa9ee0",
           "bytes_per_launch": 137175349,   # 120.40 MB read (FETCH_SIZE x 1.99944) + 16.78 MB written
           "source": "profiles/bench_linear_4096x2048x7168_counters.md"}
CALIB_COPY_BYTES = 128 << 20


def algorithmic():
    tiles_x = M * (K // 128)
    quant_x_bytes = M * K * 2 + M * K + tiles_x * 4
    quant_w_bytes = N * K * 2 + N * K + (N // 128) * (K // 128) * 4
    gemm_flops = 2 * M * N * K
    return quant_x_bytes, quant_w_bytes, gemm_flops


def quant_bytes(rows, cols, kind):
    """Algorithmic bytes of one quantizer call on a bf16 [rows, cols] input:
    input read once, each output written once."""
    n = rows * cols
    if kind in ("1x128", "128x1_t"):
        return 2 * n + n + 4 * (n // 128)
    if kind == "128x128":
        return 2 * n + n + 4 * (n // (128 * 128))
    if kind == "128x128+t":
        return 2 * n + 2 * n + 4 * (n // (128 * 128))
    if kind == "dual":
        return 2 * n + 2 * n + 2 * 4 * (n // 128)
    raise ValueError(kind)


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--launches", type=int, default=50,
                   help="back-to-back launches per kernel figure (at least 50)")
    p.add_argument("--gemm-warmup", type=int, default=300,
                   help="untimed GEMM launches before its back-to-back timing (the clock settles)")
    p.add_argument("--out", choices=["bf16", "f32"], default="bf16")
    p.add_argument("--rotate-mib", type=int, default=1100,
                   help="bytes of input/output buffers cycled through (defeats the MALL)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=M,
                   help="rows of X in the oracle's timed sample (default: all)")
    p.add_argument("--no-workloads", action="store_true",
                   help="skip the other workload shapes (dense FFN, MoE grouped, dgrad/wgrad)")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run one device copy of 128 MiB (counter calibration for rocprofv3 --pmc)")
    a = p.parse_args()
    a.launches = max(50, a.launches)
    return a


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001 - threadpoolctl is optional
        return 1


def cpu_baseline(xbits, wbits, rows):
    """The oracle, as it stands, on the first `rows` rows of X and all of W."""
    import oracle
    from fp8_block_scaled_05_amd import synth
    nthreads = blas_threads()
    x = synth.bf16_bits_to_f32(xbits[:rows])
    w = synth.bf16_bits_to_f32(wbits)
    t0 = time.perf_counter()
    a, sa = oracle.quant_1x128(x)
    b, sb = oracle.quant_128x128(w)
    t1 = time.perf_counter()
    oracle.blockscaled_gemm_ref(a, sa, b, sb)
    t2 = time.perf_counter()
    dt = t2 - t0
    flops = 2.0 * rows * N * K
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(nthreads),
            "kind": "oracle",
            "sample": (f"quantize X[:{rows}] (1x128) + W[{N},{K}] (128x128) + float64 "
                       f"per-128-K-block GEMM with its error bound for {rows} rows; "
                       f"{dt:.2f} s wall"),
            "seconds": round(dt, 3),
            "stages": {"quantize": {"seconds": round(t1 - t0, 3), "cores": 1,
                                    "note": "single-threaded numpy"},
                       "gemm": {"seconds": round(t2 - t1, 3), "cores": int(nthreads),
                                "note": "float64 BLAS"}},
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0))}


def extra_cpu_baselines(shrink=1):
    """The oracle, as it stands, on bounded samples of the other workloads.

    Each sample is drawn with its workload's recipe (same distributions and
    K; fewer rows), quantized by the oracle and multiplied by its float64
    per-128-K-block reference, so every figure includes quantization.
    Throughput is 2 * rows * cols * K of the sample over its wall time.
    Every stage is timed on its own; the full workload's oracle time is
    estimated by scaling each quantization stage by the full tensor's
    element count and each GEMM stage by the full GEMM's flops.
    `shrink` divides every row count (the tests use a small sample)."""
    import numpy as np
    import oracle
    from fp8_block_scaled_05_amd import synth
    f32 = synth.bf16_bits_to_f32
    nthreads = blas_threads()
    res = {}

    def timed(name, flops, sample, stages):
        """stages: (stage name, cores, fn, factor from the sample to the full workload)."""
        per, total, full = {}, 0.0, 0.0
        for sname, cores, fn, factor in stages:
            t0 = time.perf_counter()
            fn()
            dt = time.perf_counter() - t0
            per[sname] = {"seconds": round(dt, 3), "cores": int(cores), "to_full": round(factor, 3)}
            total += dt
            full += dt * factor
        res[name] = {"value": round(flops / total / 1e12, 6), "unit": "TFLOP/s", "kind": "oracle",
                     "sample": sample, "seconds": round(total, 3),
                     "full_workload_seconds_est": round(full, 1),
                     "cores": {"quantize": 1, "gemm": int(nthreads)}, "stages": per}

    k = 7168
    r1, r2, r4 = 1024 // shrink, 2048 // shrink, 4096 // shrink
    d = {}
    # Dense FFN [8192, 18432, 7168]: 1024 rows of X, 2048 rows (16 row
    # blocks) of the block-spread W.
    x = f32(synth.normal_bf16(synth.rng_for(3, synth.X_ID), (r1, k), 1.0, 0.001, 100.0))
    w = f32(synth.block_spread_bf16(synth.rng_for(3, synth.W_ID), (r2, k), 0.02))
    timed("ffn_8192x18432x7168", 2.0 * r1 * r2 * k,
          f"X[{r1},7168] 1x128 + W[{r2},7168] 128x128 (block spread) + GEMM {r1}x{r2}x7168", [
              ("quant_x_1x128", 1, lambda: d.update(a=oracle.quant_1x128(x)), 8192 / r1),
              ("quant_w_128x128", 1, lambda: d.update(b=oracle.quant_128x128(w)), 18432 / r2),
              ("gemm", nthreads, lambda: oracle.blockscaled_gemm_ref(*d["a"], *d["b"]),
               8192 * 18432 / (r1 * r2)),
          ])

    # MoE [32768 tokens, 16 experts of 4096 x 7168]: one expert's full
    # weight and 512 of its tokens.
    x = f32(synth.normal_bf16(synth.rng_for(4, synth.X_ID), (r1 // 2, k), 1.0, 0.001, 100.0))
    w = f32(synth.weight(4, r4, k, expert=0))
    off = np.array([0, r1 // 2], np.int32)
    timed("moe_grouped_32768x4096x7168_g16", 2.0 * (r1 // 2) * r4 * k,
          f"one expert: X[{r1 // 2},7168] 1x128 + W[{r4},7168] 128x128 + grouped GEMM {r1 // 2}x{r4}x7168", [
              ("quant_x_1x128", 1, lambda: d.update(a=oracle.quant_1x128(x)), 32768 / (r1 // 2)),
              ("quant_w_128x128", 1, lambda: d.update(b=oracle.quant_128x128(w)), 16 * 4096 / r4),
              ("grouped_gemm", nthreads,
               lambda: oracle.grouped_gemm_ref(off, *d["a"], d["b"][0][None], d["b"][1][None]),
               32768 * 4096 / ((r1 // 2) * r4)),
          ])

    # Backward [8192 tokens]: 1024 tokens.  dgrad dY[1024,2048] x W[2048,7168]
    # (W quantized 128x128, used transposed); wgrad X^T dY with both
    # operands 128x1 along the tokens.
    t, h, f = r1, 7168, 2048
    dy = f32(synth.normal_bf16(synth.rng_for(5, synth.DY_ID), (t, f), 1e-3))
    x = f32(synth.normal_bf16(synth.rng_for(5, synth.X_ID), (t, h), 1.0, 0.001, 100.0))
    w = f32(synth.weight(5, f, h))
    tok = 8192 / t

    def dgrad():
        b, sb = d["w"]
        oracle.blockscaled_gemm_ref(*d["g"], np.ascontiguousarray(b.T), np.ascontiguousarray(sb.T))

    timed("backward_dgrad_wgrad", 2.0 * (t * h * f) * 2,
          f"{t} tokens: dY 1x128 + W 128x128 + dgrad {t}x7168x2048; X and dY 128x1 + wgrad 7168x2048x{t}", [
              ("quant_dy_1x128", 1, lambda: d.update(g=oracle.quant_1x128(dy)), tok),
              ("quant_w_128x128", 1, lambda: d.update(w=oracle.quant_128x128(w)), 1.0),
              ("dgrad_gemm", nthreads, dgrad, tok),
              ("quant_x_128x1_t", 1, lambda: d.update(xt=oracle.quant_128x1_t(x)), tok),
              ("quant_dy_128x1_t", 1, lambda: d.update(gt=oracle.quant_128x1_t(dy)), tok),
              ("wgrad_gemm", nthreads, lambda: oracle.blockscaled_gemm_ref(*d["xt"], *d["gt"], "row"), tok),
          ])
    return res


def device_info(torch):
    """Name, compute units and current clock levels of cuda:0.

    The clocks are read from the driver's sysfs files; no other program is
    started, since a child process started after the GPU is initialised
    (e.g. under a profiler's preload) must not exec another program."""
    import glob
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "gcn_arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count,
            "memory_GiB": round(p.total_memory / 2 ** 30, 1)}
    for kind in ("sclk", "mclk"):
        for path in sorted(glob.glob(f"/sys/class/drm/card*/device/pp_dpm_{kind}")):
            try:
                with open(path) as f:
                    lines = [l.strip() for l in f if l.strip()]
            except OSError:
                continue
            cur = [l.split(":", 1)[-1].strip(" *") for l in lines if l.endswith("*")]
            if lines:
                info[f"{kind}_max"] = lines[-1].split(":", 1)[-1].strip(" *")
            if cur:
                info[f"{kind}_at_exit"] = cur[0]
            if lines:
                break
    return info


class Bench:
    """Library calls with prepared arguments and event timing on one stream."""

    def __init__(self, torch, fb, launches, rotate_bytes):
        self.torch, self.fb, self.L = torch, fb, fb.lib()
        self.stream = torch.cuda.current_stream()
        self.hs = ctypes.c_void_p(self.stream.cuda_stream)
        self.launches = launches
        self.rotate_bytes = rotate_bytes
        self.dev = torch.device("cuda:0")

    def check(self, status):
        if status:
            raise RuntimeError(self.fb.last_error())

    def n_sets(self, set_bytes, cap=32):
        """Buffer sets whose total exceeds the rotation size (at least 1)."""
        return max(1, min(cap, -(-self.rotate_bytes // max(1, set_bytes))))

    def timed_us(self, fn, n=None, warm=3):
        """Average microseconds per call over n back-to-back calls fn(i), with
        events recorded on the launch stream."""
        torch = self.torch
        n = n or self.launches
        for i in range(warm):
            fn(i)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(self.stream)
        for i in range(n):
            fn(i)
        t1.record(self.stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / n * 1e3

    # -- library calls on tensors (pointers only; shapes are the caller's) --
    def quant_act(self, x, q, s, tiling=0):
        rows, cols = x.shape
        ldq = cols if tiling == 0 else rows
        self.check(self.L.fp8_quant_act_1x128(x.data_ptr(), 0 if x.dtype == self.torch.bfloat16 else 1,
                                              rows, cols, cols, tiling, q.data_ptr(), ldq, s.data_ptr(),
                                              self.hs))

    def quant_w(self, w, q, s, qt=None):
        rows, cols = w.shape
        self.check(self.L.fp8_quant_w_128x128(w.data_ptr(), 0, rows, cols, cols, q.data_ptr(), cols,
                                              s.data_ptr(), qt.data_ptr() if qt is not None else None,
                                              rows if qt is not None else 0, self.hs))

    def batch_jobs(self, jobs):
        """A prepared fp8bs_quant_job array for fp8_quant_batch: jobs is a
        list of (x, tiling code, q, scale)."""
        fb = self.fb
        arr = (fb.QuantJob * len(jobs))()
        for i, (x, tiling, q, sc) in enumerate(jobs):
            rows, cols = x.shape
            arr[i] = fb.QuantJob(x.data_ptr(), 0 if x.dtype == self.torch.bfloat16 else 1, tiling, rows, cols,
                                 cols, q.data_ptr(), cols, sc.data_ptr())
        return arr

    def quant_batch(self, arr):
        self.check(self.L.fp8_quant_batch(arr, len(arr), self.hs))

    def quant_dual(self, x, q, s, qt, st):
        rows, cols = x.shape
        self.check(self.L.fp8_quant_act_dual(x.data_ptr(), 0, rows, cols, cols, q.data_ptr(), cols,
                                             s.data_ptr(), qt.data_ptr(), rows, st.data_ptr(), self.hs))

    def gemm(self, a, sa, b, sb, y, kind=0, entry="fp8_blockscaled_gemm"):
        m, k = a.shape
        n = b.shape[0]
        ydt = 0 if y.dtype == self.torch.bfloat16 else 1
        self.check(getattr(self.L, entry)(m, n, k, a.data_ptr(), k, sa.data_ptr(), b.data_ptr(), k,
                                          sb.data_ptr(), kind, y.data_ptr(), ydt, n, self.hs))

    def grouped(self, off, a, sa, b, sb, y):
        m, k = a.shape
        g, n, _ = b.shape
        self.check(self.L.fp8_blockscaled_grouped_gemm(m, n, k, g, off.data_ptr(), a.data_ptr(),
                                                       sa.data_ptr(), b.data_ptr(), sb.data_ptr(),
                                                       y.data_ptr(), 0, self.hs))

    # -- result records --
    @staticmethod
    def gemm_rec(flops, us, **extra):
        tf = flops / us / 1e6
        return {**extra, "avg_us": round(us, 2), "TFLOP/s": round(tf, 2),
                "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
                "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4), "flops": int(flops)}

    @staticmethod
    def quant_rec(nbytes, us, **extra):
        gbs = nbytes / us / 1e3
        return {**extra, "avg_us": round(us, 2), "GB/s": round(gbs, 1),
                "frac_hbm": round(gbs / PEAK_HBM_GBPS, 4), "bytes": int(nbytes)}


def rand_bf16(torch, dev, shape, std=1.0, seed=0):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return (torch.randn(shape, device=dev, generator=g) * std).to(torch.bfloat16)


def linear_kernels(B, xs, ws, ys_dtype, qx_bytes, qw_bytes, flops, gemm_warmup):
    """Back-to-back figures of the step's kernels and the library's other
    kernels on the linear workload's shapes."""
    torch, dev, n = B.torch, B.dev, B.launches
    ns = len(xs)
    a = [torch.empty((M, K), dtype=torch.uint8, device=dev) for _ in range(ns)]
    sa = [torch.empty((M, K // 128), dtype=torch.float32, device=dev) for _ in range(ns)]
    b = [torch.empty((N, K), dtype=torch.uint8, device=dev) for _ in range(ns)]
    sb = [torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev) for _ in range(ns)]
    ys = [torch.empty((M, N), dtype=ys_dtype, device=dev) for _ in range(ns)]
    for j in range(ns):
        B.quant_act(xs[j], a[j], sa[j])
        B.quant_w(ws[j], b[j], sb[j])
    torch.cuda.synchronize()
    out = {}
    qx_us = B.timed_us(lambda i: B.quant_act(xs[i % ns], a[i % ns], sa[i % ns]))
    qw_us = B.timed_us(lambda i: B.quant_w(ws[i % ns], b[i % ns], sb[i % ns]))
    both_us = B.timed_us(lambda i: (B.quant_act(xs[i % ns], a[i % ns], sa[i % ns]),
                                    B.quant_w(ws[i % ns], b[i % ns], sb[i % ns])))
    # Under sustained matrix work the chip's clock goes through a transient of
    # tens of milliseconds before it settles: `gemm_warmup` untimed launches
    # (default 300, about 33 ms) come first, and the average is taken over at
    # least 100 launches.
    n_g = max(100, 2 * n)
    gemm_us = B.timed_us(lambda i: B.gemm(a[i % ns], sa[i % ns], b[i % ns], sb[i % ns], ys[i % ns]),
                         n=n_g, warm=gemm_warmup)
    out["quant_act_1x128"] = B.quant_rec(qx_bytes, qx_us, shape=[M, K], launches=n)
    out["quant_w_128x128"] = B.quant_rec(qw_bytes, qw_us, shape=[N, K], launches=n)
    out["quantize_two_launches"] = B.quant_rec(qx_bytes + qw_bytes, both_us, launches=n,
                                               note="X 1x128 and W 128x128 as two launches, back to back")
    arrs = [B.batch_jobs([(xs[j], 0, a[j], sa[j]), (ws[j], 2, b[j], sb[j])]) for j in range(ns)]
    batch_us = B.timed_us(lambda i: B.quant_batch(arrs[i % ns]))
    out["quantize_step"] = B.quant_rec(qx_bytes + qw_bytes, batch_us, launches=n,
                                       note="the step's quantization: X 1x128 and W 128x128 in one "
                                            "fp8_quant_batch launch")
    out["blockscaled_gemm"] = B.gemm_rec(flops, gemm_us, M=M, N=N, K=K, out="bf16" if ys_dtype == torch.bfloat16 else "f32",
                                         mfma="bf16 (E4M3 widened exactly)", launches=n_g, warmup_launches=gemm_warmup)
    fp8_us = B.timed_us(lambda i: B.gemm(a[i % ns], sa[i % ns], b[i % ns], sb[i % ns], ys[i % ns],
                                         entry="fp8_blockscaled_gemm_fp8mma"), n=n_g, warm=30)
    out["blockscaled_gemm_fp8mma"] = B.gemm_rec(flops, fp8_us, mfma="fp8", launches=n_g,
                                                note="FP8 matrix instructions; outside the accuracy contract")

    # The GEMM with its output quantized 1x128 in the epilogue, against the
    # same result in two launches (float32 GEMM output, then the quantizer).
    yq = torch.empty((M, N), dtype=torch.uint8, device=dev)
    ysc = torch.empty((M, N // 128), dtype=torch.float32, device=dev)
    y32 = torch.empty((M, N), dtype=torch.float32, device=dev)

    def gemm_quant(i):
        j = i % ns
        B.check(B.L.fp8_blockscaled_gemm_quant(M, N, K, a[j].data_ptr(), K, sa[j].data_ptr(), b[j].data_ptr(), K,
                                               sb[j].data_ptr(), 0, yq.data_ptr(), N, ysc.data_ptr(), B.hs))

    def gemm_then_quant(i):
        j = i % ns
        B.gemm(a[j], sa[j], b[j], sb[j], y32)
        B.quant_act(y32, yq, ysc)
    gq_us, g2_us = B.timed_us(gemm_quant, warm=20), B.timed_us(gemm_then_quant, warm=20)
    out["blockscaled_gemm_quant_out"] = B.gemm_rec(flops, gq_us, two_launch_us=round(g2_us, 2), launches=n,
                                                   note="Y quantized 1x128 (E4M3 + scales) in the GEMM epilogue "
                                                        "vs float32 GEMM then the quantizer")
    del y32

    # Both activation tilings from one read (dual) and the 128x1 tiling alone.
    qd = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sd = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    qtd = torch.empty((K, M), dtype=torch.uint8, device=dev)
    std = torch.empty((K, M // 128), dtype=torch.float32, device=dev)
    dual_us = B.timed_us(lambda i: B.quant_dual(xs[i % ns], qd, sd, qtd, std))
    t_us = B.timed_us(lambda i: B.quant_act(xs[i % ns], qtd, std, tiling=1))
    out["quant_act_dual"] = B.quant_rec(quant_bytes(M, K, "dual"), dual_us, launches=n,
                                        note="X 1x128 and 128x1 (transposed) from one read")
    out["quant_act_128x1_t"] = B.quant_rec(quant_bytes(M, K, "128x1_t"), t_us, launches=n)

    # Dequantize 1x128 codes to bf16.
    n_deq = 4                       # 4 x (29 MB codes + 59 MB bf16 out) cycled: above the MALL
    deq_out = [torch.empty((M, K), dtype=torch.bfloat16, device=dev) for _ in range(n_deq)]

    def dequant(i):
        B.check(B.L.fp8_dequant(a[i % ns].data_ptr(), M, K, K, sa[i % ns].data_ptr(), 0,
                                deq_out[i % n_deq].data_ptr(), 0, K, B.hs))
    deq_us = B.timed_us(dequant)
    out["dequant_1x128_bf16"] = B.quant_rec(M * K * 3 + 4 * M * (K // 128), deq_us, launches=n)
    del deq_out

    # Prior-art per-tensor scalings on the same X: current (two passes) and
    # delayed (one pass, 1024-entry amax history).
    t_scale = torch.empty((1,), dtype=torch.float32, device=dev)
    t_amax = torch.empty((1,), dtype=torch.float32, device=dev)
    t_hist = torch.ones((1024,), dtype=torch.float32, device=dev)

    def tensor_q(i, hist):
        B.check(B.L.fp8_quant_tensor(xs[i % ns].data_ptr(), 0, M, K, K, 0, ctypes.c_double(0.0),
                                     hist.data_ptr() if hist is not None else None, 1024 if hist is not None else 0,
                                     qd.data_ptr(), K, t_scale.data_ptr(), t_amax.data_ptr(), B.hs))
    tc_us = B.timed_us(lambda i: tensor_q(i, None))
    td_us = B.timed_us(lambda i: tensor_q(i, t_hist))
    out["quant_tensor_current"] = B.quant_rec(M * K * 5, tc_us, launches=n,
                                              note="per-tensor scale (prior art): amax pass + code pass")
    out["quant_tensor_delayed"] = B.quant_rec(M * K * 3, td_us, launches=n,
                                              note="per-tensor scale from a 1024-entry amax history")
    return out


def other_workloads(B):
    """The dense FFN, MoE grouped and backward workloads' GEMMs and
    quantizers, each on its exact shapes.  Operands are codes and scales of
    Gaussian bf16 tensors quantized by the library (X ~ N(0,1),
    W ~ N(0,0.02), dY ~ N(0,1e-6)); the MoE expert counts are the
    workload's seeded counts.  Buffer sets rotate past the Infinity Cache."""
    from fp8_block_scaled_05_amd import synth
    torch, dev = B.torch, B.dev
    bf, u8, f32 = torch.bfloat16, torch.uint8, torch.float32
    n_gemm = max(20, B.launches // 2)

    def w_gemm(flops):
        # Untimed launches first, about 30 ms of matrix work (at least 10):
        # the chip's clock goes through a transient of tens of milliseconds
        # under sustained matrix work before it settles.
        return max(10, -(-30000 * 12 // (flops // 10**8)))
    res = {}

    def quantize_pair(x, w, w_t=False):
        a = torch.empty(x.shape, dtype=u8, device=dev)
        sa = torch.empty((x.shape[0], x.shape[1] // 128), dtype=f32, device=dev)
        B.quant_act(x, a, sa)
        b = torch.empty(w.shape, dtype=u8, device=dev)
        sb = torch.empty((w.shape[0] // 128, w.shape[1] // 128), dtype=f32, device=dev)
        bt = torch.empty((w.shape[1], w.shape[0]), dtype=u8, device=dev) if w_t else None
        B.quant_w(w, b, sb, bt)
        return a, sa, b, sb, bt

    def rotate(tensors):
        """Copies of a set of tensors so that all sets together exceed the rotation size."""
        nb = sum(t.numel() * t.element_size() for t in tensors)
        ns = B.n_sets(nb, cap=8)
        return [tensors] + [[t.clone() for t in tensors] for _ in range(ns - 1)]

    # ---- dense FFN: X [8192, 7168] x W [18432, 7168]^T -> Y bf16 [8192, 18432]
    m, n, k = 8192, 18432, 7168
    x = rand_bf16(torch, dev, (m, k), 1.0, 31)
    w = rand_bf16(torch, dev, (n, k), 0.02, 32)
    a, sa, b, sb, _ = quantize_pair(x, w)
    y = torch.empty((m, n), dtype=bf, device=dev)
    sets = rotate([a, sa, b, sb, y])
    us = B.timed_us(lambda i: B.gemm(*sets[i % len(sets)]), n=n_gemm, warm=w_gemm(2 * m * n * k))
    qa = [torch.empty((m, k), dtype=u8, device=dev), torch.empty((m, k // 128), dtype=f32, device=dev)]
    qb = [torch.empty((n, k), dtype=u8, device=dev), torch.empty((n // 128, k // 128), dtype=f32, device=dev)]
    x2, w2 = x.clone(), w.clone()
    qx_us = B.timed_us(lambda i: B.quant_act((x, x2)[i % 2], *qa))
    qw_us = B.timed_us(lambda i: B.quant_w((w, w2)[i % 2], *qb))
    res["ffn_8192x18432x7168"] = {
        "gemm": B.gemm_rec(2 * m * n * k, us, M=m, N=n, K=k, out="bf16", launches=n_gemm,
                           warmup_launches=w_gemm(2 * m * n * k)),
        "quant_x_1x128": B.quant_rec(quant_bytes(m, k, "1x128"), qx_us, shape=[m, k], launches=B.launches),
        "quant_w_128x128": B.quant_rec(quant_bytes(n, k, "128x128"), qw_us, shape=[n, k], launches=B.launches)}
    del x, w, x2, w2, a, sa, b, sb, y, sets, qa, qb
    torch.cuda.empty_cache()

    # ---- MoE grouped: 16 experts, seeded counts, X [32768, 7168], W 16 x [4096, 7168]
    counts = synth.expert_counts()
    off_h = synth.offsets_from_counts(counts)
    m, n, k, g = int(off_h[-1]), 4096, 7168, len(counts)
    off = torch.from_numpy(off_h).to(dev)
    x = rand_bf16(torch, dev, (m, k), 1.0, 41)
    w = rand_bf16(torch, dev, (g * n, k), 0.02, 42)
    a, sa, b, sb, _ = quantize_pair(x, w)
    b, sb = b.view(g, n, k), sb.view(g, n // 128, k // 128)
    y = torch.empty((m, n), dtype=bf, device=dev)
    sets = rotate([a, sa, b, sb, y])
    us = B.timed_us(lambda i: B.grouped(off, *sets[i % len(sets)]), n=n_gemm, warm=w_gemm(2 * m * n * k))
    qx_us = B.timed_us(lambda i: B.quant_act(x, a, sa))
    qw_us = B.timed_us(lambda i: B.quant_w(w, b.view(g * n, k), sb.view(g * n // 128, k // 128)))
    res["moe_grouped_32768x4096x7168_g16"] = {
        "counts": counts.tolist(),
        "gemm": B.gemm_rec(2 * m * n * k, us, M_total=m, N=n, K=k, G=g, out="bf16", launches=n_gemm,
                           warmup_launches=w_gemm(2 * m * n * k)),
        "quant_x_1x128": B.quant_rec(quant_bytes(m, k, "1x128"), qx_us, shape=[m, k], launches=B.launches),
        "quant_w_128x128": B.quant_rec(quant_bytes(g * n, k, "128x128"), qw_us, shape=[g * n, k],
                                       launches=B.launches, note="the 16 expert weights as one call")}
    del x, w, a, sa, b, sb, y, sets
    torch.cuda.empty_cache()

    # ---- backward: dgrad dX = dY W (B = W^T codes), wgrad dW = X^T dY (both 128x1 along tokens)
    t, h, f = 8192, 7168, 2048
    dy = rand_bf16(torch, dev, (t, f), 1e-3, 51)
    x = rand_bf16(torch, dev, (t, h), 1.0, 52)
    w = rand_bf16(torch, dev, (f, h), 0.02, 53)
    g_, sg_, wq, ws, wt = quantize_pair(dy, w, w_t=True)
    wst = ws.t().contiguous()
    y = torch.empty((t, h), dtype=bf, device=dev)
    sets = rotate([g_, sg_, wt, wst, y])
    dgrad_us = B.timed_us(lambda i: B.gemm(*sets[i % len(sets)]), n=n_gemm, warm=w_gemm(2 * t * h * f))
    del sets, y
    xt = torch.empty((h, t), dtype=u8, device=dev)
    sxt = torch.empty((h, t // 128), dtype=f32, device=dev)
    B.quant_act(x, xt, sxt, tiling=1)
    gq = torch.empty((t, f), dtype=u8, device=dev)
    sgq = torch.empty((t, f // 128), dtype=f32, device=dev)
    gt = torch.empty((f, t), dtype=u8, device=dev)
    sgt = torch.empty((f, t // 128), dtype=f32, device=dev)
    B.quant_dual(dy, gq, sgq, gt, sgt)
    dw = torch.empty((h, f), dtype=f32, device=dev)
    sets = rotate([xt, sxt, gt, sgt, dw])
    wgrad_us = B.timed_us(lambda i: B.gemm(*sets[i % len(sets)], kind=1), n=n_gemm, warm=w_gemm(2 * t * h * f))
    del sets
    dys = [dy] + [dy.clone() for _ in range(B.n_sets(t * f * 2 * 3, cap=16) - 1)]
    xs = [x, x.clone()]
    dual_us = B.timed_us(lambda i: B.quant_dual(dys[i % len(dys)], gq, sgq, gt, sgt))
    xt_us = B.timed_us(lambda i: B.quant_act(xs[i % 2], xt, sxt, tiling=1))
    ws_ = [w] + [w.clone() for _ in range(B.n_sets(f * h * 2 * 4, cap=16) - 1)]
    wt_us = B.timed_us(lambda i: B.quant_w(ws_[i % len(ws_)], wq, ws, wt))
    res["backward_8192x7168x2048"] = {
        "dgrad_gemm": B.gemm_rec(2 * t * h * f, dgrad_us, M=t, N=h, K=f, out="bf16",
                                 b="W^T codes from the 128x128 quantizer's transposed copy", launches=n_gemm,
                                 warmup_launches=w_gemm(2 * t * h * f)),
        "wgrad_gemm": B.gemm_rec(2 * h * f * t, wgrad_us, M=h, N=f, K=t, out="f32", b_scales="row",
                                 operands="X^T and dY^T, 128x1 tiles along the tokens", launches=n_gemm,
                                 warmup_launches=w_gemm(2 * t * h * f)),
        "quant_dy_dual": B.quant_rec(quant_bytes(t, f, "dual"), dual_us, shape=[t, f], launches=B.launches,
                                     note="dY 1x128 (dgrad) and 128x1 transposed (wgrad) from one read"),
        "quant_x_128x1_t": B.quant_rec(quant_bytes(t, h, "128x1_t"), xt_us, shape=[t, h], launches=B.launches),
        "quant_w_128x128_t": B.quant_rec(quant_bytes(f, h, "128x128+t"), wt_us, shape=[f, h], launches=B.launches,
                                         note="codes and transposed codes")}
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the quantize + GEMM path needs no collective; see the design notes).",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import fp8_block_scaled_05_amd as fb
    from fp8_block_scaled_05_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    B = Bench(torch, fb, args.launches, args.rotate_mib << 20)

    print(f"[bench] generating linear workload X[{M},{K}] W[{N},{K}]", file=sys.stderr, flush=True)
    inp = synth.workload_inputs(2)
    xbits, wbits = inp["X"], inp["W"]
    x0 = torch.from_numpy(xbits.view(np.int16)).view(torch.bfloat16).to(dev)
    w0 = torch.from_numpy(wbits.view(np.int16)).view(torch.bfloat16).to(dev)
    out_dtype = torch.bfloat16 if args.out == "bf16" else torch.float32
    set_bytes = x0.numel() * 2 + w0.numel() * 2 + M * N * (2 if args.out == "bf16" else 4)
    n_sets = B.n_sets(set_bytes)
    xs = [x0] + [x0.clone() for _ in range(n_sets - 1)]
    ws = [w0] + [w0.clone() for _ in range(n_sets - 1)]
    ys = [torch.empty((M, N), dtype=out_dtype, device=dev) for _ in range(n_sets)]
    a = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sa = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    b = torch.empty((N, K), dtype=torch.uint8, device=dev)
    sb = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)

    step_jobs = [B.batch_jobs([(xs[j], 0, a, sa), (ws[j], 2, b, sb)]) for j in range(n_sets)]

    def step(i):
        """The step's two library calls on the stream: both quantizations in
        one fp8_quant_batch launch, then the GEMM."""
        j = i % n_sets
        B.quant_batch(step_jobs[j])
        B.gemm(a, sa, b, sb, ys[j])

    step(0)
    torch.cuda.synchronize()
    if args.calib_copy:
        src = torch.empty(CALIB_COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Per-kernel figures first: seconds of GPU work, so that the timed steps
    # below run with the chip's clock settled.  (After an idle period the
    # GEMM's clock goes through a transient of tens of milliseconds under
    # sustained matrix work; see the kernel trace in profiles/.)
    qx_bytes, qw_bytes, flops = algorithmic()
    print(f"[bench] timing each kernel over at least {args.launches} back-to-back launches",
          file=sys.stderr, flush=True)
    kernels = linear_kernels(B, xs, ws, out_dtype, qx_bytes, qw_bytes, flops, args.gemm_warmup)
    workloads = None
    if not args.no_workloads:
        print("[bench] timing the other workload shapes", file=sys.stderr, flush=True)
        workloads = other_workloads(B)
        torch.cuda.empty_cache()

    print(f"[bench] warmup {args.warmup} steps, {n_sets} buffer sets "
          f"({n_sets * set_bytes / 2**20:.0f} MiB cycled)", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: exactly `steps` steps between two events on the launch
    # stream, synchronized on both sides.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(B.stream)
    for i in range(args.steps):
        step(i)
    end.record(B.stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    value = flops / (ms_step * 1e-3) / 1e12
    print(f"[bench] {ms_step * 1e3:.1f} us per step", file=sys.stderr, flush=True)

    g = kernels["blockscaled_gemm"]
    gemm_src = os.path.join(ROOT, "fp8_block_scaled_05_amd", "csrc", "gemm.hip")
    sha = hashlib.sha256(open(gemm_src, "rb").read()).hexdigest()
    traffic = TRAFFIC["bytes_per_launch"] if TRAFFIC["gemm_sha256"] == sha else None

    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3",
        "data": "synthetic",
        "config": {"workload": "linear layer: quantize X[4096,7168] 1x128 + W[2048,7168] "
                               "128x128, GEMM Y[4096,2048] with FP32 promotion per 128-K block",
                   "M": M, "N": N, "K": K, "out": args.out, "buffer_sets": n_sets,
                   "value": "2*M*N*K per whole step (both quantizers + GEMM) over the step time"},
        "device": device_info(torch),
        "roofline": {"bound": "mfma", "achieved": g["TFLOP/s"], "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": g["frac_fp8_peak"], "traffic": traffic,
                     "kernel": "blockscaled_gemm", "avg_us": g["avg_us"], "launches": g["launches"],
                     "warmup_launches": g["warmup_launches"],
                     "frac_bf16_peak": g["frac_bf16_peak"],
                     "note": "the exact GEMM runs on the bf16 matrix instructions (2.5 PFLOP/s peak)"},
        "kernels": kernels,
    }
    if workloads is not None:
        result["workloads"] = workloads
    if not args.no_cpu_baseline:
        print(f"[bench] timing the CPU oracle on {args.cpu_rows} rows", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(xbits, wbits, args.cpu_rows)
        if not args.no_workloads:
            print("[bench] timing the CPU oracle on samples of the other workloads", file=sys.stderr, flush=True)
            result["workloads"]["cpu_baseline"] = extra_cpu_baselines()
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
