"""Throughput of the FP8 block-scaled hot path on one MI355X.

One step = online 1x128 quantization of the activations X [4096, 7168] (bf16),
128x128 quantization of the weight W [2048, 7168] (bf16), and the block-scaled
FP8 GEMM Y = X W^T [4096, 2048] with FP32 promotion per 128-deep K block
(bf16 output by default).  Inputs are seeded synthetic tensors shaped like a
DeepSeek-V3 layer (hidden 7168), already resident in HBM; W steps through
several copies and X/Y through several buffers so that more than 1 GiB is
cycled and the 256 MB Infinity Cache cannot serve repeated reads.

Prints one JSON line.  `value` is whole-step throughput in TFLOP/s
(2*M*N*K per step over the measured step time, quantization included); the
`roofline` object covers the dominant kernel (the GEMM) with its average
launch duration from HIP events recorded on the stream the kernels run on,
around each kernel of every 8th timed step (events on every step would add
~10 us of their own to each step's time);
`kernels` gives the same for each kernel, the quantizers as GB/s against HBM;
`cpu_baseline` times the CPU oracle on a bounded sample of the same step.
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
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 (= f16) MFMA (the FP32-accumulating path)
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
METRIC = "FP8 block-scaled GEMM TFLOP/s (% FP8 MFMA peak); quantize GB/s (% HBM)"

# HBM bytes per GEMM launch from two rocprofv3 --pmc runs of
# `bench.py --calib-copy` (FETCH_SIZE, then WRITE_SIZE), each scaled by what
# the same counter reads for the device copy of known size that --calib-copy
# adds; valid only for the GEMM source it was measured on (sha256 of gemm.hip).
TRAFFIC = {"gemm_sha256": "3f6cf08b0c5a964d01f11c467d2f8c9eefbd5444f25db659adcecae7418dfd3f",
           "bytes_per_launch": 137155718,   # 120.38 MB read (FETCH_SIZE x 1.99948) + 16.78 MB written
           "source": "profiles/bench_linear_4096x2048x7168_counters.md"}
CALIB_COPY_BYTES = 128 << 20
# The quantizers' figures come from 50 back-to-back launches on the rotating
# buffers.  Their in-step durations from the sampled steps' events are also
# reported; on kernels this short those include a few microseconds of the
# events' own records (a kernel trace of the same steps, without events, gives
# durations within 2% of the back-to-back ones).
IN_STEP_NOTE = ("avg_us/GB/s/frac_hbm: 50 back-to-back launches on rotating buffers; "
                "in_step_events: sampled steps' events, which add their own few microseconds")


def algorithmic():
    tiles_x = M * (K // 128)
    quant_x_bytes = M * K * 2 + M * K + tiles_x * 4
    quant_w_bytes = N * K * 2 + N * K + (N // 128) * (K // 128) * 4
    gemm_flops = 2 * M * N * K
    return quant_x_bytes, quant_w_bytes, gemm_flops


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--out", choices=["bf16", "f32"], default="bf16")
    p.add_argument("--accum", choices=["fp32", "fp8_mfma"], default="fp32",
                   help="block-partial accumulation of the GEMM (see include/fp8bs.h)")
    p.add_argument("--event-every", type=int, default=8,
                   help="record per-kernel events on every Nth timed step (1 = every step)")
    p.add_argument("--rotate-mib", type=int, default=1100,
                   help="bytes of input/output buffers cycled through (defeats the MALL)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=M,
                   help="rows of X in the oracle's timed sample (default: all)")
    p.add_argument("--extra-workloads", action="store_true",
                   help="also time the GEMMs (and quantizers) of the other workload shapes: dense FFN, "
                        "MoE grouped, dgrad and wgrad (reported under extra_workloads)")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run one device copy of 128 MiB (counter calibration for rocprofv3 --pmc)")
    return p.parse_args()


def cpu_baseline(xbits, wbits, rows):
    """The oracle, as it stands, on the first `rows` rows of X and all of W."""
    import numpy as np
    import oracle
    from fp8_block_scaled_05_amd import synth
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001 - threadpoolctl is optional
        blas_threads = 1
    x = synth.bf16_bits_to_f32(xbits[:rows])
    w = synth.bf16_bits_to_f32(wbits)
    t0 = time.perf_counter()
    a, sa = oracle.quant_1x128(x)
    b, sb = oracle.quant_128x128(w)
    y, _ = oracle.blockscaled_gemm_ref(a, sa, b, sb)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * N * K
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": (f"quantize X[:{rows}] (1x128) + W[{N},{K}] (128x128) + float64 "
                       f"per-128-K-block GEMM with its error bound for {rows} rows; "
                       f"{dt:.2f} s wall; quantizer single-threaded numpy, GEMM on "
                       f"{blas_threads} BLAS threads"),
            "seconds": round(dt, 3),
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0))}


def extra_cpu_baselines(shrink=1):
    """The oracle, as it stands, on bounded samples of the other workloads.

    Each sample is drawn with its workload's recipe (same distributions and
    K; fewer rows), quantized by the oracle and multiplied by its float64
    per-128-K-block reference, so every figure includes quantization.
    Throughput is 2 * rows * cols * K of the sample over its wall time.
    `shrink` divides every row count (the tests use a small sample)."""
    import numpy as np
    import oracle
    from fp8_block_scaled_05_amd import synth
    f32 = synth.bf16_bits_to_f32
    res = {}

    def timed(name, flops, sample, fn):
        t0 = time.perf_counter()
        fn()
        dt = time.perf_counter() - t0
        res[name] = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "kind": "oracle",
                     "sample": sample, "seconds": round(dt, 3)}

    k = 7168
    r1, r2, r4 = 1024 // shrink, 2048 // shrink, 4096 // shrink
    # Dense FFN: 1024 rows of X, 2048 rows (16 row blocks) of the block-spread W.
    x = f32(synth.normal_bf16(synth.rng_for(3, synth.X_ID), (r1, k), 1.0, 0.001, 100.0))
    w = f32(synth.block_spread_bf16(synth.rng_for(3, synth.W_ID), (r2, k), 0.02))

    def ffn():
        a, sa = oracle.quant_1x128(x)
        b, sb = oracle.quant_128x128(w)
        oracle.blockscaled_gemm_ref(a, sa, b, sb)
    timed("ffn_8192x18432x7168", 2.0 * r1 * r2 * k,
          f"X[{r1},7168] 1x128 + W[{r2},7168] 128x128 (block spread) + GEMM {r1}x{r2}x7168", ffn)

    # MoE: one expert's full weight [4096, 7168] and 512 of its tokens.
    x = f32(synth.normal_bf16(synth.rng_for(4, synth.X_ID), (r1 // 2, k), 1.0, 0.001, 100.0))
    w = f32(synth.weight(4, r4, k, expert=0))

    def moe():
        a, sa = oracle.quant_1x128(x)
        b, sb = oracle.quant_128x128(w)
        oracle.grouped_gemm_ref(np.array([0, r1 // 2], np.int32), a, sa, b[None], sb[None])
    timed("moe_grouped_32768x4096x7168_g16", 2.0 * (r1 // 2) * r4 * k,
          f"one expert: X[{r1 // 2},7168] 1x128 + W[{r4},7168] 128x128 + grouped GEMM {r1 // 2}x{r4}x7168", moe)

    # Backward: 1024 tokens.  dgrad dY[1024,2048] x W[2048,7168] (W quantized
    # 128x128, used transposed); wgrad X^T dY with both operands 128x1 along
    # the tokens.
    t, h, f = r1, 7168, 2048
    dy = f32(synth.normal_bf16(synth.rng_for(5, synth.DY_ID), (t, f), 1e-3))
    x = f32(synth.normal_bf16(synth.rng_for(5, synth.X_ID), (t, h), 1.0, 0.001, 100.0))
    w = f32(synth.weight(5, f, h))

    def backward():
        g, sg = oracle.quant_1x128(dy)
        b, sb = oracle.quant_128x128(w)
        oracle.blockscaled_gemm_ref(g, sg, np.ascontiguousarray(b.T), np.ascontiguousarray(sb.T))
        xt, sxt = oracle.quant_128x1_t(x)
        gt, sgt = oracle.quant_128x1_t(dy)
        oracle.blockscaled_gemm_ref(xt, sxt, gt, sgt, "row")
    timed("backward_dgrad_wgrad", 2.0 * (t * h * f) * 2,
          f"{t} tokens: dY 1x128 + W 128x128 + dgrad {t}x7168x2048; X and dY 128x1 + wgrad 7168x2048x{t}", backward)
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


def extra_workloads(L, fb, torch, dev, hs, accum):
    """Time each other workload's kernels on operands of its exact shapes.

    Codes are uniform random E4M3 bytes without NaN, scales uniform in
    [0.5, 1.5), generated on the GPU (the values do not change the work);
    the MoE expert counts are the workload's seeded counts.  Each kernel is
    timed over back-to-back launches with events on the launch stream."""
    from fp8_block_scaled_05_amd import synth
    vp = ctypes.c_void_p

    def codes(*shape):
        return torch.randint(0, 0x7E, shape, dtype=torch.uint8, device=dev)

    def scales(*shape):
        return torch.rand(shape, device=dev) + 0.5

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(torch.cuda.current_stream())
        for _ in range(n):
            fn()
        t1.record(torch.cuda.current_stream())
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / n * 1e3

    def check(st):
        if st:
            raise RuntimeError(fb.last_error())

    out = {}

    def dense(name, m, n, k, kind, ydt, iters):
        a, sa, b = codes(m, k), scales(m, k // 128), codes(n, k)
        sb = scales(n // 128, k // 128) if kind == 0 else scales(n, k // 128)
        y = torch.empty((m, n), dtype=torch.bfloat16 if ydt == 0 else torch.float32, device=dev)
        us = timed(lambda: check(L.fp8_blockscaled_gemm(m, n, k, vp(a.data_ptr()), k, vp(sa.data_ptr()),
                                                        vp(b.data_ptr()), k, vp(sb.data_ptr()), kind,
                                                        vp(y.data_ptr()), ydt, n, accum, hs)), iters)
        out[name] = {"M": m, "N": n, "K": k, "b_scales": "block128" if kind == 0 else "row",
                     "out": "bf16" if ydt == 0 else "f32", "avg_us": round(us, 2),
                     "TFLOP/s": round(2 * m * n * k / us / 1e6, 2)}

    dense("ffn_8192x18432x7168", 8192, 18432, 7168, 0, 0, 10)
    dense("dgrad_8192x7168x2048", 8192, 7168, 2048, 0, 0, 20)
    dense("wgrad_7168x2048x8192", 7168, 2048, 8192, 1, 1, 20)

    counts = synth.expert_counts()
    off_h = synth.offsets_from_counts(counts)
    m, n, k, g = int(off_h[-1]), 4096, 7168, len(counts)
    off = torch.from_numpy(off_h).to(dev)
    a, sa = codes(m, k), scales(m, k // 128)
    b, sb = codes(g, n, k), scales(g, n // 128, k // 128)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    us = timed(lambda: check(L.fp8_blockscaled_grouped_gemm(m, n, k, g, vp(off.data_ptr()), vp(a.data_ptr()),
                                                            vp(sa.data_ptr()), vp(b.data_ptr()),
                                                            vp(sb.data_ptr()), vp(y.data_ptr()), 0, accum,
                                                            hs)), 5)
    out["moe_grouped_32768x4096x7168_g16"] = {"M_total": m, "N": n, "K": k, "G": g,
                                              "counts": counts.tolist(), "avg_us": round(us, 2),
                                              "TFLOP/s": round(2 * m * n * k / us / 1e6, 2)}
    del a, b, y
    # The MoE workload's quantizers: X [32768, 7168] 1x128, the 16 expert
    # weights as one [65536, 7168] 128x128 call.
    x = torch.randn((m, k), device=dev).to(torch.bfloat16)
    q, s1 = torch.empty((m, k), dtype=torch.uint8, device=dev), torch.empty((m, k // 128), device=dev)
    us = timed(lambda: check(L.fp8_quant_act_1x128(vp(x.data_ptr()), 0, m, k, k, 0, vp(q.data_ptr()), k,
                                                   vp(s1.data_ptr()), hs)), 10)
    byt = m * k * 3 + 4 * m * (k // 128)
    out["quant_act_1x128_32768x7168"] = {"avg_us": round(us, 2), "GB/s": round(byt / us / 1e3, 1),
                                         "frac_hbm": round(byt / us / 1e3 / PEAK_HBM_GBPS, 4)}
    del x, q, s1
    w = (torch.randn((g * n, k), device=dev) * 0.02).to(torch.bfloat16)
    q, s2 = torch.empty((g * n, k), dtype=torch.uint8, device=dev), torch.empty((g * n // 128, k // 128), device=dev)
    us = timed(lambda: check(L.fp8_quant_w_128x128(vp(w.data_ptr()), 0, g * n, k, k, vp(q.data_ptr()), k,
                                                   vp(s2.data_ptr()), None, 0, None, hs)), 10)
    byt = g * n * k * 3 + 4 * (g * n // 128) * (k // 128)
    out["quant_w_128x128_65536x7168"] = {"avg_us": round(us, 2), "GB/s": round(byt / us / 1e3, 1),
                                         "frac_hbm": round(byt / us / 1e3 / PEAK_HBM_GBPS, 4)}
    return out


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
    L = fb.lib()

    print(f"[bench] generating linear workload X[{M},{K}] W[{N},{K}]", file=sys.stderr, flush=True)
    inp = synth.workload_inputs(2)
    xbits, wbits = inp["X"], inp["W"]
    x0 = torch.from_numpy(xbits.view(np.int16)).view(torch.bfloat16).to(dev)
    w0 = torch.from_numpy(wbits.view(np.int16)).view(torch.bfloat16).to(dev)
    out_dtype = torch.bfloat16 if args.out == "bf16" else torch.float32
    set_bytes = x0.numel() * 2 + w0.numel() * 2 + M * N * (2 if args.out == "bf16" else 4)
    n_sets = max(1, -(-args.rotate_mib * (1 << 20) // set_bytes))
    xs = [x0] + [x0.clone() for _ in range(n_sets - 1)]
    ws = [w0] + [w0.clone() for _ in range(n_sets - 1)]
    ys = [torch.empty((M, N), dtype=out_dtype, device=dev) for _ in range(n_sets)]
    a = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sa = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    b = torch.empty((N, K), dtype=torch.uint8, device=dev)
    sb = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)

    stream = torch.cuda.current_stream()
    hs = ctypes.c_void_p(stream.cuda_stream)
    vp = ctypes.c_void_p
    ycode = 0 if args.out == "bf16" else 1
    accum = fb._ACCUM[args.accum]

    def step(i):
        """Three library calls on `stream`, with prepared arguments (no per-call checks)."""
        j = i % n_sets
        st = L.fp8_quant_act_1x128(vp(xs[j].data_ptr()), 0, M, K, K, 0, vp(a.data_ptr()), K,
                                   vp(sa.data_ptr()), hs)
        st |= L.fp8_quant_w_128x128(vp(ws[j].data_ptr()), 0, N, K, K, vp(b.data_ptr()), K,
                                    vp(sb.data_ptr()), None, 0, None, hs)
        st |= L.fp8_blockscaled_gemm(M, N, K, vp(a.data_ptr()), K, vp(sa.data_ptr()),
                                     vp(b.data_ptr()), K, vp(sb.data_ptr()), 0,
                                     vp(ys[j].data_ptr()), ycode, N, accum, hs)
        if st:
            raise RuntimeError(fb.last_error())

    step(0)
    torch.cuda.synchronize()
    if args.calib_copy:
        src = torch.empty(CALIB_COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    print(f"[bench] warmup {args.warmup} steps, {n_sets} buffer sets "
          f"({n_sets * set_bytes / 2**20:.0f} MiB cycled)", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: K steps.  Every event_every-th step also records events
    # around each of its kernels on the launch stream (the per-kernel and
    # roofline timings); recording them on every step would add ~10 us of
    # event overhead to each step's time.
    # (The first sampled step is not the first timed step, which follows the
    # synchronization and starts cold.)
    sampled = [i for i in range(args.steps) if i % args.event_every == args.event_every // 2]
    if not sampled:
        sampled = [args.steps - 1]
    ev = {i: [torch.cuda.Event(enable_timing=True) for _ in range(4)] for i in sampled}
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def mark(e, k):
        if e is not None:
            e[k].record(stream)

    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        j = i % n_sets
        e = ev.get(i)
        mark(e, 0)
        if L.fp8_quant_act_1x128(vp(xs[j].data_ptr()), 0, M, K, K, 0, vp(a.data_ptr()), K,
                                 vp(sa.data_ptr()), hs):
            raise RuntimeError(fb.last_error())
        mark(e, 1)
        if L.fp8_quant_w_128x128(vp(ws[j].data_ptr()), 0, N, K, K, vp(b.data_ptr()), K,
                                 vp(sb.data_ptr()), None, 0, None, hs):
            raise RuntimeError(fb.last_error())
        mark(e, 2)
        if L.fp8_blockscaled_gemm(M, N, K, vp(a.data_ptr()), K, vp(sa.data_ptr()),
                                  vp(b.data_ptr()), K, vp(sb.data_ptr()), 0,
                                  vp(ys[j].data_ptr()), ycode, N, accum, hs):
            raise RuntimeError(fb.last_error())
        mark(e, 3)
    end.record(stream)
    torch.cuda.synchronize()

    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    per = np.array([[ev[i][k].elapsed_time(ev[i][k + 1]) for k in range(3)] for i in sampled])
    avg_ms = per.mean(axis=0)
    med_ms = np.median(per, axis=0)
    min_ms = per.min(axis=0)
    qx_bytes, qw_bytes, flops = algorithmic()
    gemm_tflops = flops / (avg_ms[2] * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if args.accum == "fp32" else PEAK_FP8_TFLOPS

    # For context: the other accumulation mode's GEMM on the same codes.
    other = 1 - accum
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(5):
        L.fp8_blockscaled_gemm(M, N, K, vp(a.data_ptr()), K, vp(sa.data_ptr()), vp(b.data_ptr()), K,
                               vp(sb.data_ptr()), 0, vp(ys[0].data_ptr()), ycode, N, other, hs)
    g0.record(stream)
    n_alt = 50
    for i in range(n_alt):
        L.fp8_blockscaled_gemm(M, N, K, vp(a.data_ptr()), K, vp(sa.data_ptr()), vp(b.data_ptr()), K,
                               vp(sb.data_ptr()), 0, vp(ys[i % n_sets].data_ptr()), ycode, N, other, hs)
    g1.record(stream)
    torch.cuda.synchronize()
    alt_us = g0.elapsed_time(g1) / n_alt * 1e3
    # Further kernels of the path, timed on the rotating X buffers with events
    # on the launch stream: the dual-orientation quantizer (1x128 and 128x1
    # transposed from one read) and, for comparison, the 128x1 tiling alone.
    def timed_us(fn, n=50, warm=5):
        for i in range(warm):
            fn(i)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for i in range(n):
            fn(i)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / n * 1e3

    qd = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sd = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    qtd = torch.empty((K, M), dtype=torch.uint8, device=dev)
    std = torch.empty((K, M // 128), dtype=torch.float32, device=dev)

    def dual(i):
        if L.fp8_quant_act_dual(vp(xs[i % n_sets].data_ptr()), 0, M, K, K, vp(qd.data_ptr()), K,
                                vp(sd.data_ptr()), vp(qtd.data_ptr()), M, vp(std.data_ptr()), hs):
            raise RuntimeError(fb.last_error())

    def t128x1(i):
        if L.fp8_quant_act_1x128(vp(xs[i % n_sets].data_ptr()), 0, M, K, K, 1, vp(qtd.data_ptr()), M,
                                 vp(std.data_ptr()), hs):
            raise RuntimeError(fb.last_error())

    n_deq = 4                       # 4 x (29 MB codes + 59 MB bf16 out) cycled: above the MALL
    deq_in = [a.clone() for _ in range(n_deq)]
    deq_out = [torch.empty((M, K), dtype=torch.bfloat16, device=dev) for _ in range(n_deq)]

    def dequant(i):
        if L.fp8_dequant(vp(deq_in[i % n_deq].data_ptr()), M, K, K, vp(sa.data_ptr()), 0,
                         vp(deq_out[i % n_deq].data_ptr()), 0, K, hs):
            raise RuntimeError(fb.last_error())

    # The GEMM with its output quantized 1x128 in the epilogue, against the
    # same result in two launches (float32 GEMM output, then the quantizer).
    yq = torch.empty((M, N), dtype=torch.uint8, device=dev)
    ysc = torch.empty((M, N // 128), dtype=torch.float32, device=dev)
    y32 = torch.empty((M, N), dtype=torch.float32, device=dev)

    def gemm_quant(i):
        if L.fp8_blockscaled_gemm_quant(M, N, K, vp(a.data_ptr()), K, vp(sa.data_ptr()),
                                        vp(b.data_ptr()), K, vp(sb.data_ptr()), 0,
                                        vp(yq.data_ptr()), N, vp(ysc.data_ptr()), accum, hs):
            raise RuntimeError(fb.last_error())

    def gemm_then_quant(i):
        if L.fp8_blockscaled_gemm(M, N, K, vp(a.data_ptr()), K, vp(sa.data_ptr()),
                                  vp(b.data_ptr()), K, vp(sb.data_ptr()), 0,
                                  vp(y32.data_ptr()), 1, N, accum, hs):
            raise RuntimeError(fb.last_error())
        if L.fp8_quant_act_1x128(vp(y32.data_ptr()), 1, M, N, N, 0, vp(yq.data_ptr()), N,
                                 vp(ysc.data_ptr()), hs):
            raise RuntimeError(fb.last_error())

    # Prior-art per-tensor scalings on the same X: current (two passes) and
    # delayed (one pass, 1024-entry amax history).
    t_scale = torch.empty((1,), dtype=torch.float32, device=dev)
    t_amax = torch.empty((1,), dtype=torch.float32, device=dev)
    t_hist = torch.ones((1024,), dtype=torch.float32, device=dev)

    def tensor_current(i):
        if L.fp8_quant_tensor(vp(xs[i % n_sets].data_ptr()), 0, M, K, K, 0, ctypes.c_float(0.0), None, 0,
                              vp(a.data_ptr()), K, vp(t_scale.data_ptr()), vp(t_amax.data_ptr()), hs):
            raise RuntimeError(fb.last_error())

    def tensor_delayed(i):
        if L.fp8_quant_tensor(vp(xs[i % n_sets].data_ptr()), 0, M, K, K, 0, ctypes.c_float(0.0),
                              vp(t_hist.data_ptr()), 1024, vp(a.data_ptr()), K, vp(t_scale.data_ptr()),
                              vp(t_amax.data_ptr()), hs):
            raise RuntimeError(fb.last_error())

    tc_us, td_us = timed_us(tensor_current), timed_us(tensor_delayed)
    gq_us, g2_us = timed_us(gemm_quant), timed_us(gemm_then_quant)
    # The two step quantizers again, back to back (the per-launch events of
    # the step add a few microseconds to kernels this short).
    def quant_x(i):
        if L.fp8_quant_act_1x128(vp(xs[i % n_sets].data_ptr()), 0, M, K, K, 0, vp(a.data_ptr()), K,
                                 vp(sa.data_ptr()), hs):
            raise RuntimeError(fb.last_error())

    def quant_w(i):
        if L.fp8_quant_w_128x128(vp(ws[i % n_sets].data_ptr()), 0, N, K, K, vp(b.data_ptr()), K,
                                 vp(sb.data_ptr()), None, 0, None, hs):
            raise RuntimeError(fb.last_error())

    qx_b2b_us, qw_b2b_us = timed_us(quant_x), timed_us(quant_w)
    dual_us, t128_us, deq_us = timed_us(dual), timed_us(t128x1), timed_us(dequant)
    deq_bytes = M * K * (1 + 2) + 4 * M * (K // 128)
    dual_bytes = M * K * (2 + 1 + 1) + 2 * 4 * M * (K // 128)
    t128_bytes = qx_bytes
    qx_gbps = qx_bytes / (avg_ms[0] * 1e-3) / 1e9
    qw_gbps = qw_bytes / (avg_ms[1] * 1e-3) / 1e9
    value = flops / (ms_step * 1e-3) / 1e12

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
                   "M": M, "N": N, "K": K, "out": args.out, "accum": args.accum,
                   "buffer_sets": n_sets, "kernel_event_steps": len(sampled)},
        "device": device_info(torch),
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / peak, 4),
                     "traffic": traffic},
        "kernels": {
            "quant_act_1x128": {"avg_us": round(qx_b2b_us, 2),
                                "GB/s": round(qx_bytes / qx_b2b_us / 1e3, 1),
                                "frac_hbm": round(qx_bytes / qx_b2b_us / 1e3 / PEAK_HBM_GBPS, 4),
                                "bytes": qx_bytes, "launches": 50,
                                "in_step_events": {"avg_us": round(avg_ms[0] * 1e3, 2),
                                                   "median_us": round(med_ms[0] * 1e3, 2),
                                                   "min_us": round(min_ms[0] * 1e3, 2),
                                                   "GB/s": round(qx_gbps, 1)},
                                "note": IN_STEP_NOTE},
            "quant_w_128x128": {"avg_us": round(qw_b2b_us, 2),
                                "GB/s": round(qw_bytes / qw_b2b_us / 1e3, 1),
                                "frac_hbm": round(qw_bytes / qw_b2b_us / 1e3 / PEAK_HBM_GBPS, 4),
                                "bytes": qw_bytes, "launches": 50,
                                "in_step_events": {"avg_us": round(avg_ms[1] * 1e3, 2),
                                                   "median_us": round(med_ms[1] * 1e3, 2),
                                                   "min_us": round(min_ms[1] * 1e3, 2),
                                                   "GB/s": round(qw_gbps, 1)},
                                "note": IN_STEP_NOTE},
            "blockscaled_gemm": {"accum": args.accum, "mfma": "bf16" if args.accum == "fp32" else "fp8",
                                 "avg_us": round(avg_ms[2] * 1e3, 2), "median_us": round(med_ms[2] * 1e3, 2),
                                 "min_us": round(min_ms[2] * 1e3, 2),
                                 "TFLOP/s": round(gemm_tflops, 2),
                                 "frac_own_peak": round(gemm_tflops / peak, 4),
                                 "frac_fp8_peak": round(gemm_tflops / PEAK_FP8_TFLOPS, 4), "flops": flops},
            "quant_act_dual": {"avg_us": round(dual_us, 2),
                               "GB/s": round(dual_bytes / dual_us / 1e3, 1),
                               "frac_hbm": round(dual_bytes / dual_us / 1e3 / PEAK_HBM_GBPS, 4),
                               "bytes": dual_bytes, "launches": 50,
                               "note": "X 1x128 and 128x1 (transposed) from one read"},
            "quant_act_128x1_t": {"avg_us": round(t128_us, 2),
                                  "GB/s": round(t128_bytes / t128_us / 1e3, 1),
                                  "frac_hbm": round(t128_bytes / t128_us / 1e3 / PEAK_HBM_GBPS, 4),
                                  "bytes": t128_bytes, "launches": 50},
            "dequant_1x128_bf16": {"avg_us": round(deq_us, 2),
                                   "GB/s": round(deq_bytes / deq_us / 1e3, 1),
                                   "frac_hbm": round(deq_bytes / deq_us / 1e3 / PEAK_HBM_GBPS, 4),
                                   "bytes": deq_bytes, "launches": 50},
            "quant_tensor_current": {"avg_us": round(tc_us, 2),
                                     "GB/s": round(M * K * 5 / tc_us / 1e3, 1),
                                     "bytes": M * K * 5, "launches": 50,
                                     "note": "per-tensor scale (prior art): amax pass + code pass"},
            "quant_tensor_delayed": {"avg_us": round(td_us, 2),
                                     "GB/s": round(M * K * 3 / td_us / 1e3, 1),
                                     "bytes": M * K * 3, "launches": 50,
                                     "note": "per-tensor scale from a 1024-entry amax history"},
            "blockscaled_gemm_quant_out": {"accum": args.accum, "avg_us": round(gq_us, 2),
                                           "TFLOP/s": round(flops / (gq_us * 1e-6) / 1e12, 2),
                                           "two_launch_us": round(g2_us, 2), "launches": 50,
                                           "note": "Y quantized 1x128 (E4M3 + scales) in the GEMM "
                                                   "epilogue vs float32 GEMM then the quantizer"},
            "blockscaled_gemm_other_accum": {
                "accum": "fp8_mfma" if args.accum == "fp32" else "fp32", "avg_us": round(alt_us, 2),
                "TFLOP/s": round(flops / (alt_us * 1e-6) / 1e12, 2), "launches": n_alt},
        },
    }
    if args.extra_workloads:
        print("[bench] timing the other workload shapes", file=sys.stderr, flush=True)
        result["extra_workloads"] = extra_workloads(L, fb, torch, dev, hs, accum)
    if not args.no_cpu_baseline:
        print(f"[bench] timing the CPU oracle on {args.cpu_rows} rows", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(xbits, wbits, args.cpu_rows)
        if args.extra_workloads:
            print("[bench] timing the CPU oracle on samples of the other workloads", file=sys.stderr, flush=True)
            result["extra_workloads"]["cpu_baseline"] = extra_cpu_baselines()
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
