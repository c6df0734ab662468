"""Seeded synthetic inputs shaped like DeepSeek-V3 layers (hidden 7168, expert width 2048).

This module only draws random numbers and rounds them to bf16; it holds none
of the quantization or GEMM arithmetic, so the HIP path and the CPU oracle can
both take their inputs from it.  No dataset or trained weight is used: these
tensors stand in for real activations and weights with the shapes and value
distributions of the five workloads below.

Every tensor comes from ``numpy.random.default_rng([8, workload, tensor_id])``
(tensor ids: X=0, W=1, dY=2, expert counts=3).  A tensor is drawn as float32
``standard_normal * std``; a fraction of its entries, chosen without
replacement, is multiplied by an outlier factor; the weight of the dense FFN
workload then gets one log-uniform factor 10^U(-2, 1) per 128x128 block; last,
the values are rounded to bf16 (nearest, ties to even).  bf16 tensors are
returned as their uint16 bit patterns.

Workloads (sizes as rows x cols, row-major, K = the contiguous dimension):
  1 tiny:    X [128,512] N(0,1), 0.5% x50;  W [256,512] N(0,0.02)
  2 linear:  X [4096,7168] N(0,1), 0.1% x100;  W [2048,7168] N(0,0.02)
  3 ffn:     X [8192,7168] as 2;  W [18432,7168] N(0,0.02) with block spread
  4 moe:     16 experts; counts ~ multinomial(32768, p), p ~ Dirichlet(0.5)
             with experts 3 and 11 forced empty; X [32768,7168] as 2 (rows
             sorted by expert); W 16 x [4096,7168] N(0,0.02)
  5 backward: dY [8192,2048] N(0,1)*1e-3;  X [8192,7168] as 2;
             W [2048,7168] N(0,0.02)
"""
import numpy as np

X_ID, W_ID, DY_ID, COUNTS_ID = 0, 1, 2, 3

WORKLOADS = {
    1: "tiny: X[128,512] 1x128, W[256,512] 128x128, Y[128,256] fp32",
    2: "linear: X[4096,7168] 1x128, W[2048,7168] 128x128, Y[4096,2048]",
    3: "ffn: X[8192,7168] 1x128, W[18432,7168] 128x128 (block spread), Y[8192,18432]",
    4: "moe: 16 experts, 32768 tokens, X[tokens,7168], W 16x[4096,7168], Y[32768,4096] bf16",
    5: "backward: dgrad dY[8192,2048] x W[2048,7168]; wgrad X^T dY (128x1 along tokens)",
}


def rng_for(workload, tensor_id, sub=None):
    key = [8, workload, tensor_id] if sub is None else [8, workload, tensor_id, sub]
    return np.random.default_rng(key)


def f32_to_bf16_bits(x):
    """Round finite float32 values to bf16 (nearest, ties to even); uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Widen bf16 bit patterns (uint16) to float32, exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rng, shape, std, outlier_frac=0.0, outlier_mult=1.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    x *= np.float32(std)
    if outlier_frac > 0:
        flat = x.reshape(-1)
        k = int(round(outlier_frac * flat.size))
        idx = rng.choice(flat.size, k, replace=False)
        flat[idx] *= np.float32(outlier_mult)
    return f32_to_bf16_bits(x)


def block_spread_bf16(rng, shape, std):
    """N(0, std) with one factor 10^U(-2,1) per 128x128 block."""
    n, k = shape
    x = rng.standard_normal(shape, dtype=np.float32)
    x *= np.float32(std)
    f = (10.0 ** rng.uniform(-2.0, 1.0, size=(n // 128, k // 128))).astype(np.float32)
    x.reshape(n // 128, 128, k // 128, 128)[...] *= f[:, None, :, None]
    return f32_to_bf16_bits(x)


def activation(workload, rows, cols):
    """X of workloads 2-5: N(0,1) with 0.1% outliers x100 (workload 1: 0.5% x50)."""
    if workload == 1:
        return normal_bf16(rng_for(1, X_ID), (rows, cols), 1.0, 0.005, 50.0)
    return normal_bf16(rng_for(workload, X_ID), (rows, cols), 1.0, 0.001, 100.0)


def weight(workload, rows, cols, expert=None):
    rng = rng_for(workload, W_ID, expert)
    if workload == 3:
        return block_spread_bf16(rng, (rows, cols), 0.02)
    return normal_bf16(rng, (rows, cols), 0.02)


def expert_counts(total=32768, experts=16, empty=(3, 11)):
    """Seeded multinomial token counts per expert; some empty, some not %128."""
    rng = rng_for(4, COUNTS_ID)
    p = rng.dirichlet(np.full(experts, 0.5))
    p[list(empty)] = 0.0
    p /= p.sum()
    counts = rng.multinomial(total, p).astype(np.int64)
    assert counts.sum() == total
    assert all(counts[e] == 0 for e in empty)
    assert np.any(counts % 128 != 0)
    return counts


def offsets_from_counts(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


SHAPES = {
    1: dict(M=128, N=256, K=512),
    2: dict(M=4096, N=2048, K=7168),
    3: dict(M=8192, N=18432, K=7168),
    4: dict(M=32768, N=4096, K=7168, G=16),
    5: dict(T=8192, H=7168, F=2048),
}


def workload_inputs(workload):
    """All bf16 inputs of one workload, as uint16 bit arrays (plus offsets)."""
    s = SHAPES[workload]
    if workload in (1, 2, 3):
        return dict(X=activation(workload, s["M"], s["K"]),
                    W=weight(workload, s["N"], s["K"]))
    if workload == 4:
        counts = expert_counts(s["M"], s["G"])
        return dict(X=activation(4, s["M"], s["K"]),
                    W=np.stack([weight(4, s["N"], s["K"], e) for e in range(s["G"])]),
                    counts=counts, offsets=offsets_from_counts(counts))
    if workload == 5:
        return dict(dY=normal_bf16(rng_for(5, DY_ID), (s["T"], s["F"]), 1e-3),
                    X=activation(5, s["T"], s["H"]),
                    W=weight(5, s["F"], s["H"]))
    raise ValueError(f"unknown workload {workload}")


def sample_rows(m, n_rows=512, seed=0, must=()):
    """Seeded sorted row sample of [0, m) that always holds the rows in `must`."""
    rng = np.random.default_rng([8, 99, seed])
    extra = rng.choice(m, size=min(n_rows, m), replace=False)
    rows = np.unique(np.concatenate([np.asarray(list(must), dtype=np.int64), extra]))
    return rows[(rows >= 0) & (rows < m)]
