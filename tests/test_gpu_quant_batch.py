"""GPU parity of the batched quantizer (fp8_quant_batch): every job's codes
and scales equal the oracle's and, bit for bit, what the single calls write."""
import numpy as np
import pytest

import oracle
from fp8_block_scaled_05_amd import synth
from gpu_util import (banner, inputs, dev_bf16, dev_f32, host, f32, assert_codes_equal,
                      assert_scales_equal)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
fb = pytest.importorskip("fp8_block_scaled_05_amd")


def _same(a, b, what):
    torch.cuda.synchronize()
    assert a.shape == b.shape, what
    if a.dtype == torch.float32:
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), what
    else:
        assert torch.equal(a, b), what


def test_batch_linear_workload2():
    """X [4096, 7168] 1x128 and W [2048, 7168] 128x128 in one launch: the whole
    outputs against the oracle."""
    d = inputs(2)
    banner("batch: workload 2 X 1x128 + W 128x128")
    (qx, sx), (qw, sw) = fb.fp8_quant_batch([(dev_bf16(d["X"]), "1x128"), (dev_bf16(d["W"]), "128x128")])
    torch.cuda.synchronize()
    want_q, want_s = oracle.quant_128x128(f32(d["W"]))
    assert_scales_equal(host(sw), want_s, "W scale")
    assert_codes_equal(host(qw), want_q, "W codes")
    want_q, want_s = oracle.quant_1x128(f32(d["X"]))
    assert_scales_equal(host(sx), want_s, "X scale")
    assert_codes_equal(host(qx), want_q, "X codes")


def test_batch_eight_mixed_jobs_match_single_calls():
    """Eight jobs of both tilings and both input types, ragged row counts,
    an empty job, pitched inputs and outputs with canaries around them."""
    rng = np.random.default_rng(70)
    specs = [("1x128", "bf16", 1, 256), ("128x128", "f32", 256, 384), ("1x128", "f32", 33, 640),
             ("128x128", "bf16", 128, 128), ("1x128", "bf16", 0, 512), ("1x128", "bf16", 1000, 128),
             ("128x128", "bf16", 384, 256), ("1x128", "f32", 129, 1024)]
    jobs, outs, bufs, singles = [], [], [], []
    for i, (tiling, dt, rows, cols) in enumerate(specs):
        x = (rng.standard_normal((rows, cols)) * np.exp2(rng.uniform(-20, 20, (rows, 1)))).astype(np.float32)
        ldx = cols + 16
        xb = torch.zeros((rows, ldx), dtype=torch.bfloat16 if dt == "bf16" else torch.float32, device="cuda")
        xb[:, :cols] = dev_bf16(synth.f32_to_bf16_bits(x)) if dt == "bf16" else dev_f32(x)
        xv = xb[:, :cols]
        ldq = cols + 32
        qbuf = torch.full((rows + 2, ldq), 0xA5, dtype=torch.uint8, device="cuda")
        srows = rows if tiling == "1x128" else rows // 128
        sbuf = torch.full((srows * (cols // 128) + 16,), -5.0, device="cuda")
        q = qbuf[1:rows + 1, :cols]
        s = sbuf[8:8 + srows * (cols // 128)].view(srows, cols // 128)
        jobs.append((xv, tiling))
        outs.append((q, s))
        bufs.append((qbuf, sbuf, rows, cols, srows))
        if tiling == "1x128":
            singles.append(fb.fp8_quant_act_1x128(xv))
        else:
            q1, s1, _, _ = fb.fp8_quant_w_128x128(xv)
            singles.append((q1, s1))
    banner("batch: 8 mixed jobs")
    fb.fp8_quant_batch(jobs, outs)
    torch.cuda.synchronize()
    for i, ((q, s), (q1, s1), (qbuf, sbuf, rows, cols, srows)) in enumerate(zip(outs, singles, bufs)):
        _same(q, q1, f"job {i} codes")
        _same(s, s1, f"job {i} scales")
        qb, sb = host(qbuf), host(sbuf)
        assert np.all(qb[0] == 0xA5) and np.all(qb[-1] == 0xA5) and np.all(qb[:, cols:] == 0xA5), f"job {i}"
        assert np.all(sb[:8] == -5.0) and np.all(sb[8 + srows * (cols // 128):] == -5.0), f"job {i}"
        xv, tiling = jobs[i]
        if rows == 0:
            continue
        xf = host(xv).astype(np.float32) if xv.dtype == torch.float32 else f32(host(xv))
        want_q, want_s = oracle.quant_1x128(xf) if tiling == "1x128" else oracle.quant_128x128(xf)
        assert_scales_equal(host(s), want_s, f"job {i} scale")
        assert_codes_equal(host(q), want_q, f"job {i} codes")


def test_batch_expert_weights_match_one_call():
    """The 16 expert weights of the MoE workload as two batches of eight
    separate tensors give the bytes of one 128x128 call on all of them."""
    w = (torch.randn((16 * 4096, 7168), device="cuda") * 0.02).to(torch.bfloat16)
    banner("batch: 16 expert weights [4096, 7168] in two launches")
    q, s, _, _ = fb.fp8_quant_w_128x128(w)
    for h in range(2):
        parts = [w[(8 * h + e) * 4096:(8 * h + e + 1) * 4096] for e in range(8)]
        res = fb.fp8_quant_batch([(p, "128x128") for p in parts])
        for e, (qe, se) in enumerate(res):
            g = 8 * h + e
            _same(qe, q[g * 4096:(g + 1) * 4096], f"expert {g} codes")
            _same(se, s[g * 32:(g + 1) * 32], f"expert {g} scales")


def test_batch_streaming_store_path_matches_single_call():
    """A 128x128 job above the cached-store size (codes streamed past the
    caches) next to an activation job."""
    w = (torch.randn((28672, 7168), device="cuda") * 0.02).to(torch.bfloat16)   # 205 MB of codes
    x = torch.randn((512, 7168), device="cuda").to(torch.bfloat16)
    banner("batch: 128x128 job above the cached-store threshold")
    (qx, sx), (qw, sw) = fb.fp8_quant_batch([(x, "1x128"), (w, "128x128")])
    q1, s1, _, _ = fb.fp8_quant_w_128x128(w)
    qx1, sx1 = fb.fp8_quant_act_1x128(x)
    _same(qw, q1, "codes")
    _same(sw, s1, "scales")
    _same(qx, qx1, "act codes")
    _same(sx, sx1, "act scales")


def test_batch_errors_write_nothing():
    x = torch.ones((4, 256), dtype=torch.bfloat16, device="cuda")
    q = torch.full((4, 256), 0x11, dtype=torch.uint8, device="cuda")
    s = torch.full((4, 2), -1.0, device="cuda")
    banner("batch: a bad job stops the whole call")
    with pytest.raises(fb.Fp8bsError) as e:
        fb.fp8_quant_batch([(x, "1x128"), (x, "128x128")], [(q, s), (None, None)])
    assert "job 1" in str(e.value)
    torch.cuda.synchronize()
    assert bool((q == 0x11).all()) and bool((s == -1.0).all())
    with pytest.raises(ValueError):
        fb.fp8_quant_batch([(x, "1x128")] * 9)
    assert fb.fp8_quant_batch([]) == []
