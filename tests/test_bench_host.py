"""Host-side checks of bench.py (no GPU): its algorithmic byte and flop
counts for the linear workload (X [4096, 7168], W [2048, 7168]), the
one-GPU-only refusal, and the traffic record's tie to the GEMM source."""
import hashlib
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_algorithmic_counts():
    # Per element: 2 bytes of bf16 in, 1 code out, plus one 4-byte scale per
    # 128 elements (1x128) or per 128x128 elements; 2*M*N*K flops.
    b = _bench()
    qx, qw, flops = b.algorithmic()
    assert qx == 4096 * 7168 * 3 + 4096 * 56 * 4 == 88_997_888
    assert qw == 2048 * 7168 * 3 + 16 * 56 * 4 == 44_043_776
    assert flops == 2 * 4096 * 2048 * 7168 == 120_259_084_288
    assert b.quant_bytes(4096, 7168, "1x128") == qx and b.quant_bytes(2048, 7168, "128x128") == qw
    # the other workloads' quantizers (byte counts of the workload table)
    assert b.quant_bytes(18432, 7168, "128x128") == 396_393_984
    assert b.quant_bytes(8192, 7168, "1x128") == 177_995_776
    assert b.quant_bytes(32768, 7168, "1x128") == 711_983_104
    assert b.quant_bytes(65536, 7168, "128x128") == 1_409_400_832
    assert b.quant_bytes(8192, 2048, "1x128") == 50_855_936
    assert b.quant_bytes(8192, 2048, "dual") == 8192 * 2048 * 4 + 2 * 4 * 8192 * 16
    assert b.quant_bytes(2048, 7168, "128x128+t") == 2048 * 7168 * 4 + 16 * 56 * 4


def test_peaks_are_the_published_ones():
    b = _bench()
    assert (b.PEAK_BF16_TFLOPS, b.PEAK_FP8_TFLOPS, b.PEAK_HBM_GBPS) == (2500.0, 5000.0, 8000.0)


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""


def test_traffic_record_names_its_gemm_source():
    # The stored HBM traffic is reported only while gemm.hip is the source it
    # was measured on; the record names the profile summary it came from.
    b = _bench()
    rec = b.TRAFFIC
    assert len(rec["gemm_sha256"]) == 64 and rec["bytes_per_launch"] > 0
    assert os.path.exists(os.path.join(ROOT, rec["source"]))
    src = os.path.join(ROOT, "fp8_block_scaled_05_amd", "csrc", "gemm.hip")
    current = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if current == rec["gemm_sha256"]:
        # Counters of this source: at least the algorithmic bytes (operands
        # read once, bf16 output written once).
        operands = 4096 * 7168 + 2048 * 7168 + 4 * (4096 * 56 + 16 * 56)
        assert rec["bytes_per_launch"] >= operands + 4096 * 2048 * 2


def test_extra_oracle_samples_run():
    # The oracle leg of --extra-workloads on a reduced sample: every entry
    # names its sample and reports a positive throughput.
    b = _bench()
    res = b.extra_cpu_baselines(shrink=8)
    assert set(res) == {"ffn_8192x18432x7168", "moe_grouped_32768x4096x7168_g16", "backward_dgrad_wgrad"}
    for v in res.values():
        assert v["kind"] == "oracle" and v["unit"] == "TFLOP/s"
        assert v["value"] > 0 and v["seconds"] > 0 and v["sample"]
        assert v["cores"]["quantize"] == 1 and v["cores"]["gemm"] >= 1
        # every stage timed, the estimate scales each one up to the full workload
        assert abs(sum(st["seconds"] for st in v["stages"].values()) - v["seconds"]) < 0.01
        assert all(st["to_full"] >= 1 for st in v["stages"].values())
        assert v["full_workload_seconds_est"] >= v["seconds"]
    assert "X[128,7168]" in res["ffn_8192x18432x7168"]["sample"]
