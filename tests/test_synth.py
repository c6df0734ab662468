"""The seeded input generator: bf16 rounding, determinism and workload structure."""
import numpy as np

from fp8_block_scaled_05_amd import synth


def test_bf16_rounding_ties_to_even():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20,
                  -2.5, 3.0e38], dtype=np.float32)
    got = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    assert got.tolist()[:5] == [1.0, 1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -2.5]
    assert np.isfinite(got[5])


def test_workload1_deterministic_and_shaped():
    a = synth.workload_inputs(1)
    b = synth.workload_inputs(1)
    assert a["X"].shape == (128, 512) and a["W"].shape == (256, 512)
    assert np.array_equal(a["X"], b["X"]) and np.array_equal(a["W"], b["W"])
    x = synth.bf16_bits_to_f32(a["X"])
    assert np.sum(np.abs(x) > 20) >= 100          # the 0.5% x50 outliers


def test_expert_counts():
    c = synth.expert_counts()
    assert c.sum() == 32768 and c[3] == 0 and c[11] == 0 and np.any(c % 128)
    off = synth.offsets_from_counts(c)
    assert off[0] == 0 and off[-1] == 32768 and np.all(np.diff(off) >= 0)


def test_sample_rows():
    r = synth.sample_rows(1000, 50, must=[0, 999])
    assert r[0] == 0 and r[-1] == 999 and np.all(np.diff(r) > 0)
