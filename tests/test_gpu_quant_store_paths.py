"""The 128x128 and dual-orientation quantizers write their codes with ordinary
stores when all the codes of a call fit well inside the Infinity Cache (up to
192 MB) and with nontemporal stores above that.  Quantization is independent
per tile and block, so a tensor above that size must give exactly the bytes
of its parts, each quantized below it (the parts' path is checked against
the oracle by the other quantizer tests)."""
import pytest

from gpu_util import banner

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
fb = pytest.importorskip("fp8_block_scaled_05_amd")

COLS = 7168


def _bf16(rows, seed, std=1.0):
    g = torch.Generator(device="cuda").manual_seed(seed)
    x = torch.randn((rows, COLS), device="cuda", generator=g) * std
    x[torch.rand((rows, COLS), device="cuda", generator=g) < 1e-3] *= 100
    return x.to(torch.bfloat16)


def test_w_128x128_large_matches_halves():
    rows = 28672   # 205.5 MB of codes; each half 102.8 MB
    w = _bf16(rows, 1, 0.02)
    banner(f"w 128x128 store paths {rows}x{COLS}")
    q, s, _, _ = fb.fp8_quant_w_128x128(w)
    h = rows // 2
    q0, s0, _, _ = fb.fp8_quant_w_128x128(w[:h])
    q1, s1, _, _ = fb.fp8_quant_w_128x128(w[h:])
    torch.cuda.synchronize()
    assert torch.equal(q[:h], q0) and torch.equal(q[h:], q1)
    assert torch.equal(s[:h // 128], s0) and torch.equal(s[h // 128:], s1)


def test_w_128x128_transposed_large_matches_quarters():
    rows = 28672   # codes and transposed codes 411 MB; each quarter 103 MB
    w = _bf16(rows, 2, 0.02)
    banner(f"w 128x128 + transposed store paths {rows}x{COLS}")
    q, s, qt, st = fb.fp8_quant_w_128x128(w, transpose=True)
    r4 = rows // 4
    for i in range(4):
        qi, si, qti, sti = fb.fp8_quant_w_128x128(w[i * r4:(i + 1) * r4], transpose=True)
        torch.cuda.synchronize()
        assert torch.equal(q[i * r4:(i + 1) * r4], qi), f"quarter {i} codes"
        assert torch.equal(s[i * r4 // 128:(i + 1) * r4 // 128], si), f"quarter {i} scales"
        assert torch.equal(qt[:, i * r4:(i + 1) * r4], qti), f"quarter {i} transposed codes"
        assert torch.equal(st[:, i * r4 // 128:(i + 1) * r4 // 128], sti), f"quarter {i} transposed scales"


def test_dual_large_matches_halves():
    rows = 14336   # both outputs 205.5 MB; each half 102.8 MB
    x = _bf16(rows, 3)
    banner(f"act dual store paths {rows}x{COLS}")
    q, s, qt, st = fb.fp8_quant_act_dual(x)
    h = rows // 2
    for i in range(2):
        qi, si, qti, sti = fb.fp8_quant_act_dual(x[i * h:(i + 1) * h])
        torch.cuda.synchronize()
        assert torch.equal(q[i * h:(i + 1) * h], qi), f"half {i} codes"
        assert torch.equal(s[i * h:(i + 1) * h], si), f"half {i} scales"
        assert torch.equal(qt[:, i * h:(i + 1) * h], qti), f"half {i} transposed codes"
        assert torch.equal(st[:, i * h // 128:(i + 1) * h // 128], sti), f"half {i} transposed scales"


def test_128x1_t_large_matches_halves():
    rows = 28672   # 205.5 MB of transposed codes; each half 102.8 MB
    x = _bf16(rows, 4)
    banner(f"act 128x1_T store paths {rows}x{COLS}")
    qt, st = fb.fp8_quant_act_1x128(x, tiling="128x1_T")
    h = rows // 2
    for i in range(2):
        qti, sti = fb.fp8_quant_act_1x128(x[i * h:(i + 1) * h], tiling="128x1_T")
        torch.cuda.synchronize()
        assert torch.equal(qt[:, i * h:(i + 1) * h], qti), f"half {i} transposed codes"
        assert torch.equal(st[:, i * h // 128:(i + 1) * h // 128], sti), f"half {i} transposed scales"
