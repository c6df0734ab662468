"""The 128x128 and dual-orientation quantizers give each workgroup one
128x128 block up to 65536 blocks; beyond that a workgroup takes several
blocks in turn and loads the next block's input while it works on the
current one.  Quantization is independent per block, so a tensor beyond that
count must give exactly the bytes of its parts, each below it (the one-block
path is checked against the oracle by the other quantizer tests)."""
import pytest

from gpu_util import banner

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
fb = pytest.importorskip("fp8_block_scaled_05_amd")

COLS = 7168
ROWS = 1171 * 128                  # 1171 x 56 = 65576 blocks: more than 65536
SPLIT = 585 * 128                  # parts of 32760 and 32816 blocks


def _bf16(rows, seed, std=1.0):
    g = torch.Generator(device="cuda").manual_seed(seed)
    x = torch.randn((rows, COLS), device="cuda", generator=g) * std
    x[torch.rand((rows, COLS), device="cuda", generator=g) < 1e-3] *= 100
    return x.to(torch.bfloat16)


def _parts():
    return ((0, SPLIT), (SPLIT, ROWS))


def test_w_128x128_transposed_multiblock_matches_parts():
    w = _bf16(ROWS, 11, 0.02)
    banner(f"w 128x128 + transposed, {ROWS}x{COLS} ({ROWS // 128 * COLS // 128} blocks)")
    q, s, qt, st = fb.fp8_quant_w_128x128(w, transpose=True)
    for i, (a, b) in enumerate(_parts()):
        qi, si, qti, sti = fb.fp8_quant_w_128x128(w[a:b], transpose=True)
        torch.cuda.synchronize()
        assert torch.equal(q[a:b], qi), f"part {i} codes"
        assert torch.equal(s[a // 128:b // 128], si), f"part {i} scales"
        assert torch.equal(qt[:, a:b], qti), f"part {i} transposed codes"
        assert torch.equal(st[:, a // 128:b // 128], sti), f"part {i} transposed scales"
        del qi, si, qti, sti


def test_dual_multiblock_matches_parts():
    x = _bf16(ROWS, 12)
    banner(f"act dual, {ROWS}x{COLS} ({ROWS // 128 * COLS // 128} blocks)")
    q, s, qt, st = fb.fp8_quant_act_dual(x)
    for i, (a, b) in enumerate(_parts()):
        qi, si, qti, sti = fb.fp8_quant_act_dual(x[a:b])
        torch.cuda.synchronize()
        assert torch.equal(q[a:b], qi), f"part {i} codes"
        assert torch.equal(s[a:b], si), f"part {i} scales"
        assert torch.equal(qt[:, a:b], qti), f"part {i} transposed codes"
        assert torch.equal(st[:, a // 128:b // 128], sti), f"part {i} transposed scales"
        del qi, si, qti, sti


def test_128x1_t_multiblock_matches_parts():
    x = _bf16(ROWS, 13)
    banner(f"act 128x1_T, {ROWS}x{COLS} ({ROWS // 128 * COLS // 128} blocks)")
    qt, st = fb.fp8_quant_act_1x128(x, tiling="128x1_T")
    for i, (a, b) in enumerate(_parts()):
        qti, sti = fb.fp8_quant_act_1x128(x[a:b], tiling="128x1_T")
        torch.cuda.synchronize()
        assert torch.equal(qt[:, a:b], qti), f"part {i} transposed codes"
        assert torch.equal(st[:, a // 128:b // 128], sti), f"part {i} transposed scales"
        del qti, sti
