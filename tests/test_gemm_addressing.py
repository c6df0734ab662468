"""Host-side model of the GEMM kernel's global->LDS load addresses.

The kernel's buffer loads are range-checked by the hardware on the VGPR
offset only; the SGPR offset is added afterwards without a check.  These
tests replay the kernel's offset formulas (gemm.hip: the per-row-group
descriptors of load_stage and load_scales) for every lane, wave, row-group
load and K block of tail tiles, and assert that any access that passes the
check lies inside the rows that exist, and that every byte a real row needs
is loaded exactly once.  A negative control shows that the earlier scheme
(row-group term in the SGPR offset, one descriptor per operand) fails.
No GPU is needed.
"""
import itertools

import pytest

# (BM, BN, waves) of the three tile configurations.
CONFIGS = {"large": (256, 128, 8), "small": (128, 128, 4)}


def swz(row):
    return (row & 7) ^ ((row >> 3) & 1)


def stage_accesses(rows, ld, kb_count, nw, loads, old_scheme=False):
    """(row the lane's bytes belong to, byte offset from the tile start) of
    every 16-byte access that passes the range check."""
    out = []
    for v, wave, lane in itertools.product(range(loads), range(nw), range(64)):
        lrow = 8 * wave + (lane >> 3)
        chunk = ((lane & 7) ^ swz(lrow)) << 4
        if old_scheme:
            base, records, voff = 0, rows * ld, lrow * ld + chunk
            extra = 8 * v * nw * ld
        else:
            base = 8 * v * nw * ld
            records = max(rows - 8 * v * nw, 0) * ld
            voff, extra = lrow * ld + chunk, 0
        if voff >= records:          # out of range: reads zero, touches nothing
            continue
        for kb in range(kb_count):
            addr = base + voff + extra + kb * 128
            out.append((lrow + 8 * v * nw, addr))
    return out


@pytest.mark.parametrize("cfg", sorted(CONFIGS))
@pytest.mark.parametrize("ld_extra", [0, 16, 112])
@pytest.mark.parametrize("kb_count", [1, 3])
def test_stage_loads_stay_inside_existing_rows(cfg, ld_extra, kb_count):
    bm, bn, nw = CONFIGS[cfg]
    k = 128 * kb_count
    ld = k + ld_extra
    for tile_rows, loads in ((bm, bm // 8 // nw), (bn, bn // 8 // nw)):
        for rows in sorted({1, 7, 8, 9, 63, 64, 65, 127, 128, 129, tile_rows - 1, tile_rows}):
            if rows > tile_rows:
                continue
            acc = stage_accesses(rows, ld, kb_count, nw, loads)
            seen = set()
            for row, addr in acc:
                assert row < rows
                assert row * ld <= addr and addr + 16 <= row * ld + k, (row, addr)
                assert addr not in seen
                seen.add(addr)
            # every 16-byte piece of every existing row's K range is loaded
            assert len(seen) == rows * (k // 16)


def test_old_scheme_reads_past_the_last_row():
    """The scheme the kernel used before: the row-group term in the SGPR
    offset escapes the check, so a tail tile reads rows that do not exist."""
    bm, _, nw = CONFIGS["large"]
    rows, ld = 100, 7168
    acc = stage_accesses(rows, ld, 1, nw, bm // 8 // nw, old_scheme=True)
    assert any(row >= rows for row, _ in acc)
    assert max(addr for _, addr in acc) + 16 > rows * ld


def lane_row_kb(lane, layout):
    """(row within the wave's 16, K block within the group of 4) that a lane
    loads: A scales lane / 4 and lane % 4; per-row B scales lane % 16 and
    lane / 16 (gemm.hip: voff_s and voff_sb)."""
    if layout == "a":
        return lane >> 2, lane & 3
    return lane & 15, lane >> 4


def scale_accesses(rows, kb_count, nw, loads, layout="a"):
    """(row, K block, byte offset from the tile's first scale, LDS float
    index in the scale group) of every 4-byte scale load that passes the
    range check.  Each wave's load u lands in 64 consecutive floats of the
    group, lane by lane."""
    out = []
    groups = (kb_count + 3) // 4
    for u, wave, lane, g in itertools.product(range(loads), range(nw), range(64), range(groups)):
        base = 16 * u * nw * kb_count * 4
        records = max(rows - 16 * u * nw, 0) * kb_count * 4
        r, k = lane_row_kb(lane, layout)
        voff = ((16 * wave + r) * kb_count + k) * 4 + g * 16
        if voff >= records:
            continue
        out.append((16 * u * nw + 16 * wave + r, 4 * g + k, base + voff, 64 * (u * nw + wave) + lane))
    return out


def lds_index(row, kb, layout):
    """Where the kernel reads the scale of (row, K block) in its group: A
    scales [row][kb % 4]; per-row B scales [row / 16][kb % 4][row % 16]."""
    if layout == "a":
        return 4 * row + (kb & 3)
    return 64 * (row >> 4) + 16 * (kb & 3) + (row & 15)


@pytest.mark.parametrize("cfg", sorted(CONFIGS))
@pytest.mark.parametrize("kb_count", [1, 2, 5, 56])
@pytest.mark.parametrize("layout", ["a", "b_row"])
def test_scale_loads_stay_inside_existing_rows(cfg, kb_count, layout):
    bm, bn, nw = CONFIGS[cfg]
    for tile_rows in ((bm, bn) if layout == "a" else (bn,)):
        loads = tile_rows // 16 // nw
        for rows in sorted({1, 3, 15, 16, 17, 100, tile_rows - 1, tile_rows}):
            needed = set()
            for row, kb, addr, lds in scale_accesses(rows, kb_count, nw, loads, layout):
                assert 0 <= addr and addr + 4 <= rows * kb_count * 4, (row, kb, addr)
                if kb < kb_count:                  # a real scale: it is where it belongs
                    assert row < rows and addr == (row * kb_count + kb) * 4
                    # and the kernel reads it from the LDS slot it landed in
                    assert lds == lds_index(row, kb, layout), (row, kb, lds)
                    needed.add((row, kb))
            assert len(needed) == rows * kb_count


def test_b_row_scale_reads_are_aligned_quads():
    """The per-row B scales a lane needs for one K block and slab (columns
    c .. c + 3, c = 64 wn + 32 j + 8 rq + 4 hk) are one aligned 16-byte run
    of the scale group."""
    for wn, j, rq, hk, kb in itertools.product(range(2), range(2), range(4), range(2), range(4)):
        c = 64 * wn + 32 * j + 8 * rq + 4 * hk
        idx = [lds_index(c + t, kb, "b_row") for t in range(4)]
        assert idx == list(range(idx[0], idx[0] + 4)) and idx[0] % 4 == 0
