"""Host-side model of the GEMM's workgroup -> tile walk (gemm.hip: tile_of
and locate_tile), checked without a GPU.

- Dense: the XCD-aware renumbering followed by the kGroupM-high walk is a
  bijection from the workgroups onto the (M tile, N tile) grid for every
  grid shape, and each XCD (workgroup i runs on XCD i % 8) receives one
  contiguous range of the walk.
- Grouped: for any offset table, valid or not, the clamped group ranges are
  disjoint and inside [0, M], the launch's upper bound ceil(M / BM) + G on
  the M tiles is never exceeded, and every row of every group lies in
  exactly one tile of that group.  The kernel finds a tile's group with a
  64-lane search (prefix maximum of the clamped offsets, prefix sum of the
  tile counts); its model returns the same group and rows as the one-group-
  at-a-time rule for every tile, also with more than 64 groups.
"""
import numpy as np
import pytest

GROUP_M = 4


def tile_of(wg, n_wg, tiles_m, tiles_n):
    q, r = n_wg >> 3, n_wg & 7
    x = wg & 7
    wg = x * q + min(x, r) + (wg >> 3)
    per_group = GROUP_M * tiles_n
    g = wg // per_group
    first_m = g * GROUP_M
    gm = min(tiles_m - first_m, GROUP_M)
    in_g = wg - g * per_group
    return first_m + in_g % gm, in_g // gm, wg


@pytest.mark.parametrize("tiles_m", [1, 2, 3, 4, 5, 7, 16, 17, 32, 33, 56])
@pytest.mark.parametrize("tiles_n", [1, 2, 3, 8, 16, 31, 144])
def test_dense_walk_is_a_bijection_with_contiguous_xcd_ranges(tiles_m, tiles_n):
    n_wg = tiles_m * tiles_n
    seen = set()
    walk_of_xcd = {}
    for wg in range(n_wg):
        tm, tn, w = tile_of(wg, n_wg, tiles_m, tiles_n)
        assert 0 <= tm < tiles_m and 0 <= tn < tiles_n
        seen.add((tm, tn))
        walk_of_xcd.setdefault(wg % 8, []).append(w)
    assert len(seen) == n_wg
    ranges = sorted((min(v), max(v), len(v)) for v in walk_of_xcd.values())
    for lo, hi, n in ranges:
        assert hi - lo + 1 == n, "an XCD's share of the walk is not contiguous"
    for (_, hi, _), (lo2, _, _) in zip(ranges, ranges[1:]):
        assert lo2 == hi + 1


def group_tiles(off, m, bm):
    """locate_tile's clamped ranges: [(lo, hi, tile count)] per group."""
    out, prev_hi = [], 0
    for g in range(len(off) - 1):
        lo = max(prev_hi, min(int(off[g]), m))
        hi = max(lo, min(int(off[g + 1]), m))
        prev_hi = hi
        out.append((lo, hi, (hi - lo + bm - 1) // bm))
    return out


def locate(tm, ranges, bm):
    vm = tm
    for g, (lo, hi, cnt) in enumerate(ranges):
        if vm < cnt:
            return g, lo + vm * bm, hi
        vm -= cnt
    return None


def _tables():
    rng = np.random.default_rng(12)
    tables = [
        ([0, 100, 100, 400, 640], 640),              # valid, one empty group
        ([0, 200, 100, 900, -5, 300], 300),          # decreasing, negative, past M
        ([0, 0, 0], 10),                             # all empty, rows left over
        ([5, 5, 300], 300),                          # rows before the first offset
        ([0, 255, 256, 257, 513], 513),
    ]
    for _ in range(40):
        g = int(rng.integers(1, 20))
        m = int(rng.integers(1, 3000))
        if rng.random() < 0.5:
            cuts = np.sort(rng.integers(0, m + 1, size=g - 1))
            off = [0, *cuts.tolist(), m]
        else:
            off = rng.integers(-50, m + 50, size=g + 1).tolist()
        tables.append((off, m))
    return tables


@pytest.mark.parametrize("bm", [128, 256])
@pytest.mark.parametrize("off,m", _tables())
def test_grouped_walk_covers_every_group_row_once(off, m, bm):
    g_count = len(off) - 1
    ranges = group_tiles(off, m, bm)
    prev = 0
    for lo, hi, _ in ranges:
        assert prev <= lo <= hi <= m
        prev = hi
    tiles_m = (m + bm - 1) // bm + g_count          # the launch's bound
    assert sum(c for _, _, c in ranges) <= tiles_m
    covered = np.zeros(m, dtype=np.int64)
    for tm in range(tiles_m):
        hit = locate(tm, ranges, bm)
        if hit is None:
            continue
        g, row0, row_end = hit
        lo, hi, _ = ranges[g]
        assert lo <= row0 < hi and row_end == hi
        covered[row0:min(row0 + bm, row_end)] += 1
    want = np.zeros(m, dtype=np.int64)
    for lo, hi, _ in ranges:
        want[lo:hi] = 1
    assert (covered == want).all()
    if all(0 <= a <= b for a, b in zip(off, off[1:])) and off[0] == 0 and off[-1] == m:
        assert covered.all(), "a valid table must cover every row"


def test_walk_without_the_remainder_term_is_caught():
    """Negative control: dropping the min(x, r) term of the renumbering (the
    first r XCDs take one extra workgroup when n_wg % 8 != 0) makes two
    workgroups share a tile, which the bijection check above detects."""
    tiles_m, tiles_n = 5, 3
    n_wg = tiles_m * tiles_n
    q = n_wg >> 3
    seen = set()
    for wg in range(n_wg):
        w = (wg & 7) * q + (wg >> 3)
        per_group = GROUP_M * tiles_n
        g = w // per_group
        gm = min(tiles_m - g * GROUP_M, GROUP_M)
        in_g = w - g * per_group
        seen.add((g * GROUP_M + in_g % gm, in_g // gm))
    assert len(seen) < n_wg


def wave_locate(tm, off, m, bm):
    """The kernel's search, 64 groups per step (lane l takes group g0 + l):
    (group, first row, end row) of virtual M tile tm, or None."""
    g_count = len(off) - 1
    vm, run = tm, 0
    for g0 in range(0, g_count, 64):
        real = [g0 + l < g_count for l in range(64)]
        cg = [min(max(off[g0 + l], 0), m) if real[l] else 0 for l in range(64)]
        cn = [min(max(off[g0 + l + 1], 0), m) if real[l] else 0 for l in range(64)]
        pm = list(np.maximum.accumulate(cg))
        lo = [max(run, p) for p in pm]
        hi = [max(lo[l], cn[l]) for l in range(64)]
        cnt = [(hi[l] - lo[l] + bm - 1) // bm if real[l] else 0 for l in range(64)]
        ps = list(np.cumsum(cnt))
        hits = [l for l in range(64) if vm < ps[l]]
        if hits:
            l = hits[0]
            return g0 + l, lo[l] + (vm - (ps[l] - cnt[l])) * bm, hi[l]
        vm -= ps[63]
        run = hi[63]
    return None


def _many_group_tables():
    rng = np.random.default_rng(21)
    out = []
    for _ in range(12):
        g = int(rng.integers(60, 300))
        m = int(rng.integers(1, 20000))
        if rng.random() < 0.5:
            cuts = np.sort(rng.integers(0, m + 1, size=g - 1))
            out.append(([0, *cuts.tolist(), m], m))
        else:
            out.append((rng.integers(-50, m + 50, size=g + 1).tolist(), m))
    return out


@pytest.mark.parametrize("bm", [128, 256])
@pytest.mark.parametrize("off,m", _tables() + _many_group_tables())
def test_wave_search_matches_the_sequential_rule(off, m, bm):
    ranges = group_tiles(off, m, bm)
    tiles_m = (m + bm - 1) // bm + len(off) - 1
    for tm in range(tiles_m):
        assert wave_locate(tm, off, m, bm) == locate(tm, ranges, bm), tm
