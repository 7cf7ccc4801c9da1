"""Oracle pins for the number formats (CPU only).

The E2M1 grid and the E4M3 extremes are what the pages print; the rounding
rules are checked against a brute-force nearest search in float64 (a
different computation from the oracle's bracketing in fp32).
"""
import math
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line.split())
    return out


def test_e2m1_grid_matches_page(orc):
    for code, val in _rows("e2m1_grid.txt"):
        v = orc.e2m1_value(int(code))
        assert v == float(val)
        assert math.copysign(1.0, v) == math.copysign(1.0, float(val))


def test_e2m1_gap_ratio(orc):
    grid = [orc.e2m1_value(c) for c in range(8)]
    gaps = np.diff(grid)
    ratio = {r[0]: float(r[1]) for r in _rows("palette_stats.txt")}["gap_ratio"]
    assert gaps.max() / gaps.min() == pytest.approx(ratio, abs=5e-3)


def _e4m3_all(orc):
    return np.array([orc.e4m3_value(b) for b in range(256)], dtype=np.float64)


def test_e4m3_extremes_and_count(orc):
    v = _e4m3_all(orc)
    pos = v[:128]
    fin = pos[np.isfinite(pos)]
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert fin.max() == 448.0                       # Table 1 "6 x 448"
    assert fin[fin > 0].min() == 2.0 ** -9          # Table 1 "0.5 x 2^-9"
    assert np.count_nonzero(fin > 0) == 126
    assert np.all(np.diff(fin) > 0)                 # bytes 0..0x7E ascend
    assert np.all(v[128:255] == -v[0:127])


def test_table1_extremes_and_dynamic_range(orc):
    v = _e4m3_all(orc)
    fin = v[:127]
    smin = fin[fin > 0].min()
    rows = {r[0]: r for r in _rows("table1_formats.txt")}
    ref_range = None
    for name in ("NVFP4", "NVFP4_4over6", "NVINT4", "IF4"):
        _, group, max_elem, max_scale, min_elem, min_log2, rel, _ = rows[name]
        assert int(group) == 16
        if name in ("NVFP4", "IF4"):
            assert orc.e2m1_value(7) * fin.max() == float(max_elem) * float(max_scale)
            assert orc.e2m1_value(1) * smin == float(min_elem) * 2.0 ** int(min_log2)
        rng_ = float(max_elem) * float(max_scale) / (float(min_elem) * 2.0 ** int(min_log2))
        if name == "NVFP4":
            ref_range = rng_
        assert 100.0 * rng_ / ref_range == pytest.approx(float(rel), abs=0.05)


def _nearest_even(v, grid, even_of):
    """Brute force: argmin |v - g| in float64; ties -> the even code."""
    d = np.abs(np.float64(v) - grid.astype(np.float64))
    best = np.flatnonzero(d == d.min())
    if len(best) == 1:
        return int(best[0])
    evens = [int(b) for b in best if even_of(int(b))]
    assert len(evens) == 1
    return evens[0]


def test_e2m1_rne_bruteforce(orc):
    grid = np.array([orc.e2m1_value(c) for c in range(8)])
    rng = np.random.default_rng(0)
    vals = list(rng.uniform(0, 6, 3000).astype(np.float32))
    mids = (grid[:-1] + grid[1:]) / 2
    for m in mids:  # ties and their neighbours
        m32 = np.float32(m)
        vals += [m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(7))]
    vals += [np.float32(g) for g in grid] + [np.float32(1e-30), np.float32(6.0)]
    for v in vals:
        assert orc.e2m1_rne(v) == _nearest_even(v, grid, lambda c: c % 2 == 0), v
    # the tie readings, spelled out
    for v, code in ((0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)):
        assert orc.e2m1_rne(v) == code


def test_e4m3_rne_and_ceil_bruteforce(orc):
    fin = _e4m3_all(orc)[:127]
    rng = np.random.default_rng(1)
    vals = list((2.0 ** rng.uniform(-12, 9.2, 4000)).astype(np.float32))
    mids = (fin[:-1] + fin[1:]) / 2
    for m in mids:
        m32 = np.float32(m)
        vals += [m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e4))]
    vals += [np.float32(f) for f in fin]
    for v in vals:
        want = 0x7E if v >= 448 else _nearest_even(v, fin, lambda b: b % 2 == 0)
        assert orc.e4m3_rne(v) == want, v
        up = np.flatnonzero(fin >= np.float64(v))
        want_c = 0x7E if v >= 448 else int(up[0])
        assert orc.e4m3_ceil(v) == want_c, v
    assert orc.e4m3_rne(0.0) == 0 and orc.e4m3_ceil(0.0) == 0
    assert orc.e4m3_rne(1e6) == 0x7E and orc.e4m3_ceil(449.0) == 0x7E


def test_int4_rne_bruteforce(orc):
    grid = np.arange(8, dtype=np.float64)
    rng = np.random.default_rng(2)
    vals = list(rng.uniform(0, 7, 2000).astype(np.float32)) + [np.float32(k + 0.5) for k in range(7)]
    for v in vals:
        assert orc.int4_rne(v) == _nearest_even(v, grid, lambda c: c % 2 == 0), v


def test_philox_known_answers(orc):
    for r in _rows("philox_kat.txt"):
        ctr = [int(t, 16) for t in r[0:4]]
        key = [int(t, 16) for t in r[4:6]]
        want = [int(t, 16) for t in r[6:10]]
        assert [int(w) for w in orc.philox4x32_10(ctr, key)] == want


def test_uniform16_layout_and_uniformity(orc):
    # eight 16-bit uniforms per Philox call, in word/half order
    w = orc.philox4x32_10([5, 0, 0, 7], [123, 0])
    for j in range(8):
        want = (int(w[j >> 1]) >> (16 * (j & 1))) & 0xFFFF
        assert orc.uniform16(123, 0, 7, 40 + j) == want
    # tag changes the stream
    assert [orc.uniform16(1, 0, 0, i) for i in range(8)] != [orc.uniform16(1, 1, 0, i) for i in range(8)]
    # chi-square on the top 4 bits over 32768 draws
    u = np.array([orc.uniform16(99, 0, 3, i) for i in range(32768)])
    counts = np.bincount(u >> 12, minlength=16)
    chi2 = ((counts - 2048.0) ** 2 / 2048.0).sum()
    assert chi2 < 45.0   # 15 dof, p ~ 1e-4


def test_sr_exact_expectation_matches_closed_form(orc):
    """Enumerate all 65536 uniforms: the SR rule is unbiased and its mean
    squared error is (a - l)(u - a) -- the closed form of the palettes blog,
    section 'The two corners' -- both up to the 2^-16 resolution."""
    grid = np.array([orc.e2m1_value(c) for c in range(8)], dtype=np.float64)
    rng = np.random.default_rng(3)
    vals = [np.float32(v) for v in rng.uniform(0, 6, 12)] + [np.float32(0.3), np.float32(5.9)]
    L = orc.lib()
    for a in vals:
        q = np.array([grid[L.orc_sr_e2m1(float(a), u)] for u in range(65536)])
        j = np.searchsorted(grid, np.float64(a), side="right") - 1
        lo, hi = grid[j], grid[min(j + 1, 7)]
        gap = hi - lo
        assert abs(q.mean() - np.float64(a)) <= gap * 2.0 ** -16 + 1e-12
        closed = (np.float64(a) - lo) * (hi - np.float64(a))
        assert abs(((q - np.float64(a)) ** 2).mean() - closed) <= gap * gap * 2.0 ** -15 + 1e-12
    # values on the grid never move
    for c in range(8):
        assert L.orc_sr_e2m1(float(grid[c]), 0) == c and L.orc_sr_e2m1(float(grid[c]), 65535) == c


def test_sr_e4m3_exact_expectation(orc):
    fin = _e4m3_all(orc)[:127]
    rng = np.random.default_rng(4)
    L = orc.lib()
    for a in (2.0 ** rng.uniform(-11, 8.8, 10)).astype(np.float32):
        q = np.array([fin[L.orc_sr_e4m3(float(a), u)] for u in range(0, 65536)])
        j = np.searchsorted(fin, np.float64(a), side="right") - 1
        gap = fin[j + 1] - fin[j]
        assert abs(q.mean() - np.float64(a)) <= gap * 2.0 ** -16 + 1e-15
