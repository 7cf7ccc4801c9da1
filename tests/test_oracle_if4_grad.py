"""Oracle pins for IF4 in the backward pass: IF4 with stochastic rounding and
IF4 with MS-EDEN (IF4 page, Figure 4: IF4 also lowers the error of the
gradient quantizers, more so with MS-EDEN).  CPU only.  Each check rests on
something other than the oracle's own formulas: exact enumeration of the
16-bit uniforms, Monte Carlo against the known mean, Haar-random rotations,
float64 brute force over both branches, or a comparison with the plain
NVFP4 quantizers whose own pins are elsewhere.
"""
import numpy as np
import pytest

from nvfp4_bit_block_amd import synth

def _grids(orc):
    f = np.array([orc.e2m1_value(c) for c in range(8)], dtype=np.float64)
    return f, np.arange(8, dtype=np.float64)


def _e4(orc):
    return np.array([orc.e4m3_value(b) for b in range(128)], dtype=np.float64)


def _sr_exact(y, grid):
    """Exact expected squared error (grid units) of the library's SR rule
    'up iff u16 < p * 65536' over all 65536 uniforms: ceil(p * 65536) of
    them round up.  float64, elementwise."""
    y = np.asarray(y, dtype=np.float64)
    top = grid[-1]
    j = np.clip(np.searchsorted(grid, y, side="right") - 1, 0, len(grid) - 2)
    lo, hi = grid[j], grid[j + 1]
    p = np.where(y >= top, 0.0, (y - lo) / (hi - lo))
    n_up = np.ceil(p * 65536.0)
    pu = n_up / 65536.0
    return np.where(y >= top, 0.0, pu * (hi - y) ** 2 + (1 - pu) * (y - lo) ** 2)


def _branch(orc, z, ts, top, grid, e4):
    """The SR candidate of one block in float64: scale rounded up from
    (a/top)/s_t in fp32 as the method does, y, and exact expected SSE."""
    a = np.float32(np.abs(z).max())
    e = orc.e4m3_ceil(np.float32(np.float32(a / np.float32(top)) / np.float32(ts)))
    S = np.float64(np.float32(np.float32(e4[e]) * np.float32(ts)))
    if e == 0:
        return e, S, np.zeros(16), 0.0
    y = np.minimum(np.abs(z.astype(np.float64)) / S, top)
    return e, S, y, S * S * float(_sr_exact(y, grid).sum())


def test_sr_expected_error_closed_form_against_enumeration(orc):
    """The closed form (y - l)(u - y) the IF4 SR choice uses, on both grids,
    equals the exact enumeration over the 65536 uniforms within their
    2^-16 granularity; literal enumeration through the oracle's own SR rule
    agrees with the counting formula on a few points."""
    f, i = _grids(orc)
    rng = np.random.default_rng(31)
    for grid, is_int in ((f, False), (i, True)):
        y = np.concatenate([rng.uniform(0, grid[-1], 4000), grid, grid[:-1] + 1e-3])
        y32 = y.astype(np.float32)
        closed = np.array([orc.sr_expected_sq(v, is_int) for v in y32], dtype=np.float64)
        exact = _sr_exact(y32, grid)
        gap = np.diff(grid).max()
        assert np.all(np.abs(closed - exact) <= gap * gap * 2.0 ** -16 + 1e-7)
    # literal enumeration (E2M1 via the oracle's SR rule) for three values
    for v in (np.float32(0.3), np.float32(2.7), np.float32(4.9)):
        codes = np.array([orc.sr_e2m1(v, u) for u in range(65536)])
        err = ((f[codes] - np.float64(v)) ** 2).mean()
        assert err == pytest.approx(float(_sr_exact(v, f)), rel=1e-12)


def test_if4_sr_choice_is_the_smaller_exact_expectation(orc):
    """Per 16-group IF4-SR keeps the branch (E2M1 under the rounded-up scale
    of a/6, or integers under that of a/7) whose exact expected squared
    error is the smaller: checked in float64 against the enumeration of the
    uniforms, wherever the two differ by more than the 2^-16 granularity."""
    x = synth.weight(48, 256, seed=21)
    x[:8] = synth.gaussian(8, 256, seed=22)
    q = orc.quantize(x, fmt=orc.FMT_IF4, rounding=orc.SR, seed=3)
    ts = q["ts"]
    assert ts == np.float32(np.float32(np.abs(x).max()) / np.float32(2688.0))
    f, i = _grids(orc)
    e4 = _e4(orc)
    n_int = decided = 0
    for r in range(x.shape[0]):
        for b in range(x.shape[1] // 16):
            z = x[r, 16 * b:16 * b + 16]
            ef, Sf, _, Ef = _branch(orc, z, ts, 6.0, f, e4)
            ei, Si, _, Ei = _branch(orc, z, ts, 7.0, i, e4)
            byte = int(q["scales"][r, b])
            flag = byte >> 7
            assert (byte & 0x7F) == (ei if flag else ef)
            n_int += flag
            tol = 16 * (Sf * Sf * 4.0 + Si * Si) * 2.0 ** -16 + 1e-30
            if abs(Ef - Ei) > tol:
                decided += 1
                assert flag == int(Ei < Ef)
    assert 0 < n_int < x.size // 16
    assert decided > 0.9 * (x.size // 16)


def test_if4_sr_never_worse_than_nvfp4_sr(orc):
    """The FP4 branch of IF4-SR is NVFP4 SR at the same tensor scale, so the
    expected error of every block is at most NVFP4 SR's; and over many
    streams the measured error is lower (IF4 page, Figure 4)."""
    x = synth.weight(32, 256, seed=23)
    qi = orc.quantize(x, fmt=orc.FMT_IF4, rounding=orc.SR)
    qn = orc.quantize(x, rounding=orc.SR)
    assert qi["ts"] == qn["ts"]
    f, i = _grids(orc)
    e4 = _e4(orc)
    for r in range(x.shape[0]):
        for b in range(x.shape[1] // 16):
            z = x[r, 16 * b:16 * b + 16]
            _, _, _, En = _branch(orc, z, qn["ts"], 6.0, f, e4)
            flag = qi["scales"][r, b] >> 7
            _, _, _, Ei = _branch(orc, z, qi["ts"], 7.0 if flag else 6.0, i if flag else f, e4)
            assert Ei <= En * (1 + 1e-6) + 16 * En * 2.0 ** -16 + 1e-30
    mi = mn = 0.0
    for t in range(8):
        for fmt, acc in ((orc.FMT_IF4, "i"), (orc.FMT_NVFP4, "n")):
            q = orc.quantize(x, fmt=fmt, rounding=orc.SR, seed=1, stream=t)
            e = float(np.mean((orc.dequantize(q["codes"], q["scales"], q["ts"], fmt=fmt) - x) ** 2))
            if acc == "i":
                mi += e
            else:
                mn += e
    assert mi < 0.9 * mn


def test_if4_sr_mc_unbiased(orc):
    """Mean over 400 Philox streams of the dequantized IF4-SR tensor is x
    (heavy-tailed weight-like rows, both branches occurring), to the
    precision the per-element closed-form variance S^2 (y - l)(u - y)
    predicts; the scales and the branch choice do not depend on the stream."""
    x = synth.weight(16, 256, seed=24)
    T = 400
    acc = np.zeros(x.shape)
    for t in range(T):
        q = orc.quantize(x, fmt=orc.FMT_IF4, rounding=orc.SR, seed=9, stream=t)
        if t == 0:
            scales0 = q["scales"].copy()
        assert np.array_equal(q["scales"], scales0)
        acc += orc.dequantize(q["codes"], q["scales"], q["ts"], fmt=orc.FMT_IF4).astype(np.float64)
    flags = np.repeat(scales0 >> 7, 16, axis=1).astype(bool)
    assert 0 < np.count_nonzero(flags) < flags.size
    f, i = _grids(orc)
    e4 = _e4(orc)
    S = e4[np.repeat(scales0 & 0x7F, 16, axis=1)] * np.float64(q["ts"])
    y = np.abs(x) / S
    var = S * S * np.where(flags, _sr_exact(np.minimum(y, 7.0), i), _sr_exact(np.minimum(y, 6.0), f))
    bias = acc / T - x
    se = np.sqrt(var / T)
    assert abs(bias.sum()) < 5 * np.sqrt((var / T).sum()) + 1e-9
    # elementwise: within 6 standard errors, plus the 2^-16 granularity of
    # the uniforms (an element one ulp above a level rounds up with
    # probability 2^-16, possibly never in T draws)
    assert np.all(np.abs(bias) <= 6 * se + S * 2.0 ** -16 + 4.0 * S / T)


def test_if4_sr_grid_blocks_are_exact(orc):
    """A block of integers under an exact scale is coded by the INT branch
    with zero error, whatever the random stream; a block of E2M1 values by
    the FP4 branch."""
    ts = np.float32(1.0 / 32)   # every block's scale (a/6 or a/7) / s_t is an E4M3 value
    ints = np.array([7, 6, 5, 4, 3, 2, 1, 0, -1, -2, -3, -4, -5, -6, -7, 0], np.float32)
    fp = np.array([6, 4, 3, 2, 1.5, 1, 0.5, 0, -6, -4, -3, -2, -1.5, -1, -0.5, 0], np.float32)
    x = np.stack([ints, fp, ints * np.float32(0.25), fp * np.float32(8)])
    for t in range(5):
        q = orc.quantize(x, fmt=orc.FMT_IF4, rounding=orc.SR, seed=4, stream=t, ts_in=float(ts))
        assert list(q["scales"][:, 0] >> 7) == [1, 0, 1, 0]
        d = orc.dequantize(q["codes"], q["scales"], q["ts"], fmt=orc.FMT_IF4)
        assert np.array_equal(d, x)


# ------------------------------------------------------------------ IF4 with MS-EDEN
def _haar(n, rng):
    g = rng.standard_normal((n, n))
    qm, r = np.linalg.qr(g)
    return qm * np.sign(np.diag(r))[None, :]


@pytest.mark.parametrize("group", [128, 16])
def test_if4_mseden_unbiased_under_haar_rotation(orc, group):
    """EDEN's guarantee holds for any deterministic coding of the group,
    so also for IF4's per-block choice: with uniformly random rotations the
    estimate's projection on x is 1 (RTN IF4 is the biased control)."""
    rng = np.random.default_rng(41)
    x = rng.standard_normal(128)
    x[7] = -5.0
    T = 3000
    Qs = np.stack([_haar(128, rng) for _ in range(T)])
    Z = np.einsum("tij,j->ti", Qs, x).astype(np.float32)
    q = orc.quantize(Z, fmt=orc.FMT_IF4, rounding=orc.MSEDEN, eden_group=group, seed=5, stream=group)
    assert 0 < np.count_nonzero(q["scales"] >> 7) < q["scales"].size
    zh = orc.dequantize(q["codes"], q["scales"], q["ts"], fmt=orc.FMT_IF4).astype(np.float64)
    r = orc.quantize(Z, fmt=orc.FMT_IF4)
    zr = orc.dequantize(r["codes"], r["scales"], r["ts"], fmt=orc.FMT_IF4).astype(np.float64)
    nx = x @ x
    pe = np.einsum("tij,ti->tj", Qs, zh) @ x / nx
    pr = np.einsum("tij,ti->tj", Qs, zr) @ x / nx
    assert abs(pe.mean() - 1.0) < 4 * pe.std() / np.sqrt(T)
    assert abs(pr.mean() - 1.0) > 4 * pr.std() / np.sqrt(T)


def test_if4_mseden_rht_mc_unbiased_on_gradient_slice(orc):
    """Monte Carlo over randomized Hadamard rotations (signs and streams
    redrawn per trial) on the 64x128 gradient slice: projection 1."""
    x, _ = synth.gradient(256, 256, seed=1)
    x = x[:64, :128].copy()
    T = 300
    acc = np.zeros(x.shape)
    for t in range(T):
        w = orc.signs_words(synth.mc_signs(t))
        q = orc.quantize(x, fmt=orc.FMT_IF4, rounding=orc.MSEDEN, rht_on=True, signs_w=w, seed=1, stream=t)
        acc += orc.dequantize(q["codes"], q["scales"], q["ts"], fmt=orc.FMT_IF4, inv_signs_w=w)
    nx = float((x.astype(np.float64) ** 2).sum())
    pe = float((acc / T * x).sum()) / nx
    assert abs(pe - 1.0) < 1.5e-3


def test_if4_mseden_choice_is_bruteforce_minimum(orc):
    """Each block keeps the branch with the smaller squared error at its
    exact scale (a/6 on the E2M1 grid, a/7 on the integers), each branch
    coded elementwise to the nearest level (float64 brute force); the
    target scale is the kept scale times the group's correction."""
    x = synth.gaussian(16, 256, seed=42)
    q = orc.quantize(x, fmt=orc.FMT_IF4, rounding=orc.MSEDEN, want_tb=True)
    f, i = _grids(orc)
    d_flag = q["scales"] >> 7
    for r in range(x.shape[0]):
        for g in range(x.shape[1] // 128):
            zg = x[r, 128 * g:128 * g + 128].astype(np.float64)
            rec = np.zeros(128)
            s_keep = np.zeros(8)
            for b in range(8):
                z = zg[16 * b:16 * b + 16]
                a = np.abs(z).max()
                sse, recs, sc = {}, {}, {}
                for name, grid, top in (("fp", f, 6.0), ("int", i, 7.0)):
                    s = a / top
                    y = np.abs(z) / s
                    recs[name] = np.sign(z) * grid[np.argmin(np.abs(y[:, None] - grid[None, :]), axis=1)] * s
                    sse[name] = ((z - recs[name]) ** 2).sum()
                    sc[name] = s
                k = "int" if d_flag[r, 8 * g + b] else "fp"
                other = "fp" if k == "int" else "int"
                assert sse[k] <= sse[other] * (1 + 1e-5) + 1e-30
                rec[16 * b:16 * b + 16] = recs[k]
                s_keep[b] = sc[k]
            c = (zg @ zg) / (zg @ rec)
            np.testing.assert_allclose(q["tb"][r, 8 * g:8 * g + 8], s_keep * c, rtol=2e-6)


def test_if4_lowers_gradient_error_with_sr_and_mseden(orc):
    """IF4 page, Figure 4: in the backward pass IF4 improves on NVFP4 with
    SR, and with MS-EDEN.  On the contaminated gradient under the rotation
    both IF4 variants have lower error than their NVFP4 counterparts, and
    IF4 MS-EDEN stays more than 2x below IF4 SR (QII abstract's gap)."""
    x, signs = synth.gradient(256, 1024, seed=1)
    w = orc.signs_words(signs)
    mse = {}
    for fmt in (orc.FMT_NVFP4, orc.FMT_IF4):
        for rnd in (orc.SR, orc.MSEDEN):
            tot = 0.0
            for t in range(3):
                q = orc.quantize(x, fmt=fmt, rounding=rnd, rht_on=True, signs_w=w, seed=5, stream=t)
                d = orc.dequantize(q["codes"], q["scales"], q["ts"], fmt=fmt, inv_signs_w=w)
                tot += float(np.mean((d.astype(np.float64) - x) ** 2))
            mse[(fmt, rnd)] = tot
    assert mse[(orc.FMT_IF4, orc.SR)] < 0.9 * mse[(orc.FMT_NVFP4, orc.SR)]
    assert mse[(orc.FMT_IF4, orc.MSEDEN)] < 0.9 * mse[(orc.FMT_NVFP4, orc.MSEDEN)]
    assert mse[(orc.FMT_IF4, orc.SR)] / mse[(orc.FMT_IF4, orc.MSEDEN)] > 2.0
