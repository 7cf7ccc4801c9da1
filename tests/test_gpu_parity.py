"""GPU <-> oracle parity of the quantizers, the rotation and dequantization,
called through the C ABI (the Python binding marshals arguments only).

Rotation off: packed codes, scales and the tensor scale are bit-exact.
Rotation on: the contract's tolerance (<= 1e-5 of codes one level apart,
rotated values within 1e-5 of their group's largest magnitude).  The
butterfly kernels (fp32 input; both axes at once) run the transform's stages
in the oracle's order and are bit-exact in practice; bf16 input rotates on
the matrix cores, which round the same exact products' sums in another
order.
Sizes span several workgroups and a ragged tail.
"""
import numpy as np
import pytest

import oracle
from nvfp4_bit_block_amd import synth
from gpu_util import assert_bit_exact, assert_rotated_close, assert_rotation_values_close, q_to_host, to_device

pytestmark = pytest.mark.gpu

ROUNDINGS = [("rtn", oracle.RTN, 128), ("sr", oracle.SR, 128), ("eden128", oracle.MSEDEN, 128),
             ("eden16", oracle.MSEDEN, 16)]


@pytest.fixture(scope="module")
def nv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nvfp4_bit_block_amd as m
    m.lib()
    return m


def _run(nv, x, dtype, rnd, axis, signs, seed=11, stream=5, group=128, if4=False):
    xt = to_device(x, dtype)
    if if4:
        q = nv.quantize_if4(xt, axis=axis, rht_signs=signs)
    else:
        q = nv.quantize_nvfp4(xt, rounding=rnd, axis=axis, rht_signs=signs, seed=seed,
                              stream_id=stream, eden_group=group)
    return q_to_host(q)


def _ref(x, rnd, axis, signs, seed=11, stream=5, group=128, fmt=oracle.FMT_NVFP4):
    w = None if signs is None else oracle.signs_words(signs)
    return oracle.quantize(x, fmt=fmt, rounding=rnd, axis=axis, rht_on=signs is not None,
                           signs_w=w, seed=seed, stream=stream, eden_group=group)


# shapes (rows, cols): quantized dim must be a multiple of 128 for rotation and
# MS-EDEN-128, of 16 otherwise; several workgroups plus ragged tails.
ROW_SHAPES = [(256, 256), (37, 1152), (1, 128), (300, 384)]
COL_SHAPES = [(256, 256), (1152, 37), (128, 1), (512, 200), (384, 72), (400, 200)]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("name,rnd,group", ROUNDINGS)
@pytest.mark.parametrize("axis", [0, 1])
def test_quantize_bit_exact_rotation_off(nv, dtype, name, rnd, group, axis):
    shapes = ROW_SHAPES if axis == 0 else COL_SHAPES
    for i, (r, c) in enumerate(shapes):
        if rnd == oracle.MSEDEN and group == 128 and (c if axis == 0 else r) % 128:
            continue                 # the correction group needs whole 128-groups
        x = synth.gradient(r, c, seed=100 + i)[0] if dtype == "bf16" else synth.gaussian(r, c, seed=100 + i)
        g = _run(nv, x, dtype, rnd, axis, None, group=group)
        ref = _ref(x, rnd, axis, None, group=group)
        assert_bit_exact(g, ref, f"{name} {dtype} axis{axis} {r}x{c}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("name,rnd,group", ROUNDINGS)
@pytest.mark.parametrize("axis", [0, 1])
def test_quantize_rotation_on(nv, dtype, name, rnd, group, axis):
    rng = np.random.default_rng(7)
    signs = synth.signs_from_rng(rng)
    shapes = [(256, 256), (40, 1024)] if axis == 0 else [(256, 256), (1024, 40), (384, 72)]
    for i, (r, c) in enumerate(shapes):
        x = synth.gradient(r, c, seed=200 + i)[0] if dtype == "bf16" else synth.gaussian(r, c, seed=200 + i)
        g = _run(nv, x, dtype, rnd, axis, signs, group=group)
        ref = _ref(x, rnd, axis, signs, group=group)
        assert_rotated_close(g, ref, what=f"{name} {dtype} axis{axis} {r}x{c}")


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_if4_bit_exact(nv, axis, dtype):
    for i, (r, c) in enumerate([(256, 256), (64, 1040), (1040, 64)] if axis == 0 else
                               [(256, 256), (1040, 64), (64, 1040)]):
        x = synth.weight(r, c, seed=300 + i)
        if dtype == "fp32":
            x = synth.gaussian(r, c, seed=300 + i) * np.float32(3.0)
        g = _run(nv, x, dtype, oracle.RTN, axis, None, if4=True)
        ref = _ref(x, oracle.RTN, axis, None, fmt=oracle.FMT_IF4)
        assert_bit_exact(g, ref, f"if4 {dtype} axis{axis} {r}x{c}")
        assert np.any(g["scales"] >= 0x80) and np.any(g["scales"] < 0x80)


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_four_over_six_bit_exact(nv, axis, dtype):
    """Four Over Six (RTN, block maximum mapped to 6 or 4): codes, scales and
    the tensor scale bit-exact; both candidates are taken somewhere."""
    shapes = ROW_SHAPES if axis == 0 else COL_SHAPES
    n4 = 0
    for i, (r, c) in enumerate(shapes):
        x = synth.gradient(r, c, seed=500 + i)[0] if dtype == "bf16" else synth.gaussian(r, c, seed=500 + i)
        g = q_to_host(nv.quantize_nvfp4(to_device(x, dtype), axis=axis, scale_rule="4over6"))
        ref = oracle.quantize(x, fmt=oracle.FMT_NVFP4_4OVER6, axis=axis)
        assert_bit_exact(g, ref, f"4over6 {dtype} axis{axis} {r}x{c}")
        rtn = oracle.quantize(x, axis=axis, ts_in=float(ref["ts"]))
        n4 += int(np.sum(ref["scales"] != rtn["scales"]))
    assert n4 > 0


@pytest.mark.parametrize("axis", [0, 1])
def test_four_over_six_rotation_and_given_scale(nv, axis):
    import torch
    rng = np.random.default_rng(17)
    signs = synth.signs_from_rng(rng)
    x = synth.gradient(256, 384, seed=510)[0]
    if axis == 1:
        x = np.ascontiguousarray(x[:, :256])
    w = oracle.signs_words(signs)
    g = q_to_host(nv.quantize_nvfp4(to_device(x, "bf16"), axis=axis, rht_signs=signs, scale_rule="4over6"))
    ref = oracle.quantize(x, fmt=oracle.FMT_NVFP4_4OVER6, axis=axis, rht_on=True, signs_w=w)
    assert_rotated_close(g, ref, what=f"4over6 rotation axis{axis}")
    ts = np.float32(0.0123)
    g = q_to_host(nv.quantize_nvfp4(to_device(x, "bf16"), axis=axis, scale_rule="4over6",
                                    tensor_scale_in=torch.tensor([ts], device="cuda:0")))
    ref = oracle.quantize(x, fmt=oracle.FMT_NVFP4_4OVER6, axis=axis, ts_in=float(ts))
    assert_bit_exact(g, ref, f"4over6 given scale axis{axis}")


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_scale_search_bit_exact(nv, axis, dtype):
    """RTN with a searched block scale: codes, scales, tensor scale bit-exact,
    including rows so small that the standard scale byte underflows to 0."""
    shapes = ROW_SHAPES if axis == 0 else COL_SHAPES
    moved = 0
    for i, (r, c) in enumerate(shapes):
        x = synth.gradient(r, c, seed=700 + i)[0] if dtype == "bf16" else synth.gaussian(r, c, seed=700 + i)
        g = q_to_host(nv.quantize_nvfp4(to_device(x, dtype), axis=axis, scale_rule="search"))
        ref = oracle.quantize(x, fmt=oracle.FMT_NVFP4_SEARCH, axis=axis)
        assert_bit_exact(g, ref, f"search {dtype} axis{axis} {r}x{c}")
        moved += int(np.sum(ref["scales"] != oracle.quantize(x, axis=axis)["scales"]))
    assert moved > 0
    rng = np.random.default_rng(41)
    x = rng.standard_normal((96, 256)).astype(np.float32)
    x *= (2.0 ** -(np.arange(96) % 31)).astype(np.float32)[:, None]
    if axis == 1:
        x = np.ascontiguousarray(x.T)
    if dtype == "bf16":
        x = synth.to_bf16_f32(x)
    g = q_to_host(nv.quantize_nvfp4(to_device(x, dtype), axis=axis, scale_rule="search"))
    ref = oracle.quantize(x, fmt=oracle.FMT_NVFP4_SEARCH, axis=axis)
    assert_bit_exact(g, ref, f"search tiny rows {dtype} axis{axis}")
    assert np.any(oracle.quantize(x, axis=axis)["scales"] == 0)


def test_scale_search_rotation_and_given_scale(nv):
    import torch
    rng = np.random.default_rng(43)
    signs = synth.signs_from_rng(rng)
    w = oracle.signs_words(signs)
    x = synth.gradient(256, 384, seed=710)[0]
    g = q_to_host(nv.quantize_nvfp4(to_device(x, "bf16"), rht_signs=signs, scale_rule="search"))
    ref = oracle.quantize(x, fmt=oracle.FMT_NVFP4_SEARCH, rht_on=True, signs_w=w)
    assert_rotated_close(g, ref, what="search rotation")
    ts = np.float32(0.0117)
    g = q_to_host(nv.quantize_nvfp4(to_device(x, "bf16"), scale_rule="search",
                                    tensor_scale_in=torch.tensor([ts], device="cuda:0")))
    ref = oracle.quantize(x, fmt=oracle.FMT_NVFP4_SEARCH, ts_in=float(ts))
    assert_bit_exact(g, ref, "search given scale")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("group,rot", [(128, True), (16, True), (128, False), (16, False)])
def test_dual_axis_mseden(nv, dtype, group, rot):
    """MS-EDEN along both axes from one read equals the oracle's axis-0 and
    axis-1 quantizations (and the two separate GPU calls, bit for bit);
    shapes with a partial column tile."""
    rng = np.random.default_rng(19)
    signs = synth.signs_from_rng(rng) if rot else None
    w = None if signs is None else oracle.signs_words(signs)
    for i, (r, c) in enumerate([(256, 384), (128, 128), (384, 1152)]):
        x = synth.gradient(r, c, seed=600 + i)[0] if dtype == "bf16" else synth.gaussian(r, c, seed=600 + i)
        xt = to_device(x, dtype)
        qr, qc = nv.quantize_nvfp4_dual(xt, rht_signs=signs, seed=3, stream_id=2, eden_group=group)
        gr, gc = q_to_host(qr), q_to_host(qc)
        for axis, g in ((0, gr), (1, gc)):
            ref = oracle.quantize(x, rounding=oracle.MSEDEN, axis=axis, rht_on=rot, signs_w=w, seed=3,
                                  stream=2, eden_group=group)
            what = f"dual {dtype} g{group} rot{rot} axis{axis} {r}x{c}"
            if rot:
                assert_rotated_close(g, ref, what=what)
            else:
                assert_bit_exact(g, ref, what)
            sep = q_to_host(nv.quantize_nvfp4(xt, rounding="mseden", axis=axis, rht_signs=signs, seed=3,
                                              stream_id=2, eden_group=group))
            if rot and dtype == "bf16":
                # the separate calls rotate on the matrix cores
                assert_rotated_close(g, sep, what=what + " vs separate call")
            else:
                assert_bit_exact(g, sep, what + " vs separate call")


def test_dual_axis_given_scale(nv):
    import torch
    x = synth.gradient(256, 256, seed=610)[0]
    ts = np.float32(2.5e-3)
    qr, qc = nv.quantize_nvfp4_dual(to_device(x, "bf16"), tensor_scale_in=torch.tensor([ts], device="cuda:0"),
                                    seed=4)
    for axis, q in ((0, qr), (1, qc)):
        ref = oracle.quantize(x, rounding=oracle.MSEDEN, axis=axis, ts_in=float(ts), seed=4)
        assert_bit_exact(q_to_host(q), ref, f"dual given scale axis{axis}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("axis", [0, 1])
def test_rht_values(nv, axis, dtype):
    """fp32 input: the butterfly stages in the oracle's order, bit-exact
    (signed zeros included); bf16 input: the matrix-core product, within the
    rotation tolerance of each group's largest value."""
    import torch
    rng = np.random.default_rng(8)
    signs = synth.signs_from_rng(rng)
    x = synth.gradient(256, 384, seed=9)[0]
    z = nv.rht(to_device(x, dtype), signs, axis=axis).cpu().numpy()
    view = x if axis == 0 else np.ascontiguousarray(x.T)
    ref = oracle.rht(view, oracle.signs_words(signs))
    assert_rotation_values_close(z, ref, what=f"rotation {dtype} axis{axis}")
    if dtype == "fp32":
        assert np.array_equal(z.view(np.uint32), ref.view(np.uint32))
    else:
        # both round sums of the same exact products: far inside the tolerance
        assert_rotation_values_close(z, ref, tol=1e-6, what=f"rotation {dtype} axis{axis}")
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_rht_signed_zero_cancellations(nv, dtype):
    """Inputs whose rotated values cancel to exactly zero in many butterflies:
    the butterfly kernels (fp32 input) match the oracle bit for bit, the sign
    of every zero included; the matrix-core kernels (bf16) match it as values
    (a zero of either sign)."""
    rng = np.random.default_rng(21)
    signs = synth.signs_from_rng(rng)
    x = np.repeat(rng.choice(np.array([1.0, -1.0, 0.5, 0.0], dtype=np.float32), (64, 8)), 16, axis=1)
    x[:, ::3] *= -1
    for axis in (0, 1):
        exact = dtype == "fp32"
        xin = x if axis == 0 else np.ascontiguousarray(x.T)
        z = nv.rht(to_device(xin, dtype), signs, axis=axis).cpu().numpy()
        ref = oracle.rht(x, oracle.signs_words(signs))
        assert np.count_nonzero(ref == 0) > 100
        if exact:
            assert np.array_equal(z.view(np.uint32), ref.view(np.uint32))
        else:
            assert np.array_equal(z, ref)  # values; -0 == +0
        for rnd, name in ((oracle.RTN, "rtn"), (oracle.MSEDEN, "mseden")):
            g = q_to_host(nv.quantize_nvfp4(to_device(xin, dtype), rounding=name, axis=axis, rht_signs=signs))
            r = oracle.quantize(xin, rounding=rnd, axis=axis, rht_on=True, signs_w=oracle.signs_words(signs))
            if exact:
                assert_bit_exact(g, r, f"zero cancellations {name} {dtype} axis{axis}")
            else:
                assert_rotated_close(g, r, frac=0.0, what=f"zero cancellations {name} {dtype} axis{axis}")


def _negative_zero_groups(signs, rows, cols, seed):
    """bf16-exact input whose 128-groups are, by row: Gaussian; half of the
    group -0 after the sign flips and the other half cancelling exactly (the
    last butterfly then gives (-0) - (+0) = -0); the same at quarter scale;
    all zeros of random signs.  The oracle's rotation of such groups has
    outputs of both zero signs."""
    rng = np.random.default_rng(seed)
    flip = np.where(np.asarray(signs) > 0, -1.0, 1.0).astype(np.float32)
    x = synth.to_bf16_f32(rng.standard_normal((rows, cols)).astype(np.float32))
    for r in range(rows):
        kind = r % 4
        for g0 in range(0, cols, 128):
            if kind == 0 or (g0 // 128 + r) % 3 == 0:
                continue                                         # stays Gaussian
            seg = np.empty(128, dtype=np.float32)
            if kind == 3:
                seg[:] = np.where(rng.integers(0, 2, 128) > 0, -0.0, 0.0)
            else:
                part = 64 if kind == 1 else 32
                neg = -0.0 * flip                                # flip * neg = -0
                alt = flip * np.where(np.arange(128) % 2 == 0, 1.0, -1.0).astype(np.float32) * 0.75
                pos = (np.arange(128) // part) % 2 == 0
                seg[:] = np.where(pos, neg, alt)
            x[r, g0:g0 + 128] = seg
    return x


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_rotation_negative_zero_outputs(nv, dtype):
    """Rotated outputs that are -0 in the oracle: the butterfly kernels (fp32
    input, also both axes at once) give -0 too, while other groups of the
    same waves take the fast stages -- rotation values, RTN, SR and MS-EDEN
    codes; the matrix-core kernels (bf16) give the same values, a zero of
    either sign."""
    import torch
    rng = np.random.default_rng(34)
    signs = synth.signs_from_rng(rng)
    w = oracle.signs_words(signs)
    x = _negative_zero_groups(signs, 128, 768, seed=35)
    ref_rot = oracle.rht(x, w)
    assert np.count_nonzero((ref_rot == 0) & np.signbit(ref_rot)) > 50
    assert np.count_nonzero((ref_rot == 0) & ~np.signbit(ref_rot)) > 50
    for axis in (0, 1):
        exact = dtype == "fp32"
        xin = x if axis == 0 else np.ascontiguousarray(x.T)
        z = nv.rht(to_device(xin, dtype), signs, axis=axis).cpu().numpy()
        if exact:
            assert np.array_equal(z.view(np.uint32), ref_rot.view(np.uint32)), f"rotation axis{axis}"
        else:
            assert_rotation_values_close(z, ref_rot, tol=1e-6, what=f"rotation axis{axis}")
            assert np.all(z[ref_rot == 0] == 0), f"rotation axis{axis}: exact zeros"
        for name, rnd in (("rtn", oracle.RTN), ("sr", oracle.SR), ("mseden", oracle.MSEDEN)):
            g = q_to_host(nv.quantize_nvfp4(to_device(xin, dtype), rounding=name, axis=axis, rht_signs=signs,
                                            seed=6, stream_id=2))
            r = oracle.quantize(xin, rounding=rnd, axis=axis, rht_on=True, signs_w=w, seed=6, stream=2)
            if exact:
                assert_bit_exact(g, r, f"-0 outputs {name} {dtype} axis{axis}")
            else:
                assert_rotated_close(g, r, frac=0.0, what=f"-0 outputs {name} {dtype} axis{axis}")
    xt = x.T.copy()        # both axes at once quantize along the rows of their input
    qr, qc = nv.quantize_nvfp4_dual(to_device(xt, dtype), rht_signs=signs, seed=8)
    for axis, q in ((0, qr), (1, qc)):
        r = oracle.quantize(xt, rounding=oracle.MSEDEN, axis=axis, rht_on=True, signs_w=w, seed=8)
        if dtype == "fp32":
            assert_bit_exact(q_to_host(q), r, f"-0 outputs dual {dtype} axis{axis}")
        else:
            assert_rotated_close(q_to_host(q), r, frac=0.0, what=f"-0 outputs dual {dtype} axis{axis}")
    torch.cuda.synchronize()


def test_tensor_scale_in(nv):
    import torch
    x = synth.gaussian(128, 512, seed=12)
    ts = torch.tensor([0.0123], dtype=torch.float32, device="cuda:0")
    for rnd in (oracle.RTN, oracle.SR, oracle.MSEDEN):
        q = q_to_host(nv.quantize_nvfp4(to_device(x, "fp32"), rounding=rnd, seed=3, stream_id=1,
                                        tensor_scale_in=ts))
        ref = oracle.quantize(x, rounding=rnd, seed=3, stream=1, ts_in=np.float32(0.0123))
        assert_bit_exact(q, ref, f"ts_in rounding {rnd}")


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("group", [128, 16])
def test_mseden_given_scale_rotation(nv, axis, group):
    """MS-EDEN with a given tensor scale and the rotation: codes and scales in
    one pass, each block's scale rounded with the uniform at its position in
    its Philox word (bf16: the matrix-core kernels; fp32: the butterflies).
    Several tiles, a ragged tail, every position 0..7 of the uniforms."""
    import torch
    rng = np.random.default_rng(47)
    signs = synth.signs_from_rng(rng)
    w = oracle.signs_words(signs)
    shapes = [(200, 1024), (33, 384)] if axis == 0 else [(1024, 200), (384, 33)]
    for dtype in ("bf16", "fp32"):
        for i, (r, c) in enumerate(shapes):
            x = synth.gradient(r, c, seed=900 + i)[0]
            amax = float(np.max(np.abs(x)))
            ts = np.float32(amax / 2688.0)
            g = q_to_host(nv.quantize_nvfp4(to_device(x, dtype), rounding=oracle.MSEDEN, axis=axis,
                                            rht_signs=signs, seed=13, stream_id=3, eden_group=group,
                                            tensor_scale_in=torch.tensor([ts], device="cuda:0")))
            ref = oracle.quantize(x, rounding=oracle.MSEDEN, axis=axis, rht_on=True, signs_w=w, seed=13, stream=3,
                                  eden_group=group, ts_in=float(ts))
            assert g["ts"] == float(ts)
            assert_rotated_close(g, ref, what=f"mseden given scale {dtype} axis{axis} group{group} {r}x{c}")
            assert len(np.unique(ref["scales"])) > 8


def upload(nv, ref, fmt):
    """A QTensor on the device holding the oracle's packed output."""
    import torch
    return nv.QTensor(torch.from_numpy(ref["codes"]).to("cuda:0"),
                      torch.from_numpy(ref["scales"]).to("cuda:0"),
                      torch.tensor([ref["ts"]], dtype=torch.float32, device="cuda:0"), fmt)


@pytest.mark.parametrize("fmt", ["nvfp4", "if4"])
def test_dequantize_bit_exact(nv, fmt):
    import torch
    x = synth.weight(96, 512, seed=13)
    ofmt = oracle.FMT_IF4 if fmt == "if4" else oracle.FMT_NVFP4
    q = oracle.quantize(x, fmt=ofmt) if fmt == "if4" else oracle.quantize(x, rounding=oracle.SR, seed=4)
    ref = oracle.dequantize(q["codes"], q["scales"], q["ts"], fmt=ofmt)
    qt = upload(nv, q, nv.FORMAT_IF4 if fmt == "if4" else nv.FORMAT_NVFP4)
    d = nv.dequantize(qt).cpu().numpy()
    assert np.array_equal(d.view(np.uint32), ref.view(np.uint32))
    d16 = nv.dequantize(qt, out_dtype=torch.bfloat16).float().cpu().numpy()
    assert np.array_equal(d16, synth.to_bf16_f32(ref))


def test_dequantize_inverse_rotation(nv):
    rng = np.random.default_rng(14)
    signs = synth.signs_from_rng(rng)
    w = oracle.signs_words(signs)
    x = synth.gradient(64, 1024, seed=15)[0]
    q = oracle.quantize(x, rounding=oracle.MSEDEN, rht_on=True, signs_w=w, seed=1)
    ref = oracle.dequantize(q["codes"], q["scales"], q["ts"], inv_signs_w=w)
    d = nv.dequantize(upload(nv, q, nv.FORMAT_NVFP4), inv_rht_signs=signs).cpu().numpy()
    assert np.max(np.abs(d - ref)) <= 1e-5 * np.abs(ref).max()


def test_deterministic_replay(nv):
    x = synth.gradient(512, 1024, seed=16)[0]
    xt = to_device(x, "bf16")
    signs = synth.signs_from_rng(np.random.default_rng(3))
    a = q_to_host(nv.quantize_nvfp4(xt, rounding="sr", rht_signs=signs, seed=9, stream_id=2))
    b = q_to_host(nv.quantize_nvfp4(xt, rounding="sr", rht_signs=signs, seed=9, stream_id=2))
    assert_bit_exact(a, b, "replay")
    c = q_to_host(nv.quantize_nvfp4(xt, rounding="sr", rht_signs=signs, seed=9, stream_id=3))
    assert not np.array_equal(a["codes"], c["codes"])


@pytest.mark.parametrize("axis", [0, 1])
def test_mseden_group16_block_count_not_multiple_of_8(nv, axis):
    """MS-EDEN with 16-element groups on shapes whose block count is not a
    multiple of 8: the scale pass codes the last, partial Philox call (and
    a tensor below one call) like the rest."""
    for i, (r, c) in enumerate([(37, 80), (5, 48), (1, 16), (261, 208)]):
        x = synth.gradient(r, c, seed=900 + i)[0]
        xin = x if axis == 0 else np.ascontiguousarray(x.T)
        g = _run(nv, xin, "bf16", oracle.MSEDEN, axis, None, group=16)
        ref = _ref(xin, oracle.MSEDEN, axis, None, group=16)
        assert g["scales"].size % 8 != 0
        assert_bit_exact(g, ref, f"eden16 axis{axis} {r}x{c}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_columns_unaligned_rows_and_many_tiles(nv, dtype):
    """Column-wise quantization where every tile takes the element-wise path
    (a leading dimension that leaves rows unaligned), and a tensor of whole
    tiles plus a ragged tile column."""
    import torch
    rng = np.random.default_rng(41)
    signs = synth.signs_from_rng(rng)
    x = synth.gradient(384, 520, seed=42)[0] if dtype == "bf16" else synth.gaussian(384, 520, seed=42)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    full = torch.from_numpy(np.pad(x, ((0, 0), (0, 3)))).to(tdt).to("cuda:0")
    view = full[:, :520]                       # ld = 523 elements: rows not 16-byte aligned
    for name, rnd in (("rtn", oracle.RTN), ("mseden", oracle.MSEDEN)):
        g = q_to_host(nv.quantize_nvfp4(view, rounding=name, axis=1, seed=3))
        assert_bit_exact(g, oracle.quantize(x, rounding=rnd, axis=1, seed=3), f"unaligned {name} {dtype}")
    # 2048 x 1000: 16 x 15 interior tiles (bf16) plus a ragged tile column
    y = synth.gradient(2048, 1000, seed=43)[0] if dtype == "bf16" else synth.gaussian(2048, 1000, seed=43)
    for name, rnd in (("rtn", oracle.RTN), ("mseden", oracle.MSEDEN)):
        g = q_to_host(nv.quantize_nvfp4(to_device(y, dtype), rounding=name, axis=1, rht_signs=signs, seed=5))
        r = oracle.quantize(y, rounding=rnd, axis=1, rht_on=True, signs_w=oracle.signs_words(signs), seed=5)
        if dtype == "bf16":  # the matrix-core rotation
            assert_rotated_close(g, r, what=f"many tiles {name} {dtype}")
        else:
            assert_bit_exact(g, r, f"many tiles {name} {dtype}")


@pytest.mark.parametrize("axis", [0, 1])
def test_matrix_core_rotation_layouts(nv, axis):
    """The matrix-core rotation (bf16) on layouts its tiling treats apart:
    strided views (axis 0: per-group addresses instead of one contiguous
    tile; axis 1: a leading dimension above the row length), a last tile with
    one 128-row group of two and a ragged column tile (axis 1), a group count
    that leaves the last 32-group tile partial (axis 0), and a view offset by
    8 (axis 0) or 4 (axis 1: rows not 16-byte aligned, the butterfly kernel
    instead) elements."""
    import torch
    rng = np.random.default_rng(47)
    signs = synth.signs_from_rng(rng)
    w = oracle.signs_words(signs)
    x = synth.gradient(384, 840, seed=48)[0]
    full = torch.from_numpy(x).to(torch.bfloat16).to("cuda:0")
    cases = [("dense", x[:-1, :640] if axis == 0 else x[:, :200], None),
             ("strided", x[:, 64:576], (64, 576)),
             ("unaligned", x[:, 4:516] if axis == 1 else x[:, 8:520], (4, 516) if axis == 1 else (8, 520))]
    for name, xv, cut in cases:
        xv = np.ascontiguousarray(xv)
        t = to_device(xv, "bf16") if cut is None else full[:, cut[0]:cut[1]]
        for rn, rnd in (("rtn", oracle.RTN), ("sr", oracle.SR), ("mseden", oracle.MSEDEN)):
            g = q_to_host(nv.quantize_nvfp4(t, rounding=rn, axis=axis, rht_signs=signs, seed=2, stream_id=1))
            r = oracle.quantize(xv, rounding=rnd, axis=axis, rht_on=True, signs_w=w, seed=2, stream=1)
            assert_rotated_close(g, r, what=f"{name} {rn} axis{axis} {xv.shape}")
        z = nv.rht(t, signs, axis=axis).cpu().numpy()
        assert_rotation_values_close(z, oracle.rht(xv if axis == 0 else np.ascontiguousarray(xv.T), w),
                                     what=f"{name} rotation axis{axis}")


@pytest.mark.parametrize("group", [128, 16])
@pytest.mark.parametrize("axis", [0, 1])
def test_matrix_core_mseden_small_blocks(nv, axis, group):
    """MS-EDEN on the matrix cores with 128-groups scaled to about 1e-18 (block
    maxima below 2^-50, where the kernels leave the wave to the exact rule
    instead of the fused sums) and all-zero groups, among Gaussian ones: the
    waves that hold them and those that do not both match the oracle under
    the rotation rule."""
    rng = np.random.default_rng(53)
    signs = synth.signs_from_rng(rng)
    x = synth.gaussian(256, 512, seed=54)
    if axis == 0:
        x[5:9, 128:256] *= np.float32(1e-18)       # groups of rows 5..8
        x[40, 256:384] = 0.0
        x[200:202, :] *= np.float32(3e-19)
    else:
        x[128:256, 7:11] *= np.float32(1e-18)      # groups of columns 7..10
        x[0:128, 300] = 0.0
        x[:, 450:452] *= np.float32(3e-19)
    x = synth.to_bf16_f32(x)
    g = _run(nv, x, "bf16", "mseden", axis, signs, group=group)
    r = _ref(x, oracle.MSEDEN, axis, signs, group=group)
    assert_rotated_close(g, r, what=f"small blocks axis{axis} group{group}")


def test_strided_input(nv):
    """A row-major view with leading dimension above the row length."""
    import torch
    x = synth.gaussian(64, 320, seed=17)
    full = torch.from_numpy(x).to("cuda:0")
    view = full[:, 32:288]
    assert view.stride(0) == 320
    for axis in (0, 1):
        g = q_to_host(nv.quantize_nvfp4(view, rounding="rtn", axis=axis))
        ref = oracle.quantize(np.ascontiguousarray(x[:, 32:288]), axis=axis)
        assert_bit_exact(g, ref, f"strided axis{axis}")


def test_zero_tensor_and_empty(nv):
    import torch
    z = torch.zeros((16, 256), dtype=torch.bfloat16, device="cuda:0")
    for rnd in ("rtn", "sr", "mseden"):
        h = q_to_host(nv.quantize_nvfp4(z, rounding=rnd))
        assert h["ts"] == 1.0 and not h["scales"].any() and not h["codes"].any()
    e = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda:0")
    h = q_to_host(nv.quantize_nvfp4(e))
    assert h["ts"] == 1.0 and h["codes"].size == 0


def test_negative_zero_sign_kept(nv):
    x = np.zeros((1, 16), dtype=np.float32)
    x[0, :8] = -0.0
    x[0, 8] = 1.0
    x[0, 9] = -1e-6
    g = _run(nv, x, "fp32", oracle.RTN, 0, None)
    ref = _ref(x, oracle.RTN, 0, None)
    assert_bit_exact(g, ref, "signed zeros")
