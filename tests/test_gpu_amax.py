"""The tensor maximum handed between calls on the GPU: an MS-EDEN call with
amax_out writes max|x| of its raw input (exactly), without changing its own
results; a call with amax_in codes exactly as the oracle does with the tensor
scale amax_in / (6 * 448) (or / (6 * 256) for Four Over Six) -- and so as
the call without it when amax_in is the input's maximum."""
import numpy as np
import pytest

import oracle
from nvfp4_bit_block_amd import synth
from gpu_util import assert_bit_exact, q_to_host, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import torch
    assert torch.cuda.is_available()
    import nvfp4_bit_block_amd as m
    m.lib()
    return m


def _dev_scalar(v):
    import torch
    return torch.tensor([v], dtype=torch.float32, device="cuda:0")


def _same(a, b, what):
    ha, hb = q_to_host(a), q_to_host(b)
    assert ha["ts"] == hb["ts"], what
    assert np.array_equal(ha["codes"], hb["codes"]) and np.array_equal(ha["scales"], hb["scales"]), what


# (rows, cols): multiples of 128 along both axes, several tiles and a ragged
# tile count; a tensor with a lone large value in its last row
SHAPES = [(256, 384), (640, 1024), (128, 4096)]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("rot", [False, True])
@pytest.mark.parametrize("group", [128, 16])
def test_amax_out_mseden(nv, dtype, axis, rot, group):
    import torch
    rng = np.random.default_rng(51)
    signs = synth.signs_from_rng(rng) if rot else None
    for r, c in SHAPES:
        x = synth.gradient(r, c, seed=52 + r)[0].copy()
        x[-1, c // 3] = np.float32(-1232.0)        # the maximum, negative, in the last row
        if dtype == "fp32":
            x = x * np.float32(1.1)                # values off the bf16 grid
        xd = to_device(x, dtype)
        am = _dev_scalar(-1.0)
        q = nv.quantize_nvfp4(xd, rounding="mseden", axis=axis, rht_signs=signs, seed=5, eden_group=group,
                              amax_out=am)
        q0 = nv.quantize_nvfp4(xd, rounding="mseden", axis=axis, rht_signs=signs, seed=5, eden_group=group)
        torch.cuda.synchronize()
        assert float(am.cpu()[0]) == float(np.abs(x).max()), f"{dtype} axis{axis} {r}x{c}"
        _same(q, q0, f"amax_out changes nothing: {dtype} axis{axis} rot{rot} g{group} {r}x{c}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("axis", [0, 1])
def test_amax_in(nv, dtype, axis):
    import torch
    x = synth.weight(384, 512, seed=53)
    if dtype == "fp32":
        x = x * np.float32(1.1)                    # values off the bf16 grid
    xd = to_device(x, dtype)
    m = float(np.abs(x).max())
    view = x
    calls = [  # name, library call, oracle format, oracle rounding, top
        ("rtn", lambda a: nv.quantize_nvfp4(xd, axis=axis, amax_in=a), oracle.FMT_NVFP4, oracle.RTN, 6 * 448),
        ("sr", lambda a: nv.quantize_nvfp4(xd, rounding="sr", axis=axis, seed=7, amax_in=a), oracle.FMT_NVFP4,
         oracle.SR, 6 * 448),
        ("if4", lambda a: nv.quantize_if4(xd, axis=axis, amax_in=a), oracle.FMT_IF4, oracle.RTN, 6 * 448),
        ("4over6", lambda a: nv.quantize_nvfp4(xd, axis=axis, scale_rule="4over6", amax_in=a),
         oracle.FMT_NVFP4_4OVER6, oracle.RTN, 6 * 256),
        ("search", lambda a: nv.quantize_nvfp4(xd, axis=axis, scale_rule="search", amax_in=a),
         oracle.FMT_NVFP4_SEARCH, oracle.RTN, 6 * 448),
    ]
    for name, call, fmt, rnd, top in calls:
        # the input's own maximum: the oracle's computed tensor scale
        g = q_to_host(call(_dev_scalar(m)))
        ref = oracle.quantize(view, fmt=fmt, rounding=rnd, axis=axis, seed=7)
        assert_bit_exact(g, ref, f"{name} amax_in = max|x|, {dtype} axis{axis}")
        # another maximum: the tensor scale it gives
        a = np.float32(m * 3.0)
        ts = np.float32(a / np.float32(top))
        g = q_to_host(call(_dev_scalar(float(a))))
        ref = oracle.quantize(view, fmt=fmt, rounding=rnd, axis=axis, seed=7, ts_in=ts)
        assert_bit_exact(g, ref, f"{name} amax_in = 3 max|x|, {dtype} axis{axis}")
        # zero: tensor scale 1
        g = q_to_host(call(_dev_scalar(0.0)))
        ref = oracle.quantize(view, fmt=fmt, rounding=rnd, axis=axis, seed=7, ts_in=np.float32(1.0))
        assert_bit_exact(g, ref, f"{name} amax_in = 0, {dtype} axis{axis}")
    torch.cuda.synchronize()


def test_amax_empty_tensor(nv):
    import torch
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda:0")
    am = _dev_scalar(-1.0)
    q = nv.quantize_nvfp4(x, rounding="mseden", amax_out=am)
    torch.cuda.synchronize()
    assert float(am.cpu()[0]) == 0.0 and float(q.tensor_scale.cpu()[0]) == 1.0
    q = nv.quantize_nvfp4(x, amax_in=_dev_scalar(5.0))
    assert float(q.tensor_scale.cpu()[0]) == 1.0


def test_amax_handoff_mlp_shapes(nv):
    """The training step's hand-off at the full weight shape: W's column-wise
    MS-EDEN (rotation on) gives max|W| to W's row-wise RTN, whose results
    equal the oracle's."""
    import torch
    rng = np.random.default_rng(4)
    W = synth.to_bf16_f32((0.02 * rng.standard_normal((11008, 4096))).astype(np.float32))
    signs = synth.signs_from_rng(rng)
    Wd = to_device(W, "bf16")
    am = _dev_scalar(0.0)
    nv.quantize_nvfp4(Wd, rounding="mseden", axis=1, rht_signs=signs, seed=9, amax_out=am)
    q = nv.quantize_nvfp4(Wd, amax_in=am)
    q0 = nv.quantize_nvfp4(Wd)
    torch.cuda.synchronize()
    assert float(am.cpu()[0]) == float(np.abs(W).max())
    _same(q, q0, "W row-wise RTN with the handed maximum")
    # sampled rows against the oracle (the whole tensor is slow on the CPU)
    rows = np.sort(rng.choice(W.shape[0], 24, replace=False))
    ts = np.float32(np.float32(np.abs(W).max()) / np.float32(6 * 448))
    ref = oracle.quantize(W[rows], ts_in=ts)
    h = q_to_host(q)
    assert h["ts"] == float(ts)
    assert np.array_equal(h["codes"][rows], ref["codes"]) and np.array_equal(h["scales"][rows], ref["scales"])
