"""GPU <-> oracle parity of IF4 for gradients: IF4 with stochastic rounding
and IF4 with MS-EDEN (nvfp4_quantize_if4 with rounding SR / MSEDEN), through
the C ABI.  Rotation off: codes, scale bytes (with the INT flag) and the
tensor scale are bit-exact on the same Philox streams.  Rotation on: the
contract's tolerance (at most 1e-5 of codes or scales one level apart; in
practice bit-exact).  Also: a given tensor scale, the tensor maximum handed
between calls, dequantization, the GEMM on the IF4 gradient operands, and
the 4096 x 4096 gradient at full size.
"""
import numpy as np
import pytest

import oracle
from nvfp4_bit_block_amd import synth
from gpu_util import assert_bit_exact, assert_rotated_close, q_to_host, to_device

pytestmark = pytest.mark.gpu

MODES = [("sr", oracle.SR, 128), ("eden128", oracle.MSEDEN, 128), ("eden16", oracle.MSEDEN, 16)]
ROW_SHAPES = [(256, 256), (37, 1152), (1, 128), (300, 384)]
COL_SHAPES = [(256, 256), (1152, 37), (128, 1), (512, 200), (384, 72)]


@pytest.fixture(scope="module")
def nv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nvfp4_bit_block_amd as m
    m.lib()
    return m


def _data(r, c, dtype, seed):
    # weight-like heavy-tailed rows make both branches occur; bf16 inputs are
    # the bf16-rounded values
    x = synth.weight(r, c, seed=seed) if r * c > 0 else np.zeros((r, c), np.float32)
    return synth.to_bf16_f32(x) if dtype == "bf16" else x


def _run(nv, x, dtype, rnd, axis, signs, group, seed=13, stream=3, **kw):
    q = nv.quantize_if4(to_device(x, dtype), rounding=rnd, axis=axis, rht_signs=signs, seed=seed,
                        stream_id=stream, eden_group=group, **kw)
    return q_to_host(q)


def _ref(x, rnd, axis, signs, group, seed=13, stream=3, ts_in=None):
    w = None if signs is None else oracle.signs_words(signs)
    return oracle.quantize(x, fmt=oracle.FMT_IF4, rounding=rnd, axis=axis, rht_on=signs is not None, signs_w=w,
                           seed=seed, stream=stream, eden_group=group, ts_in=ts_in)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("name,rnd,group", MODES)
@pytest.mark.parametrize("axis", [0, 1])
def test_if4_grad_bit_exact_rotation_off(nv, dtype, name, rnd, group, axis):
    n_int = 0
    for i, (r, c) in enumerate(ROW_SHAPES if axis == 0 else COL_SHAPES):
        if rnd == oracle.MSEDEN and group == 128 and (c if axis == 0 else r) % 128:
            continue
        x = _data(r, c, dtype, 300 + i)
        g = _run(nv, x, dtype, rnd, axis, None, group)
        ref = _ref(x, rnd, axis, None, group)
        assert_bit_exact(g, ref, f"IF4 {name} {dtype} axis{axis} {r}x{c}")
        n_int += int(np.count_nonzero(ref["scales"] >> 7))
    assert n_int > 0


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("name,rnd,group", MODES)
@pytest.mark.parametrize("axis", [0, 1])
def test_if4_grad_rotation_on(nv, dtype, name, rnd, group, axis):
    signs = synth.signs_from_rng(np.random.default_rng(17))
    shapes = [(256, 256), (40, 1024)] if axis == 0 else [(256, 256), (1024, 40), (384, 72)]
    for i, (r, c) in enumerate(shapes):
        x = synth.gradient(r, c, seed=310 + i)[0]
        g = _run(nv, x, dtype, rnd, axis, signs, group)
        ref = _ref(x, rnd, axis, signs, group)
        assert_rotated_close(g, ref, what=f"IF4 {name} {dtype} axis{axis} {r}x{c}")


@pytest.mark.parametrize("name,rnd,group", MODES)
@pytest.mark.parametrize("axis", [0, 1])
def test_if4_grad_given_scale(nv, name, rnd, group, axis):
    """tensor_scale_in: MS-EDEN codes and rounds its scales in one pass."""
    import torch
    x = _data(256, 256, "fp32", 320)
    for ts in (np.float32(np.abs(x).max() / 2688.0), np.float32(0.002), np.float32(1.0)):
        tsd = torch.tensor([ts], dtype=torch.float32, device="cuda:0")
        g = _run(nv, x, "fp32", rnd, axis, None, group, tensor_scale_in=tsd)
        ref = _ref(x, rnd, axis, None, group, ts_in=float(ts))
        assert_bit_exact(g, ref, f"IF4 {name} axis{axis} ts={ts}")


def test_if4_grad_amax_handoff(nv):
    """MS-EDEN writes max|x| (amax_out); SR without rotation takes it (amax_in)
    and gives the results of the call that finds it itself."""
    import torch
    x = _data(512, 384, "bf16", 321)
    xt = to_device(x, "bf16")
    am = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    qe = nv.quantize_if4(xt, rounding="mseden", axis=1, rht_signs=synth.signs_from_rng(np.random.default_rng(3)),
                         amax_out=am)
    assert float(am.cpu()[0]) == np.float32(np.abs(x).max())
    plain = q_to_host(nv.quantize_if4(xt, rounding="sr", seed=2))
    handed = q_to_host(nv.quantize_if4(xt, rounding="sr", seed=2, amax_in=am))
    assert_bit_exact(handed, plain, "IF4 SR with amax_in")
    assert_bit_exact(handed, _ref(x, oracle.SR, 0, None, 128, seed=2, stream=0), "IF4 SR vs oracle")
    ref_e = _ref(x, oracle.MSEDEN, 1, synth.signs_from_rng(np.random.default_rng(3)), 128, seed=0, stream=0)
    assert_rotated_close(q_to_host(qe), ref_e, what="IF4 MS-EDEN with amax_out")


@pytest.mark.parametrize("name,rnd", [("sr", oracle.SR), ("eden", oracle.MSEDEN)])
def test_if4_grad_dequantize(nv, name, rnd):
    x = _data(128, 512, "fp32", 322)
    q = nv.quantize_if4(to_device(x, "fp32"), rounding=rnd, seed=5)
    h = q_to_host(q)
    d = nv.dequantize(q).cpu().numpy()
    assert np.array_equal(d, oracle.dequantize(h["codes"], h["scales"], h["ts"], fmt=oracle.FMT_IF4))


def test_if4_grad_gemm(nv):
    """Weight gradient from IF4 MS-EDEN operands quantized along the
    reduction dimension: the INT-flag-aware GEMM against the oracle's fp64
    GEMM on the same packed operands."""
    dy, x, s = synth.wgrad(1024, 384, seed=3)
    a = nv.quantize_if4(to_device(dy, "bf16"), rounding="mseden", axis=1, rht_signs=s, seed=1)
    b = nv.quantize_if4(to_device(x, "bf16"), rounding="mseden", axis=1, rht_signs=s, seed=2)
    c = nv.gemm_nvfp4(a, b).cpu().numpy()
    ha, hb = q_to_host(a), q_to_host(b)
    ref = oracle.gemm_full(ha, hb, fmt=oracle.FMT_IF4)
    err = np.linalg.norm(c - ref) / np.linalg.norm(ref)
    assert err <= 1e-3, err
    assert np.count_nonzero(ha["scales"] >> 7) > 0 and np.count_nonzero(hb["scales"] >> 7) > 0


@pytest.mark.parametrize("name,rnd", [("sr", oracle.SR), ("eden", oracle.MSEDEN)])
def test_if4_grad_full_gradient_4096(nv, name, rnd):
    """The 4096 x 4096 gradient (5 % outliers at 10x), rows, with the
    randomized Hadamard rotation: the whole tensor against the oracle."""
    g, signs = synth.gradient(4096, 4096, seed=1)
    got = _run(nv, g, "bf16", rnd, 0, signs, 128, seed=1, stream=0)
    ref = _ref(g, rnd, 0, signs, 128, seed=1, stream=0)
    assert_rotated_close(got, ref, what=f"IF4 {name} gradient 4096^2")
