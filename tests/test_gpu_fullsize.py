"""Parity at the workloads' full sizes, in the launch configuration the
benchmark uses: the 4096^2 gradient (rotation + SR and MS-EDEN), the 8192^2
IF4 weight, the 16384 x 4096 weight-gradient pair (column-wise rotation +
MS-EDEN, then the GEMM), and the MLP up-projection step's six quantizations
and three GEMMs.  Quantizer outputs are compared whole against the oracle;
GEMM outputs on sampled entries that the oracle computes one by one (fp64)."""
import numpy as np
import pytest

import oracle
from nvfp4_bit_block_amd import synth
from gpu_util import assert_bit_exact, assert_rotated_close, q_to_host, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nvfp4_bit_block_amd as m
    m.lib()
    return m


def upload(nv, ref):
    import torch
    return nv.QTensor(torch.from_numpy(ref["codes"]).to("cuda:0"),
                      torch.from_numpy(ref["scales"]).to("cuda:0"),
                      torch.tensor([ref["ts"]], dtype=torch.float32, device="cuda:0"), nv.FORMAT_NVFP4)


def sampled_gemm_check(nv, qa_ref, qb_ref, c, n=512, seed=0):
    M, N = c.shape
    rng = np.random.default_rng(seed)
    im = np.concatenate([rng.integers(0, M, n), [0, M - 1, M - 1]])
    in_ = np.concatenate([rng.integers(0, N, n), [0, N - 1, 0]])
    ref = oracle.gemm_entries(qa_ref, qb_ref, im, in_)
    got = c[im, in_].astype(np.float64)
    err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert err <= 1e-3, err
    return err


def test_gradient_4096_rotation_sr_and_mseden(nv):
    x, signs = synth.gradient(4096, 4096, seed=1)
    w = oracle.signs_words(signs)
    xt = to_device(x, "bf16")
    for name, rnd in (("sr", oracle.SR), ("mseden", oracle.MSEDEN)):
        g = q_to_host(nv.quantize_nvfp4(xt, rounding=name, rht_signs=signs, seed=1, stream_id=0))
        ref = oracle.quantize(x, rounding=rnd, rht_on=True, signs_w=w, seed=1, stream=0)
        assert_rotated_close(g, ref, what=f"gradient {name}")


def test_weight_8192_if4(nv):
    x = synth.weight(8192, 8192, seed=2)
    g = q_to_host(nv.quantize_if4(to_device(x, "bf16")))
    ref = oracle.quantize(x, fmt=oracle.FMT_IF4)
    assert_bit_exact(g, ref, "weight if4")


def test_wgrad_16384x4096(nv):
    dy, x, signs = synth.wgrad(16384, 4096, seed=3)
    w = oracle.signs_words(signs)
    qa = nv.quantize_nvfp4(to_device(dy, "bf16"), rounding="mseden", axis=1, rht_signs=signs, seed=5)
    qb = nv.quantize_nvfp4(to_device(x, "bf16"), rounding="mseden", axis=1, rht_signs=signs, seed=6)
    ra = oracle.quantize(dy, rounding=oracle.MSEDEN, axis=1, rht_on=True, signs_w=w, seed=5)
    rb = oracle.quantize(x, rounding=oracle.MSEDEN, axis=1, rht_on=True, signs_w=w, seed=6)
    assert_rotated_close(q_to_host(qa), ra, what="dY col")
    assert_rotated_close(q_to_host(qb), rb, what="X col")
    c = nv.gemm_nvfp4(upload(nv, ra), upload(nv, rb)).cpu().numpy()
    assert c.shape == (4096, 4096)
    assert sampled_gemm_check(nv, ra, rb, c) <= 1e-5


@pytest.fixture(scope="module")
def mlp():
    return synth.mlp_step()


@pytest.mark.parametrize("name", ["X_rtn", "W_rtn", "dY_row", "W_col", "dY_col", "X_col"])
def test_mlp_step_quantizations(nv, mlp, name):
    x, wt, dy, signs = mlp
    w = oracle.signs_words(signs)
    src = {"X": x, "W": wt, "dY": dy}[name.split("_")[0]]
    kind = name.split("_")[1]
    if kind == "rtn":
        g = q_to_host(nv.quantize_nvfp4(to_device(src, "bf16")))
        ref = oracle.quantize(src)
        assert_bit_exact(g, ref, name)
    else:
        axis = 0 if kind == "row" else 1
        g = q_to_host(nv.quantize_nvfp4(to_device(src, "bf16"), rounding="mseden", axis=axis,
                                        rht_signs=signs, seed=7, stream_id=3))
        ref = oracle.quantize(src, rounding=oracle.MSEDEN, axis=axis, rht_on=True, signs_w=w, seed=7,
                              stream=3)
        assert_rotated_close(g, ref, what=name)


def test_weight_8192_if4_gemm(nv):
    """The 8192^2 IF4 weight as the B operand of a GEMM with a 4096 x 8192
    activation (IF4 as well), quantized on the GPU and checked bit-exact
    first; sampled entries of C against the oracle's fp64 GEMM."""
    import torch
    wt = synth.weight(8192, 8192, seed=2)
    x = synth.to_bf16_f32(synth.gaussian(4096, 8192, seed=9))
    gw = nv.quantize_if4(to_device(wt, "bf16"))
    gx = nv.quantize_if4(to_device(x, "bf16"))
    rw = oracle.quantize(wt, fmt=oracle.FMT_IF4)
    rx = oracle.quantize(x, fmt=oracle.FMT_IF4)
    assert_bit_exact(q_to_host(gw), rw, "weight if4")
    assert_bit_exact(q_to_host(gx), rx, "x if4")
    c = nv.gemm_nvfp4(gx, gw, out_dtype=torch.float32).cpu().numpy()
    M, N = c.shape
    rng = np.random.default_rng(11)
    im = np.concatenate([rng.integers(0, M, 512), [0, M - 1]])
    in_ = np.concatenate([rng.integers(0, N, 512), [0, N - 1]])
    ref = oracle.gemm_entries(rx, rw, im, in_, fmt=oracle.FMT_IF4)
    got = c[im, in_].astype(np.float64)
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) <= 1e-5


def test_mlp_dy_dual_axis(nv, mlp):
    """dY of the MLP step quantized along both axes from one read: the same
    outputs as the oracle's row-wise and column-wise RHT + MS-EDEN."""
    _, _, dy, signs = mlp
    w = oracle.signs_words(signs)
    qr, qc = nv.quantize_nvfp4_dual(to_device(dy, "bf16"), rht_signs=signs, seed=7, stream_id=3)
    for axis, q in ((0, qr), (1, qc)):
        ref = oracle.quantize(dy, rounding=oracle.MSEDEN, axis=axis, rht_on=True, signs_w=w, seed=7, stream=3)
        assert_rotated_close(q_to_host(q), ref, what=f"dY dual axis{axis}")


def test_mlp_forward_scale_search(nv, mlp):
    """The forward operands with a searched block scale, full size, bit-exact;
    then Y = X W^T on sampled entries."""
    import torch
    x, wt, _, _ = mlp
    gx = nv.quantize_nvfp4(to_device(x, "bf16"), scale_rule="search")
    gw = nv.quantize_nvfp4(to_device(wt, "bf16"), scale_rule="search")
    rx = oracle.quantize(x, fmt=oracle.FMT_NVFP4_SEARCH)
    rw = oracle.quantize(wt, fmt=oracle.FMT_NVFP4_SEARCH)
    assert_bit_exact(q_to_host(gx), rx, "X search")
    assert_bit_exact(q_to_host(gw), rw, "W search")
    c = nv.gemm_nvfp4(gx, gw, out_dtype=torch.float32).cpu().numpy()
    sampled_gemm_check(nv, rx, rw, c, seed=5)


def test_mlp_forward_four_over_six(nv, mlp):
    """The forward pass with Four Over Six scaling of X and W: both operands
    bit-exact at full size, then Y = X W^T on sampled entries."""
    import torch
    x, wt, _, _ = mlp
    gx = nv.quantize_nvfp4(to_device(x, "bf16"), scale_rule="4over6")
    gw = nv.quantize_nvfp4(to_device(wt, "bf16"), scale_rule="4over6")
    rx = oracle.quantize(x, fmt=oracle.FMT_NVFP4_4OVER6)
    rw = oracle.quantize(wt, fmt=oracle.FMT_NVFP4_4OVER6)
    assert_bit_exact(q_to_host(gx), rx, "X 4over6")
    assert_bit_exact(q_to_host(gw), rw, "W 4over6")
    c = nv.gemm_nvfp4(gx, gw, out_dtype=torch.float32).cpu().numpy()
    sampled_gemm_check(nv, rx, rw, c, seed=4)


@pytest.mark.parametrize("which", ["Y", "dX", "dW"])
def test_mlp_step_gemms(nv, mlp, which):
    import torch
    x, wt, dy, signs = mlp
    w = oracle.signs_words(signs)
    if which == "Y":
        ra, rb = oracle.quantize(x), oracle.quantize(wt)
        out = torch.bfloat16
    elif which == "dX":
        ra = oracle.quantize(dy, rounding=oracle.MSEDEN, rht_on=True, signs_w=w, seed=1)
        rb = oracle.quantize(wt, rounding=oracle.MSEDEN, axis=1, rht_on=True, signs_w=w, seed=2)
        out = torch.bfloat16
    else:
        ra = oracle.quantize(dy, rounding=oracle.MSEDEN, axis=1, rht_on=True, signs_w=w, seed=3)
        rb = oracle.quantize(x, rounding=oracle.MSEDEN, axis=1, rht_on=True, signs_w=w, seed=4)
        out = torch.float32
    qa, qb = upload(nv, ra), upload(nv, rb)
    # the contract (fp32 output): relative Frobenius error <= 1e-3
    c32 = nv.gemm_nvfp4(qa, qb, out_dtype=torch.float32).cpu().numpy()
    assert sampled_gemm_check(nv, ra, rb, c32) <= 1e-5
    if out == torch.bfloat16:
        # the step's bf16 output: the fp32 result rounded once more
        c16 = nv.gemm_nvfp4(qa, qb, out_dtype=torch.bfloat16).float().cpu().numpy()
        rng = np.random.default_rng(1)
        im, in_ = rng.integers(0, c16.shape[0], 512), rng.integers(0, c16.shape[1], 512)
        ref = oracle.gemm_entries(ra, rb, im, in_)
        assert np.all(np.abs(c16[im, in_] - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6 * np.abs(ref).max())
