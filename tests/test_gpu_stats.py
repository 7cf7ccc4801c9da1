"""Statistical properties of the GPU quantizers on the pages' workloads:
the SR error closed form on the 256x256 N(0,1) case, Monte-Carlo
unbiasedness of SR and MS-EDEN on a 64x128 slice of the gradient case
(1000 trials, rotation signs and Philox streams redrawn per trial), and the
MS-EDEN error gain over SR (more than 2x, Quartet II abstract)."""
import numpy as np
import pytest

import oracle
from nvfp4_bit_block_amd import synth
from gpu_util import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nvfp4_bit_block_amd as m
    m.lib()
    return m


def test_sr_error_closed_form_256(nv):
    import torch
    x = synth.gaussian(256, 256, seed=0)
    xt = to_device(x, "fp32")
    T = 1000
    acc = torch.zeros((256, 256), dtype=torch.float64, device="cuda:0")
    acc2 = torch.zeros_like(acc)
    for t in range(T):
        q = nv.quantize_nvfp4(xt, rounding="sr", seed=0, stream_id=t)
        d = nv.dequantize(q).double()
        acc += d
        acc2 += (d - xt.double()) ** 2
    # closed form S^2 (y - l)(u - y) from the oracle's (deterministic) scales
    ref = oracle.quantize(x, rounding=oracle.SR, seed=0, stream=0)
    grid = np.array([oracle.e2m1_value(c) for c in range(8)], dtype=np.float64)
    e4 = np.array([oracle.e4m3_value(b) for b in range(128)], dtype=np.float64)
    S = e4[np.repeat(ref["scales"], 16, axis=1)] * np.float64(ref["ts"])
    y = np.minimum(np.abs(x) / S, 6.0)
    j = np.clip(np.searchsorted(grid, y, side="right") - 1, 0, 6)
    closed = S * S * np.clip((y - grid[j]) * (grid[j + 1] - y), 0, None)
    emp = acc2.cpu().numpy() / T
    assert emp.sum() == pytest.approx(closed.sum(), rel=0.02)
    bias = acc.cpu().numpy() / T - x
    assert np.abs(bias).max() < 6 * np.sqrt(closed.max() / T)
    assert abs(bias.sum()) < 5 * np.sqrt(closed.sum() / T)


def _mc_projection(nv, x, rounding, T=1000):
    import torch
    xt = to_device(x, "bf16")
    acc = torch.zeros(x.shape, dtype=torch.float64, device="cuda:0")
    for t in range(T):
        signs = synth.mc_signs(t)
        q = nv.quantize_nvfp4(xt, rounding=rounding, rht_signs=signs, seed=1, stream_id=t)
        acc += nv.dequantize(q, inv_rht_signs=signs).double()
    mean = acc.cpu().numpy() / T
    x64 = x.astype(np.float64)
    return float((mean * x64).sum() / (x64 * x64).sum()), mean


def test_mc_unbiased_gradient_slice(nv):
    x, _ = synth.gradient(4096, 4096, seed=1)
    x = np.ascontiguousarray(x[:64, :128])
    p_sr, _ = _mc_projection(nv, x, "sr")
    p_ed, mean_ed = _mc_projection(nv, x, "mseden")
    p_rtn, _ = _mc_projection(nv, x, "rtn", T=300)
    assert abs(p_sr - 1.0) < 1.5e-3
    assert abs(p_ed - 1.0) < 1.5e-3
    assert abs(p_rtn - 1.0) > 2e-3      # negative control: RTN is biased
    # elementwise: the MS-EDEN mean error shrinks like 1/sqrt(T)
    rel = np.linalg.norm(mean_ed - x) / np.linalg.norm(x)
    assert rel < 0.02


def test_mseden_error_below_half_of_sr(nv):
    x, signs = synth.gradient(4096, 4096, seed=1)
    xt = to_device(x, "bf16")
    mse = {}
    for r in ("sr", "mseden"):
        q = nv.quantize_nvfp4(xt, rounding=r, rht_signs=signs, seed=2, stream_id=0)
        d = nv.dequantize(q, inv_rht_signs=signs)
        mse[r] = float(((d.double() - xt.double()) ** 2).mean())
    assert mse["sr"] / mse["mseden"] > 2.0
