"""Large-size parity: tensors whose byte offsets pass 2^32 and GEMM shapes
near the addressing limits.  Inputs are generated on the device; only
sampled rows and columns go to the oracle, which is exact for them because
each output row depends only on its own input row (or column) once the
tensor scale is given (RTN: per block; MS-EDEN: per 128-group)."""
import numpy as np
import pytest

import oracle
from nvfp4_bit_block_amd import synth
from gpu_util import assert_bit_exact, assert_rotated_close, q_to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nvfp4_bit_block_amd as m
    m.lib()
    return m


@pytest.fixture(scope="module")
def big():
    """65536 x 32768 bf16 (2^31 elements, 4 GiB): element offsets of the last
    rows exceed 2^31 and byte offsets 2^32."""
    import torch
    g = torch.Generator(device="cuda:0")
    g.manual_seed(123)
    x = torch.randn((65536, 32768), generator=g, device="cuda:0", dtype=torch.float32).to(torch.bfloat16)
    torch.cuda.synchronize()
    yield x
    del x
    torch.cuda.empty_cache()


def _rows(q, idx):
    return {"codes": q.codes[idx].cpu().numpy(), "scales": q.scales[idx].cpu().numpy(),
            "ts": float(q.tensor_scale.cpu().numpy()[0])}


def test_rtn_beyond_4gib_rows_and_columns(nv, big):
    import torch
    ts = np.float32(0.0021)
    tsd = torch.tensor([ts], device="cuda:0")
    rows = np.array([0, 1, 31999, 65534, 65535])
    xr = big[torch.from_numpy(rows).to("cuda:0")].float().cpu().numpy()
    q = nv.quantize_nvfp4(big, tensor_scale_in=tsd)
    assert_bit_exact(_rows(q, torch.from_numpy(rows).to("cuda:0")), oracle.quantize(xr, ts_in=float(ts)),
                     "rtn rows of a 4 GiB tensor")
    del q
    cols = np.array([0, 7, 16383, 32767])
    xc = big[:, torch.from_numpy(cols).to("cuda:0")].float().cpu().numpy()     # [65536 x 4]
    q = nv.quantize_nvfp4(big, axis=1, tensor_scale_in=tsd)
    assert_bit_exact(_rows(q, torch.from_numpy(cols).to("cuda:0")),
                     oracle.quantize(np.ascontiguousarray(xc), axis=1, ts_in=float(ts)),
                     "rtn columns of a 4 GiB tensor")


def test_mseden_rotation_beyond_4gib(nv, big):
    """Rotation + MS-EDEN with a given tensor scale on rows of the 4 GiB
    tensor.  Codes against the oracle on those rows; the scale of each block is
    stochastic (Philox keyed by the global block index), so it is checked to
    be the E4M3 value just below or just above the oracle's target t_b / s_t."""
    import torch
    ts = np.float32(0.0009)
    tsd = torch.tensor([ts], device="cuda:0")
    signs = synth.signs_from_rng(np.random.default_rng(5))
    w = oracle.signs_words(signs)
    rows = np.array([2, 40000, 65535])
    sel = torch.from_numpy(rows).to("cuda:0")
    xr = big[sel].float().cpu().numpy()
    q = nv.quantize_nvfp4(big, rounding="mseden", rht_signs=signs, seed=9, stream_id=1, tensor_scale_in=tsd)
    g = _rows(q, sel)
    ref = oracle.quantize(xr, rounding=oracle.MSEDEN, rht_on=True, signs_w=w, seed=9, stream=1,
                          ts_in=float(ts), want_tb=True)
    assert g["ts"] == ref["ts"]
    assert_rotated_close({"codes": g["codes"], "scales": ref["scales"], "ts": g["ts"]}, ref,
                         what="mseden codes of rows of a 4 GiB tensor")
    grid = np.array([oracle.e4m3_value(b) for b in range(127)], dtype=np.float64)
    target = np.minimum(ref["tb"].astype(np.float64) / np.float64(ts), 448.0).ravel()
    lo = np.searchsorted(grid, target, side="right") - 1
    hi = np.minimum(lo + (grid[lo] < target), 126)
    e = g["scales"].ravel().astype(np.int64)
    assert np.all((e == lo) | (e == hi))
    assert np.any(e != lo) and np.any(e == lo)     # both directions of the rounding occur


def _random_operand(torch, rows, K, seed):
    g = torch.Generator(device="cuda:0")
    g.manual_seed(seed)
    codes = torch.randint(0, 256, (rows, K // 2), generator=g, device="cuda:0", dtype=torch.uint8)
    scales = torch.randint(0x30, 0x48, (rows, K // 16), generator=g, device="cuda:0", dtype=torch.uint8)
    return codes, scales


@pytest.mark.parametrize("K", [1 << 22, (1 << 22) - 16])
def test_gemm_long_k(nv, K):
    """K = 2^22 on the vector-load path and K = 2^22 - 16 on the element-wise
    path (K % 64 != 0): 256 x 256 outputs, sampled entries against the fp64
    oracle."""
    import torch
    ac, asc = _random_operand(torch, 256, K, 1)
    bc, bsc = _random_operand(torch, 256, K, 2)
    ts = torch.tensor([0.5], device="cuda:0")
    a = nv.QTensor(ac, asc, ts, nv.FORMAT_NVFP4)
    b = nv.QTensor(bc, bsc, ts, nv.FORMAT_NVFP4)
    c = nv.gemm_nvfp4(a, b).cpu().numpy()
    rng = np.random.default_rng(3)
    im = np.concatenate([rng.integers(0, 256, 12), [0, 255]])
    in_ = np.concatenate([rng.integers(0, 256, 12), [255, 0]])
    ra = {"codes": ac.cpu().numpy(), "scales": asc.cpu().numpy(), "ts": np.float32(0.5)}
    rb = {"codes": bc.cpu().numpy(), "scales": bsc.cpu().numpy(), "ts": np.float32(0.5)}
    ref = oracle.gemm_entries(ra, rb, im, in_)
    got = c[im, in_].astype(np.float64)
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) <= 1e-3


def test_gemm_operand_beyond_4gib(nv):
    """A = 2^22 x 4096 (8 GiB of codes; row offsets pass 2^32), B = 256 x 4096,
    C bf16 [2^22 x 256] (16384 tiles): sampled entries, including the last
    rows, against the oracle on the sampled rows."""
    import torch
    M, N, K = 1 << 22, 256, 4096
    ac, asc = _random_operand(torch, M, K, 4)
    bc, bsc = _random_operand(torch, N, K, 5)
    ts = torch.tensor([0.25], device="cuda:0")
    a = nv.QTensor(ac, asc, ts, nv.FORMAT_NVFP4)
    b = nv.QTensor(bc, bsc, ts, nv.FORMAT_NVFP4)
    c = nv.gemm_nvfp4(a, b, out_dtype=torch.bfloat16)
    rng = np.random.default_rng(6)
    im = np.concatenate([rng.integers(0, M, 30), [M - 1, M - 2, (1 << 21) + 5]])
    in_ = np.concatenate([rng.integers(0, N, 30), [N - 1, 0, 17]])
    sel = torch.from_numpy(im).to("cuda:0")
    got = c[sel, torch.from_numpy(in_).to("cuda:0")].float().cpu().numpy().astype(np.float64)
    ra = {"codes": ac[sel].cpu().numpy(), "scales": asc[sel].cpu().numpy(), "ts": np.float32(0.25)}
    rb = {"codes": bc.cpu().numpy(), "scales": bsc.cpu().numpy(), "ts": np.float32(0.25)}
    ref = oracle.gemm_entries(ra, rb, np.arange(im.size), in_)
    # bf16 output: one more rounding (2^-9 relative) on top of the fp32 result
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-3 * np.abs(ref).max())
    del c, ac, asc
    torch.cuda.empty_cache()
