"""GPU GEMM with its output coded as NVFP4 in the same kernel
(nvfp4_gemm_nvfp4_rtn) against the oracle: the oracle's product, as fp32,
coded by the oracle's RTN with the same given tensor scale.

Where the product is exact in fp32 (operands whose block scales are all 1.0,
so every product is a multiple of 1/4 and every sum stays far below 2^24
quarter units) the codes must be bit-exact.  For general operands the fp32
accumulation differs from the fp64 product by rounding, so a code can sit on
the other side of a rounding boundary: at most 1e-5 of codes and scales may
differ, by one level.  The fused path must also equal, bit for bit, the
library's own fp32 GEMM followed by its RTN quantizer with the same tensor
scale."""
import numpy as np
import pytest

import oracle
from gpu_util import assert_bit_exact, assert_rotated_close, q_to_host

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


def unit_scale_operand(rng, rows, K):
    """Random E2M1 codes, every block scale E4M3 1.0 (byte 0x38), tensor scale 1."""
    return {"codes": rng.integers(0, 256, (rows, K // 2), dtype=np.uint8),
            "scales": np.full((rows, K // 16), 0x38, dtype=np.uint8), "ts": 1.0}


def exact_product(a, b):
    da = oracle.dequantize(a["codes"], a["scales"], a["ts"]).astype(np.float64)
    db = oracle.dequantize(b["codes"], b["scales"], b["ts"]).astype(np.float64)
    return da @ db.T


@pytest.mark.parametrize("M,N,K", [(300, 272, 128), (513, 528, 64), (64, 16, 16), (257, 1040, 80),
                                   (4100, 4512, 64)])
def test_gemm_rtn_bit_exact_on_exact_products(nv, M, N, K):
    import torch
    rng = np.random.default_rng(M + 3 * N + 7 * K)
    a, b = unit_scale_operand(rng, M, K), unit_scale_operand(rng, N, K)
    c = exact_product(a, b)
    assert np.all(c == c.astype(np.float32))
    ts = np.float32(np.abs(c).max() / (6 * 448))
    ref = oracle.quantize(c.astype(np.float32), ts_in=ts)
    amax = torch.full((1,), -1.0, dtype=torch.float32, device="cuda:0")
    q = nv.gemm_nvfp4_rtn(upload(nv, a), upload(nv, b),
                          torch.tensor([ts], dtype=torch.float32, device="cuda:0"), amax_out=amax)
    assert_bit_exact(q_to_host(q), ref, f"gemm rtn {M}x{N}x{K}")
    assert float(amax.cpu()[0]) == float(np.abs(c).max())


@pytest.mark.parametrize("M,N,K", [(256, 512, 512), (200, 304, 1040)])
def test_gemm_rtn_against_oracle_product(nv, M, N, K):
    import torch
    rng = np.random.default_rng(M * N + K)
    a = oracle.quantize(rng.standard_normal((M, K)).astype(np.float32))
    b = oracle.quantize((0.05 * rng.standard_normal((N, K))).astype(np.float32), rounding=oracle.SR, seed=3)
    c = oracle.gemm_full(a, b)
    ts = np.float32(np.abs(c).max() / (6 * 448))
    ref = oracle.quantize(c.astype(np.float32), ts_in=ts)
    amax = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    q = nv.gemm_nvfp4_rtn(upload(nv, a), upload(nv, b),
                          torch.tensor([ts], dtype=torch.float32, device="cuda:0"), amax_out=amax)
    assert_rotated_close(q_to_host(q), ref, frac=1e-5, what=f"gemm rtn {M}x{N}x{K}")
    assert abs(float(amax.cpu()[0]) - np.abs(c).max()) <= 1e-5 * np.abs(c).max()


def test_gemm_rtn_equals_gemm_then_quantizer(nv):
    """Same fp32 values, same RTN: the fused output equals the library's fp32
    GEMM followed by its RTN quantizer, and max |C| equals the fp32 C's."""
    import torch
    rng = np.random.default_rng(11)
    M, N, K = 1000, 1536, 1024
    a = upload(nv, oracle.quantize(rng.standard_normal((M, K)).astype(np.float32)))
    b = upload(nv, oracle.quantize((0.02 * rng.standard_normal((N, K))).astype(np.float32)))
    c32 = nv.gemm_nvfp4(a, b)
    ts = (c32.abs().max() / 2688.0).reshape(1).contiguous()
    q_ref = nv.quantize_nvfp4(c32, rounding="rtn", tensor_scale_in=ts)
    amax = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    q = nv.gemm_nvfp4_rtn(a, b, ts, amax_out=amax)
    assert torch.equal(q.codes, q_ref.codes) and torch.equal(q.scales, q_ref.scales)
    assert float(amax.cpu()[0]) == float(c32.abs().max().cpu())


def test_gemm_rtn_empty_and_no_amax(nv):
    import torch
    z = torch.zeros((0, 32), dtype=torch.uint8, device="cuda:0")
    e = nv.QTensor(z, torch.zeros((0, 4), dtype=torch.uint8, device="cuda:0"),
                   torch.ones(1, dtype=torch.float32, device="cuda:0"), nv.FORMAT_NVFP4)
    rng = np.random.default_rng(2)
    b = upload(nv, unit_scale_operand(rng, 32, 64))
    amax = torch.full((1,), -1.0, dtype=torch.float32, device="cuda:0")
    q = nv.gemm_nvfp4_rtn(e, b, e.tensor_scale, amax_out=amax)
    assert q.codes.shape == (0, 16) and float(amax.cpu()[0]) == 0.0
    a = unit_scale_operand(rng, 40, 64)
    c = exact_product(a, {"codes": b.codes.cpu().numpy(), "scales": b.scales.cpu().numpy(), "ts": 1.0})
    ts = np.float32(np.abs(c).max() / (6 * 448))
    q = nv.gemm_nvfp4_rtn(upload(nv, a), b, torch.tensor([ts], dtype=torch.float32, device="cuda:0"))
    assert_bit_exact(q_to_host(q), oracle.quantize(c.astype(np.float32), ts_in=ts), "gemm rtn, no amax")
