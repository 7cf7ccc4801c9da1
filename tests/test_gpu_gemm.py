"""GPU block-scaled FP4 GEMM against the oracle's fp64 GEMM on the same
packed operands (quantized by the oracle, uploaded).  Bar: relative Frobenius
error <= 1e-3 with fp32 output; the dequantized products are exact in fp16,
so the only error is fp32 accumulation order."""
import numpy as np
import pytest

import oracle
from nvfp4_bit_block_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nvfp4_bit_block_amd as m
    m.lib()
    return m


def upload(nv, ref, fmt=None):
    import torch
    return nv.QTensor(torch.from_numpy(ref["codes"]).to("cuda:0"),
                      torch.from_numpy(ref["scales"]).to("cuda:0"),
                      torch.tensor([ref["ts"]], dtype=torch.float32, device="cuda:0"),
                      nv.FORMAT_NVFP4 if fmt is None else fmt)


def rel_fro(got, ref):
    return float(np.linalg.norm(got.astype(np.float64) - ref) / np.linalg.norm(ref))


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (300, 200, 528), (1, 17, 64), (513, 259, 1024),
                                   (64, 640, 2064), (768, 512, 4096)])
def test_gemm_small_shapes(nv, M, N, K):
    import torch
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    a = oracle.quantize(rng.standard_normal((M, K)).astype(np.float32))
    b = oracle.quantize((0.02 * rng.standard_normal((N, K))).astype(np.float32), rounding=oracle.SR, seed=1)
    ref = oracle.gemm_full(a, b)
    c = nv.gemm_nvfp4(upload(nv, a), upload(nv, b)).cpu().numpy()
    assert c.shape == (M, N)
    assert rel_fro(c, ref) <= 1e-3
    assert rel_fro(c, ref) <= 1e-5   # in practice: fp32 accumulation only
    c16 = nv.gemm_nvfp4(upload(nv, a), upload(nv, b), out_dtype=torch.bfloat16).float().cpu().numpy()
    # bf16 output: the fp32 result rounded once more (2^-9 relative) plus accumulation noise
    assert np.all(np.abs(c16 - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6 * np.abs(ref).max())


def test_gemm_ldc_and_strided_output(nv):
    import torch
    rng = np.random.default_rng(5)
    a = oracle.quantize(rng.standard_normal((130, 256)).astype(np.float32))
    b = oracle.quantize(rng.standard_normal((70, 256)).astype(np.float32))
    ref = oracle.gemm_full(a, b)
    big = torch.full((130, 96), -7.0, dtype=torch.float32, device="cuda:0")
    out = big[:, 10:80]
    nv.gemm_nvfp4(upload(nv, a), upload(nv, b), out=out)
    h = big.cpu().numpy()
    assert rel_fro(h[:, 10:80], ref) <= 1e-5
    assert np.all(h[:, :10] == -7.0) and np.all(h[:, 80:] == -7.0)


@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
@pytest.mark.parametrize("M,N,ldc", [(300, 259, 264), (70, 202, 208), (257, 520, 520)])
def test_gemm_output_rows_with_aligned_stride(nv, dtype, M, N, ldc):
    """Output rows whose starts are 16-byte aligned (full-width stores) with a
    ragged last column group and ragged rows: every element of [M x N] is
    written once and the columns N .. ldc-1 of each row stay untouched."""
    import torch
    rng = np.random.default_rng(M + N + ldc)
    K = 320
    a = oracle.quantize(rng.standard_normal((M, K)).astype(np.float32))
    b = oracle.quantize(rng.standard_normal((N, K)).astype(np.float32))
    ref = oracle.gemm_full(a, b)
    td = getattr(torch, dtype)
    big = torch.full((M, ldc), -7.0, dtype=td, device="cuda:0")
    nv.gemm_nvfp4(upload(nv, a), upload(nv, b), out=big[:, :N])
    h = big.float().cpu().numpy()
    if dtype == "float32":
        assert rel_fro(h[:, :N], ref) <= 1e-5
    else:
        assert np.all(np.abs(h[:, :N] - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6 * np.abs(ref).max())
    assert np.all(h[:, N:] == -7.0)


def test_gemm_more_tiles_than_workgroups(nv):
    """17 x 18 = 306 output tiles of 256 x 256, more than one per compute
    unit, so workgroups take several tiles each; ragged in M and N.  Checked
    on the first, last and one random row and column of every tile (every
    tile's corners and the ragged edges), in fp32 and bf16."""
    import torch
    rng = np.random.default_rng(306)
    M, N, K = 4100, 4500, 64
    a = oracle.quantize(rng.standard_normal((M, K)).astype(np.float32))
    b = oracle.quantize(rng.standard_normal((N, K)).astype(np.float32))

    def picks(n):
        out = []
        for t0 in range(0, n, 256):
            t1 = min(t0 + 256, n)
            out += [t0, int(rng.integers(t0, t1)), t1 - 1]
        return np.array(out)
    rows, cols = picks(M), picks(N)
    im, in_ = np.repeat(rows, cols.size), np.tile(cols, rows.size)
    ref = oracle.gemm_entries(a, b, im, in_)
    c = nv.gemm_nvfp4(upload(nv, a), upload(nv, b)).cpu().numpy()[im, in_]
    assert rel_fro(c, ref) <= 1e-5
    c16 = nv.gemm_nvfp4(upload(nv, a), upload(nv, b), out_dtype=torch.bfloat16).float().cpu().numpy()[im, in_]
    assert np.all(np.abs(c16 - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6 * np.abs(ref).max())


def test_gemm_rotated_operands_match_unrotated_product(nv):
    """With the same signs on both operands, (H D a) . (H D b) = a . b: the
    GEMM of rotated, MS-EDEN-quantized operands estimates A B^T."""
    rng = np.random.default_rng(6)
    signs = synth.signs_from_rng(rng)
    w = oracle.signs_words(signs)
    A = rng.standard_normal((128, 1024)).astype(np.float32)
    B = rng.standard_normal((96, 1024)).astype(np.float32)
    qa = oracle.quantize(A, rounding=oracle.MSEDEN, rht_on=True, signs_w=w, seed=1)
    qb = oracle.quantize(B, rounding=oracle.MSEDEN, rht_on=True, signs_w=w, seed=2)
    c = nv.gemm_nvfp4(upload(nv, qa), upload(nv, qb)).cpu().numpy()
    ref = A.astype(np.float64) @ B.T.astype(np.float64)
    assert rel_fro(c, oracle.gemm_full(qa, qb)) <= 1e-5
    assert rel_fro(c, ref) < 0.2     # a 4-bit estimate of the exact product


def test_gemm_subnormal_and_zero_scales(nv):
    """Rows spanning 2^0 .. 2^-30 in magnitude under one tensor scale give
    subnormal and zero E4M3 block scales; all-zero blocks give scale 0."""
    rng = np.random.default_rng(7)
    A = rng.standard_normal((96, 512)).astype(np.float32)
    A *= (2.0 ** -(np.arange(96) % 31)).astype(np.float32)[:, None]
    A[5, 32:64] = 0.0
    B = rng.standard_normal((64, 512)).astype(np.float32)
    B *= (2.0 ** -(np.arange(64) % 17)).astype(np.float32)[:, None]
    qa, qb = oracle.quantize(A), oracle.quantize(B, rounding=oracle.SR, seed=3)
    assert np.any((qa["scales"] > 0) & (qa["scales"] < 8))       # subnormal E4M3 scales
    assert np.any(qa["scales"] == 0)
    ref = oracle.gemm_full(qa, qb)
    c = nv.gemm_nvfp4(upload(nv, qa), upload(nv, qb)).cpu().numpy()
    assert rel_fro(c, ref) <= 1e-5
    # row by row as well: tiny rows must not be swamped by large ones
    for r in (0, 9, 20, 30, 60, 90):
        nr = np.linalg.norm(ref[r])
        if nr > 0:
            assert np.linalg.norm(c[r] - ref[r]) <= 1e-5 * nr


# ---------------------------------------------------------------- IF4 operands
@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (300, 200, 528), (1, 17, 64), (513, 259, 1024),
                                   (64, 640, 2064)])
def test_gemm_if4_operands(nv, M, N, K):
    """IF4 operands (INT-flagged blocks hold integers 0..7): the oracle's fp64
    GEMM on the same packed operands; also IF4 x NVFP4 (an NVFP4 tensor is an
    IF4 tensor without flags)."""
    import torch
    a = oracle.quantize(synth.weight(M, K, seed=M + K), fmt=oracle.FMT_IF4)
    b = oracle.quantize(synth.weight(N, K, seed=N + 2 * K), fmt=oracle.FMT_IF4)
    assert np.any(a["scales"] >= 0x80) and np.any(a["scales"] < 0x80)
    ref = oracle.gemm_full(a, b, fmt=oracle.FMT_IF4)
    c = nv.gemm_nvfp4(upload(nv, a, nv.FORMAT_IF4), upload(nv, b, nv.FORMAT_IF4)).cpu().numpy()
    assert rel_fro(c, ref) <= 1e-3
    assert rel_fro(c, ref) <= 1e-5
    bn = oracle.quantize(synth.gaussian(N, K, seed=N + 3 * K))
    ref = oracle.gemm_full(a, bn, fmt=oracle.FMT_IF4)
    c = nv.gemm_nvfp4(upload(nv, a, nv.FORMAT_IF4), upload(nv, bn)).cpu().numpy()
    assert rel_fro(c, ref) <= 1e-5
    c16 = nv.gemm_nvfp4(upload(nv, a, nv.FORMAT_IF4), upload(nv, bn), out_dtype=torch.bfloat16)
    c16 = c16.float().cpu().numpy()
    assert np.all(np.abs(c16 - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6 * np.abs(ref).max())


def test_gemm_if4_every_code_and_flag(nv):
    """Every nibble 0..15 under both flags, with subnormal and normal scales,
    in one operand; the other operand is a one-hot selector, so each output
    entry is one dequantized value times a known scale."""
    K = 256
    rng = np.random.default_rng(31)
    codes = rng.integers(0, 256, (64, K // 2), dtype=np.uint8)
    codes[0, :8] = np.array([0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE], dtype=np.uint8)
    scales = rng.integers(1, 0x7F, (64, K // 16), dtype=np.uint8)
    scales[:, ::2] |= 0x80                  # every other block INT-flagged
    scales[1, :] = np.arange(1, 17) | 0x80   # small (subnormal) scales
    a = {"codes": codes, "scales": scales, "ts": np.float32(0.75)}
    eye = np.eye(K, dtype=np.float32)
    b = oracle.quantize(eye)
    assert np.all(b["scales"][b["scales"] != 0] == 0x7E)     # the one-hot blocks: 6 x 448
    ref = oracle.gemm_full(a, b, fmt=oracle.FMT_IF4)
    c = nv.gemm_nvfp4(upload(nv, a, nv.FORMAT_IF4), upload(nv, b)).cpu().numpy().astype(np.float64)
    # one exact product per entry; the GPU then rounds twice in fp32 (the
    # scale product, then the result), the oracle scales in fp64
    assert np.all(np.abs(c - ref) <= 2.0 ** -22 * np.abs(ref))
    assert np.array_equal(c == 0, ref == 0)
