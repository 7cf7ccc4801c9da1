"""Seeded random sweep of the quantizer options against the oracle: dtype,
axis, rounding and format, scale rule, rotation, a given tensor scale,
ragged shapes and value distributions (Gaussian, heavy-tailed, sparse with
exact zeros, tiny and huge magnitudes).  Rotation off: bit-exact; rotation
on: the rotation contract.
Followed by random GEMM shapes on the swept operands."""
import numpy as np
import pytest

import oracle
from nvfp4_bit_block_amd import synth
from gpu_util import assert_bit_exact, assert_rotated_close, q_to_host, to_device

pytestmark = pytest.mark.gpu

MODES = [  # (name, oracle format, oracle rounding, binding kwargs)
    ("rtn", oracle.FMT_NVFP4, oracle.RTN, dict(rounding="rtn")),
    ("sr", oracle.FMT_NVFP4, oracle.SR, dict(rounding="sr")),
    ("mseden128", oracle.FMT_NVFP4, oracle.MSEDEN, dict(rounding="mseden", eden_group=128)),
    ("mseden16", oracle.FMT_NVFP4, oracle.MSEDEN, dict(rounding="mseden", eden_group=16)),
    ("if4", oracle.FMT_IF4, oracle.RTN, None),
    ("4over6", oracle.FMT_NVFP4_4OVER6, oracle.RTN, dict(scale_rule="4over6")),
    ("search", oracle.FMT_NVFP4_SEARCH, oracle.RTN, dict(scale_rule="search")),
]
# IF4 for gradients (swept on cases of their own, so that the cases above
# keep their draws)
MODES_IF4_GRAD = [
    ("if4_sr", oracle.FMT_IF4, oracle.SR, dict(rounding="sr", if4=True)),
    ("if4_mseden128", oracle.FMT_IF4, oracle.MSEDEN, dict(rounding="mseden", eden_group=128, if4=True)),
    ("if4_mseden16", oracle.FMT_IF4, oracle.MSEDEN, dict(rounding="mseden", eden_group=16, if4=True)),
]


def _values(rng, rows, cols, kind, dtype):
    if kind == "gauss":
        x = rng.standard_normal((rows, cols))
    elif kind == "heavy":
        x = rng.standard_t(3.0, (rows, cols)) * np.exp(rng.normal(0, 1.5, (rows, 1)))
    elif kind == "sparse":
        x = rng.standard_normal((rows, cols)) * (rng.random((rows, cols)) < 0.3)
        x[rng.random((rows, cols)) < 0.1] = -0.0
    elif kind == "tiny":
        x = rng.standard_normal((rows, cols)) * 2.0 ** -100
    else:  # "huge"
        x = rng.standard_normal((rows, cols)) * 2.0 ** 90
    x = x.astype(np.float32)
    return synth.to_bf16_f32(x) if dtype == "bf16" else x


def _case(i, modes=MODES, base=2026):
    rng = np.random.default_rng([base, i])
    name, fmt, rnd, kw = modes[i % len(modes)]
    dtype = ("bf16", "fp32")[rng.integers(0, 2)]
    axis = int(rng.integers(0, 2))
    rot = bool(rng.integers(0, 2))
    need128 = rot or name.endswith("mseden128")
    k_unit = 128 if need128 else 16
    K = int(rng.integers(1, 5 if need128 else 24)) * k_unit
    R = int(rng.integers(1, 200))
    kind = ("gauss", "heavy", "sparse", "tiny", "huge")[rng.integers(0, 5)]
    given = bool(rng.integers(0, 4) == 0)
    rows, cols = (R, K) if axis == 0 else (K, R)
    x = _values(rng, rows, cols, kind, dtype)
    signs = synth.signs_from_rng(rng) if rot else None
    return dict(name=name, fmt=fmt, rnd=rnd, kw=kw, dtype=dtype, axis=axis, rot=rot, x=x, signs=signs,
                kind=kind, given=given, seed=int(rng.integers(0, 1 << 30)), stream=int(rng.integers(0, 9)))


@pytest.fixture(scope="module")
def nv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nvfp4_bit_block_amd as m
    m.lib()
    return m


def _run(nv, c):
    import torch
    x = to_device(c["x"], c["dtype"])
    ts = None
    if c["given"]:
        amax = float(np.max(np.abs(c["x"]))) if c["x"].size else 1.0
        ts = np.float32(amax / 2688.0) if amax > 0 else np.float32(1.0)
    tsd = None if ts is None else torch.tensor([ts], device="cuda:0")
    if c["kw"] is None:
        q = nv.quantize_if4(x, axis=c["axis"], rht_signs=c["signs"], tensor_scale_in=tsd)
    elif c["kw"].get("if4"):
        kw = {k: v for k, v in c["kw"].items() if k != "if4"}
        q = nv.quantize_if4(x, axis=c["axis"], rht_signs=c["signs"], seed=c["seed"], stream_id=c["stream"],
                            tensor_scale_in=tsd, **kw)
    else:
        q = nv.quantize_nvfp4(x, axis=c["axis"], rht_signs=c["signs"], seed=c["seed"], stream_id=c["stream"],
                              tensor_scale_in=tsd, **c["kw"])
    w = None if c["signs"] is None else oracle.signs_words(c["signs"])
    ref = oracle.quantize(c["x"], fmt=c["fmt"], rounding=c["rnd"], axis=c["axis"], rht_on=c["rot"], signs_w=w,
                          seed=c["seed"], stream=c["stream"],
                          eden_group=c["kw"].get("eden_group", 128) if c["kw"] else 128,
                          ts_in=None if ts is None else float(ts))
    return q, ref


@pytest.mark.parametrize("i", range(70))
def test_quantize_sweep(nv, i):
    c = _case(i)
    q, ref = _run(nv, c)
    what = (f"case {i}: {c['name']} {c['dtype']} axis{c['axis']} {c['x'].shape} rot={c['rot']} "
            f"{c['kind']} given_ts={c['given']}")
    g = q_to_host(q)
    if c["rot"]:
        assert_rotated_close(g, ref, what=what)
    else:
        assert_bit_exact(g, ref, what)


@pytest.mark.parametrize("i", range(30))
def test_if4_gradient_sweep(nv, i):
    c = _case(i, MODES_IF4_GRAD, 2028)
    q, ref = _run(nv, c)
    what = (f"IF4 gradient case {i}: {c['name']} {c['dtype']} axis{c['axis']} {c['x'].shape} rot={c['rot']} "
            f"{c['kind']} given_ts={c['given']}")
    g = q_to_host(q)
    if c["rot"]:
        assert_rotated_close(g, ref, what=what)
    else:
        assert_bit_exact(g, ref, what)


@pytest.mark.parametrize("i", range(8))
def test_gemm_sweep(nv, i):
    """Random M, N, K (K a multiple of 16, ragged against the 256 x 256 tile
    and the 64-wide K chunk), NVFP4 or IF4 operands, fp32 or bf16 output."""
    import torch
    rng = np.random.default_rng([2027, i])
    M, N = int(rng.integers(1, 600)), int(rng.integers(1, 600))
    K = int(rng.integers(1, 40)) * 16
    fmt = (oracle.FMT_NVFP4, oracle.FMT_IF4)[i % 2]
    a = synth.to_bf16_f32(rng.standard_normal((M, K)).astype(np.float32))
    b = synth.to_bf16_f32((0.05 * rng.standard_t(4.0, (N, K))).astype(np.float32))
    quant = (lambda t: nv.quantize_if4(t)) if fmt == oracle.FMT_IF4 else (lambda t: nv.quantize_nvfp4(t))
    qa, qb = quant(to_device(a, "bf16")), quant(to_device(b, "bf16"))
    out_dtype = (torch.float32, torch.bfloat16)[rng.integers(0, 2)]
    c = nv.gemm_nvfp4(qa, qb, out_dtype=out_dtype).float().cpu().numpy().astype(np.float64)
    ra, rb = oracle.quantize(a, fmt=fmt), oracle.quantize(b, fmt=fmt)
    assert_bit_exact(q_to_host(qa), ra, f"gemm sweep {i} A")
    ref = oracle.gemm_full(ra, rb, fmt=fmt)
    if out_dtype == torch.bfloat16:
        # a bf16 result carries its own rounding (up to 2^-9 relative, about
        # 1.1e-3 in Frobenius norm): compare with the reference rounded alike
        ref = synth.to_bf16_f32(ref.astype(np.float32)).astype(np.float64)
    err = np.linalg.norm(c - ref) / max(np.linalg.norm(ref), 1e-30)
    assert err <= 1e-3, f"gemm sweep {i}: {M}x{N}x{K} {out_dtype} rel. Frobenius error {err:.2e}"
