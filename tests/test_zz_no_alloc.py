"""The allocation-free entry point nvfp4_quantize_nvfp4_noalloc, called
through the C ABI: its results equal those of nvfp4_quantize_nvfp4 with a
workspace, bit for bit, on two calls in a row (the second on a smaller
input, reusing the scratch the first left behind), for every rounding and
both axes; requests beyond its scratch are refused before anything runs."""
import ctypes

import numpy as np
import pytest

from nvfp4_bit_block_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nvfp4_bit_block_amd as m
    m.lib()
    return m


def _qt(nv, R, K):
    import torch
    return nv.QTensor(torch.full((R, K // 2), 0xAB, dtype=torch.uint8, device="cuda:0"),
                      torch.full((R, K // 16), 0xCD, dtype=torch.uint8, device="cuda:0"),
                      torch.full((1,), -7.0, dtype=torch.float32, device="cuda:0"))


def _noalloc(nv, x, q, **kw):
    """One call of the C entry point (arguments marshalled by hand)."""
    import torch
    rows, cols = x.shape
    o = nv._opts(kw.get("rounding", nv.RTN), kw.get("axis", 0), kw.get("rht_signs"), kw.get("seed", 0),
                 kw.get("stream_id", 0), kw.get("eden_group", 128), None)
    rc = nv.lib().nvfp4_quantize_nvfp4_noalloc(
        ctypes.c_void_p(x.data_ptr()), 1 if x.dtype == torch.bfloat16 else 0, rows, cols, x.stride(0),
        ctypes.byref(o), ctypes.c_void_p(q.codes.data_ptr()), ctypes.c_void_p(q.scales.data_ptr()),
        ctypes.c_void_p(q.tensor_scale.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return rc


CASES = [("rtn", dict(rounding=0)), ("sr_rot", dict(rounding=1, rot=True, seed=5, stream_id=2)),
         ("eden128_rot", dict(rounding=2, rot=True, seed=7)), ("eden16", dict(rounding=2, eden_group=16, seed=9))]


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("name,kw", CASES)
def test_noalloc_matches_workspace_entry(nv, name, kw, axis):
    import torch
    kw = dict(kw)
    signs = synth.signs_from_rng(np.random.default_rng(5)) if kw.pop("rot", False) else None
    # first a large call, then a smaller one over the scratch the first left
    for i, (r, c) in enumerate([(1024, 2048), (256, 384)]):
        x = torch.from_numpy(synth.gradient(r, c, seed=40 + i)[0]).to(torch.bfloat16).to("cuda:0")
        R, K = (r, c) if axis == 0 else (c, r)
        got = _qt(nv, R, K)
        assert _noalloc(nv, x, got, axis=axis, rht_signs=signs, **kw) == 0, nv.lib().nvfp4_last_error()
        torch.cuda.synchronize()
        want = nv.quantize_nvfp4(x, axis=axis, rht_signs=signs, **kw)
        torch.cuda.synchronize()
        assert torch.equal(got.codes, want.codes), f"{name} axis {axis} call {i}: codes"
        assert torch.equal(got.scales, want.scales), f"{name} axis {axis} call {i}: scales"
        assert torch.equal(got.tensor_scale, want.tensor_scale), f"{name} axis {axis} call {i}: tensor scale"


def test_noalloc_binding_and_limits(nv):
    import torch
    x = torch.from_numpy(synth.gaussian(128, 256, seed=3)).to("cuda:0")
    q = nv.quantize_nvfp4_noalloc(x, _qt(nv, 128, 256), rounding="mseden")
    want = nv.quantize_nvfp4(x, rounding="mseden")
    assert torch.equal(q.codes, want.codes) and torch.equal(q.scales, want.scales)
    # an empty tensor: the tensor scale is 1
    e = _qt(nv, 0, 256)
    assert _noalloc(nv, torch.empty((0, 256), device="cuda:0"), e) == 0
    assert float(e.tensor_scale.cpu()[0]) == 1.0
    # MS-EDEN on more blocks than the scratch holds: refused on the host
    # (shape only; the pointers are never used)
    o = nv._opts(nv.MSEDEN, 0, None, 0, 0, 128, None)
    big = nv.lib().nvfp4_quantize_nvfp4_noalloc(ctypes.c_void_p(256), 1, 1 << 16, 6272, 6272, ctypes.byref(o),
                                                ctypes.c_void_p(256), ctypes.c_void_p(256), ctypes.c_void_p(256),
                                                None)
    assert big == -6 and b"scratch" in nv.lib().nvfp4_last_error()
    torch.cuda.synchronize()
