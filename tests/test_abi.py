"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments with the documented status codes
before enqueuing anything (the checks are host-side; no call here reaches a
launch)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")

OK, INVALID, SHAPE, MISALIGNED, WS_SMALL, HIP_ERR, UNSUPPORTED = 0, -1, -2, -3, -4, -5, -6
FAKE = 0x7f0000000000   # 256-byte aligned, never dereferenced


@pytest.fixture(scope="module")
def nv():
    import nvfp4_bit_block_amd as m
    if not os.path.exists(m.LIB_PATH):
        from nvfp4_bit_block_amd import build
        build.build()
    m.lib()
    return m


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(nvfp4_[a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


def test_header_functions_exported(nv):
    names = declared_functions()
    assert len(names) >= 10
    L = nv.lib()
    for n in names:
        assert hasattr(L, n), n


def test_version_and_strings(nv):
    L = nv.lib()
    assert nv.abi_version() == 5
    for st, text in ((OK, b"ok"), (INVALID, b"invalid argument"), (SHAPE, b"bad shape"),
                     (MISALIGNED, b"misaligned pointer or stride"), (WS_SMALL, b"workspace too small"),
                     (HIP_ERR, b"HIP error"), (UNSUPPORTED, b"unsupported")):
        assert L.nvfp4_status_string(st) == text


def _opts(nv, **kw):
    o = nv._Opts()
    nv.lib().nvfp4_opts_init(ctypes.byref(o))
    for k, v in kw.items():
        setattr(o, k, v)
    return o


def _q(nv, rows=64, cols=256, ld=None, dtype=1, x=FAKE, codes=FAKE, scales=FAKE, ts=FAKE, ws=FAKE,
       ws_bytes=1 << 30, fn="nvfp4_quantize_nvfp4", **kw):
    o = _opts(nv, **kw)
    f = getattr(nv.lib(), fn)
    return f(ctypes.c_void_p(x), dtype, rows, cols, cols if ld is None else ld, ctypes.byref(o),
             ctypes.c_void_p(codes), ctypes.c_void_p(scales), ctypes.c_void_p(ts), ctypes.c_void_p(ws),
             ws_bytes, None)


def test_workspace_size(nv):
    L = nv.lib()
    o = _opts(nv)
    assert L.nvfp4_workspace_size(64, 256, ctypes.byref(o)) == 16384
    o = _opts(nv, rounding=2)
    assert L.nvfp4_workspace_size(64, 256, ctypes.byref(o)) == 16384 + 64 * 16 * 4
    o = _opts(nv, rounding=2, axis=1)
    assert L.nvfp4_workspace_size(256, 64, ctypes.byref(o)) == 16384 + 64 * 16 * 4
    assert L.nvfp4_workspace_size(-1, 4, ctypes.byref(o)) == 0


def test_quantize_rejections(nv):
    L = nv.lib()
    assert _q(nv, cols=100) == SHAPE                      # K % 16
    assert _q(nv, cols=144, rht=1) == SHAPE               # K % 128 with rotation
    assert _q(nv, cols=144, rounding=2) == SHAPE          # MS-EDEN group 128
    assert _q(nv, rows=144, cols=64, axis=1, rht=1) == SHAPE   # axis 1: K = rows
    assert _q(nv, rows=100, cols=64, axis=1) == SHAPE     # axis 1: K = rows
    assert _q(nv, rounding=7) == INVALID
    assert _q(nv, axis=2) == INVALID
    assert _q(nv, rht=3) == INVALID
    assert _q(nv, rounding=2, eden_group=32) == INVALID
    assert _q(nv, dtype=5) == INVALID
    assert _q(nv, rows=-1) == INVALID
    assert _q(nv, ld=128) == SHAPE                        # ld < cols
    assert _q(nv, x=0) == INVALID
    assert _q(nv, codes=0) == INVALID
    assert _q(nv, ts=0) == INVALID
    assert _q(nv, x=FAKE + 8) == MISALIGNED
    assert _q(nv, ld=260, dtype=1) == MISALIGNED          # 520-byte rows
    # axis 1: rows of up to 16 MiB pass the shape checks (and fail later, on
    # the workspace); one element more is unsupported
    assert _q(nv, rows=128, axis=1, ld=1 << 23, ws_bytes=100) == WS_SMALL
    assert _q(nv, rows=128, axis=1, ld=(1 << 23) + 8, ws_bytes=100) == UNSUPPORTED
    assert _q(nv, rows=128, axis=1, ld=1 << 22, dtype=0, ws_bytes=100) == WS_SMALL
    assert _q(nv, rows=128, axis=1, ld=(1 << 22) + 4, dtype=0, ws_bytes=100) == UNSUPPORTED
    assert _q(nv, codes=FAKE + 4) == MISALIGNED
    assert _q(nv, ws=FAKE + 16) == MISALIGNED
    assert _q(nv, ws_bytes=100) == WS_SMALL
    # IF4 takes all three roundings (SR and MS-EDEN for gradients); the MS-EDEN
    # workspace holds the target scales, so a small one is rejected
    assert _q(nv, fn="nvfp4_quantize_if4", rounding=1, ws_bytes=100) == WS_SMALL   # accepted (fails later)
    assert _q(nv, fn="nvfp4_quantize_if4", rounding=2, ws_bytes=16384) == WS_SMALL
    assert _q(nv, fn="nvfp4_quantize_if4", rounding=3) == INVALID
    assert _q(nv, fn="nvfp4_quantize_if4", rounding=2, amax_out=FAKE, ws_bytes=100) == WS_SMALL
    assert _q(nv, scale_rule=3) == INVALID
    assert _q(nv, scale_rule=2, rounding=1) == INVALID        # scale search: RTN only
    assert _q(nv, scale_rule=1, rounding=1) == INVALID        # Four Over Six: RTN only
    assert _q(nv, scale_rule=1, rounding=2) == INVALID
    assert _q(nv, fn="nvfp4_quantize_if4", scale_rule=1) == INVALID
    # amax_out: MS-EDEN with a computed tensor scale only; amax_in: no
    # rotation, no given tensor scale, not MS-EDEN; both 4-byte aligned
    assert _q(nv, rounding=2, amax_out=FAKE, ws_bytes=100) == WS_SMALL   # accepted (fails later)
    assert _q(nv, rounding=2, axis=1, rows=256, cols=64, amax_out=FAKE, ws_bytes=100) == WS_SMALL
    assert _q(nv, rounding=0, amax_out=FAKE) == UNSUPPORTED
    assert _q(nv, rounding=2, amax_out=FAKE, tensor_scale_in=FAKE) == UNSUPPORTED
    assert _q(nv, rounding=2, amax_out=FAKE + 2) == MISALIGNED
    assert _q(nv, amax_in=FAKE, ws_bytes=100) == WS_SMALL                 # RTN: accepted
    assert _q(nv, rounding=1, amax_in=FAKE, ws_bytes=100) == WS_SMALL     # SR
    assert _q(nv, fn="nvfp4_quantize_if4", amax_in=FAKE, ws_bytes=100) == WS_SMALL
    assert _q(nv, rounding=2, amax_in=FAKE) == UNSUPPORTED
    assert _q(nv, rht=1, amax_in=FAKE) == UNSUPPORTED
    assert _q(nv, amax_in=FAKE, tensor_scale_in=FAKE) == UNSUPPORTED
    assert _q(nv, amax_in=FAKE + 1) == MISALIGNED
    _q(nv, cols=100)
    assert b"multiple of 16" in L.nvfp4_last_error()


def test_dual_rejections_and_workspace(nv):
    L = nv.lib()
    P = ctypes.c_void_p
    o = _opts(nv, rounding=2)
    w0 = L.nvfp4_workspace_size(128, 256, ctypes.byref(_opts(nv, rounding=2)))
    w1 = L.nvfp4_workspace_size(128, 256, ctypes.byref(_opts(nv, rounding=2, axis=1)))
    assert L.nvfp4_workspace_size_dual(128, 256, ctypes.byref(o)) == w0 + w1

    def d(rows=128, cols=256, ws_bytes=1 << 30, **kw):
        oo = _opts(nv, **({"rounding": 2} | kw))
        return L.nvfp4_quantize_nvfp4_dual(P(FAKE), 1, rows, cols, cols, ctypes.byref(oo), P(FAKE), P(FAKE),
                                           P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), ws_bytes, None)
    assert d(rounding=0) == INVALID                  # MS-EDEN only
    assert d(rows=100) == SHAPE                      # the column-wise K = rows
    assert d(cols=200) == SHAPE
    assert d(rows=144) == SHAPE                      # group 128 along the rows
    assert d(rows=144, eden_group=16) == SHAPE       # group 16: still whole 128-row tiles
    assert d(ws_bytes=w0) == WS_SMALL
    assert d(amax_out=FAKE) == UNSUPPORTED
    assert d(amax_in=FAKE) == UNSUPPORTED


def test_dequantize_and_gemm_rejections(nv):
    L = nv.lib()
    P = ctypes.c_void_p
    assert L.nvfp4_dequantize(P(FAKE), P(FAKE), P(FAKE), 4, 100, 0, None, 0, P(FAKE), None) == SHAPE
    assert L.nvfp4_dequantize(P(FAKE), P(FAKE), P(FAKE), 4, 64, 3, None, 0, P(FAKE), None) == INVALID
    assert L.nvfp4_dequantize(P(FAKE), P(FAKE), P(FAKE), 4, 64, 0, None, 9, P(FAKE), None) == INVALID
    w = (ctypes.c_uint32 * 4)()
    assert L.nvfp4_dequantize(P(FAKE), P(FAKE), P(FAKE), 4, 64, 0, w, 0, P(FAKE), None) == SHAPE
    assert L.nvfp4_dequantize(P(0), P(FAKE), P(FAKE), 4, 64, 0, None, 0, P(FAKE), None) == INVALID
    assert L.nvfp4_dequantize(P(FAKE + 2), P(FAKE), P(FAKE), 4, 64, 0, None, 0, P(FAKE), None) == MISALIGNED
    assert L.nvfp4_dequantize(P(0), P(0), P(0), 0, 64, 0, None, 0, P(0), None) == OK   # empty
    g = L.nvfp4_gemm_nvfp4
    assert g(P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 8, 8, 40, P(FAKE), 0, 8, None) == SHAPE
    assert g(P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 8, 8, 64, P(FAKE), 0, 4, None) == SHAPE
    assert g(P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 8, 8, 64, P(FAKE), 3, 8, None) == INVALID
    assert g(P(FAKE), P(FAKE), P(FAKE), P(0), P(FAKE), P(FAKE), 8, 8, 64, P(FAKE), 0, 8, None) == INVALID
    assert g(P(FAKE + 4), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 8, 8, 64, P(FAKE), 0, 8, None) == MISALIGNED
    assert g(P(0), P(0), P(0), P(0), P(0), P(0), 0, 8, 64, P(0), 0, 8, None) == OK      # empty
    # the 256-row operand panel must fit a 32-bit buffer range
    assert g(P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 8, 8, 16777216, P(FAKE), 0, 8,
             None) == UNSUPPORTED
    q = L.nvfp4_gemm_nvfp4_rtn
    ops = [P(FAKE)] * 6
    assert q(*ops, 8, 24, 64, P(FAKE), P(FAKE), P(FAKE), None, None) == SHAPE        # N % 16
    assert q(*ops, 8, 32, 40, P(FAKE), P(FAKE), P(FAKE), None, None) == SHAPE        # K % 16
    assert q(*ops, 8, 32, 64, P(0), P(FAKE), P(FAKE), None, None) == INVALID         # no c_ts
    assert q(*ops, 8, 32, 64, P(FAKE), P(FAKE + 8), P(FAKE), None, None) == MISALIGNED
    assert q(*ops, 8, 32, 64, P(FAKE), P(FAKE), P(FAKE), P(FAKE + 2), None) == MISALIGNED
    assert q(P(0), P(0), P(0), P(0), P(0), P(0), 0, 32, 64, P(0), P(0), P(0), None, None) == OK  # empty
    assert L.nvfp4_rht(P(FAKE), 1, 4, 100, 100, 0, w, P(FAKE), None) == SHAPE
    assert L.nvfp4_rht(P(FAKE), 1, 4, 128, 128, 0, None, P(FAKE), None) == INVALID


# ---------------------------------------------------------------- the binding's own checks
# The C ABI sees raw pointers only, so the Python binding checks every tensor
# it hands over (shape, dtype, layout, device) and raises before any call;
# these cases need no GPU: host tensors are rejected as such, and wrongly
# shaped ones by their shape before the device is looked at.

def _raises(nv, fn, match):
    with pytest.raises(nv.NvFp4Error, match=match):
        fn()


def test_binding_rejects_host_and_misshaped_tensors(nv):
    import torch
    x = torch.zeros((64, 256), dtype=torch.bfloat16)
    _raises(nv, lambda: nv.quantize_nvfp4(x), "device tensor")
    _raises(nv, lambda: nv.quantize_nvfp4(x[:, ::2]), "unit stride")
    _raises(nv, lambda: nv.quantize_nvfp4(torch.zeros(64, 256, 2)), "2-D")
    _raises(nv, lambda: nv.quantize_nvfp4(torch.zeros((64, 256), dtype=torch.float16)), "dtype")
    _raises(nv, lambda: nv.rht(x, np.zeros(128, np.uint8)), "device tensor")
    _raises(nv, lambda: nv.rht(x.t(), np.zeros(128, np.uint8)), "unit stride")
    # a caller-supplied output of the wrong shape, dtype or layout
    good = nv.QTensor(torch.zeros((64, 128), dtype=torch.uint8), torch.zeros((64, 16), dtype=torch.uint8),
                      torch.zeros(1))
    bad_codes = nv.QTensor(torch.zeros((64, 64), dtype=torch.uint8), good.scales, good.tensor_scale)
    bad_scales = nv.QTensor(good.codes, torch.zeros((16, 64), dtype=torch.uint8), good.tensor_scale)
    bad_dtype = nv.QTensor(good.codes.to(torch.int32), good.scales, good.tensor_scale)
    strided = nv.QTensor(torch.zeros((64, 256), dtype=torch.uint8)[:, ::2], good.scales, good.tensor_scale)
    bad_ts = nv.QTensor(good.codes, good.scales, torch.zeros(1, dtype=torch.float64))
    for q, msg in ((bad_codes, "codes has shape"), (bad_scales, "scales has shape"),
                   (bad_dtype, "codes has dtype"), (strided, "contiguous"), (bad_ts, "tensor_scale has dtype")):
        _raises(nv, lambda: nv.quantize_nvfp4(x, out=q), "device tensor")   # the input is checked first
        _raises(nv, lambda: nv._check_qtensor(q, "out", rows=64, k=256), msg)
        _raises(nv, lambda: nv.dequantize(q) if q is not bad_codes else nv._check_qtensor(q, "q", k=256), msg)
    # correct shapes on the host: rejected for their device
    _raises(nv, lambda: nv.dequantize(good), "device tensor")
    _raises(nv, lambda: nv.gemm_nvfp4(good, good), "device tensor")
    _raises(nv, lambda: nv.gemm_nvfp4_rtn(good, good, torch.ones(1)), "device tensor")
    # GEMM and dequantize outputs
    _raises(nv, lambda: nv._check_tensor(torch.zeros(64, 63), "out", shape=(64, 64)), "shape")
    _raises(nv, lambda: nv._check_tensor(torch.zeros(64, 64, dtype=torch.float16), "out",
                                         dtypes=(torch.float32, torch.bfloat16)), "dtype")
    _raises(nv, lambda: nv._check_tensor(torch.zeros(1), "tensor_scale", min_numel=2), "at least")
    _raises(nv, lambda: nv._check_tensor(torch.zeros(64, 64).t(), "out", dense=True), "contiguous")
    _raises(nv, lambda: nv._check_qtensor(nv.QTensor(torch.zeros((4, 4), dtype=torch.uint8),
                                                      torch.zeros((4, 1), dtype=torch.uint8), torch.zeros(1)),
                                          "a"), "multiple of 16")
