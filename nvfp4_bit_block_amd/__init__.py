"""nvfp4_bit_block_amd -- NVFP4 microscaled quantization (randomized Hadamard
rotation, RTN, stochastic rounding, MS-EDEN), IF4, dequantization and the
block-scaled FP4 GEMM on AMD Instinct MI355X (gfx950).

This module is argument marshalling over the C ABI of ``libnvfp4.so``
(``include/nvfp4.h``): PyTorch provides device memory and the current HIP
stream, every step of the computation runs in the library's HIP kernels.
There is no CPU fallback: without the built library (or without a GPU) every
compute call raises.
"""
import ctypes
import os
from dataclasses import dataclass

import numpy as np

__all__ = [
    "RTN", "SR", "MSEDEN", "FORMAT_NVFP4", "FORMAT_IF4", "QTensor", "NvFp4Error",
    "lib", "signs_to_words", "workspace_size", "quantize_nvfp4", "quantize_if4",
    "dequantize", "gemm_nvfp4", "rht", "abi_version", "SCALE_MAX6", "SCALE_4OVER6", "SCALE_SEARCH",
    "quantize_nvfp4_dual", "workspace_size_dual", "gemm_nvfp4_rtn", "quantize_nvfp4_noalloc",
]

RTN, SR, MSEDEN = 0, 1, 2
FORMAT_NVFP4, FORMAT_IF4 = 0, 1
SCALE_MAX6, SCALE_4OVER6, SCALE_SEARCH = 0, 1, 2
_F32, _BF16 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

_ROUNDING = {"rtn": RTN, "sr": SR, "mseden": MSEDEN, "ms-eden": MSEDEN, RTN: RTN, SR: SR,
             MSEDEN: MSEDEN}


class NvFp4Error(RuntimeError):
    pass


class _Opts(ctypes.Structure):
    _fields_ = [
        ("rounding", ctypes.c_int32),
        ("axis", ctypes.c_int32),
        ("rht", ctypes.c_int32),
        ("rht_signs", ctypes.c_uint32 * 4),
        ("seed", ctypes.c_uint64),
        ("stream", ctypes.c_uint32),
        ("eden_group", ctypes.c_int32),
        ("tensor_scale_in", ctypes.c_void_p),
        ("scale_rule", ctypes.c_int32),
        ("amax_out", ctypes.c_void_p),
        ("amax_in", ctypes.c_void_p),
    ]


_lib = None


def lib():
    """Load libnvfp4.so (built by ``nvfp4_bit_block_amd.build``).  Import
    torch first so that the library binds to torch's HIP runtime."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise NvFp4Error(f"{LIB_PATH} is missing: build it with `python -m nvfp4_bit_block_amd.build`"
                         " (or __graft_entry__.build())")
    import torch  # noqa: F401  (binds the HIP runtime before the library loads)
    L = ctypes.CDLL(LIB_PATH)
    P, I64, INT, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.nvfp4_opts_init.restype = None
    L.nvfp4_opts_init.argtypes = [ctypes.POINTER(_Opts)]
    L.nvfp4_workspace_size.restype = SZ
    L.nvfp4_workspace_size.argtypes = [I64, I64, ctypes.POINTER(_Opts)]
    L.nvfp4_workspace_size_dual.restype = SZ
    L.nvfp4_workspace_size_dual.argtypes = [I64, I64, ctypes.POINTER(_Opts)]
    L.nvfp4_quantize_nvfp4_dual.restype = INT
    L.nvfp4_quantize_nvfp4_dual.argtypes = [P, INT, I64, I64, I64, ctypes.POINTER(_Opts), P, P, P, P, P, P,
                                            P, SZ, P]
    for name in ("nvfp4_quantize_nvfp4", "nvfp4_quantize_if4"):
        f = getattr(L, name)
        f.restype = INT
        f.argtypes = [P, INT, I64, I64, I64, ctypes.POINTER(_Opts), P, P, P, P, SZ, P]
    L.nvfp4_quantize_nvfp4_noalloc.restype = INT
    L.nvfp4_quantize_nvfp4_noalloc.argtypes = [P, INT, I64, I64, I64, ctypes.POINTER(_Opts), P, P, P, P]
    L.nvfp4_dequantize.restype = INT
    L.nvfp4_dequantize.argtypes = [P, P, P, I64, I64, INT, P, INT, P, P]
    for name in ("nvfp4_gemm_nvfp4", "nvfp4_gemm_if4"):
        getattr(L, name).restype = INT
        getattr(L, name).argtypes = [P, P, P, P, P, P, I64, I64, I64, P, INT, I64, P]
    L.nvfp4_gemm_nvfp4_rtn.restype = INT
    L.nvfp4_gemm_nvfp4_rtn.argtypes = [P, P, P, P, P, P, I64, I64, I64, P, P, P, P, P]
    L.nvfp4_rht.restype = INT
    L.nvfp4_rht.argtypes = [P, INT, I64, I64, I64, INT, P, P, P]
    L.nvfp4_status_string.restype = ctypes.c_char_p
    L.nvfp4_status_string.argtypes = [INT]
    L.nvfp4_last_error.restype = ctypes.c_char_p
    L.nvfp4_last_error.argtypes = []
    L.nvfp4_abi_version.restype = INT
    L.nvfp4_abi_version.argtypes = []
    _lib = L
    return L


def abi_version():
    return int(lib().nvfp4_abi_version())


def _check(rc):
    if rc != 0:
        L = lib()
        raise NvFp4Error(f"{L.nvfp4_status_string(rc).decode()} ({rc}): {L.nvfp4_last_error().decode()}")


def signs_to_words(signs):
    """128 flags (1 = negate) or 4 uint32 words -> 4 uint32 words (bit k of
    the vector is bit k % 32 of word k // 32)."""
    a = np.asarray(signs)
    if a.size == 4 and a.dtype != np.uint8:
        return np.ascontiguousarray(a, dtype=np.uint32)
    a = a.astype(np.uint8).reshape(128)
    w = np.zeros(4, dtype=np.uint32)
    for k in np.flatnonzero(a):
        w[k // 32] |= np.uint32(1 << (k % 32))
    return w


def _stream(torch):
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t, torch):
    if t.dtype == torch.bfloat16:
        return _BF16
    if t.dtype == torch.float32:
        return _F32
    raise NvFp4Error(f"input dtype {t.dtype} is not float32 or bfloat16")


def _check_tensor(t, name, shape=None, dtypes=None, dev=None, dense=False, min_numel=None, where=True):
    """Host-side checks of a tensor handed to the library (the C ABI sees
    raw pointers only, so a wrong size or layout would become an
    out-of-bounds device access).  Shape, dtype and layout are checked
    before the device, so that the messages name the first real problem."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise NvFp4Error(f"{name} must be a torch tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise NvFp4Error(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise NvFp4Error(f"{name} holds {t.numel()} elements, at least {min_numel} needed")
    if dtypes is not None and t.dtype not in dtypes:
        raise NvFp4Error(f"{name} has dtype {t.dtype}, expected one of {tuple(dtypes)}")
    if dense and not t.is_contiguous():
        raise NvFp4Error(f"{name} must be contiguous")
    if where:
        _check_where(t, name, dev)


def _check_where(t, name, dev=None):
    if not t.is_cuda:
        raise NvFp4Error(f"{name} must be a device tensor")
    if dev is not None and t.device != dev:
        raise NvFp4Error(f"{name} is on {t.device}, expected {dev}")


def _check_input(x, name="x"):
    """A 2-D float32/bfloat16 input with unit stride along its last axis."""
    import torch
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise NvFp4Error(f"{name} must be a 2-D torch tensor")
    if x.size(1) > 1 and x.stride(1) != 1:
        raise NvFp4Error(f"{name} must have unit stride along its last dimension")
    if x.size(0) > 1 and x.stride(0) < x.size(1):
        raise NvFp4Error(f"{name} has a row stride below its row length")
    _check_tensor(x, name, dtypes=(torch.float32, torch.bfloat16))


def _check_qtensor(q, name, rows=None, k=None, dev=None):
    """A packed tensor: codes [rows, k/2] and scales [rows, k/16] uint8,
    contiguous, and a float32 tensor scale, all on one device."""
    import torch
    if not isinstance(q, QTensor):
        raise NvFp4Error(f"{name} must be a QTensor")
    if q.codes.dim() != 2 or q.scales.dim() != 2:
        raise NvFp4Error(f"{name}: codes and scales must be 2-D")
    r = q.codes.shape[0] if rows is None else rows
    kk = q.codes.shape[1] * 2 if k is None else k
    if kk % 16:
        raise NvFp4Error(f"{name}: K = {kk} is not a multiple of 16")
    dev = q.codes.device if dev is None else dev
    parts = ((q.codes, f"{name}.codes", dict(shape=(r, kk // 2), dtypes=(torch.uint8,), dense=True)),
             (q.scales, f"{name}.scales", dict(shape=(r, kk // 16), dtypes=(torch.uint8,), dense=True)),
             (q.tensor_scale, f"{name}.tensor_scale", dict(dtypes=(torch.float32,), min_numel=1)))
    for t, n, kw in parts:   # shapes and layouts first, then where the parts live
        _check_tensor(t, n, where=False, **kw)
    for t, n, _ in parts:
        _check_where(t, n, dev)


def _check_scalar(t, name, dev):
    import torch
    if t is not None:
        _check_tensor(t, name, dtypes=(torch.float32,), dev=dev, min_numel=1)


_SCALE_RULE = {"max6": SCALE_MAX6, "4over6": SCALE_4OVER6, "four_over_six": SCALE_4OVER6,
               "search": SCALE_SEARCH, SCALE_MAX6: SCALE_MAX6, SCALE_4OVER6: SCALE_4OVER6,
               SCALE_SEARCH: SCALE_SEARCH}


def _opts(rounding, axis, rht_signs, seed, stream_id, eden_group, tensor_scale_in, scale_rule=SCALE_MAX6,
          amax_out=None, amax_in=None):
    o = _Opts()
    lib().nvfp4_opts_init(ctypes.byref(o))
    o.rounding = _ROUNDING[rounding.lower() if isinstance(rounding, str) else rounding]
    o.axis = int(axis)
    if rht_signs is not None:
        o.rht = 1
        w = signs_to_words(rht_signs)
        for i in range(4):
            o.rht_signs[i] = int(w[i])
    o.seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    o.stream = int(stream_id) & 0xFFFFFFFF
    o.eden_group = int(eden_group)
    o.tensor_scale_in = None if tensor_scale_in is None else tensor_scale_in.data_ptr()
    o.scale_rule = _SCALE_RULE[scale_rule.lower() if isinstance(scale_rule, str) else scale_rule]
    o.amax_out = None if amax_out is None else amax_out.data_ptr()
    o.amax_in = None if amax_in is None else amax_in.data_ptr()
    return o


@dataclass
class QTensor:
    """Packed NVFP4 / IF4 tensor in the library's layout: codes [rows_out,
    K/2] uint8 (low nibble = even element), scales [rows_out, K/16] uint8
    (E4M3, bit 7 = INT flag for IF4), tensor scale [1] float32 -- all on the
    device."""
    codes: "object"
    scales: "object"
    tensor_scale: "object"
    format: int = FORMAT_NVFP4

    @property
    def rows(self):
        return self.codes.shape[0]

    @property
    def k(self):
        return self.codes.shape[1] * 2


def workspace_size(rows, cols, rounding=RTN, axis=0, tensor_scale_in=None):
    o = _opts(rounding, axis, None, 0, 0, 128, tensor_scale_in)
    return int(lib().nvfp4_workspace_size(int(rows), int(cols), ctypes.byref(o)))


def _quantize(fn, x, rounding, axis, rht_signs, seed, stream_id, eden_group, tensor_scale_in,
              out, workspace, fmt, scale_rule=SCALE_MAX6, amax_out=None, amax_in=None):
    import torch
    L = lib()
    _check_input(x)
    rows, cols = x.shape
    ld = x.stride(0) if rows > 1 else cols
    dev = x.device
    for t, n in ((amax_out, "amax_out"), (amax_in, "amax_in"), (tensor_scale_in, "tensor_scale_in")):
        _check_scalar(t, n, dev)
    o = _opts(rounding, axis, rht_signs, seed, stream_id, eden_group, tensor_scale_in, scale_rule,
              amax_out, amax_in)
    R, K = (rows, cols) if axis == 0 else (cols, rows)
    if out is None:
        out = QTensor(torch.empty((R, K // 2), dtype=torch.uint8, device=dev),
                      torch.empty((R, K // 16), dtype=torch.uint8, device=dev),
                      torch.empty(1, dtype=torch.float32, device=dev), fmt)
    else:
        if K % 16 == 0:
            _check_qtensor(out, "out", rows=R, k=K, dev=dev)
        out.format = fmt
    wsz = int(L.nvfp4_workspace_size(rows, cols, ctypes.byref(o)))
    if workspace is None or workspace.numel() < wsz:
        workspace = torch.empty(max(wsz, 256), dtype=torch.uint8, device=dev)
    else:
        _check_tensor(workspace, "workspace", dtypes=(torch.uint8,), dev=dev, dense=True)
    rc = fn(ctypes.c_void_p(x.data_ptr()), _dtype_code(x, torch), rows, cols, ld, ctypes.byref(o),
            ctypes.c_void_p(out.codes.data_ptr()), ctypes.c_void_p(out.scales.data_ptr()),
            ctypes.c_void_p(out.tensor_scale.data_ptr()), ctypes.c_void_p(workspace.data_ptr()),
            workspace.numel(), _stream(torch))
    _check(rc)
    return out


def quantize_nvfp4(x, rounding=RTN, axis=0, rht_signs=None, seed=0, stream_id=0, eden_group=128,
                   tensor_scale_in=None, out=None, workspace=None, scale_rule=SCALE_MAX6,
                   amax_out=None, amax_in=None):
    """NVFP4 quantization of a 2-D float32/bfloat16 device tensor (see
    ``nvfp4_quantize_nvfp4`` in include/nvfp4.h).  rht_signs: 128 flags or 4
    words enable the randomized Hadamard rotation.  scale_rule "4over6"
    selects Four Over Six block scaling, "search" a searched block scale
    (both RTN only).  amax_out (MS-EDEN) receives max|x|; amax_in (no
    rotation, not MS-EDEN) supplies it instead of a pass over x: float32
    device tensors.  Returns a QTensor."""
    return _quantize(lib().nvfp4_quantize_nvfp4, x, rounding, axis, rht_signs, seed, stream_id,
                     eden_group, tensor_scale_in, out, workspace, FORMAT_NVFP4, scale_rule,
                     amax_out, amax_in)


def quantize_nvfp4_noalloc(x, out, rounding=RTN, axis=0, rht_signs=None, seed=0, stream_id=0, eden_group=128,
                           tensor_scale_in=None, scale_rule=SCALE_MAX6, amax_out=None, amax_in=None):
    """quantize_nvfp4 through ``nvfp4_quantize_nvfp4_noalloc``: no workspace,
    the library's per-GPU scratch instead, and nothing allocated -- so the
    caller passes the output QTensor `out` (codes [R, K/2], scales [R, K/16],
    tensor scale [1]).  Calls that overlap on one GPU race on that scratch."""
    L = lib()
    _check_input(x)
    rows, cols = x.shape
    ld = x.stride(0) if rows > 1 else cols
    dev = x.device
    for t, n in ((amax_out, "amax_out"), (amax_in, "amax_in"), (tensor_scale_in, "tensor_scale_in")):
        _check_scalar(t, n, dev)
    R, K = (rows, cols) if axis == 0 else (cols, rows)
    if K % 16 == 0:
        _check_qtensor(out, "out", rows=R, k=K, dev=dev)
    o = _opts(rounding, axis, rht_signs, seed, stream_id, eden_group, tensor_scale_in, scale_rule, amax_out,
              amax_in)
    import torch
    rc = L.nvfp4_quantize_nvfp4_noalloc(ctypes.c_void_p(x.data_ptr()), _dtype_code(x, torch), rows, cols, ld,
                                        ctypes.byref(o), ctypes.c_void_p(out.codes.data_ptr()),
                                        ctypes.c_void_p(out.scales.data_ptr()),
                                        ctypes.c_void_p(out.tensor_scale.data_ptr()), _stream(torch))
    _check(rc)
    out.format = FORMAT_NVFP4
    return out


def quantize_nvfp4_dual(x, rht_signs=None, seed=0, stream_id=0, eden_group=128, tensor_scale_in=None,
                        out_rows=None, out_cols=None, workspace=None):
    """MS-EDEN of a 2-D device tensor along both axes from one read (see
    ``nvfp4_quantize_nvfp4_dual``): returns (row-wise QTensor [rows, cols],
    column-wise QTensor [cols, rows]), equal to two quantize_nvfp4 calls with
    rounding "mseden" and axis 0 / axis 1."""
    import torch
    L = lib()
    _check_input(x)
    rows, cols = x.shape
    ld = x.stride(0) if rows > 1 else cols
    dev = x.device
    _check_scalar(tensor_scale_in, "tensor_scale_in", dev)
    o = _opts(MSEDEN, 0, rht_signs, seed, stream_id, eden_group, tensor_scale_in)

    def alloc(R, K):
        return QTensor(torch.empty((R, K // 2), dtype=torch.uint8, device=dev),
                       torch.empty((R, K // 16), dtype=torch.uint8, device=dev),
                       torch.empty(1, dtype=torch.float32, device=dev), FORMAT_NVFP4)
    qr = out_rows if out_rows is not None else alloc(rows, cols)
    qc = out_cols if out_cols is not None else alloc(cols, rows)
    if rows % 16 == 0 and cols % 16 == 0:
        _check_qtensor(qr, "out_rows", rows=rows, k=cols, dev=dev)
        _check_qtensor(qc, "out_cols", rows=cols, k=rows, dev=dev)
    wsz = int(L.nvfp4_workspace_size_dual(rows, cols, ctypes.byref(o)))
    if workspace is None or workspace.numel() < wsz:
        workspace = torch.empty(max(wsz, 256), dtype=torch.uint8, device=dev)
    else:
        _check_tensor(workspace, "workspace", dtypes=(torch.uint8,), dev=dev, dense=True)
    rc = L.nvfp4_quantize_nvfp4_dual(ctypes.c_void_p(x.data_ptr()), _dtype_code(x, torch), rows, cols, ld,
                                     ctypes.byref(o), ctypes.c_void_p(qr.codes.data_ptr()),
                                     ctypes.c_void_p(qr.scales.data_ptr()),
                                     ctypes.c_void_p(qr.tensor_scale.data_ptr()),
                                     ctypes.c_void_p(qc.codes.data_ptr()), ctypes.c_void_p(qc.scales.data_ptr()),
                                     ctypes.c_void_p(qc.tensor_scale.data_ptr()),
                                     ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), _stream(torch))
    _check(rc)
    return qr, qc


def workspace_size_dual(rows, cols, eden_group=128, tensor_scale_in=None):
    o = _opts(MSEDEN, 0, None, 0, 0, eden_group, tensor_scale_in)
    return int(lib().nvfp4_workspace_size_dual(int(rows), int(cols), ctypes.byref(o)))


def quantize_if4(x, rounding=RTN, axis=0, rht_signs=None, seed=0, stream_id=0, eden_group=128,
                 tensor_scale_in=None, out=None, workspace=None, amax_out=None, amax_in=None):
    """IF4 quantization (per-16 FP4/INT4 choice): RTN keeps the branch with
    the lower squared error; SR the one with the lower expected error of
    stochastic rounding; MS-EDEN codes both by RTN under exact scales, keeps
    the better and folds the EDEN correction into the stochastic scale (see
    ``nvfp4_quantize_if4``).  Returns a QTensor of format FORMAT_IF4."""
    return _quantize(lib().nvfp4_quantize_if4, x, rounding, axis, rht_signs, seed, stream_id, eden_group,
                     tensor_scale_in, out, workspace, FORMAT_IF4, amax_out=amax_out, amax_in=amax_in)


def dequantize(q, inv_rht_signs=None, out_dtype=None, out=None):
    """Decode a QTensor to [rows_out, K] float32 (or bfloat16), optionally
    undoing the rotation."""
    import torch
    _check_qtensor(q, "q")
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((q.rows, q.k), dtype=out_dtype, device=q.codes.device)
    else:
        _check_tensor(out, "out", shape=(q.rows, q.k), dtypes=(torch.float32, torch.bfloat16),
                      dev=q.codes.device, dense=True)
    w = None
    if inv_rht_signs is not None:
        w = signs_to_words(inv_rht_signs)
    rc = lib().nvfp4_dequantize(ctypes.c_void_p(q.codes.data_ptr()), ctypes.c_void_p(q.scales.data_ptr()),
                                ctypes.c_void_p(q.tensor_scale.data_ptr()), q.rows, q.k, q.format,
                                None if w is None else w.ctypes.data_as(ctypes.c_void_p),
                                _dtype_code(out, torch), ctypes.c_void_p(out.data_ptr()), _stream(torch))
    _check(rc)
    return out


def gemm_nvfp4(a, b, out_dtype=None, out=None):
    """C = (ts_a ts_b) * A_hat @ B_hat^T for two K-major NVFP4 or IF4
    QTensors (A: [M, K], B: [N, K]); C is [M, N] float32 (or bfloat16)."""
    import torch
    _check_qtensor(a, "a")
    _check_qtensor(b, "b", dev=a.codes.device)
    if a.k != b.k:
        raise NvFp4Error(f"K mismatch: {a.k} vs {b.k}")
    if a.format not in (FORMAT_NVFP4, FORMAT_IF4) or b.format not in (FORMAT_NVFP4, FORMAT_IF4):
        raise NvFp4Error("operands must be NVFP4 or IF4 QTensors")
    # IF4 operands go through the entry point that decodes INT-flagged blocks
    fn = lib().nvfp4_gemm_nvfp4 if a.format == b.format == FORMAT_NVFP4 else lib().nvfp4_gemm_if4
    out_dtype = out_dtype or torch.float32
    M, N = a.rows, b.rows
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.codes.device)
    else:
        _check_tensor(out, "out", shape=(M, N), dtypes=(torch.float32, torch.bfloat16), dev=a.codes.device)
        if (N > 1 and out.stride(1) != 1) or (M > 1 and out.stride(0) < N):
            raise NvFp4Error("out must have unit stride along its last dimension and a row stride >= N")
    ldc = out.stride(0) if M > 1 else N
    rc = fn(ctypes.c_void_p(a.codes.data_ptr()), ctypes.c_void_p(a.scales.data_ptr()),
                                ctypes.c_void_p(a.tensor_scale.data_ptr()),
                                ctypes.c_void_p(b.codes.data_ptr()), ctypes.c_void_p(b.scales.data_ptr()),
                                ctypes.c_void_p(b.tensor_scale.data_ptr()), M, N, a.k,
                                ctypes.c_void_p(out.data_ptr()), _dtype_code(out, torch), ldc,
                                _stream(torch))
    _check(rc)
    return out


def gemm_nvfp4_rtn(a, b, tensor_scale, amax_out=None, out=None):
    """The NVFP4 GEMM with its output [M, N] coded as NVFP4 (RTN along N,
    tensor scale `tensor_scale`, a float32 device tensor [1]) in the same
    kernel.  Returns a QTensor (rows M, K = N) that holds `tensor_scale`;
    amax_out (float32 device [1]) receives max |C|.  `out` may give a
    preallocated QTensor."""
    import torch
    _check_qtensor(a, "a")
    dev = a.codes.device
    _check_qtensor(b, "b", dev=dev)
    if a.k != b.k:
        raise NvFp4Error(f"K mismatch: {a.k} vs {b.k}")
    if a.format != FORMAT_NVFP4 or b.format != FORMAT_NVFP4:
        raise NvFp4Error("operands must be NVFP4 QTensors")
    if tensor_scale is None:
        raise NvFp4Error("tensor_scale is required")
    _check_scalar(tensor_scale, "tensor_scale", dev)
    _check_scalar(amax_out, "amax_out", dev)
    M, N = a.rows, b.rows
    if out is None:
        out = QTensor(torch.empty((M, N // 2), dtype=torch.uint8, device=dev),
                      torch.empty((M, N // 16), dtype=torch.uint8, device=dev), tensor_scale, FORMAT_NVFP4)
    elif N % 16 == 0:
        _check_qtensor(out, "out", rows=M, k=N, dev=dev)
    rc = lib().nvfp4_gemm_nvfp4_rtn(
        ctypes.c_void_p(a.codes.data_ptr()), ctypes.c_void_p(a.scales.data_ptr()),
        ctypes.c_void_p(a.tensor_scale.data_ptr()), ctypes.c_void_p(b.codes.data_ptr()),
        ctypes.c_void_p(b.scales.data_ptr()), ctypes.c_void_p(b.tensor_scale.data_ptr()), M, N, a.k,
        ctypes.c_void_p(tensor_scale.data_ptr()), ctypes.c_void_p(out.codes.data_ptr()),
        ctypes.c_void_p(out.scales.data_ptr()),
        None if amax_out is None else ctypes.c_void_p(amax_out.data_ptr()), _stream(torch))
    _check(rc)
    return out


def rht(x, signs, axis=0, out=None):
    """The rotation step alone: rotated fp32 values [rows_out, K]."""
    import torch
    _check_input(x)
    rows, cols = x.shape
    R, K = (rows, cols) if axis == 0 else (cols, rows)
    if out is None:
        out = torch.empty((R, K), dtype=torch.float32, device=x.device)
    else:
        _check_tensor(out, "out", shape=(R, K), dtypes=(torch.float32,), dev=x.device, dense=True)
    w = signs_to_words(signs)
    ld = x.stride(0) if rows > 1 else cols
    rc = lib().nvfp4_rht(ctypes.c_void_p(x.data_ptr()), _dtype_code(x, torch), rows, cols, ld, int(axis),
                         w.ctypes.data_as(ctypes.c_void_p), ctypes.c_void_p(out.data_ptr()), _stream(torch))
    _check(rc)
    return out
