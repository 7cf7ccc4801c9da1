"""CPU oracle for NVFP4 / MS-EDEN / IF4 quantization and the block-scaled
FP4 GEMM -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product (``nvfp4_bit_block_amd``)
never imports it, and the two share no code.

This module is argument marshalling over ``liboracle.so`` (plain C, see
``oracle.c`` for the method, its sources and the readings taken).
"""
import ctypes
import os

import numpy as np

from . import build as _build

FMT_NVFP4, FMT_IF4, FMT_NVINT4, FMT_NVFP4_4OVER6, FMT_NVFP4_SEARCH = 0, 1, 2, 3, 4
RTN, SR, MSEDEN = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_U32 = ctypes.c_uint32
_U64 = ctypes.c_uint64
_F32 = ctypes.c_float
_INT = ctypes.c_int


def lib():
    """Load liboracle.so, building it first when it is missing or stale."""
    global _lib
    if _lib is not None:
        return _lib
    so = _build.LIB
    src = os.path.join(_HERE, "oracle.c")
    if not os.path.exists(so) or os.path.getmtime(so) < os.path.getmtime(src):
        _build.build()
    L = ctypes.CDLL(so)
    L.orc_e2m1_value.restype = _F32
    L.orc_e2m1_value.argtypes = [_INT]
    L.orc_e4m3_value.restype = _F32
    L.orc_e4m3_value.argtypes = [_INT]
    for name in ("orc_e4m3_rne_sat", "orc_e4m3_ceil_sat", "orc_e2m1_rne", "orc_int4_rne"):
        getattr(L, name).restype = _INT
        getattr(L, name).argtypes = [_F32]
    for name in ("orc_sr_e2m1", "orc_sr_e4m3"):
        getattr(L, name).restype = _INT
        getattr(L, name).argtypes = [_F32, _U32]
    L.orc_sr_expected_sq.restype = _F32
    L.orc_sr_expected_sq.argtypes = [_F32, _INT]
    L.orc_e2m1_rne_run.restype = None
    L.orc_e2m1_rne_run.argtypes = [_U32, _U64, _P]
    L.orc_e4m3_run.restype = None
    L.orc_e4m3_run.argtypes = [_U32, _U64, _INT, _P]
    L.orc_sr_e4m3_pairs.restype = None
    L.orc_sr_e4m3_pairs.argtypes = [_P, _P, _U64, _P]
    L.orc_philox4x32_10.restype = None
    L.orc_philox4x32_10.argtypes = [_P, _P, _P]
    L.orc_uniform16.restype = _U32
    L.orc_uniform16.argtypes = [_U64, _U32, _U32, _U64]
    L.orc_fwht128.restype = None
    L.orc_fwht128.argtypes = [_P]
    L.orc_rht128.restype = None
    L.orc_rht128.argtypes = [_P, _P, _P]
    L.orc_irht128.restype = None
    L.orc_irht128.argtypes = [_P, _P, _P]
    L.orc_pairwise_sum.restype = _F32
    L.orc_pairwise_sum.argtypes = [_P, _INT]
    L.orc_quantize.restype = _INT
    L.orc_quantize.argtypes = [_P, _I64, _I64, _I64, _INT, _INT, _INT, _INT, _P, _U64, _U32,
                               _INT, _P, _P, _P, _P, _P, _P]
    L.orc_dequantize.restype = _INT
    L.orc_dequantize.argtypes = [_P, _P, _F32, _I64, _I64, _INT, _P, _P]
    L.orc_gemm_entries.restype = _INT
    L.orc_gemm_entries.argtypes = [_P, _P, _F32, _P, _P, _F32, _I64, _I64, _I64, _INT,
                                   _P, _P, _I64, _P]
    L.orc_gemm_full.restype = _INT
    L.orc_gemm_full.argtypes = [_P, _P, _F32, _P, _P, _F32, _I64, _I64, _I64, _INT, _P]
    L.orc_num_threads.restype = _INT
    L.orc_num_threads.argtypes = []
    L.orc_set_num_threads.restype = None
    L.orc_set_num_threads.argtypes = [_INT]
    _lib = L
    return L


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def signs_words(signs):
    """128 sign flags (1 = negate) -> four uint32 words, bit k of the vector
    is bit (k % 32) of word k // 32."""
    s = np.asarray(signs, dtype=np.uint8).reshape(128)
    w = np.zeros(4, dtype=np.uint32)
    for k in range(128):
        if s[k]:
            w[k // 32] |= np.uint32(1 << (k % 32))
    return w


# ---------------------------------------------------------------- scalars
def e2m1_value(nibble):
    return float(lib().orc_e2m1_value(int(nibble)))


def e4m3_value(byte):
    return float(lib().orc_e4m3_value(int(byte)))


def e4m3_rne(v):
    return int(lib().orc_e4m3_rne_sat(float(v)))


def e4m3_ceil(v):
    return int(lib().orc_e4m3_ceil_sat(float(v)))


def e2m1_rne(a):
    return int(lib().orc_e2m1_rne(float(a)))


def int4_rne(a):
    return int(lib().orc_int4_rne(float(a)))


def sr_e2m1(a, u16):
    return int(lib().orc_sr_e2m1(float(a), int(u16)))


def sr_e4m3(a, u16):
    return int(lib().orc_sr_e4m3(float(a), int(u16)))


def sr_expected_sq(a, is_int=False):
    """(a - l)(u - a) on the E2M1 grid (or integers 0..7), fp32."""
    return float(lib().orc_sr_expected_sq(float(a), int(bool(is_int))))


def e2m1_rne_run(bits_lo, count):
    """Packed RTN nibbles of the fp32 bit patterns bits_lo .. bits_lo+count-1
    (sign<<3 | E2M1_RNE(min(|y|, 6)), two per byte)."""
    out = np.empty(count // 2, dtype=np.uint8)
    lib().orc_e2m1_rne_run(int(bits_lo), int(count), _ptr(out))
    return out


def e4m3_run(bits_lo, count, ceil_mode=False):
    """E4M3 bytes (RNE, or rounded up) of the fp32 bit patterns
    bits_lo .. bits_lo+count-1."""
    out = np.empty(count, dtype=np.uint8)
    lib().orc_e4m3_run(int(bits_lo), int(count), int(bool(ceil_mode)), _ptr(out))
    return out


def sr_e4m3_pairs(a, u16):
    """E4M3 bytes of the stochastic scale rounding, orc_sr_e4m3(a[i], u16[i])."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u16 = np.ascontiguousarray(u16, dtype=np.uint16)
    assert a.shape == u16.shape
    out = np.empty(a.shape, dtype=np.uint8)
    lib().orc_sr_e4m3_pairs(_ptr(a), _ptr(u16), int(a.size), _ptr(out))
    return out


def philox4x32_10(ctr, key):
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, dtype=np.uint32)
    lib().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def uniform16(seed, tag, stream, idx):
    return int(lib().orc_uniform16(int(seed), int(tag), int(stream), int(idx)))


def pairwise_sum(v):
    v = np.ascontiguousarray(v, dtype=np.float32)
    return float(lib().orc_pairwise_sum(_ptr(v), int(v.size)))


# ---------------------------------------------------------------- rotation
def fwht128(v):
    v = np.ascontiguousarray(v, dtype=np.float32).copy()
    assert v.size == 128
    lib().orc_fwht128(_ptr(v))
    return v


def rht(x, signs_w):
    """Rotate every 128-group along the last axis of x (fp32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.shape[-1] % 128 == 0
    w = np.ascontiguousarray(signs_w, dtype=np.uint32)
    flat = x.reshape(-1, 128)
    out = np.empty_like(flat)
    L = lib()
    for i in range(flat.shape[0]):
        L.orc_rht128(_ptr(flat[i]), _ptr(w), _ptr(out[i]))
    return out.reshape(x.shape)


def irht(z, signs_w):
    z = np.ascontiguousarray(z, dtype=np.float32)
    w = np.ascontiguousarray(signs_w, dtype=np.uint32)
    flat = z.reshape(-1, 128)
    out = np.empty_like(flat)
    L = lib()
    for i in range(flat.shape[0]):
        L.orc_irht128(_ptr(flat[i]), _ptr(w), _ptr(out[i]))
    return out.reshape(z.shape)


# ---------------------------------------------------------------- quantize
class OracleError(RuntimeError):
    pass


def quantize(x, fmt=FMT_NVFP4, rounding=RTN, axis=0, rht_on=False, signs_w=None, seed=0,
             stream=0, eden_group=128, ts_in=None, want_z=False, want_tb=False):
    """Quantize a 2-D fp32 array (bf16 inputs are passed as their exact fp32
    values).  Returns dict(codes [R, K/2] u8, scales [R, K/16] u8, ts float,
    z [R, K] f32 (rotated values) if asked, tb [R, K/16] f32 if asked)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    R, K = (rows, cols) if axis == 0 else (cols, rows)
    codes = np.zeros((R, K // 2), dtype=np.uint8)
    scales = np.zeros((R, max(K // 16, 0)), dtype=np.uint8)
    ts = np.zeros(1, dtype=np.float32)
    z = np.zeros((R, K), dtype=np.float32) if want_z else None
    tb = np.zeros((R, K // 16), dtype=np.float32) if (want_tb and rounding == MSEDEN) else None
    w = None if signs_w is None else np.ascontiguousarray(signs_w, dtype=np.uint32)
    tsi = None if ts_in is None else np.array([ts_in], dtype=np.float32)
    rc = lib().orc_quantize(_ptr(x), rows, cols, cols, fmt, rounding, axis, int(bool(rht_on)),
                            _ptr(w), int(seed), int(stream), int(eden_group), _ptr(tsi),
                            _ptr(codes), _ptr(scales), _ptr(ts), _ptr(z), _ptr(tb))
    if rc != 0:
        raise OracleError(f"orc_quantize failed with status {rc}")
    out = {"codes": codes, "scales": scales, "ts": float(ts[0])}
    if want_z:
        out["z"] = z
    if tb is not None:
        out["tb"] = tb
    return out


def dequantize(codes, scales, ts, fmt=FMT_NVFP4, inv_signs_w=None):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    R, K = codes.shape[0], codes.shape[1] * 2
    out = np.zeros((R, K), dtype=np.float32)
    w = None if inv_signs_w is None else np.ascontiguousarray(inv_signs_w, dtype=np.uint32)
    rc = lib().orc_dequantize(_ptr(codes), _ptr(scales), float(ts), R, K, fmt, _ptr(w), _ptr(out))
    if rc != 0:
        raise OracleError(f"orc_dequantize failed with status {rc}")
    return out


# ---------------------------------------------------------------- GEMM
def gemm_entries(a, b, im, in_, fmt=FMT_NVFP4):
    """C[m, n] for the listed index pairs, fp64.  a, b: dicts from quantize
    (K-major operands)."""
    ac, asc = np.ascontiguousarray(a["codes"]), np.ascontiguousarray(a["scales"])
    bc, bsc = np.ascontiguousarray(b["codes"]), np.ascontiguousarray(b["scales"])
    M, N, K = ac.shape[0], bc.shape[0], ac.shape[1] * 2
    assert bc.shape[1] * 2 == K
    im = np.ascontiguousarray(im, dtype=np.int64)
    in_ = np.ascontiguousarray(in_, dtype=np.int64)
    out = np.zeros(im.size, dtype=np.float64)
    rc = lib().orc_gemm_entries(_ptr(ac), _ptr(asc), float(a["ts"]), _ptr(bc), _ptr(bsc),
                                float(b["ts"]), M, N, K, fmt, _ptr(im), _ptr(in_), im.size,
                                _ptr(out))
    if rc != 0:
        raise OracleError(f"orc_gemm_entries failed with status {rc}")
    return out


def gemm_full(a, b, fmt=FMT_NVFP4):
    ac, asc = np.ascontiguousarray(a["codes"]), np.ascontiguousarray(a["scales"])
    bc, bsc = np.ascontiguousarray(b["codes"]), np.ascontiguousarray(b["scales"])
    M, N, K = ac.shape[0], bc.shape[0], ac.shape[1] * 2
    out = np.zeros((M, N), dtype=np.float64)
    rc = lib().orc_gemm_full(_ptr(ac), _ptr(asc), float(a["ts"]), _ptr(bc), _ptr(bsc),
                             float(b["ts"]), M, N, K, fmt, _ptr(out))
    if rc != 0:
        raise OracleError(f"orc_gemm_full failed with status {rc}")
    return out


def num_threads():
    return int(lib().orc_num_threads())


def set_num_threads(n):
    lib().orc_set_num_threads(int(n))
