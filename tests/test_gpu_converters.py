"""Exhaustive device checks of the conversions the kernels rely on, against
the oracle's rules (and, for the divisions, the device's IEEE division).

The quantizers code RTN blocks with gfx950's packed fp32 -> E2M1 conversion
(e2m1x16_rne), divide the block maximum by 6 and 7 with a corrected
reciprocal product (div_by), round block scales with e4m3_rne_sat /
e4m3_ceil_sat, and decode codes with the packed E2M1 -> fp32 conversion;
the GEMM decodes operands with the packed E2M1 -> fp16 conversion, its
scales with the E4M3 -> fp16 conversion, and IF4 operands by table.  Each
test below runs the library's own device function (tests/convcheck.hip
includes the kernels' header) over its whole input domain:

- e2m1x16_rne on every fp32 bit pattern that is not a NaN, both signs (the
  E2M1 range [0, 6], the saturation range above it, the infinities), against
  the nibble sign<<3 | E2M1_RNE(min(|y|, 6)) of the oracle's block coding;
- e4m3_rne_sat and e4m3_ceil_sat on every finite v >= 0 and +inf;
- e4m3_sr_sat (MS-EDEN's stochastic scale rounding, an integer addition on
  the bit pattern in the normal range) on every fp32 value in [0, 448] with
  a uniform per value, and at every decision boundary: for each of the
  65536 uniforms, the values whose position in the gap sits exactly on the
  threshold and one unit either side, in every binade and every gap;
- div_by<6>, div_by<7> on every finite a >= 0, against the IEEE quotient;
- every code byte through both E2M1 decoders and both IF4 tables, every
  scale byte through the E4M3 decoders, and every (scale byte, code byte)
  pair through the GEMM's operand decoding, against the oracle's values.
"""
import ctypes
import os
import time

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_build", "libconvcheck.so")
CHUNK = 1 << 28   # fp32 patterns per device call (128 MiB of packed codes)
POS_INF = 0x7F800000


@pytest.fixture(scope="module")
def cc():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert os.path.exists(LIB), f"{LIB} is missing: run __graft_entry__.build()"
    torch.cuda.init()
    lib = ctypes.CDLL(LIB)
    u32, P = ctypes.c_uint32, ctypes.c_void_p
    lib.convcheck_e2m1_rne.argtypes = [u32, u32, P]
    lib.convcheck_e4m3.argtypes = [u32, u32, ctypes.c_int, P]
    lib.convcheck_e4m3_sr.argtypes = [P, P, u32, P]
    lib.convcheck_div_by.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_ulonglong), ctypes.POINTER(u32)]
    lib.convcheck_decoders.argtypes = [P] * 7
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _first_diff(got, want, lo, per_byte):
    i = int(np.flatnonzero(got != want)[0])
    return f"pattern {lo + per_byte * i:#010x}: device {got[i]:#04x}, oracle {want[i]:#04x}"


@pytest.mark.parametrize("sign", [0, 0x80000000], ids=["positive", "negative"])
def test_e2m1_rne_every_pattern(cc, orc, sign):
    """0 .. +inf (or -0 .. -inf): 2^31 - 2^23 + 1 patterns; the run is padded
    to a multiple of 16 with NaN patterns past the infinity, which are not
    compared."""
    end = POS_INF + 16          # exclusive, a multiple of 16
    t0 = time.time()
    for lo in range(0, end, CHUNK):
        n = min(CHUNK, end - lo)
        got = np.empty(n // 2, dtype=np.uint8)
        assert cc.convcheck_e2m1_rne(sign | lo, n, _ptr(got)) == 0
        want = orc.e2m1_rne_run(sign | lo, n)
        keep = min(n, POS_INF + 1 - lo)        # patterns up to the infinity
        if keep < n:
            # compare the whole bytes, then the low nibble of the last one
            got_b, want_b = got[: keep // 2], want[: keep // 2]
            if keep % 2:
                assert (got[keep // 2] & 15) == (want[keep // 2] & 15), f"pattern {sign | POS_INF:#010x}"
        else:
            got_b, want_b = got, want
        assert np.array_equal(got_b, want_b), _first_diff(got_b, want_b, sign | lo, 2)
    print(f"e2m1 RTN, {'negative' if sign else 'positive'} patterns: {time.time() - t0:.1f} s", flush=True)


@pytest.mark.parametrize("ceil_mode", [0, 1], ids=["rne", "ceil"])
def test_e4m3_block_scale_every_value(cc, orc, ceil_mode):
    end = POS_INF + 1            # every finite v >= 0 and +inf
    t0 = time.time()
    for lo in range(0, end, CHUNK):
        n = min(CHUNK, end - lo)
        got = np.empty(n, dtype=np.uint8)
        assert cc.convcheck_e4m3(lo, n, ceil_mode, _ptr(got)) == 0
        want = orc.e4m3_run(lo, n, ceil_mode)
        assert np.array_equal(got, want), _first_diff(got, want, lo, 1)
    print(f"e4m3 {'ceil' if ceil_mode else 'rne'}: {time.time() - t0:.1f} s", flush=True)


def _uniforms_of(bits):
    """A 16-bit uniform per value: the high half of a multiplicative hash of
    its bit pattern, so that neighbouring values meet unrelated uniforms."""
    return ((bits.astype(np.uint32) * np.uint32(0x9E3779B1)) >> np.uint32(16)).astype(np.uint16)


def _sr_compare(cc, orc, a, u, what):
    got = np.empty(a.size, dtype=np.uint8)
    assert cc.convcheck_e4m3_sr(_ptr(a), _ptr(u), a.size, _ptr(got)) == 0
    want = orc.sr_e4m3_pairs(a, u)
    if not np.array_equal(got, want):
        i = int(np.flatnonzero(got != want)[0])
        raise AssertionError(f"{what}: a bits {a.view(np.uint32)[i]:#010x}, u16 {u[i]}: device {got[i]:#04x}, "
                             f"oracle {want[i]:#04x}")


def test_e4m3_sr_every_value(cc, orc):
    """Every fp32 value in [0, 448] (the range the MS-EDEN scale reaches after
    its clamp), then -0, +inf, NaN and values above 448."""
    end = 0x43E00000 + 1           # 448 = 0x43E00000
    t0 = time.time()
    for lo in range(0, end, CHUNK):
        bits = np.arange(lo, min(lo + CHUNK, end), dtype=np.uint32)
        _sr_compare(cc, orc, bits.view(np.float32), _uniforms_of(bits), "e4m3 SR")
    odd = np.array([0x80000000, 0x7F800000, 0x7FC00000, 0x43E00001, 0x43E0FFFF, 0x44000000, 0x7F7FFFFF], np.uint32)
    for u in (0, 1, 0x8000, 0xFFFF):
        _sr_compare(cc, orc, odd.view(np.float32), np.full(odd.size, u, np.uint16), "e4m3 SR outside [0, 448]")
    print(f"e4m3 SR: {time.time() - t0:.1f} s", flush=True)


def test_e4m3_sr_decision_boundaries(cc, orc):
    """The decision u16 < frac * 65536 at its threshold, for every uniform:
    normal values with the 20 mantissa bits below the kept three equal to
    16 u16 - 1, 16 u16, 16 u16 + 1 (binades 2^-6 .. 2^8, every gap), and
    E4M3-subnormal values (f + u16 / 65536) * 2^-9 and their fp32
    neighbours."""
    u = np.arange(65536, dtype=np.int64)
    A, U = [], []
    for E in range(-6, 9):
        for q in range(8):
            for d in (-1, 0, 1):
                m = np.clip(16 * u + d, 0, (1 << 20) - 1)
                A.append((((E + 127) << 23) | (q << 20) | m).astype(np.uint32))
                U.append(u)
    for f in range(8):
        b = ((f + u / 65536.0) * 2.0 ** -9).astype(np.float32).view(np.uint32)
        for d in (-1, 0, 1):
            A.append((b.astype(np.int64) + d).clip(0).astype(np.uint32))
            U.append(u)
    bits, uu = np.concatenate(A), np.concatenate(U).astype(np.uint16)
    keep = bits <= 0x43E00000
    _sr_compare(cc, orc, bits[keep].view(np.float32), uu[keep], "e4m3 SR boundary")


@pytest.mark.parametrize("d", [6, 7])
def test_div_by_every_finite(cc, d):
    bad, first = ctypes.c_ulonglong(), ctypes.c_uint32()
    assert cc.convcheck_div_by(d, ctypes.byref(bad), ctypes.byref(first)) == 0
    assert bad.value == 0, f"{bad.value} quotients a / {d} differ, e.g. a bits {first.value:#010x}"


def _f16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def test_decoders_every_byte(cc, orc):
    code_f32 = np.empty(256 * 16, np.float32)
    code_f16, lut_fp, lut_int = (np.empty(256 * 8, np.uint16) for _ in range(3))
    scale_f16 = np.empty(512, np.uint16)
    scale_f32 = np.empty(256, np.float32)
    ops = np.empty(127 * 256 * 24, np.uint16)
    assert cc.convcheck_decoders(_ptr(code_f32), _ptr(code_f16), _ptr(lut_fp), _ptr(lut_int), _ptr(scale_f16),
                                 _ptr(scale_f32), _ptr(ops)) == 0
    e2m1 = np.array([orc.e2m1_value(n) for n in range(16)], np.float32)
    ints = np.array([(-1.0 if n & 8 else 1.0) * (n & 7) for n in range(16)], np.float32)
    e4m3 = np.array([orc.e4m3_value(e) for e in range(256)], np.float32)
    b = np.arange(256)
    lo, hi = b & 15, b >> 4
    # byte b repeated in every byte of both words: element 2i low nibble, 2i+1 high
    want16 = np.stack([e2m1[lo], e2m1[hi]] * 8, axis=1)
    want8 = np.stack([e2m1[lo], e2m1[hi]] * 4, axis=1)
    assert np.array_equal(code_f32.reshape(256, 16), want16), "E2M1 -> fp32 conversion"
    assert np.array_equal(np.signbit(code_f32.reshape(256, 16)), np.signbit(want16)), "sign of zero (fp32)"
    assert np.array_equal(_f16(code_f16).reshape(256, 8), want8), "E2M1 -> fp16 conversion"
    assert np.array_equal(_f16(lut_fp).reshape(256, 8), want8), "E2M1 table"
    assert np.array_equal(_f16(lut_int).reshape(256, 8), np.stack([ints[lo], ints[hi]] * 4, axis=1)), "INT table"
    # scale bytes: both halves of the fp16 conversion, NaN exactly at 0x7F / 0xFF
    s16 = _f16(scale_f16).reshape(256, 2)
    nan = np.isnan(e4m3)
    assert np.array_equal(np.isnan(s16[:, 0]), nan) and np.array_equal(np.isnan(s16[:, 1]), nan)
    assert np.array_equal(s16[~nan, 0], e4m3[~nan]) and np.array_equal(s16[~nan, 1], e4m3[~nan]), "E4M3 -> fp16"
    assert np.array_equal(scale_f32[:127], e4m3[:127]), "E4M3 value (quantizers)"
    # GEMM operands: E4M3 scale byte e (0..126) times every code, both paths
    o = _f16(ops).reshape(127, 256, 3, 8)
    sc = e4m3[:127, None, None]
    assert np.array_equal(o[:, :, 0], sc * want8[None]), "GEMM operand decoding (E2M1 conversion)"
    assert np.array_equal(o[:, :, 1], sc * want8[None]), "GEMM operand decoding (E2M1 table)"
    assert np.array_equal(o[:, :, 2], sc * np.stack([ints[lo], ints[hi]] * 4, axis=1)[None]), \
        "GEMM operand decoding (INT table)"
