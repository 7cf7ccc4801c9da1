"""The quantizers divide with a refined hardware reciprocal (rcp_rn / div_rn
in common.hpp) instead of the IEEE division sequence.  These tests check,
on the device, that the refined results are the correctly rounded ones:

- the reciprocal for every b in [2^-60, 2^61) (every significand of 121
  binades) against the device's IEEE reciprocal;
- the quotient for every significand of b against a spread of 4096
  significands of a (the whole product of significands, 2^46 pairs, is
  covered by tests/division_exhaustive.py);
- random pairs across the whole range, zeros, values outside the refined
  range and non-finite ones, against the host's IEEE float32 division.
"""
import ctypes
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_build", "libdivcheck.so")


@pytest.fixture(scope="module")
def dc():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert os.path.exists(LIB), f"{LIB} is missing: run __graft_entry__.build()"
    lib = ctypes.CDLL(LIB)
    u32, u64p, u32p = ctypes.c_uint32, ctypes.POINTER(ctypes.c_ulonglong), ctypes.POINTER(ctypes.c_uint32)
    lib.divcheck_rcp.argtypes = [u32, u32, u64p, u32p]
    lib.divcheck_div.argtypes = [u32, u32, u32, u64p, u32p, u32p]
    lib.divcheck_pairs.argtypes = [ctypes.c_void_p] * 4 + [u32]
    return lib


def test_reciprocal_every_b_in_range(dc):
    bad, fb = ctypes.c_ulonglong(), ctypes.c_uint32()
    assert dc.divcheck_rcp(127 - 60, 121, ctypes.byref(bad), ctypes.byref(fb)) == 0
    assert bad.value == 0, f"{bad.value} reciprocals differ, e.g. b bits {fb.value:#010x}"


def test_quotient_every_b_spread_a(dc):
    bad, fa, fb = ctypes.c_ulonglong(), ctypes.c_uint32(), ctypes.c_uint32()
    # a significands 0x1234 + 2047 k (mod 2^23), k < 4096: spread over the binade
    assert dc.divcheck_div(0x1234, 2047, 4096, ctypes.byref(bad), ctypes.byref(fa), ctypes.byref(fb)) == 0
    assert bad.value == 0, f"{bad.value} quotients differ, e.g. {fa.value:#010x} / {fb.value:#010x}"
    # the significands next to 1 and 2, where the quotient crosses a binade
    for lo in (0, (1 << 23) - 4096):
        assert dc.divcheck_div(lo, 1, 4096, ctypes.byref(bad), ctypes.byref(fa), ctypes.byref(fb)) == 0
        assert bad.value == 0, f"{bad.value} quotients differ, e.g. {fa.value:#010x} / {fb.value:#010x}"


def test_against_host_division(dc):
    rng = np.random.default_rng(77)
    n = 1 << 20
    # log-uniform magnitudes over [2^-70, 2^70]: inside and outside the refined range
    a = np.exp2(rng.uniform(-70, 70, n)).astype(np.float32)
    b = np.exp2(rng.uniform(-70, 70, n)).astype(np.float32)
    a[:1000] = 0.0
    a[1000:1010] = np.inf
    b[1010:1020] = np.inf
    a[1020:1030] = np.nan
    b[1030:1040] = np.float32(2.0 ** -140)              # subnormal divisor
    a[1040:1050] = np.float32(2.0 ** -140)              # subnormal dividend
    q, r = np.empty_like(a), np.empty_like(a)
    ptr = lambda x: x.ctypes.data_as(ctypes.c_void_p)
    assert dc.divcheck_pairs(ptr(a), ptr(b), ptr(q), ptr(r), n) == 0
    with np.errstate(all="ignore"):
        want_q = a / b
        want_r = np.float32(1.0) / b
    nan = np.isnan(want_q)
    assert np.array_equal(np.isnan(q), nan)
    diff = np.flatnonzero(q[~nan].view(np.uint32) != want_q[~nan].view(np.uint32))
    assert diff.size == 0, f"{diff.size} quotients differ, e.g. {a[~nan][diff[0]]!r} / {b[~nan][diff[0]]!r}"
    diff = np.flatnonzero(r.view(np.uint32) != want_r.view(np.uint32))
    assert diff.size == 0, f"{diff.size} reciprocals differ, e.g. 1 / {b[diff[0]]!r}"
