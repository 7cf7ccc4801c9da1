"""Every pair of significands (2^23 x 2^23) through div_rn on the device,
against the device's IEEE quotient, in 64 launches with a progress line
each (about a minute on one MI355X):

    python tests/division_exhaustive.py

Not collected by pytest; tests/test_gpu_division.py runs a spread of the
same check."""
import ctypes
import os
import sys
import time

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_build", "libdivcheck.so")


def main():
    lib = ctypes.CDLL(LIB)
    u32, u64p, u32p = ctypes.c_uint32, ctypes.POINTER(ctypes.c_ulonglong), ctypes.POINTER(ctypes.c_uint32)
    lib.divcheck_div.argtypes = [u32, u32, u32, u64p, u32p, u32p]
    bad, fa, fb = ctypes.c_ulonglong(), ctypes.c_uint32(), ctypes.c_uint32()
    total = 0
    t0 = time.time()
    per = (1 << 23) // 64
    for s in range(64):
        st = lib.divcheck_div(s * per, 1, per, ctypes.byref(bad), ctypes.byref(fa), ctypes.byref(fb))
        if st != 0:
            print(f"HIP error {st}", flush=True)
            return 2
        total += bad.value
        print(f"slice {s + 1}/64: a significands {s * per:#08x}..{(s + 1) * per - 1:#08x}, "
              f"mismatches {bad.value}" + (f" (e.g. {fa.value:#010x} / {fb.value:#010x})" if bad.value else "")
              + f", {time.time() - t0:.1f} s", flush=True)
    print(f"checked {(1 << 46)} quotients of significands: {total} mismatches", flush=True)
    return 0 if total == 0 else 1


if __name__ == "__main__":
    sys.exit(main())
