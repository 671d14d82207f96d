"""The GPU quantizer divides each element by its row scale with a reciprocal
and two fused multiply-adds instead of a full IEEE division.  The codes are
defined by the correctly rounded quotient fl32(x / s) (Llama 3 FP8 page,
§3.1), so the method must give that quotient bit for bit.  This checks it on
the CPU with the C library's correctly rounded fmaf: random scales over the
whole range a row scale takes, any finite x (overflowing quotients too), and
every x within a few ulps of s times an E4M3 or E5M2 value or rounding
midpoint (where a one-ulp error would flip a code).  The GPU tests then compare the kernels' codes with the oracle."""
import ctypes
import os
import subprocess
import tempfile

import numpy as np
import pytest

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def lib():
    global _lib
    if _lib is None:
        out = os.path.join(tempfile.mkdtemp(prefix="fp8divpin_"), "libdiv_pin.so")
        subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-fno-fast-math",
                        "-ffp-contract=off", os.path.join(_HERE, "pins", "div_pin.c"), "-o", out, "-lm"],
                       check=True)
        L = ctypes.CDLL(out)
        L.pin_div_random.restype = ctypes.c_uint64
        L.pin_div_random.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.POINTER(ctypes.c_float),
                                     ctypes.POINTER(ctypes.c_float)]
        L.pin_div_boundaries.restype = ctypes.c_uint64
        L.pin_div_boundaries.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.POINTER(ctypes.c_uint64)]
        L.pin_div_any_x.restype = ctypes.c_uint64
        L.pin_div_any_x.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.POINTER(ctypes.c_float),
                                    ctypes.POINTER(ctypes.c_float)]
        _lib = L
    return _lib


def test_random_scales_and_elements():
    bx, bs = ctypes.c_float(0), ctypes.c_float(0)
    bad = lib().pin_div_random(1 << 28, 1, ctypes.byref(bx), ctypes.byref(bs))
    assert bad == 0, f"{bad} mismatches, e.g. x={bx.value!r} s={bs.value!r}"


def test_any_finite_x_including_overflowing_quotients():
    """A static or stale scale can make x / s overflow fp32; the method must
    then still give a quotient past both formats' saturation points."""
    bx, bs = ctypes.c_float(0), ctypes.c_float(0)
    bad = lib().pin_div_any_x(1 << 26, 3, ctypes.byref(bx), ctypes.byref(bs))
    assert bad == 0, f"{bad} mismatches, e.g. x={bx.value!r} s={bs.value!r}"


@pytest.mark.parametrize("fmt", [0, 1], ids=["e4m3", "e5m2"])
def test_fp8_boundaries_for_many_scales(fmt):
    rng = np.random.default_rng(7)
    special = [1.0, 1e-12, np.nextafter(np.float32(2.0), np.float32(0)), 1.5, 1.0 + 2.0 ** -23,
               448.0 / 448.0, 2.0 ** -40, 3.0, 7.0 / 448.0, 1.0 / 3.0]
    mant = rng.integers(0, 1 << 23, 4000, dtype=np.uint32)
    expo = rng.integers(127 - 40, 127 + 60, 4000, dtype=np.uint32)
    rand = ((expo << 23) | mant).view(np.float32)
    scales = np.concatenate([np.array(special, np.float32), rand]).astype(np.float32)
    checked = ctypes.c_uint64(0)
    bad = lib().pin_div_boundaries(scales.ctypes.data, scales.size, 3, fmt, ctypes.byref(checked))
    assert checked.value > 10_000_000
    assert bad == 0, f"{bad} of {checked.value} boundary quotients differ from IEEE division"
