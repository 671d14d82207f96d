"""Shared test helpers: torch-side E4M3 tables and the C pin library."""
import ctypes
import os
import subprocess
import tempfile

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_pin_lib = None


def torch_e4m3_values():
    """float64 value of each of the 256 codes, decoded by PyTorch's float8_e4m3fn."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_e5m2_values():
    """float64 value of each of the 256 codes, decoded by PyTorch's float8_e5m2."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e5m2).to(torch.float64).numpy()


def torch_encode_e5m2(v):
    """PyTorch's float32 -> float8_e5m2 cast, as uint8 codes."""
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(torch.float8_e5m2).view(torch.uint8).numpy()


def torch_encode(v):
    """PyTorch's float32 -> float8_e4m3fn cast, as uint8 codes."""
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_lib():
    """Compile tests/pins/encode_pin.c into a temp dir and load it."""
    global _pin_lib
    if _pin_lib is None:
        out = os.path.join(tempfile.mkdtemp(prefix="fp8pins_"), "libencode_pin.so")
        subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-fno-fast-math",
                        "-ffp-contract=off", os.path.join(_HERE, "pins", "encode_pin.c"), "-o", out, "-lm"],
                       check=True)
        L = ctypes.CDLL(out)
        L.pin_encode_range.restype = ctypes.c_uint64
        L.pin_encode_range.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                                       ctypes.POINTER(ctypes.c_uint32)]
        L.pin_encode_one.restype = ctypes.c_uint8
        L.pin_encode_one.argtypes = [ctypes.c_void_p, ctypes.c_float]
        L.pin_encode_range_n.restype = ctypes.c_uint64
        L.pin_encode_range_n.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64,
                                         ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint32)]
        L.pin_encode_one_n.restype = ctypes.c_uint8
        L.pin_encode_one_n.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_float]
        _pin_lib = L
    return _pin_lib


def read_fixed_points(name="e4m3_fixed_points.txt"):
    rows = []
    with open(os.path.join(_HERE, "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, value = line.split()[:2]
            rows.append((int(code, 16), float(value)))
    return rows


def read_quant_examples():
    """[(row float32, scale bits or None, codes uint8)] from quant_worked_examples.txt."""
    ex, cur = [], {}
    with open(os.path.join(_HERE, "golden", "quant_worked_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            cur[key.strip()] = val.split()
            if key.strip() == "codes":
                row = np.array([float(v) for v in cur["row"]], dtype=np.float32)
                sc = None if cur["scale"][0] == "-" else int(cur["scale"][0], 16)
                codes = np.array([int(c, 16) for c in cur["codes"]], dtype=np.uint8)
                assert row.size == codes.size
                ex.append((row, sc, codes))
                cur = {}
    return ex


def _code_key(c):
    """Order of E4M3 codes by value (-0 and +0 share 0): magnitude bits,
    negated for the sign bit."""
    c = np.asarray(c, dtype=np.int64)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


def fp8out_admissible(q, s, ref, absref, rel_abs=1e-3, rel_ref=2.0 ** -22):
    """Which FP8-output codes and scales are consistent with *some* fp32
    output y32 within the GEMM bound b = rel_abs * absref + rel_ref * |ref|
    of the exact scaled product ref (the output the FP32 accumulation may
    produce in any order), quantized per row as the pages define it
    (s = max(fl32(max|y32| / 448), 1e-12f), codes E4M3(fl32(y32 / s))).

    Returns dict(scale_ok [M] bool: s within [S(lo), S(hi)] where lo / hi
    bound the row maximum of |y32|; scale_ambiguous [M]: S(lo) != S(hi);
    code_ok [M,N]: q between the codes of the lowest and highest quotient
    (ref -+ b) / s can take; code_ambiguous [M,N]: those two codes differ,
    i.e. the interval holds an E4M3 rounding boundary)."""
    import oracle
    ref = np.asarray(ref, np.float64)
    b = rel_abs * np.asarray(absref, np.float64) + rel_ref * np.abs(ref)
    s = np.asarray(s, np.float32)
    lo = np.maximum(np.abs(ref) - b, 0.0).max(axis=1) if ref.shape[1] else np.zeros(ref.shape[0])
    hi = (np.abs(ref) + b).max(axis=1) if ref.shape[1] else np.zeros(ref.shape[0])
    lo32 = np.nextafter(lo.astype(np.float32), np.float32(0))      # <= lo
    hi32 = np.nextafter(hi.astype(np.float32), np.float32(np.inf))  # >= hi
    floor = np.float32(1e-12)
    s_lo = np.maximum(lo32 / np.float32(448.0), floor)
    s_hi = np.maximum(hi32 / np.float32(448.0), floor)
    scale_ok = (s >= s_lo) & (s <= s_hi)
    sd = s.astype(np.float64)[:, None]
    eps = 2.0 ** -23   # the quotient's own fp32 rounding, widened
    z_lo = (ref - b) / sd
    z_hi = (ref + b) / sd
    z_lo = z_lo - np.abs(z_lo) * eps
    z_hi = z_hi + np.abs(z_hi) * eps
    c_lo = oracle.encode(np.nextafter(z_lo.astype(np.float32), np.float32(-np.inf)))
    c_hi = oracle.encode(np.nextafter(z_hi.astype(np.float32), np.float32(np.inf)))
    k, k_lo, k_hi = _code_key(q), _code_key(c_lo), _code_key(c_hi)
    return dict(scale_ok=scale_ok, scale_ambiguous=s_lo != s_hi,
                code_ok=(k >= k_lo) & (k <= k_hi), code_ambiguous=k_lo != k_hi)
