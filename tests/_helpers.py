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
