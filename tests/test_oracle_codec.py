"""Pins of the oracle's E4M3 codec (CPU only).

The codec is pinned to things other than itself:
  - the E4M3 endpoints the pages state (tests/golden/e4m3_fixed_points.txt);
  - PyTorch's float8_e4m3fn, the type the Llama 3 FP8 page's §3.1 conversion
    snippet casts to: its decode of all 256 codes, and its cast of finite
    values with |v| <= 464 (beyond that PyTorch returns NaN, the overflow the
    same page's §4.1 warns about, while the method saturates to +-448);
  - an independent brute-force nearest-value encoder over all 2^32 fp32
    bit patterns (tests/pins/encode_pin.c);
  - structure: monotone magnitudes, sign symmetry, round trip.
"""
import ctypes

import numpy as np
import pytest

import oracle
from tests._helpers import pin_lib, read_fixed_points, torch_e4m3_values, torch_encode

ALL_CODES = np.arange(256, dtype=np.uint8)


def test_fixed_points_from_pages():
    for code, value in read_fixed_points():
        assert oracle.decode([code])[0] == value, hex(code)
        assert oracle.encode(np.array([value], dtype=np.float32))[0] == code, value


def test_decode_matches_pytorch_float8_e4m3fn_on_all_256_codes():
    ours = oracle.decode(ALL_CODES)
    ref = torch_e4m3_values()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zero is kept
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def test_decode_structure():
    v = oracle.decode(ALL_CODES)
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0), "magnitudes must increase with the code"
    assert np.array_equal(v[0x80:0xFF], -pos)
    assert pos[1] == 2.0 ** -9 and pos[8] == 2.0 ** -6 and pos[-1] == 448.0
    # every value is a multiple of 2^-9 below 2^17 (what makes the GEMM sum exact)
    assert np.all(np.mod(pos * 512, 1) == 0) and pos.max() * 512 == 229376


def test_round_trip_all_finite_codes():
    v = oracle.decode(ALL_CODES)
    finite = ~np.isnan(v)
    back = oracle.encode(v[finite].astype(np.float32))
    assert np.array_equal(back, ALL_CODES[finite])


def test_special_inputs():
    vals = np.array([np.nan, -np.nan, np.inf, -np.inf, 449.0, 464.0, 465.0, 1e30, -1e30, 0.0, -0.0,
                     2.0 ** -10, -(2.0 ** -10), 1e-45, -1e-45], dtype=np.float32)
    got = oracle.encode(vals)
    want = [0x7F, 0xFF, 0x7E, 0xFE, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x00, 0x80, 0x00, 0x80, 0x00, 0x80]
    assert got.tolist() == want


def _sample_finite_le_464(n, seed):
    """fp32 values with |v| <= 464: uniform bit patterns per binade, plus every
    E4M3 midpoint and its fp32 neighbours (the rounding-decision points)."""
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 0x43E80000 + 1, size=n, dtype=np.uint32)  # 0x43E80000 = 464.0f
    v = bits.view(np.float32)
    mags = oracle.decode(ALL_CODES[:0x7F])
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    mids = np.concatenate([mids, [np.float32(464.0)]])
    neigh = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    out = np.concatenate([v, neigh, mags.astype(np.float32)])
    out = np.concatenate([out, -out])
    return out[np.abs(out) <= 464.0]


def test_encode_matches_pytorch_cast_for_finite_values_up_to_464():
    v = _sample_finite_le_464(1 << 20, seed=1)
    ours = np.empty(v.size, dtype=np.uint8)
    # the Python wrapper calls the C encoder element by element; keep it fast
    enc = ctypes.CFUNCTYPE(ctypes.c_uint8, ctypes.c_float)(oracle.encode_fn_address())
    for i, x in enumerate(v.tolist()):
        ours[i] = enc(x)
    assert np.array_equal(ours, torch_encode(v))


def test_pytorch_cast_overflows_where_the_method_saturates():
    # Documents the reading: PyTorch gives NaN above 464, the method saturates.
    v = np.array([465.0, 1000.0, -2000.0], dtype=np.float32)
    assert np.all(np.isin(torch_encode(v), [0x7F, 0xFF]))
    assert oracle.encode(v).tolist() == [0x7E, 0x7E, 0xFE]


def test_encode_exhaustive_against_brute_force_all_fp32_patterns():
    mags = np.ascontiguousarray(torch_e4m3_values()[:0x7F], dtype=np.float64)
    L = pin_lib()
    first = ctypes.c_uint32(0)
    bad = L.pin_encode_range(ctypes.c_void_p(oracle.encode_fn_address()), ctypes.c_void_p(mags.ctypes.data),
                             0, 1 << 32, ctypes.byref(first))
    assert bad == 0, f"{bad} mismatches, first fp32 pattern 0x{first.value:08x}"


def test_brute_force_pin_catches_a_planted_encoder_mistake():
    """The exhaustive pin must fail for an encoder that rounds ties away from zero."""
    mags = np.ascontiguousarray(torch_e4m3_values()[:0x7F], dtype=np.float64)
    L = pin_lib()

    @ctypes.CFUNCTYPE(ctypes.c_uint8, ctypes.c_float)
    def ties_away(v):
        c = oracle.lib().oracle_e4m3_encode(v)
        a = abs(float(v))
        lo = int(c & 0x7F)
        if lo < 0x7E and a == (mags[lo] + mags[lo + 1]) / 2:
            return (c & 0x80) | (lo + 1)
        return c

    first = ctypes.c_uint32(0)
    # 232 is a tie the correct encoder sends down to the even code 0x76 (224)
    u = int(np.array([232.0], dtype=np.float32).view(np.uint32)[0])
    bad = L.pin_encode_range(ctypes.cast(ties_away, ctypes.c_void_p), ctypes.c_void_p(mags.ctypes.data),
                             u - 4, u + 4, ctypes.byref(first))
    assert bad >= 1


@pytest.mark.parametrize("v", [2.0 ** -10, 3 * 2.0 ** -10, 232.0, 7.5 * 2.0 ** -9, 447.0, 460.0, 1e-40])
def test_brute_force_agrees_on_hand_cases(v):
    mags = np.ascontiguousarray(torch_e4m3_values()[:0x7F], dtype=np.float64)
    got = pin_lib().pin_encode_one(ctypes.c_void_p(mags.ctypes.data), v)
    assert got == oracle.encode(np.array([v], dtype=np.float32))[0]
