"""Pins of the oracle's E5M2 codec and of its KV-cache functions (CPU only).

The E5M2 codec is pinned like the E4M3 one:
  - the E5M2 endpoints the pages state (tests/golden/e5m2_fixed_points.txt);
  - PyTorch's float8_e5m2 (the KV-cache dtype of the DeepSeek V4 950 page's
    deployment command, §3): its decode of all 256 codes and its cast of
    finite values below 59392 (above that PyTorch goes to infinity while the
    cache codec saturates at 57344);
  - the independent brute-force nearest-value encoder over all 2^32 fp32 bit
    patterns (tests/pins/encode_pin.c with the 124 finite E5M2 magnitudes).
The KV functions (per-channel scales, paged quantize and read back) are
pinned by: the per-channel maximum landing exactly on the format's largest
code, the codec's error bound on the read back, a pure-Python loop over the
block table that casts with PyTorch, and the skip / zero rules for slots
outside the cache.
"""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from tests._helpers import (pin_lib, read_fixed_points, torch_e4m3_values, torch_e5m2_values, torch_encode,
                            torch_encode_e5m2)

ALL_CODES = np.arange(256, dtype=np.uint8)
E5M2_FINITE = 124  # codes 0x00..0x7B


def _e5m2_enc():
    return ctypes.CFUNCTYPE(ctypes.c_uint8, ctypes.c_float)(oracle.e5m2_encode_fn_address())


def test_e5m2_fixed_points_from_pages():
    for code, value in read_fixed_points("e5m2_fixed_points.txt"):
        assert oracle.e5m2_decode([code])[0] == value, hex(code)
        assert oracle.e5m2_encode(np.array([value], dtype=np.float32))[0] == code, value


def test_e5m2_decode_matches_pytorch_on_all_256_codes():
    ours = oracle.e5m2_decode(ALL_CODES)
    ref = torch_e5m2_values()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert set(np.nonzero(np.isnan(ref))[0].tolist()) == {0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF}
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert ours[0x7C] == np.inf and ours[0xFC] == -np.inf


def test_e5m2_decode_structure():
    v = oracle.e5m2_decode(ALL_CODES)
    pos = v[:E5M2_FINITE]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(v[0x80:0x80 + E5M2_FINITE], -pos)
    # smallest subnormal 2^-16, smallest normal 2^-14, largest 57344 = 1.75 * 2^15
    assert pos[1] == 2.0 ** -16 and pos[4] == 2.0 ** -14 and pos[-1] == 57344.0
    # 4 values per binade above 2^-14, spaced 2^(e-2)
    for e in range(-14, 16):
        b = pos[(pos >= 2.0 ** e) & (pos < 2.0 ** (e + 1))]
        assert np.array_equal(b, 2.0 ** e * np.array([1.0, 1.25, 1.5, 1.75])[:b.size]) and b.size == 4


def test_e5m2_round_trip_all_finite_codes():
    v = oracle.e5m2_decode(ALL_CODES)
    fin = np.isfinite(v)
    assert np.array_equal(oracle.e5m2_encode(v[fin].astype(np.float32)), ALL_CODES[fin])


def test_e5m2_special_inputs():
    vals = np.array([np.nan, -np.nan, np.inf, -np.inf, 57345.0, 61440.0, 1e30, -1e30, 0.0, -0.0,
                     2.0 ** -17, -(2.0 ** -17), 3 * 2.0 ** -18, 1e-45], dtype=np.float32)
    got = oracle.e5m2_encode(vals)
    want = [0x7F, 0xFF, 0x7B, 0xFB, 0x7B, 0x7B, 0x7B, 0xFB, 0x00, 0x80, 0x00, 0x80, 0x01, 0x00]
    assert got.tolist() == want


def test_e5m2_encode_matches_pytorch_below_59392():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 0x47680000, size=1 << 19, dtype=np.uint32)  # 0x47680000 = 59392.0f
    mags = oracle.e5m2_decode(ALL_CODES[:E5M2_FINITE])
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    v = np.concatenate([bits.view(np.float32), mids, np.nextafter(mids, np.float32(0)),
                        np.nextafter(mids, np.float32(1e9)), mags.astype(np.float32)])
    v = np.concatenate([v, -v])
    v = v[np.abs(v) < 59392.0]
    enc = _e5m2_enc()
    ours = np.fromiter((enc(x) for x in v.tolist()), dtype=np.uint8, count=v.size)
    assert np.array_equal(ours, torch_encode_e5m2(v))


def test_e5m2_encode_exhaustive_against_brute_force_all_fp32_patterns():
    mags = np.ascontiguousarray(torch_e5m2_values()[:E5M2_FINITE], dtype=np.float64)
    first = ctypes.c_uint32(0)
    bad = pin_lib().pin_encode_range_n(ctypes.c_void_p(oracle.e5m2_encode_fn_address()),
                                       ctypes.c_void_p(mags.ctypes.data), E5M2_FINITE, 0, 1 << 32,
                                       ctypes.byref(first))
    assert bad == 0, f"{bad} mismatches, first fp32 pattern 0x{first.value:08x}"


def test_brute_force_e5m2_pin_catches_a_planted_mistake():
    """An encoder that truncates instead of rounding must fail the pin."""
    mags = np.ascontiguousarray(torch_e5m2_values()[:E5M2_FINITE], dtype=np.float64)

    @ctypes.CFUNCTYPE(ctypes.c_uint8, ctypes.c_float)
    def truncating(v):
        c = oracle.lib().oracle_e5m2_encode(v)
        lo = int(c & 0x7F)
        if lo > 0 and mags[lo] > abs(float(v)):
            return (c & 0x80) | (lo - 1)
        return c

    u = int(np.array([1.2], dtype=np.float32).view(np.uint32)[0])  # 1.2 rounds up to 1.25
    first = ctypes.c_uint32(0)
    bad = pin_lib().pin_encode_range_n(ctypes.cast(truncating, ctypes.c_void_p), ctypes.c_void_p(mags.ctypes.data),
                                       E5M2_FINITE, u, u + 4, ctypes.byref(first))
    assert bad >= 1


FMT_MAX = {oracle.E4M3: 448.0, oracle.E5M2: 57344.0}
FMT_TOP = {oracle.E4M3: 0x7E, oracle.E5M2: 0x7B}


def _kv(T, C, seed):
    return synth.kv_activations(T, C, seed=seed)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_channel_scale_puts_each_channel_max_on_the_top_code(fmt):
    kv = _kv(96, 160, seed=1)
    kv[:, 7] = 0.0  # an all-zero channel takes the 1e-12 floor
    s = oracle.kv_channel_scales(kv, fmt)
    assert s[7] == np.float32(1e-12)
    slot = np.arange(96, dtype=np.int32)
    cache = oracle.kv_quantize(kv, s, fmt, slot, 96)
    top = (cache & 0x7F).max(axis=0)
    live = np.abs(kv).max(axis=0) > 0
    assert np.all(top[live] == FMT_TOP[fmt])
    assert np.all(cache[:, 7] & 0x7F == 0)
    # the scale is the channel maximum over the format's maximum, to fp32 rounding
    amax = np.abs(kv.astype(np.float64)).max(axis=0)
    assert np.allclose(s[live], amax[live] / FMT_MAX[fmt], rtol=2.0 ** -24, atol=0)


@pytest.mark.parametrize("fmt,rel,sub", [(oracle.E4M3, 2.0 ** -4, 2.0 ** -10), (oracle.E5M2, 2.0 ** -3, 2.0 ** -17)])
def test_read_back_within_the_codec_error_bound(fmt, rel, sub):
    """Half a quantum: |x - x'| <= max(rel * |x|, sub * s) for each element."""
    T, C, B = 200, 96, 16
    kv = _kv(T, C, seed=2)
    s = oracle.kv_channel_scales(kv, fmt)
    slot = synth.kv_slot_mapping(T, B, num_blocks=T // B + 3, seed=2)
    cache = oracle.kv_quantize(kv, s, fmt, slot, (T // B + 3) * B)
    back = oracle.kv_dequantize(cache, slot, s, fmt).astype(np.float64)
    err = np.abs(back - kv)
    bound = np.maximum(rel * np.abs(kv.astype(np.float64)), sub * s[None, :].astype(np.float64)) * (1 + 2.0 ** -20)
    assert np.all(err <= bound)
    # and the error is not trivially zero: the codec really rounds
    assert err.max() > 0


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_paged_write_and_read_against_a_python_loop(fmt):
    T, C, B, nb = 37, 24, 8, 9
    kv = _kv(T, C, seed=3)
    s = oracle.kv_channel_scales(kv, fmt) * np.float32(1.5)  # a stale scale: nothing saturates
    slot = synth.kv_slot_mapping(T, B, nb, seed=3)
    slot[[4, 20]] = -1  # padding tokens
    slot[30] = nb * B + 5  # beyond the cache: skipped too
    ns = nb * B
    prior = np.full((ns, C), 0x11, dtype=np.uint8)
    cache = oracle.kv_quantize(kv, s, fmt, slot, ns, cache=prior)
    want = prior.copy()
    cast = torch_encode if fmt == oracle.E4M3 else torch_encode_e5m2
    table = torch_e4m3_values() if fmt == oracle.E4M3 else torch_e5m2_values()
    for t in range(T):
        if 0 <= slot[t] < ns:
            want[slot[t]] = cast((kv[t] / s).astype(np.float32))
    assert np.array_equal(cache, want)
    back = oracle.kv_dequantize(cache, slot, s, fmt)
    for t in range(T):
        if 0 <= slot[t] < ns:
            assert np.array_equal(back[t], (table[cache[slot[t]]].astype(np.float32) * s))
        else:
            assert np.all(back[t] == 0)


def test_saturation_at_the_format_maximum():
    """A stale (too small) scale makes values overflow: they saturate, never NaN/inf."""
    kv = np.array([[1000.0, -1e6, 3.0, 0.5]], dtype=np.float32)
    s = np.ones(4, dtype=np.float32)
    c4 = oracle.kv_quantize(kv, s, oracle.E4M3, np.array([0], np.int32), 1)
    c5 = oracle.kv_quantize(kv, s, oracle.E5M2, np.array([0], np.int32), 1)
    assert c4[0].tolist() == [0x7E, 0xFE, 0x44, 0x30]
    assert c5[0].tolist() == [0x64, 0xFB, 0x42, 0x38]
