"""Pins of the oracle's IEEE binary16 rounding (CPU only).

The 16-bit read back of the FP8 KV cache (the 512K-context page, §3.3: FP8
takes the place of an FP16 KV cache) rounds fl32(dec(code) * scale) to the
nearest binary16 value, ties to even.  The oracle's encoder is pinned against
  - PyTorch's float32 -> float16 cast on random fp32 bit patterns (one
    rounding from a value exactly representable in both);
  - numpy's float64 -> float16 conversion on random doubles (a direct
    conversion, one rounding);
  - every exact tie between adjacent binary16 values and the fp32 neighbours
    on both sides, with the even code worked out from the code's last bit;
  - the IEEE boundary values: the largest finite value 65504, the overflow
    threshold 65520, the smallest subnormal 2^-24 and the half of it;
and a planted ties-away rounding is caught by the tie set.
"""
import numpy as np
import torch

import oracle


def _torch_fp16_bits(v32):
    return torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32)).to(torch.float16) \
        .view(torch.int16).numpy().view(np.uint16)


def test_fp16_matches_torch_on_random_fp32_patterns():
    rng = np.random.default_rng(16)
    bits = rng.integers(0, 2 ** 32, 400000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    # also the magnitudes where binary16 lives (2^-26 .. 2^17)
    mag = (rng.random(400000) * 2.0 ** rng.integers(-26, 17, 400000)).astype(np.float32)
    v = np.concatenate([v, mag, -mag])
    ours = oracle.fp16_from_double(v.astype(np.float64))
    assert np.array_equal(ours, _torch_fp16_bits(v))


def test_fp16_matches_numpy_on_random_doubles():
    rng = np.random.default_rng(17)
    v = rng.standard_normal(300000) * 2.0 ** rng.integers(-28, 18, 300000)
    ours = oracle.fp16_from_double(v)
    assert np.array_equal(ours, v.astype(np.float16).view(np.uint16))


def _all_ties():
    """Midpoints between every pair of adjacent finite binary16 magnitudes
    (codes c, c + 1 for c in 0 .. 0x7BFE, and 65504 .. 65536), with the code
    ties-to-even picks (the even one of c, c + 1)."""
    codes = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = codes.view(np.float16).astype(np.float64)
    hi = (codes + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2.0                      # 12 significant bits: exact in fp32
    even = np.where(codes % 2 == 0, codes, codes + 1).astype(np.uint16)
    # the last finite value 65504 (0x7BFF, odd) and 2^16 (0x7C00 would be next): ties go up, to infinity
    mid = np.append(mid, (65504.0 + 65536.0) / 2.0)
    even = np.append(even, np.uint16(0x7C00))
    return mid, even


def test_fp16_ties_go_to_the_even_code_and_neighbours_to_the_nearest():
    mid, even = _all_ties()
    m32 = mid.astype(np.float32)
    assert np.array_equal(m32.astype(np.float64), mid), "midpoints must be exact in fp32"
    ours = oracle.fp16_from_double(mid)
    assert np.array_equal(ours, even)
    assert np.array_equal(oracle.fp16_from_double(-mid), even | np.uint16(0x8000))
    below = np.nextafter(m32, np.float32(0)).astype(np.float64)
    above = np.nextafter(m32, np.float32(np.inf)).astype(np.float64)
    for v in (mid, below, above, -below, -above):
        assert np.array_equal(oracle.fp16_from_double(v), _torch_fp16_bits(v.astype(np.float32)))


def test_planted_ties_away_rounding_is_caught():
    mid, even = _all_ties()
    codes = np.arange(0, 0x7BFF, dtype=np.uint16)
    away = np.append(codes + 1, np.uint16(0x7C00)).astype(np.uint16)   # ties away from zero: always up
    assert not np.array_equal(away, oracle.fp16_from_double(mid))
    assert np.sum(away != even) == (0x7BFF + 1) // 2   # every tie whose lower neighbour is even


def test_fp16_boundaries():
    f = lambda v: int(oracle.fp16_from_double(np.array([v], np.float64))[0])
    assert f(65504.0) == 0x7BFF
    assert f(np.nextafter(65520.0, 0.0)) == 0x7BFF
    assert f(65520.0) == 0x7C00                      # overflow threshold: rounds to infinity
    assert f(1e6) == 0x7C00 and f(-1e6) == 0xFC00
    assert f(float("inf")) == 0x7C00
    assert f(2.0 ** -24) == 0x0001                  # smallest subnormal
    assert f(2.0 ** -25) == 0x0000                  # its half: tie to the even code 0
    assert f(np.nextafter(2.0 ** -25, 1.0)) == 0x0001
    assert f(3 * 2.0 ** -25) == 0x0002              # tie between 1 and 2 (x 2^-24): even 2
    assert f(2.0 ** -14) == 0x0400                  # smallest normal
    assert f(-0.0) == 0x8000 and f(0.0) == 0x0000
    assert f(1.0) == 0x3C00 and f(-2.0) == 0xC000
    assert (f(float("nan")) & 0x7E00) == 0x7E00
