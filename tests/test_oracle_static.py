"""Pins of the oracle's static / hybrid activation scales (DeepSeek V4 950
page: §3.1 static scale from the P99.9 percentile of calibration data, §2.4
per-token + per-tensor hybrid, §4.2 values above a calibrated percentile
clipped): the static quantizer against PyTorch's clamp + float8_e4m3fn cast,
the clipped per-token quantizer against the plain absmax quantizer (the clip
above the maximum is a no-op) and against PyTorch, and the nearest-rank
percentile against numpy's inverted-CDF percentile and hand-worked ranks."""
import numpy as np
import pytest
import torch

import oracle


def torch_cast_saturating(q):
    t = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float32))
    return torch.clamp(t, -448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("scale", [1.0, 0.02, 3.5e-3, 1e-12, 7.0])
def test_static_quantizer_matches_torch(scale):
    rng = np.random.default_rng(int(scale * 1e6) % 1000)
    x = (rng.standard_normal((16, 256)) * rng.choice([0.01, 1.0, 30.0, 1e4], (16, 1))).astype(np.float32)
    s = np.float32(scale)
    want = torch_cast_saturating(x / s)
    got = oracle.quantize_static(x, s)
    assert np.array_equal(got, want)


def test_static_quantizer_saturates():
    x = np.array([[448.0, 449.0, 1e6, -1e6, 464.0, -0.0, 0.0]], np.float32)
    q = oracle.quantize_static(x, np.float32(1.0))
    assert list(q[0]) == [0x7E, 0x7E, 0x7E, 0xFE, 0x7E, 0x80, 0x00]


def test_clipped_quantizer_reduces_to_absmax_when_clip_is_large():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((32, 300)) * 5).astype(np.float32)
    q1, s1 = oracle.quantize_rows(x)
    q2, s2 = oracle.quantize_rows_clipped(x, np.float32(np.inf))
    assert np.array_equal(q1, q2) and np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
    q3, s3 = oracle.quantize_rows_clipped(x, np.abs(x).max())
    assert np.array_equal(q1, q3) and np.array_equal(s1.view(np.uint32), s3.view(np.uint32))


def test_clipped_quantizer_matches_torch():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((8, 512)).astype(np.float32)
    x[:, 7] *= 200.0                      # outlier channel
    clip = np.float32(20.0)
    q, s = oracle.quantize_rows_clipped(x, clip)
    amax = np.minimum(np.abs(x).max(axis=1), clip)
    want_s = np.maximum(amax / np.float32(448.0), np.float32(1e-12)).astype(np.float32)
    assert np.array_equal(s.view(np.uint32), want_s.view(np.uint32))
    assert np.array_equal(q, torch_cast_saturating(x / want_s[:, None]))
    assert np.all(q[:, 7] & 0x7F == 0x7E)   # the clipped outliers saturate


def test_percentile_hand_worked():
    v = np.arange(1, 1001, dtype=np.float32)
    assert oracle.percentile_nearest_rank(v, 999, 1000) == 999.0      # r = ceil(999.0) = 999
    assert oracle.percentile_nearest_rank(v, 9999, 10000) == 1000.0   # r = ceil(999.9) = 1000
    assert oracle.percentile_nearest_rank(v, 1, 2) == 500.0
    assert oracle.percentile_nearest_rank(v, 1, 1) == 1000.0
    assert oracle.percentile_nearest_rank(-v, 1, 1000) == 1.0         # magnitudes; r = 1
    assert oracle.percentile_nearest_rank(np.array([-3.0], np.float32), 999, 1000) == 3.0
    assert oracle.static_scale(448.0) == np.float32(1.0)
    assert oracle.static_scale(0.0) == np.float32(1e-12)


def test_percentile_matches_numpy_inverted_cdf():
    rng = np.random.default_rng(3)
    for n in (1, 2, 7, 1000, 4097, 100003):
        x = rng.standard_normal(n).astype(np.float32) * 3
        x[: n // 50] = np.round(x[: n // 50])          # ties
        for num, den in ((999, 1000), (9999, 10000), (1, 2), (1, 1), (1, 3)):
            want = np.percentile(np.abs(x), 100.0 * num / den, method="inverted_cdf")
            got = oracle.percentile_nearest_rank(x, num, den)
            # inverted_cdf = smallest value whose empirical CDF >= p (the nearest rank)
            assert got == np.float32(want), (n, num, den)
