"""Pins of the oracle's per-row absmax quantizer (CPU only).

Pinned against:
  - hand-worked examples (tests/golden/quant_worked_examples.txt);
  - the per-row conversion of the Llama 3 FP8 page, §3.1, formed in numpy
    float32 (row max |x| / 448 floored at 1e-12, IEEE quotient) with only
    the final cast done by PyTorch's float8_e4m3fn, bit for bit on codes and
    scales.  The quotients never exceed 448.00003, inside the range where
    PyTorch's cast and the saturating encoder agree;
  - invariants: the absmax element of each row encodes to +-448, and no code
    is NaN (the NaN/Inf scan of the same page's §4.1).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests._helpers import read_quant_examples


def _library_cast_pin(x: np.ndarray):
    """The per-row conversion the Llama 3 FP8 page describes in §3.1 (scale =
    row max |x| / 448 with a 1e-12 floor, codes = the E4M3 cast of x / scale),
    formed here in numpy float32 (IEEE division, correctly rounded), with only
    the final cast of each quotient done by PyTorch's float8_e4m3fn, the
    library routine that page's conversion relies on."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    scale = np.maximum(amax / np.float32(448.0), np.float32(1e-12)).astype(np.float32)
    quot = (x / scale[:, None]).astype(np.float32)
    q = torch.from_numpy(quot).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return q, scale


@pytest.mark.parametrize("i", range(5))
def test_worked_examples(i):
    row, scale_bits, codes = read_quant_examples()[i]
    q, s = oracle.quantize_rows(row[None, :])
    assert q[0].tolist() == codes.tolist()
    if scale_bits is not None:
        assert int(s.view(np.uint32)[0]) == scale_bits


def _special_rows(K):
    rng = np.random.default_rng(7)
    rows = [
        np.zeros(K),                                          # all zero -> floor scale
        np.where(np.arange(K) % 2 == 0, 0.0, -0.0),           # signed zeros
        np.full(K, 1e-20),                                    # all below the floor
        np.eye(1, K, K // 3)[0] * 3.5,                        # single non-zero
        rng.standard_normal(K) * 1e-30,                       # tiny but not below clamp? (it is: 1e-30/448)
        np.concatenate([[1e4], rng.standard_normal(K - 1) * 1e-3]),  # huge outlier: subnormal codes
        -np.abs(rng.standard_normal(K)),                      # all negative
        rng.standard_normal(K) * 3e38 / 10,                   # near fp32 max
        np.full(K, 448.0),
        (rng.integers(-8, 9, K) * 2.0 ** -9),                 # exact grid values
    ]
    return np.array(rows, dtype=np.float32)


@pytest.mark.parametrize("K", [16, 256, 4096])
def test_matches_library_cast_on_synthetic_and_special_rows(K):
    x, _ = synth.activations(64, K, synth.n_outlier_channels(K) or 1, 50.0, seed=3)
    x = np.concatenate([x, _special_rows(K)])
    q, s = oracle.quantize_rows(x)
    tq, ts = _library_cast_pin(x)
    assert np.array_equal(s.view(np.uint32), ts.view(np.uint32))
    assert np.array_equal(q, tq)


def test_matches_library_cast_on_weight_rows():
    w = synth.weights(512, 1024, seed=5)
    q, s = oracle.quantize_rows(w)
    tq, ts = _library_cast_pin(w)
    assert np.array_equal(s.view(np.uint32), ts.view(np.uint32))
    assert np.array_equal(q, tq)


def test_invariants_absmax_maps_to_448_and_no_nan_codes():
    x, _ = synth.activations(128, 2048, 20, 50.0, seed=11)
    q, s = oracle.quantize_rows(x)
    am = np.argmax(np.abs(x), axis=1)
    top = q[np.arange(x.shape[0]), am]
    assert np.all(np.isin(top, [0x7E, 0xFE]))
    assert not np.any(np.isin(q, [0x7F, 0xFF]))
    assert np.all(s > 0) and np.all(np.isfinite(s))


def test_scale_floor_is_the_fp32_nearest_to_1e_12():
    q, s = oracle.quantize_rows(np.zeros((1, 16), dtype=np.float32))
    assert int(s.view(np.uint32)[0]) == 0x2B8CBCCC
    assert np.all(q == 0)
