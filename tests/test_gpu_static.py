"""GPU parity of the static / hybrid activation scales (through the C ABI):
the calibration percentile (exact radix select) equals the oracle's
nearest-rank percentile bit for bit; static and clipped quantization give the
oracle's codes and scales bit for bit, including saturated quotients; the
calibrated static scale feeds the GEMM end to end."""
import numpy as np
import pytest
import torch

import fp8_w8a8_quantized_quantize_amd as fp8
import oracle
import synth
from tests._gpu import DEV, assert_codes_equal, assert_scales_equal, log, to_dev, to_host

pytestmark = pytest.mark.gpu


def _calib_data(n, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n).astype(np.float32)
    x[rng.integers(0, n, max(1, n // 1000))] *= 300.0   # rare outliers
    x[: n // 20] = np.round(x[: n // 20] * 4) / 4      # ties
    if n > 4:
        x[:3] = [-0.0, 0.0, -x[3]]
    return x


@pytest.mark.parametrize("n", [1, 7, 1000, 65536 + 17, (1 << 22) + 5])
@pytest.mark.parametrize("num,den", [(999, 1000), (9999, 10000), (1, 2), (1, 1), (1, 1000)])
def test_calibration_percentile_exact(n, num, den):
    x = _calib_data(n, seed=n + num)
    value, scale = fp8.fp8_calibrate_percentile(to_dev(x), num, den)
    want = oracle.percentile_nearest_rank(x, num, den)
    assert to_host(value)[0].view(np.uint32) == np.float32(want).view(np.uint32), (n, num, den)
    assert to_host(scale)[0].view(np.uint32) == oracle.static_scale(want).view(np.uint32)


def test_static_quantization_with_calibrated_scale():
    w = synth.WORKLOADS["llama3-70b-decode-gateup"]
    x, _ = synth.activations(64, w["K"], synth.workload_outliers(w), w["mult"], seed=5)
    value, scale = fp8.fp8_calibrate_percentile(to_dev(x), 999, 1000)
    s = to_host(scale)[0]
    assert s == oracle.static_scale(oracle.percentile_nearest_rank(x, 999, 1000))
    q, scales = fp8.fp8_quantize_static(to_dev(x), scale)
    want = oracle.quantize_static(x, s)
    assert_codes_equal(to_host(q), want, "static codes")
    assert np.all(to_host(scales) == s)
    sat = np.count_nonzero((want & 0x7F) == 0x7E)
    log(f"  static: {sat} saturated codes of {want.size}")
    assert sat > 0   # the P99.9 scale makes the outlier channels saturate


@pytest.mark.parametrize("rows,K", [(3, 48), (64, 8192), (9, 28672), (600, 1040)])
def test_static_and_clipped_shapes(rows, K):
    x, _ = synth.activations(rows, K, max(1, synth.n_outlier_channels(K)), 50.0, seed=rows + K)
    s = np.float32(0.0123)
    q, sc = fp8.fp8_quantize_static(to_dev(x), to_dev(np.array([s], np.float32)))
    assert_codes_equal(to_host(q), oracle.quantize_static(x, s), f"static rows={rows} K={K}")
    clip = np.float32(6.0)
    q2, s2 = fp8.fp8_quantize_per_token_clipped(to_dev(x), to_dev(np.array([clip], np.float32)))
    oq, os_ = oracle.quantize_rows_clipped(x, clip)
    assert_scales_equal(to_host(s2), os_, f"clipped scales rows={rows} K={K}")
    assert_codes_equal(to_host(q2), oq, f"clipped codes rows={rows} K={K}")


def test_static_scale_through_the_gemm():
    """Calibrate on one batch, quantize another with the static scale, run the
    GEMM with the per-row copies of that scale as s_tok."""
    M, N, K = 200, 512, 1024
    cal, _ = synth.activations(256, K, synth.n_outlier_channels(K), 50.0, seed=31)
    x, _ = synth.activations(M, K, synth.n_outlier_channels(K), 50.0, seed=32)
    wt = synth.weights(N, K, seed=33)
    qw, sc = oracle.quantize_rows(wt)
    _, scale = fp8.fp8_calibrate_percentile(to_dev(cal), 999, 1000)
    qa, st = fp8.fp8_quantize_static(to_dev(x), scale)
    y = to_host(fp8.fp8_gemm_scaled(qa, st, to_dev(qw), to_dev(sc)))
    s = to_host(scale)[0]
    oqa = oracle.quantize_static(x, s)
    assert_codes_equal(to_host(qa), oqa, "static codes")
    ref, absref = oracle.gemm_ref(oqa, np.full(M, s, np.float32), qw, sc)
    r = oracle.tolerance_check(y, ref, absref)
    assert r["ok"], r


def test_static_scale_far_below_the_data_saturates():
    """x / s overflowing fp32 must still give the saturated code (+-448)."""
    x = np.array([[3e38, -3e38, 1e30, -1e27] + [1.0] * 12], np.float32)
    s = np.float32(1e-12)
    q, _ = fp8.fp8_quantize_static(to_dev(x), to_dev(np.array([s], np.float32)))
    want = oracle.quantize_static(x, s)
    assert want[0, :4].tolist() == [0x7E, 0xFE, 0x7E, 0xFE]
    assert_codes_equal(to_host(q), want, "static overflow")
