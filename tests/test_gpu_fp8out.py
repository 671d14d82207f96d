"""GPU parity of the FP8-output GEMM (fp8_gemm_scaled_fp8out, through the C ABI):
  - the fp32 output y32 within the GEMM tolerance of the exact product;
  - the output codes and scales bit exact against the oracle's quantizer
    applied to the GPU's own y32 (the accumulation order decides y32's last
    bits; the quantization of a given y32 is fixed);
  - the codes and scales against the oracle's own FP8 output (oracle.fp8out_ref:
    the exact product rounded once to fp32, then quantized): a scale may differ
    only where the row maximum is within the y32 bound of a scale step, a code
    only where the exact quotient lies within the y32 bound of an E4M3
    rounding boundary, and at most 1 % of the codes may differ at all (the
    fp32 accumulation error is far below the bound, so a systematic bias of
    y32 that the bound would still allow shows up here as a mismatch rate);
  - the decoded output within E4M3 resolution of the exact product.
Shapes cover the skinny kernel (with and without split K), the MFMA kernel and
the tiled fallback."""
import numpy as np
import pytest
import torch

import fp8_w8a8_quantized_quantize_amd as fp8
import oracle
import synth
from tests._gpu import DEV, assert_codes_equal, assert_scales_equal, log, to_dev, to_host
from tests._helpers import fp8out_admissible

pytestmark = pytest.mark.gpu


def _problem(M, N, K, seed):
    x, _ = synth.activations(M, K, max(1, synth.n_outlier_channels(K)), 50.0, seed=seed)
    w = synth.weights(N, K, seed=seed)
    qa, st = oracle.quantize_rows(x)
    qw, sc = oracle.quantize_rows(w)
    return qa, st, qw, sc


def _check_y32(y32, ref, absref, what):
    err = np.abs(y32.astype(np.float64) - ref)
    bound = 1e-3 * absref + 2.0 ** -22 * np.abs(ref)
    worst = float(np.max(err / np.maximum(bound, 1e-300)))
    log(f"  {what}: y32 worst/bound={worst:.3g}")
    assert np.all(err <= bound), f"{what}: y32 outside tolerance"


def _check_decoded(q, s, ref, absref, what):
    dec = oracle.decode(q) * s[:, None].astype(np.float64)
    bound = 1e-3 * absref + 2.0 ** -4 * np.abs(ref) * 1.001 + s[:, None].astype(np.float64) * 2.0 ** -10
    assert np.all(np.abs(dec - ref) <= bound), f"{what}: decoded FP8 output outside E4M3 resolution"


def _check_against_oracle_output(q, s, ref, absref, o_q, o_s, what, max_rate=0.01):
    """GPU codes / scales against oracle.fp8out_ref's (o_q, o_s) on the rows
    given (ref, absref: the exact product and its absolute sum there)."""
    r = fp8out_admissible(q, s, ref, absref)
    assert r["scale_ok"].all(), f"{what}: an output scale outside every y32 the bound allows"
    same = s.view(np.uint32) == o_s.view(np.uint32)
    assert np.all(same | r["scale_ambiguous"]), f"{what}: output scale differs where the row maximum is unambiguous"
    assert r["code_ok"].all(), f"{what}: an output code outside every y32 the bound allows"
    mism = (q != o_q) & same[:, None]
    assert not np.any(mism & ~r["code_ambiguous"]), f"{what}: code differs from the oracle away from a boundary"
    rate = float(mism.mean()) if mism.size else 0.0
    log(f"  {what}: scales equal {same.mean():.4f}, codes equal {1 - rate:.6f}, "
        f"ambiguous codes {r['code_ambiguous'].mean():.4f}")
    assert rate <= max_rate, f"{what}: {rate:.4%} of the codes differ from the oracle's FP8 output"


# (M, N, K): skinny, skinny split-K (4 and 8 parts), MFMA (K % 128 == 0), tiled (K % 128 != 0),
# and a 144 MB fp32 output with a ragged last row tile
SHAPES = [(8, 512, 1024), (16, 4096 + 32, 512), (64, 1024, 4096), (40, 1008, 8240),
          (200, 320, 640), (300, 1024, 4096), (129, 512, 400), (513, 256, 2064), (4400, 8192, 256)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_fp8out_against_oracle(M, N, K):
    log(f"fp8out M={M} N={N} K={K}")
    qa, st, qw, sc = _problem(M, N, K, seed=M + 3 * N)
    a, b, c, d = to_dev(qa), to_dev(st), to_dev(qw), to_dev(sc)
    y32_d = torch.empty((M, N), dtype=torch.float32, device=DEV)
    q_d, s_d = fp8.fp8_gemm_scaled_fp8out(a, b, c, d, y32_out=y32_d)
    y32, q, s = to_host(y32_d), to_host(q_d), to_host(s_d)
    ref, absref = oracle.gemm_ref(qa, st, qw, sc)
    _check_y32(y32, ref, absref, f"M={M} N={N} K={K}")
    oq, os_ = oracle.quantize_rows(y32)
    assert_scales_equal(s, os_, "output scales vs oracle quantizer on y32")
    assert_codes_equal(q, oq, "output codes vs oracle quantizer on y32")
    _check_decoded(q, s, ref, absref, "decoded output")
    _, o_q, o_s = oracle.fp8out_ref(qa, st, qw, sc)
    _check_against_oracle_output(q, s, ref, absref, o_q, o_s, f"M={M} N={N} K={K} vs oracle FP8 output")
    # y32 staged in the workspace instead: same bytes
    q2, s2 = fp8.fp8_gemm_scaled_fp8out(a, b, c, d)
    assert np.array_equal(to_host(q2), q) and np.array_equal(to_host(s2).view(np.uint32), s.view(np.uint32))
    # the BF16 GEMM rounds the same fp32 values
    ybf = to_host(fp8.fp8_gemm_scaled(a, b, c, d))
    want = oracle.bf16_from_double(y32.astype(np.float64))
    assert np.array_equal(ybf, want), "BF16 output is not the RNE rounding of the fp32 output"


def test_fp8out_chains_into_the_next_layer():
    """The codes and scales of one layer's FP8 output feed the next GEMM's
    activation inputs directly (the unified FP8 dataflow)."""
    M, N1, N2, K = 16, 1024, 512, 2048
    qa, st, qw1, sc1 = _problem(M, N1, K, seed=21)
    w2 = synth.weights(N2, N1, seed=22)
    qw2, sc2 = oracle.quantize_rows(w2)
    q1, s1 = fp8.fp8_gemm_scaled_fp8out(to_dev(qa), to_dev(st), to_dev(qw1), to_dev(sc1))
    y2 = to_host(fp8.fp8_gemm_scaled(q1, s1, to_dev(qw2), to_dev(sc2)))
    ref, absref = oracle.gemm_ref(to_host(q1), to_host(s1), qw2, sc2)
    r = oracle.tolerance_check(y2, ref, absref)
    assert r["ok"], r


def test_fp8out_empty_and_zero_k():
    qw = torch.zeros((32, 0), dtype=torch.uint8, device=DEV)
    qa = torch.zeros((4, 0), dtype=torch.uint8, device=DEV)
    q, s = fp8.fp8_gemm_scaled_fp8out(qa, torch.ones(4, device=DEV), qw, torch.ones(32, device=DEV))
    assert np.all(to_host(q) == 0)
    assert np.all(to_host(s).view(np.uint32) == 0x2B8CBCCC)   # all-zero rows: the 1e-12 floor
    q, s = fp8.fp8_gemm_scaled_fp8out(torch.empty((0, 64), dtype=torch.uint8, device=DEV),
                                      torch.ones(0, device=DEV), torch.zeros((32, 64), dtype=torch.uint8, device=DEV),
                                      torch.ones(32, device=DEV))
    assert q.shape == (0, 32)


def test_fp8out_decode_workload_full_size():
    """The 70B down-projection decode shape (split K), full size: codes and
    scales exact against the oracle quantizer on y32 and against the oracle's
    own FP8 output (full exact product); y32 on every element."""
    w = synth.WORKLOADS["llama3-70b-decode-down"]
    M, N, K = w["M"], w["N"], w["K"]
    x, _ = synth.activations(M, K, synth.workload_outliers(w), w["mult"], seed=0)
    qa, st = oracle.quantize_rows(x)
    wt = synth.weights(N, K, seed=0)
    qw, sc = oracle.quantize_rows(wt)
    del wt
    y32_d = torch.empty((M, N), dtype=torch.float32, device=DEV)
    q_d, s_d = fp8.fp8_gemm_scaled_fp8out(to_dev(qa), to_dev(st), to_dev(qw), to_dev(sc), y32_out=y32_d)
    y32, q, s = to_host(y32_d), to_host(q_d), to_host(s_d)
    oq, os_ = oracle.quantize_rows(y32)
    assert_scales_equal(s, os_, "workload output scales")
    assert_codes_equal(q, oq, "workload output codes")
    ref, absref = oracle.gemm_ref(qa, st, qw, sc)
    _check_y32(y32, ref, absref, "workload")
    _, o_q, o_s = oracle.fp8out_ref(qa, st, qw, sc)
    _check_against_oracle_output(q, s, ref, absref, o_q, o_s, "workload vs oracle FP8 output")
