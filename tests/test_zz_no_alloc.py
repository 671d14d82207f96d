"""GPU test of the allocation-free fused call (fp8_quant_gemm_fused_noalloc,
through the C ABI): on two calls in a row -- the second with a smaller
problem, so stale scratch contents from the first are present -- its codes,
scales and BF16 output are the same bytes as fp8_quant_gemm_fused's with a
caller workspace (same kernels, same inputs), and the outputs are within the
GEMM tolerance of the oracle on sampled elements.  The first problem is the
70B down-projection decode shape (staged codes and split-K partial sums in
the scratch array), the second a smaller decode shape, the third an MFMA
(prefill-sized M) problem."""
import ctypes

import numpy as np
import pytest
import torch

import fp8_w8a8_quantized_quantize_amd as fp8
import oracle
import synth
from tests._gpu import DEV, assert_codes_equal, assert_scales_equal, assert_within_tolerance, log, to_dev, to_host

pytestmark = pytest.mark.gpu


def _problem(M, N, K, seed):
    x, _ = synth.activations(M, K, max(1, synth.n_outlier_channels(K)), 50.0, seed=seed)
    w = synth.weights(N, K, seed=seed)
    qw, sc = fp8.fp8_quantize_per_token(to_dev(w))
    return x, qw, sc


def _noalloc_raw(xd, qw, sc, y, qa, st):
    """Call the entry point through ctypes with raw pointers (the C ABI)."""
    M, K = xd.shape
    N = qw.shape[0]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return fp8.lib().fp8_quant_gemm_fused_noalloc(
        ctypes.c_void_p(xd.data_ptr()), K, ctypes.c_void_p(qw.data_ptr()), K, ctypes.c_void_p(sc.data_ptr()),
        ctypes.c_void_p(y.data_ptr()), N, M, N, K, ctypes.c_void_p(qa.data_ptr()), ctypes.c_void_p(st.data_ptr()),
        stream)


def _run_and_compare(M, N, K, seed):
    log(f"noalloc M={M} N={N} K={K}")
    x, qw, sc = _problem(M, N, K, seed)
    xd = to_dev(x)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    qa = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    st = torch.empty(M, dtype=torch.float32, device=DEV)
    assert _noalloc_raw(xd, qw, sc, y, qa, st) == fp8.FP8_OK
    y_ref = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    qa_ref = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    st_ref = torch.empty(M, dtype=torch.float32, device=DEV)
    fp8.fp8_quant_gemm_fused(xd, qw, sc, y=y_ref, qa_out=qa_ref, s_tok_out=st_ref)
    yh, qh, sh = to_host(y), to_host(qa), to_host(st)
    assert_codes_equal(qh, to_host(qa_ref), "codes vs the workspace call")
    assert_scales_equal(sh, to_host(st_ref), "scales vs the workspace call")
    assert np.array_equal(yh, to_host(y_ref)), "BF16 output differs from the workspace call"
    # and against the oracle
    q_o, s_o = oracle.quantize_rows(x)
    assert_codes_equal(qh, q_o, "codes vs oracle")
    assert_scales_equal(sh, s_o, "scales vs oracle")
    rng = np.random.default_rng(seed)
    ms, ns = rng.integers(0, M, 4096), rng.integers(0, N, 4096)
    ref, ab = oracle.gemm_ref_sampled(q_o, s_o, to_host(qw), to_host(sc), ms, ns)
    assert_within_tolerance(yh[ms, ns], ref, ab, "noalloc sampled")


def test_noalloc_two_calls_second_smaller():
    assert fp8.fp8_workspace_bytes(64, 8192, 28672) <= fp8.FP8_NOALLOC_SCRATCH_BYTES
    _run_and_compare(64, 8192, 28672, seed=71)    # staged codes + split-K partial sums in the scratch
    _run_and_compare(16, 2048, 4096, seed=72)     # smaller: stale contents of the first call present
    _run_and_compare(1024, 1024, 2048, seed=73)   # MFMA path, staged codes only


def test_noalloc_binding_and_limit():
    x, qw, sc = _problem(8, 512, 1024, seed=74)
    xd = to_dev(x)
    y = torch.empty((8, 512), dtype=torch.bfloat16, device=DEV)
    fp8.fp8_quant_gemm_fused_noalloc(xd, qw, sc, y)
    y_ref = fp8.fp8_quant_gemm_fused(xd, qw, sc)
    assert np.array_equal(to_host(y), to_host(y_ref))
    # beyond the scratch array: rejected on the host, nothing enqueued
    big_m = fp8.FP8_NOALLOC_SCRATCH_BYTES // 4096 + 1024
    with pytest.raises(fp8.Fp8Error) as e:
        fp8.fp8_quant_gemm_fused_noalloc(torch.empty((big_m, 4096), device=DEV),
                                         torch.empty((256, 4096), dtype=torch.uint8, device=DEV),
                                         torch.ones(256, device=DEV),
                                         torch.empty((big_m, 256), dtype=torch.bfloat16, device=DEV))
    assert e.value.code == fp8.FP8_ERR_WORKSPACE
