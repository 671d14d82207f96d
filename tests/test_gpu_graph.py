"""The library's calls captured in a HIP graph (how the benchmark times the
launch-bound decode step): every replay, with eager work and synchronisation
between replays, must reproduce the eager result bit for bit."""
import numpy as np
import pytest
import torch

import fp8_w8a8_quantized_quantize_amd as fp8
import synth
from tests._gpu import DEV, log, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,N,K", [(8, 4096, 1024), (64, 2048, 4096), (300, 1024, 1024)])
def test_fused_step_graph_replays_match_eager(M, N, K):
    log(f"graph M={M} N={N} K={K}")
    x, _ = synth.activations(M, K, max(1, synth.n_outlier_channels(K)), 50.0, seed=21)
    w = synth.weights(N, K, seed=21)
    xd = to_dev(x)
    qw, sc = fp8.fp8_quantize_per_token(to_dev(w))
    ws = torch.zeros(max(1, fp8.fp8_workspace_bytes(M, N, K)), dtype=torch.uint8, device=DEV)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    qa, st = fp8.fp8_quantize_per_token(xd)
    y2 = torch.empty_like(y)
    fp8.fp8_quant_gemm_fused(xd, qw, sc, y=y, ws=ws)
    eager = to_host(y).copy()
    fp8.fp8_gemm_scaled(qa, st, qw, sc, y=y2, ws=ws)
    eager2 = to_host(y2).copy()

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fp8.fp8_quant_gemm_fused(xd, qw, sc, y=y, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        fp8.fp8_quant_gemm_fused(xd, qw, sc, y=y, ws=ws)
        fp8.fp8_gemm_scaled(qa, st, qw, sc, y=y2, ws=ws)
    for r in range(3):
        y.zero_()
        y2.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(y), eager), f"replay {r}: fused output differs from eager"
        assert np.array_equal(to_host(y2), eager2), f"replay {r}: GEMM output differs from eager"
        # eager work between replays
        fp8.fp8_quant_gemm_fused(xd, qw, sc, y=y, ws=ws)
        assert np.array_equal(to_host(y), eager)
