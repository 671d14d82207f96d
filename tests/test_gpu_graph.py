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


def _replay_check(capture, outputs, what):
    """Capture `capture()` in a graph; every replay (with eager work and
    synchronisation between replays) must reproduce the eager outputs."""
    capture()
    torch.cuda.synchronize()
    eager = [to_host(o).copy() for o in outputs]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        capture()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        capture()
    for r in range(3):
        for o in outputs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outputs, eager):
            assert np.array_equal(to_host(o), e), f"{what}: replay {r} differs from eager"
        capture()   # eager work between replays
        torch.cuda.synchronize()


def test_kv_codec_graph_replays_match_eager():
    T, C, B, nb = 2000, 576, 16, 200
    kv = to_dev(synth.kv_activations(T, C, seed=31))
    slot = to_dev(synth.kv_slot_mapping(T, B, nb, seed=31))
    scales = torch.empty(C, dtype=torch.float32, device=DEV)
    ws = torch.empty(fp8.fp8_kv_scales_workspace_bytes(T, C), dtype=torch.uint8, device=DEV)
    cache = torch.zeros((nb * B, C), dtype=torch.uint8, device=DEV)
    out = torch.empty((T, C), dtype=torch.float32, device=DEV)

    def step():
        fp8.fp8_kv_channel_scales(kv, "e5m2", scales=scales, ws=ws)
        fp8.fp8_kv_quantize_paged(kv, scales, slot, cache, "e5m2")
        fp8.fp8_kv_dequantize_paged(cache, slot, scales, "e5m2", out=out)

    _replay_check(step, [scales, cache, out], "kv codec")


def test_grouped_moe_step_graph_replays_match_eager():
    """Per-token quantization + grouped GEMM (experts with partly filled and
    several row tiles, so both the skipped fragments and the weight touch run)."""
    T, E, N, K = 600, 6, 512, 1024
    loads = np.array([300, 1, 95, 513, 0, 191], np.int32)
    rng = np.random.default_rng(37)
    off = to_dev(np.concatenate([[0], np.cumsum(loads)]).astype(np.int32))
    rt = to_dev(rng.integers(0, T, int(loads.sum())).astype(np.int32))
    x = to_dev(synth.activations(T, K, 10, 50.0, seed=37)[0])
    qw, sc = fp8.fp8_quantize_per_token(to_dev(synth.weights(E * N, K, seed=37)))
    qw, sc = qw.view(E, N, K), sc.view(E, N)
    qa = torch.empty((T, K), dtype=torch.uint8, device=DEV)
    st = torch.empty(T, dtype=torch.float32, device=DEV)
    y = torch.empty((int(loads.sum()), N), dtype=torch.bfloat16, device=DEV)

    def step():
        fp8.fp8_quantize_per_token(x, q=qa, scales=st)
        fp8.fp8_gemm_grouped_scaled(qa, st, rt, off, qw, sc, y=y)

    _replay_check(step, [qa, st, y], "grouped moe step")


@pytest.mark.parametrize("M,N,K", [(8, 4096, 1024), (64, 8192, 28672), (300, 1024, 1024)])
def test_mx_step_graph_replays_match_eager(M, N, K):
    x = to_dev(synth.activations(M, K, max(1, synth.n_outlier_channels(K)), 50.0, seed=33)[0])
    qw, sw = fp8.fp8_quantize_mx(to_dev(synth.weights(N, K, seed=33)))
    qa = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    sa = torch.empty((K // 128, M, 4), dtype=torch.uint8, device=DEV)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(max(1, fp8.fp8_mx_workspace_bytes(M, N, K)), dtype=torch.uint8, device=DEV)

    def step():
        fp8.fp8_quantize_mx(x, q=qa, scales=sa)
        fp8.fp8_gemm_mx(qa, sa, qw, sw, y=y, ws=ws)

    _replay_check(step, [qa, sa, y], f"mx M={M} N={N} K={K}")


def test_static_and_fp8out_graph_replays_match_eager():
    M, N, K = 64, 2048, 4096
    x = to_dev(synth.activations(M, K, 41, 50.0, seed=35)[0])
    qw, sc = fp8.fp8_quantize_per_token(to_dev(synth.weights(N, K, seed=35)))
    value, scale = fp8.fp8_calibrate_percentile(x, 999, 1000)
    qs = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    ss = torch.empty(M, dtype=torch.float32, device=DEV)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    q_out = torch.empty((M, N), dtype=torch.uint8, device=DEV)
    s_out = torch.empty(M, dtype=torch.float32, device=DEV)
    ws = torch.empty(max(1, fp8.fp8_workspace_bytes(M, N, K), fp8.fp8_fp8out_workspace_bytes(M, N, K)),
                     dtype=torch.uint8, device=DEV)

    def step():
        fp8.fp8_calibrate_percentile(x, 999, 1000)
        fp8.fp8_quantize_static(x, scale, q=qs, scales_out=ss)
        fp8.fp8_gemm_scaled(qs, ss, qw, sc, y=y, ws=ws)
        fp8.fp8_gemm_scaled_fp8out(qs, ss, qw, sc, q_out=q_out, s_out=s_out, ws=ws)

    _replay_check(step, [qs, ss, y, q_out, s_out], "static + fp8out")
