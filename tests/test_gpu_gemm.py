"""GPU parity of the scaled FP8 GEMM (skinny decode and tiled MFMA paths), the
fused quantize+GEMM call and the grouped MoE GEMM, through the C ABI.

Bar: every checked output satisfies
    |y - ref| <= 1e-3 * sum_k |a_k w_k| * s_tok * s_ch + 2^-8 * |ref|
against the oracle's exact reference; integer-valued special cases must be
bit exact; the fused call must reproduce quantize-then-GEMM bit for bit."""
import numpy as np
import pytest
import torch

import fp8_w8a8_quantized_quantize_amd as fp8
import oracle
import synth
from tests._gpu import DEV, assert_codes_equal, assert_scales_equal, assert_within_tolerance, log, to_dev, to_host

pytestmark = pytest.mark.gpu

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def _quantized_problem(M, N, K, seed, n_out=None):
    x, _ = synth.activations(M, K, n_out if n_out is not None else max(1, synth.n_outlier_channels(K)), 50.0,
                             seed=seed)
    w = synth.weights(N, K, seed=seed)
    qa, st = oracle.quantize_rows(x)
    qw, sc = oracle.quantize_rows(w)
    return x, qa, st, qw, sc


def _gemm(qa, st, qw, sc):
    y = fp8.fp8_gemm_scaled(to_dev(qa), to_dev(st), to_dev(qw), to_dev(sc))
    return to_host(y)


# M <= 64 runs the skinny kernel, larger M the tiled one; shapes span several
# tiles with ragged M, N and K tails.  (64, 1024, 4096), (40, 1000, 8240) and
# (17, 300, 16384) have few weight rows and long K: the skinny kernel splits
# K there (4, 8 and 16 parts; the 8240 one ends in a partial 128-byte chunk).
SHAPES = [(1, 16, 16), (8, 200, 160), (16, 4096 + 48, 512), (33, 300, 1040), (64, 520, 2064),
          (64, 1024, 4096), (40, 1000, 8240), (17, 300, 16384),
          (65, 272, 384), (200, 700, 1168), (513, 257, 2064), (300, 1024, 4096),
          (129, 1000, 640), (777, 264, 1280), (256, 256, 128),
          # one row of MFMA tiles with empty 32-row fragments (M <= 192) and just past it
          (96, 520, 1024), (192, 264, 256), (193, 264, 256)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_full_compare(M, N, K):
    log(f"gemm M={M} N={N} K={K}")
    _, qa, st, qw, sc = _quantized_problem(M, N, K, seed=M * 7 + N)
    y = _gemm(qa, st, qw, sc)
    ref, ab = oracle.gemm_ref(qa, st, qw, sc)
    assert_within_tolerance(y, ref, ab, f"M={M} N={N} K={K}")


@pytest.mark.parametrize("M", [8, 64, 256])
def test_small_integer_codes_are_bit_exact(M):
    # codes +-1, +-2, +-4 with unit scales, K = 16: integer results <= 256, exact in bf16
    rng = np.random.default_rng(M)
    pool = np.array([0x38, 0x40, 0x48, 0xB8, 0xC0, 0xC8], np.uint8)
    N, K = 48, 16
    qa, qw = rng.choice(pool, (M, K)), rng.choice(pool, (N, K))
    ones_m, ones_n = np.ones(M, np.float32), np.ones(N, np.float32)
    y = _gemm(qa, ones_m, qw, ones_n)
    ref, _ = oracle.gemm_ref(qa, ones_m, qw, ones_n)
    assert np.array_equal(y, oracle.bf16_from_double(ref))


@pytest.mark.parametrize("M", [16, 64, 128])
def test_operand_layout_one_hot(M):
    # weight row n selects activation column col[n]: y[m, n] = dec(qa[m, col[n]]) * s_tok[m] * s_ch[n]
    rng = np.random.default_rng(1)
    N, K = 64, 256
    qa = rng.choice(FINITE, (M, K)).astype(np.uint8)
    col = rng.permutation(K)[:N]
    qw = np.zeros((N, K), np.uint8)
    qw[np.arange(N), col] = 0x38
    st = np.ones(M, np.float32)
    sc = np.ones(N, np.float32)
    y = _gemm(qa, st, qw, sc)
    ref, _ = oracle.gemm_ref(qa, st, qw, sc)
    assert np.array_equal(y, oracle.bf16_from_double(ref))


@pytest.mark.parametrize("M", [8, 64, 128])
def test_all_subnormal_operands(M):
    # every code is an E4M3 subnormal (E = 0): probes MFMA subnormal handling
    rng = np.random.default_rng(2)
    N, K = 96, 512
    sub = np.array([c | s for c in range(1, 8) for s in (0, 0x80)], np.uint8)
    qa, qw = rng.choice(sub, (M, K)), rng.choice(sub, (N, K))
    st = rng.uniform(0.5, 2, M).astype(np.float32)
    sc = rng.uniform(0.5, 2, N).astype(np.float32)
    y = _gemm(qa, st, qw, sc)
    ref, ab = oracle.gemm_ref(qa, st, qw, sc)
    assert_within_tolerance(y, ref, ab, f"subnormal M={M}")
    assert np.count_nonzero(y) > 0


def test_k_zero_gives_zero_and_empty_is_noop():
    qa = torch.empty((8, 0), dtype=torch.uint8, device=DEV)
    qw = torch.empty((32, 0), dtype=torch.uint8, device=DEV)
    y = fp8.fp8_gemm_scaled(qa, torch.ones(8, device=DEV), qw, torch.ones(32, device=DEV))
    assert np.all(to_host(y) == 0)
    qa = torch.empty((100, 0), dtype=torch.uint8, device=DEV)
    y = fp8.fp8_gemm_scaled(qa, torch.ones(100, device=DEV), qw, torch.ones(32, device=DEV))
    assert np.all(to_host(y) == 0)
    y = fp8.fp8_gemm_scaled(torch.empty((0, 64), dtype=torch.uint8, device=DEV), torch.ones(0, device=DEV),
                            torch.zeros((32, 64), dtype=torch.uint8, device=DEV), torch.ones(32, device=DEV))
    assert y.shape == (0, 32)


def test_strided_operands_and_output():
    M, N, K = 40, 96, 256
    _, qa, st, qw, sc = _quantized_problem(M, N, K, seed=5)
    A = torch.zeros((M, K + 64), dtype=torch.uint8, device=DEV)
    A[:, :K] = to_dev(qa)
    W = torch.zeros((N, K + 32), dtype=torch.uint8, device=DEV)
    W[:, :K] = to_dev(qw)
    Y = torch.zeros((M, N + 8), dtype=torch.bfloat16, device=DEV)
    fp8.fp8_gemm_scaled(A[:, :K], to_dev(st), W[:, :K], to_dev(sc), y=Y[:, :N])
    yh = to_host(Y)
    ref, ab = oracle.gemm_ref(qa, st, qw, sc)
    assert_within_tolerance(yh[:, :N], ref, ab, "strided")
    assert np.all(yh[:, N:] == 0)


def test_split_k_strided_output_and_stale_workspace():
    """A split-K shape with strided operands and output, through a workspace
    that holds garbage on entry (its contents must not matter)."""
    M, N, K = 48, 1000, 8192 + 16
    _, qa, st, qw, sc = _quantized_problem(M, N, K, seed=9)
    A = torch.zeros((M, K + 48), dtype=torch.uint8, device=DEV)
    A[:, :K] = to_dev(qa)
    W = torch.zeros((N, K + 16), dtype=torch.uint8, device=DEV)
    W[:, :K] = to_dev(qw)
    Y = torch.zeros((M, N + 3), dtype=torch.bfloat16, device=DEV)
    need = fp8.fp8_workspace_bytes(M, N, K)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=DEV)
    fp8.fp8_gemm_scaled(A[:, :K], to_dev(st), W[:, :K], to_dev(sc), y=Y[:, :N], ws=ws)
    yh = to_host(Y)
    ref, ab = oracle.gemm_ref(qa, st, qw, sc)
    assert_within_tolerance(yh[:, :N], ref, ab, "split-k strided")
    assert np.all(yh[:, N:] == 0)
    y2 = to_host(fp8.fp8_gemm_scaled(to_dev(qa), to_dev(st), to_dev(qw), to_dev(sc)))
    assert np.array_equal(y2, yh[:, :N])


# M <= 16 rows whose codes fit in LDS and whose fp32 values fit in registers
# (K <= 4096 for M <= 8, K <= 2048 for M <= 16), with N <= 8192, take the
# one-kernel path; the rest quantize first.
FUSED_SHAPES = [(1, 16, 16), (8, 512, 1024), (5, 4096 + 48, 272), (16, 300, 4096), (12, 3000, 4112),
                (8, 1000, 8192), (16, 100, 4112), (8, 8192 + 16, 1024), (17, 300, 640), (200, 300, 640)]


@pytest.mark.parametrize("M,N,K", FUSED_SHAPES)
def test_fused_equals_quantize_then_gemm(M, N, K):
    log(f"fused M={M} N={N} K={K}")
    x, qa, st, qw, sc = _quantized_problem(M, N, K, seed=11)
    xd, qwd, scd = to_dev(x), to_dev(qw), to_dev(sc)
    qa_out = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    st_out = torch.empty(M, dtype=torch.float32, device=DEV)
    y_f = fp8.fp8_quant_gemm_fused(xd, qwd, scd, qa_out=qa_out, s_tok_out=st_out)
    q2, s2 = fp8.fp8_quantize_per_token(xd)
    y_s = fp8.fp8_gemm_scaled(q2, s2, qwd, scd)
    y_f2 = fp8.fp8_quant_gemm_fused(xd, qwd, scd)  # workspace-staged codes
    assert_codes_equal(to_host(qa_out), qa, "fused codes")
    assert_scales_equal(to_host(st_out), st, "fused scales")
    assert np.array_equal(to_host(y_f), to_host(y_s))
    assert np.array_equal(to_host(y_f2), to_host(y_s))
    st_only = torch.empty(M, dtype=torch.float32, device=DEV)
    y_f3 = fp8.fp8_quant_gemm_fused(xd, qwd, scd, s_tok_out=st_only)
    assert_scales_equal(to_host(st_only), st, "fused scales only")
    assert np.array_equal(to_host(y_f3), to_host(y_s))
    ref, ab = oracle.gemm_ref(qa, st, qw, sc)
    assert_within_tolerance(to_host(y_f), ref, ab, "fused")


def test_repeatable_bits():
    for (M, N, K) in [(64, 4096, 2048), (64, 1024, 8192), (512, 512, 1024)]:
        _, qa, st, qw, sc = _quantized_problem(M, N, K, seed=3)
        a, b, c, d = to_dev(qa), to_dev(st), to_dev(qw), to_dev(sc)
        y1 = to_host(fp8.fp8_gemm_scaled(a, b, c, d))
        y2 = to_host(fp8.fp8_gemm_scaled(a, b, c, d))
        assert np.array_equal(y1, y2)


# ---------------------------------------------------------------- workloads --

def _tile_samples(row0, rows, N, rng, per_tile=2, tile=256):
    """per_tile random elements inside every tile x tile block of the output
    rows [row0, row0 + rows) x columns [0, N) (blocks clipped at the edges),
    so that no output tile of any kernel (256 x 256 or smaller) goes unchecked."""
    ms, ns = [], []
    for r in range(0, rows, tile):
        h = min(tile, rows - r)
        for c in range(0, N, tile):
            wd = min(tile, N - c)
            ms.append(row0 + r + rng.integers(0, h, per_tile))
            ns.append(c + rng.integers(0, wd, per_tile))
    if not ms:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    return np.concatenate(ms), np.concatenate(ns)


def _sample_pairs(M, N, count, rng):
    """count random elements, the first and last rows and one column in full,
    and two random elements of every 256 x 256 output tile."""
    tm, tn = _tile_samples(0, M, N, rng)
    ms = np.concatenate([rng.integers(0, M, count), np.full(N, 0), np.full(N, M - 1), np.arange(M), tm])
    ns = np.concatenate([rng.integers(0, N, count), np.arange(N), np.arange(N), np.full(M, rng.integers(0, N)), tn])
    return ms, ns


@pytest.mark.parametrize("name", ["tiny", "llama3-8b-decode-up", "llama3-70b-decode-gateup",
                                  "llama3-70b-decode-down", "llama3-70b-tp4-gateup", "llama3-70b-tp4-down",
                                  "llama3-70b-prefill"])
def test_workload_fused(name):
    """Full-size workloads through the fused call (the path the benchmark times):
    codes and scales bit exact on every element, outputs on sampled elements
    (two full rows, one full column, 4096 random, two in every 256 x 256
    output tile), full compare for the tiny one."""
    w = synth.WORKLOADS[name]
    M, N, K = w["M"], w["N"], w["K"]
    log(f"workload {name}: M={M} N={N} K={K}")
    x, _ = synth.activations(M, K, synth.workload_outliers(w), w["mult"], seed=0)
    wt = synth.weights(N, K, seed=0)
    qw_d, sc_d = fp8.fp8_quantize_per_token(to_dev(wt))   # offline weight conversion on the GPU
    qw, sc = oracle.quantize_rows(wt)
    assert_scales_equal(to_host(sc_d), sc, name + " weight scales")
    assert_codes_equal(to_host(qw_d), qw, name + " weight codes")
    del wt
    qa_out = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    st_out = torch.empty(M, dtype=torch.float32, device=DEV)
    y = to_host(fp8.fp8_quant_gemm_fused(to_dev(x), qw_d, sc_d, qa_out=qa_out, s_tok_out=st_out))
    qa, st = oracle.quantize_rows(x)
    assert_codes_equal(to_host(qa_out), qa, name + " activation codes")
    assert_scales_equal(to_host(st_out), st, name + " activation scales")
    if M * N <= 1 << 16:
        ref, ab = oracle.gemm_ref(qa, st, qw, sc)
        assert_within_tolerance(y, ref, ab, name)
    else:
        ms, ns = _sample_pairs(M, N, 4096, np.random.default_rng(0))
        ref, ab = oracle.gemm_ref_sampled(qa, st, qw, sc, ms, ns)
        assert_within_tolerance(y[ms, ns], ref, ab, name + " sampled")
    assert np.all(np.isfinite(oracle.bf16_bits_to_f64(y)))


# ------------------------------------------------------------------ grouped --

def _grouped_problem(T, E, topk, N, K, seed, zipf=1.1):
    te, rt, off = synth.routing(T, E, topk, zipf, seed=seed)
    x, _ = synth.activations(T, K, max(1, synth.n_outlier_channels(K)), 50.0, seed=seed)
    qa, st = oracle.quantize_rows(x)
    w = synth.expert_weights(E, N, K, seed=seed)
    qw, sc = oracle.quantize_rows(w.reshape(E * N, K))
    return rt, off, qa, st, qw.reshape(E, N, K), sc.reshape(E, N)


def _grouped(qa, st, rt, off, qw, sc):
    y = fp8.fp8_gemm_grouped_scaled(to_dev(qa), to_dev(st), to_dev(rt), to_dev(off), to_dev(qw), to_dev(sc))
    return to_host(y)


@pytest.mark.parametrize("T,E,topk,N,K", [(40, 6, 2, 272, 160), (300, 8, 3, 256, 1024), (129, 3, 1, 520, 2064),
                                           (257, 70, 4, 520, 1152)])
def test_grouped_full_compare(T, E, topk, N, K):
    log(f"grouped T={T} E={E} topk={topk} N={N} K={K}")
    rt, off, qa, st, qw, sc = _grouped_problem(T, E, topk, N, K, seed=T)
    y = _grouped(qa, st, rt, off, qw, sc)
    R = rt.size
    rs, ns = np.repeat(np.arange(R), N), np.tile(np.arange(N), R)
    ref, ab = oracle.grouped_ref_sampled(qa, st, rt, off, qw, sc, rs, ns)
    assert_within_tolerance(y.reshape(-1), ref, ab, f"grouped T={T}")


def test_grouped_with_empty_experts():
    T, N, K = 50, 256, 256
    rng = np.random.default_rng(3)
    loads = np.array([0, 20, 0, 0, 75, 5, 0], np.int32)  # experts with no rows, incl. first and last
    off = np.concatenate([[0], np.cumsum(loads)]).astype(np.int32)
    R = int(off[-1])
    rt = rng.integers(0, T, R).astype(np.int32)
    E = loads.size
    qa = rng.choice(FINITE, (T, K)).astype(np.uint8)
    st = rng.uniform(0.01, 1, T).astype(np.float32)
    qw = rng.choice(FINITE, (E, N, K)).astype(np.uint8)
    sc = rng.uniform(0.01, 1, (E, N)).astype(np.float32)
    y = _grouped(qa, st, rt, off, qw, sc)
    rs, ns = np.repeat(np.arange(R), N), np.tile(np.arange(N), R)
    ref, ab = oracle.grouped_ref_sampled(qa, st, rt, off, qw, sc, rs, ns)
    assert_within_tolerance(y.reshape(-1), ref, ab, "grouped empty experts")


@pytest.mark.parametrize("K", [128, 256, 384, 640])
def test_grouped_partial_row_tiles(K):
    """Expert loads at and around every 32-row boundary of a 256-row tile:
    the last row tile of an expert computes only the 32-row activation
    fragments that hold real rows, dealt alternately to the two waves along
    M, so each count of live fragments (1 to 4 per wave, both waves) occurs.
    K of 1, 2, 3 and 5 stages of 128 covers each way the weight lines of a
    later stage are touched ahead (none, in the prologue, in the loop)."""
    T, N = 700, 512
    loads = np.array([1, 31, 32, 33, 63, 64, 65, 95, 96, 97, 127, 128, 129, 159, 160, 161, 191, 192, 193,
                      223, 224, 225, 255, 256, 257, 300, 511, 512, 513], np.int32)
    log(f"grouped partial tiles: {loads.size} experts, R={int(loads.sum())} N={N} K={K}")
    rng = np.random.default_rng(11)
    off = np.concatenate([[0], np.cumsum(loads)]).astype(np.int32)
    R = int(off[-1])
    rt = rng.integers(0, T, R).astype(np.int32)
    E = loads.size
    qa = rng.choice(FINITE, (T, K)).astype(np.uint8)
    st = rng.uniform(0.01, 1, T).astype(np.float32)
    qw = rng.choice(FINITE, (E, N, K)).astype(np.uint8)
    sc = rng.uniform(0.01, 1, (E, N)).astype(np.float32)
    y = _grouped(qa, st, rt, off, qw, sc)
    rs, ns = np.repeat(np.arange(R), N), np.tile(np.arange(N), R)
    ref, ab = oracle.grouped_ref_sampled(qa, st, rt, off, qw, sc, rs, ns)
    assert_within_tolerance(y.reshape(-1), ref, ab, "grouped partial row tiles")


def test_grouped_moe_workload():
    w = synth.WORKLOADS["moe-64x2048x7168"]
    T, E, k, N, K = w["T"], w["E"], w["topk"], w["N"], w["K"]
    log(f"grouped workload T={T} E={E} top-{k} N={N} K={K}")
    te, rt, off = synth.routing(T, E, k, w["zipf"], seed=0)
    x, _ = synth.activations(T, K, synth.workload_outliers(w), w["mult"], seed=0)
    qa_d, st_d = fp8.fp8_quantize_per_token(to_dev(x))
    qa, st = oracle.quantize_rows(x)
    assert_codes_equal(to_host(qa_d), qa, "moe activation codes")
    assert_scales_equal(to_host(st_d), st, "moe activation scales")
    qw = np.empty((E, N, K), np.uint8)
    sc = np.empty((E, N), np.float32)
    qw_d = torch.empty((E, N, K), dtype=torch.uint8, device=DEV)
    sc_d = torch.empty((E, N), dtype=torch.float32, device=DEV)
    for e0 in range(0, E, 16):
        we = synth.expert_weights(E, N, K, seed=0, experts=range(e0, e0 + 16)).reshape(16 * N, K)
        qe, se = oracle.quantize_rows(we)
        qw[e0:e0 + 16], sc[e0:e0 + 16] = qe.reshape(16, N, K), se.reshape(16, N)
        fp8.fp8_quantize_per_token(to_dev(we), q=qw_d[e0:e0 + 16].view(16 * N, K), scales=sc_d[e0:e0 + 16].view(-1))
    assert_codes_equal(to_host(qw_d), qw, "expert weight codes")
    y = to_host(fp8.fp8_gemm_grouped_scaled(qa_d, st_d, to_dev(rt), to_dev(off), qw_d, sc_d))
    R = rt.size
    rng = np.random.default_rng(0)
    # every expert's first and last routed row in full, random elements, and
    # two elements in every 256-row x 256-column output tile of every expert
    rows = np.unique(np.concatenate([off[:-1][np.diff(off) > 0], off[1:][np.diff(off) > 0] - 1]))
    tiles = [_tile_samples(int(off[e]), int(off[e + 1] - off[e]), N, rng) for e in range(E)]
    rs = np.concatenate([np.repeat(rows, N), rng.integers(0, R, 8192)] + [t[0] for t in tiles])
    ns = np.concatenate([np.tile(np.arange(N), rows.size), rng.integers(0, N, 8192)] + [t[1] for t in tiles])
    ref, ab = oracle.grouped_ref_sampled(qa, st, rt, off, qw, sc, rs, ns)
    assert_within_tolerance(y[rs, ns], ref, ab, "moe sampled")
