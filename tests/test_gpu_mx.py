"""GPU parity of the block-scaled ("MX") path (through the C ABI): the
quantizer's codes and exponent bytes equal the oracle's bit for bit; the
block-scaled GEMM (skinny decode kernel, split-K, and the MFMA kernel) is
within the stated tolerance of the oracle's reference, on ragged and full
sizes."""
import numpy as np
import pytest
import torch

import fp8_w8a8_quantized_quantize_amd as fp8
import oracle
import synth
from tests._gpu import DEV, assert_codes_equal, assert_within_tolerance, log, to_dev, to_host

pytestmark = pytest.mark.gpu


def chunk_major(sc):
    """Oracle scale bytes [rows, K/32] -> the library's layout [K/128, rows, 4]."""
    rows, nb = sc.shape
    return np.ascontiguousarray(sc.reshape(rows, nb // 4, 4).transpose(1, 0, 2))


def _rows_with_edges(rows, K, seed):
    x, _ = synth.activations(rows, K, max(1, K // 100), 50.0, seed=seed)
    if rows >= 4 and K >= 128:
        x[0, :32] = 0.0
        x[0, 32:64] *= 1e-30                       # tiny block (fp32 subnormal quotients)
        x[1, :32] = 448.0 * 2.0 ** np.arange(-16, 16, dtype=np.float32)   # maximum 448 * 2^15
        x[1, 32:64] = np.float32(3e38) * np.where(np.arange(32) % 2, 1, -1)  # near FLT_MAX
        x[2, :32] = np.float32(448.0 * 4)              # block maximum exactly 448 * 2^2
        x[2, 32] = np.nextafter(np.float32(448.0 * 8), np.float32(1e9))
        x[3, ::7] = -0.0
    return x


@pytest.mark.parametrize("rows,K,ld", [(1, 128, 128), (3, 256, 260), (4, 128, 128), (77, 1152, 1152),
                                       (600, 4096, 4096), (9, 28672, 28672)])
def test_quantize_mx_bit_exact(rows, K, ld):
    x = _rows_with_edges(rows, K, seed=rows + K)
    buf = np.zeros((rows, ld), np.float32)
    buf[:, :K] = x
    xd = to_dev(buf)[:, :K]
    q, sc = fp8.fp8_quantize_mx(xd)
    wq, wsc = oracle.quantize_mx(x)
    assert_codes_equal(to_host(q), wq, f"mx codes rows={rows} K={K}")
    assert_codes_equal(to_host(sc), chunk_major(wsc), f"mx scales rows={rows} K={K}")


GEMM_SHAPES = [(1, 16, 128), (8, 272, 512), (17, 300, 1024), (64, 1000, 4096), (40, 1000, 8320),
               (64, 8192, 28672), (65, 256, 256), (200, 300, 512), (256, 512, 1024), (300, 1040, 2048)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_mx_within_tolerance(M, N, K):
    x = _rows_with_edges(M, K, seed=M * 7 + N)
    x = np.where(np.abs(x) > 1e30, np.float32(1.0), x)   # keep sums finite
    w = synth.weights(N, K, seed=M + N)
    qa, sa = oracle.quantize_mx(x)
    qw, sw = oracle.quantize_mx(w)
    log(f"  mx gemm M={M} N={N} K={K} ws={fp8.fp8_mx_workspace_bytes(M, N, K)}")
    y = fp8.fp8_gemm_mx(to_dev(qa), to_dev(chunk_major(sa)), to_dev(qw), to_dev(chunk_major(sw)))
    if M * N <= 300 * 1040:
        ref, ab = oracle.gemm_mx_ref(qa, sa, qw, sw)
        assert_within_tolerance(to_host(y), ref, ab, f"mx M={M} N={N} K={K}")
    else:
        rng = np.random.default_rng(M + N + K)
        ms, ns = rng.integers(0, M, 20000), rng.integers(0, N, 20000)
        ref, ab = oracle.gemm_mx_ref_sampled(qa, sa, qw, sw, ms, ns)
        assert_within_tolerance(to_host(y)[ms, ns], ref, ab, f"mx M={M} N={N} K={K} (sampled)")


def test_gemm_mx_strided_output_and_stale_workspace():
    M, N, K = 64, 8192, 28672   # split-K plan
    x, _ = synth.activations(M, K, 287, 50.0, seed=9)
    w = synth.weights(N, K, seed=9)
    qa, sa = oracle.quantize_mx(x)
    qw, sw = oracle.quantize_mx(w)
    ws = torch.full((fp8.fp8_mx_workspace_bytes(M, N, K),), 0x7F, dtype=torch.uint8, device=DEV)
    yb = torch.full((M, N + 24), -7.0, dtype=torch.bfloat16, device=DEV)
    fp8.fp8_gemm_mx(to_dev(qa), to_dev(chunk_major(sa)), to_dev(qw), to_dev(chunk_major(sw)), y=yb[:, :N], ws=ws)
    got = to_host(yb)
    rng = np.random.default_rng(3)
    ms, ns = rng.integers(0, M, 20000), rng.integers(0, N, 20000)
    ref, ab = oracle.gemm_mx_ref_sampled(qa, sa, qw, sw, ms, ns)
    assert_within_tolerance(got[ms, ns], ref, ab, "mx split-K strided")
    pad = got[:, N:].view(np.uint16) if got.dtype != np.uint16 else got[:, N:]
    assert np.all(pad == np.uint16(0xC0E0))   # -7.0 untouched


@pytest.mark.parametrize("name", ["llama3-8b-decode-up", "llama3-70b-prefill"])
def test_mx_end_to_end_full_size(name):
    """The block-scaled step at full size: quantize x and W on the GPU, then the
    GEMM, against the oracle on sampled outputs (codes and scales in full)."""
    w = synth.WORKLOADS[name]
    M, N, K = w["M"], w["N"], w["K"]
    x, wt = synth.make_dense(name, seed=0)
    log(f"  mx full size {name}: M={M} N={N} K={K}")
    qa, sa = fp8.fp8_quantize_mx(to_dev(x))
    qw, sw = fp8.fp8_quantize_mx(to_dev(wt))
    y = fp8.fp8_gemm_mx(qa, sa, qw, sw)
    oqa, osa = oracle.quantize_mx(x)
    assert_codes_equal(to_host(qa), oqa, "activation codes")
    assert_codes_equal(to_host(sa), chunk_major(osa), "activation scales")
    oqw, osw = oracle.quantize_mx(wt)
    assert_codes_equal(to_host(sw), chunk_major(osw), "weight scales")
    qw_h = to_host(qw)
    assert_codes_equal(qw_h, oqw, "weight codes")
    rng = np.random.default_rng(1)
    ms, ns = rng.integers(0, M, 20000), rng.integers(0, N, 20000)
    ref, ab = oracle.gemm_mx_ref_sampled(oqa, osa, oqw, osw, ms, ns)
    assert_within_tolerance(to_host(y)[ms, ns], ref, ab, f"mx {name}")


@pytest.mark.parametrize("M,N,K", [(8, 64, 512), (48, 80, 1024), (128, 256, 768)])
def test_gemm_mx_random_codes_and_scales(M, N, K):
    """Codes and exponent bytes drawn directly (every block its own scale, a
    spread of 2^-8 .. 2^8): a kernel that pairs a lane's data with another
    block's scale cannot stay within tolerance."""
    rng = np.random.default_rng(M * N + K)
    qa = rng.integers(0, 256, (M, K), dtype=np.uint8)
    qw = rng.integers(0, 256, (N, K), dtype=np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x3F
    qw[(qw & 0x7F) == 0x7F] = 0x41
    sa = rng.integers(119, 136, (M, K // 32), dtype=np.uint8)
    sw = rng.integers(119, 136, (N, K // 32), dtype=np.uint8)
    y = fp8.fp8_gemm_mx(to_dev(qa), to_dev(chunk_major(sa)), to_dev(qw), to_dev(chunk_major(sw)))
    ref, ab = oracle.gemm_mx_ref(qa, sa, qw, sw)
    assert_within_tolerance(to_host(y), ref, ab, f"mx random M={M} N={N} K={K}")
