"""GPU parity of the per-token/per-channel E4M3 quantizer (through the C ABI):
codes and scale bits must equal the oracle's exactly."""
import numpy as np
import pytest
import torch

import fp8_w8a8_quantized_quantize_amd as fp8
import oracle
import synth
from tests._gpu import DEV, assert_codes_equal, assert_scales_equal, log, to_dev, to_host

pytestmark = pytest.mark.gpu


def _run(x_np, ld=None):
    rows, K = x_np.shape
    if ld is None or ld == K:
        x = to_dev(x_np)
    else:
        buf = torch.full((rows, ld), float("nan"), dtype=torch.float32, device=DEV)
        buf[:, :K] = to_dev(x_np)
        x = buf[:, :K]
    q, s = fp8.fp8_quantize_per_token(x)
    return to_host(q), to_host(s)


def _check(x_np, what, ld=None):
    q, s = _run(x_np, ld)
    oq, os_ = oracle.quantize_rows(x_np)
    assert_scales_equal(s, os_, what)
    assert_codes_equal(q, oq, what)


# the last two rows take the two-pass loop kernel: rows too long for registers
# (K > 32768 with 256 threads per row, K > 65536 with 1024 for short batches)
@pytest.mark.parametrize("rows,K,ld", [(1, 16, 16), (3, 48, 64), (77, 1040, 1040), (5, 4112, 4128),
                                       (2, 16400, 16400), (9, 28672, 28672), (300, 256, 260),
                                       (600, 33024, 33040), (2, 65600, 65600)])
def test_shapes_and_strides(rows, K, ld):
    log(f"quantize rows={rows} K={K} ld={ld}")
    x, _ = synth.activations(rows, K, max(1, synth.n_outlier_channels(K)), 50.0, seed=rows + K)
    _check(x, f"rows={rows} K={K}", ld)


def test_special_rows():
    K = 512
    rng = np.random.default_rng(0)
    rows = [np.zeros(K), np.where(np.arange(K) % 2 == 0, 0.0, -0.0), np.full(K, 1e-20),
            np.eye(1, K, 100)[0] * -3.5, np.concatenate([[1e4], rng.standard_normal(K - 1) * 1e-3]),
            rng.standard_normal(K) * 3e37, np.full(K, 448.0), rng.integers(-8, 9, K) * 2.0 ** -9,
            rng.standard_normal(K) * 1e-39]
    x = np.array(rows, dtype=np.float32)
    _check(x, "special rows")


def test_zero_k_gives_floor_scales_and_empty_rows_are_a_noop():
    x = torch.empty((4, 0), dtype=torch.float32, device=DEV)
    q, s = fp8.fp8_quantize_per_token(x)
    assert np.all(to_host(s).view(np.uint32) == 0x2B8CBCCC)
    q, s = fp8.fp8_quantize_per_token(torch.empty((0, 64), dtype=torch.float32, device=DEV))
    assert q.shape == (0, 64)


DENSE = ["tiny", "llama3-8b-decode-up", "llama3-70b-decode-gateup", "llama3-70b-decode-down",
         "llama3-70b-tp4-gateup", "llama3-70b-tp4-down",
         "llama3-70b-prefill"]


@pytest.mark.parametrize("name", DENSE + ["moe-64x2048x7168"])
def test_workload_activations(name):
    w = synth.WORKLOADS[name]
    M = w["M"] if w["kind"] == "dense" else w["T"]
    log(f"quantize activations of {name}: {M} x {w['K']}")
    x, _ = synth.activations(M, w["K"], synth.workload_outliers(w), w["mult"], seed=0)
    _check(x, name + " activations")


@pytest.mark.parametrize("name", DENSE)
def test_workload_weights(name):
    w = synth.WORKLOADS[name]
    log(f"quantize weights of {name}: {w['N']} x {w['K']}")
    _check(synth.weights(w["N"], w["K"], seed=0), name + " weights")


def test_moe_expert_weights():
    w = synth.WORKLOADS["moe-64x2048x7168"]
    E, N, K = w["E"], w["N"], w["K"]
    log(f"quantize expert weights: {E} x {N} x {K}")
    for e0 in range(0, E, 16):
        ws = synth.expert_weights(E, N, K, seed=0, experts=range(e0, e0 + 16)).reshape(16 * N, K)
        _check(ws, f"experts {e0}..{e0 + 15}")


def test_device_cast_sweep_all_fp32_magnitudes_up_to_448():
    """Every fp32 bit pattern with |v| <= 448, both signs, through the quantizer.

    Each row starts with 448, so its scale is fl32(448 / 448) = 1 and the
    division is exact: the codes are the device cast of the raw values."""
    K = 16384
    per_row = K - 1
    top = int(np.array([448.0], np.float32).view(np.uint32)[0])  # 0x43E00000
    total = top + 1
    chunk_rows = 8192
    chunk = chunk_rows * per_row
    for sign in (0, 0x80000000):
        start = 0
        while start < total:
            n = min(chunk, total - start)
            rows = (n + per_row - 1) // per_row
            bits = torch.arange(start, start + rows * per_row, dtype=torch.int64, device=DEV)
            bits = torch.clamp(bits, max=top) | sign
            vals = bits.to(torch.int32).view(torch.float32).view(rows, per_row) if sign == 0 else \
                (bits - (1 << 32)).to(torch.int32).view(torch.float32).view(rows, per_row)
            x = torch.empty((rows, K), dtype=torch.float32, device=DEV)
            x[:, 0] = 448.0
            x[:, 1:] = vals
            q, s = fp8.fp8_quantize_per_token(x)
            assert torch.all(s == 1.0).item()
            xh = to_host(x)
            want = oracle.encode(xh)
            got = to_host(q)
            assert_codes_equal(got, want, f"sweep sign={sign >> 31} start=0x{start:08x}")
            start += n
        log(f"  sweep sign={sign >> 31} done ({total} patterns)")


def _boundary_rows(n_rows, seed):
    """Rows whose first element A sets the scale s = fl32(A / 448) (A spans
    1e-9 .. 1e30 log-uniformly) and whose other elements lie within two ulps
    of s times an E4M3 magnitude or a midpoint between two neighbouring
    magnitudes -- the quotients x / s where an error of one ulp would change
    the code.  Both signs; the rest of the row is zero."""
    from tests._helpers import torch_e4m3_values
    mags = np.unique(np.abs(torch_e4m3_values()[np.isfinite(torch_e4m3_values())])).astype(np.float64)
    pts = np.concatenate([mags, 0.5 * (mags[1:] + mags[:-1])])
    pts = pts[pts <= 440.0]
    rng = np.random.default_rng(seed)
    K = 16 * ((len(pts) * 5 * 2 + 1 + 15) // 16)
    x = np.zeros((n_rows, K), np.float32)
    for i in range(n_rows):
        A = np.float32(10.0 ** rng.uniform(-9, 30))
        s = np.float32(A) / np.float32(448.0)
        vals = []
        for p in pts:
            x0 = np.float32(p * np.float64(s))
            lo = x0
            for _ in range(2):
                lo = np.nextafter(lo, np.float32(0))
            v = lo
            for _ in range(5):
                vals.append(v)
                v = np.nextafter(v, np.float32(np.inf))
        vals = np.array(vals, np.float32)
        row = np.concatenate([[A], vals, -vals]).astype(np.float32)
        x[i, :row.size] = row
    return x


def test_boundary_quotients_with_random_scales():
    x = _boundary_rows(64, seed=5)
    log(f"boundary rows {x.shape}")
    _check(x, "boundary quotients")


def test_fused_path_codes_on_boundary_quotients():
    """The fused decode kernel quantizes in its own prologue: its codes and
    scales (returned through qa_out / s_tok_out) must equal the oracle's."""
    x = _boundary_rows(8, seed=6)[:, :4096]
    M, K = x.shape
    N = 64
    qw = torch.full((N, K), 0x38, dtype=torch.uint8, device=DEV)
    sc = torch.ones(N, dtype=torch.float32, device=DEV)
    qa_out = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    st_out = torch.empty(M, dtype=torch.float32, device=DEV)
    fp8.fp8_quant_gemm_fused(to_dev(x), qw, sc, qa_out=qa_out, s_tok_out=st_out)
    oq, os_ = oracle.quantize_rows(x)
    assert_scales_equal(to_host(st_out), os_, "fused boundary scales")
    assert_codes_equal(to_host(qa_out), oq, "fused boundary codes")
