"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and rejects bad arguments on the host before any launch (CPU only:
only error paths and empty problems are called, none of which reach the HIP
runtime)."""
import ctypes
import os
import re

import pytest

import fp8_w8a8_quantized_quantize_amd as fp8
from fp8_w8a8_quantized_quantize_amd import (FP8_ERR_INVALID_ARGUMENT, FP8_ERR_UNSUPPORTED, FP8_ERR_WORKSPACE,
                                             FP8_OK)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8w8a8.h")

P = 0x10000     # a 16-byte-aligned fake device address: never dereferenced on these paths
Q = 0x20000
MIS = 0x10008   # 8-byte aligned only
S0 = ctypes.c_void_p(0)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(fp8_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    L = fp8.lib()
    names = declared_functions()
    assert set(names) == set(fp8.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for code, name in [(0, "FP8_OK"), (1, "FP8_ERR_INVALID_ARGUMENT"), (2, "FP8_ERR_UNSUPPORTED"),
                       (3, "FP8_ERR_WORKSPACE"), (4, "FP8_ERR_DEVICE")]:
        assert fp8.fp8_status_string(code) == name
    assert fp8.fp8_status_string(99) == "FP8_ERR_UNKNOWN"


def test_workspace_bytes():
    # fused path stages M*K codes and M scales, each rounded up to 256 bytes
    assert fp8.fp8_workspace_bytes(8, 14336, 4096) == 8 * 4096 + 256
    assert fp8.fp8_workspace_bytes(8192, 8192, 8192) == 8192 * 8192 + 8192 * 4
    assert fp8.fp8_workspace_bytes(0, 5, 16) == 0
    assert fp8.fp8_workspace_bytes(-1, 5, 16) == ctypes.c_size_t(-1).value
    assert fp8.fp8_grouped_workspace_bytes(4096, 32768, 64, 2048, 7168) == 0
    # split-K decode shape: fp32 partial sums for 4 splits follow the staged codes
    assert fp8.fp8_workspace_bytes(64, 8192, 28672) == 64 * 28672 + 256 + 4 * 64 * 8192 * 4
    # FP8-output GEMM: the fp32 output staged (256-byte rounded), then the GEMM's own needs
    assert fp8.fp8_fp8out_workspace_bytes(8, 14336, 4096) == 8 * 14336 * 4
    assert fp8.fp8_fp8out_workspace_bytes(64, 8192, 28672) == 64 * 8192 * 4 + 4 * 64 * 8192 * 4
    assert fp8.fp8_fp8out_workspace_bytes(-1, 5, 16) == ctypes.c_size_t(-1).value


def fo(*a):
    return fp8.lib().fp8_gemm_scaled_fp8out(*a)


def test_fp8out_validation():
    # qa, lda, s_tok, qw, ldw, s_ch, q_out, ldq, s_out, y32_out, M, N, K, ws, ws_bytes, stream
    need = fp8.fp8_fp8out_workspace_bytes(4, 32, 64)
    base = [P, 64, P, Q, 64, P, Q, 32, P, 0, 4, 32, 64, P, need, S0]

    def with_(**kw):
        a = list(base)
        idx = dict(qa=0, lda=1, st=2, qw=3, ldw=4, sc=5, qo=6, ldq=7, so=8, y32=9, M=10, N=11, K=12, ws=13, wsb=14)
        for k, v in kw.items():
            a[idx[k]] = v
        return fo(*a)

    assert with_(N=40, ldq=48) == FP8_ERR_UNSUPPORTED            # output rows must be 16-multiples
    assert with_(K=40, lda=48, ldw=48) == FP8_ERR_UNSUPPORTED
    assert with_(wsb=need - 1) == FP8_ERR_WORKSPACE
    assert with_(ws=0) == FP8_ERR_INVALID_ARGUMENT
    assert with_(ws=MIS) == FP8_ERR_UNSUPPORTED
    assert with_(qo=0) == FP8_ERR_INVALID_ARGUMENT
    assert with_(so=0) == FP8_ERR_INVALID_ARGUMENT
    assert with_(ldq=24) == FP8_ERR_INVALID_ARGUMENT              # ldq < N
    assert with_(ldq=40) == FP8_ERR_UNSUPPORTED                   # code rows not 16-byte strided
    assert with_(y32=MIS) == FP8_ERR_UNSUPPORTED
    assert with_(M=0, qa=0, st=0, qo=0, so=0) == FP8_OK          # empty: no-op


def q(*a):
    return fp8.lib().fp8_quantize_per_token(*a)


def test_quantize_validation():
    # x, rows, K, ldx, q, ldq, scales, stream
    assert q(P, 4, 15, 16, Q, 16, P, S0) == FP8_ERR_UNSUPPORTED          # K % 16
    assert q(P, 4, 16, 8, Q, 16, P, S0) == FP8_ERR_INVALID_ARGUMENT      # ldx < K
    assert q(P, 4, 16, 16, Q, 8, P, S0) == FP8_ERR_INVALID_ARGUMENT      # ldq < K
    assert q(0, 4, 16, 16, Q, 16, P, S0) == FP8_ERR_INVALID_ARGUMENT     # null x
    assert q(P, 4, 16, 16, 0, 16, P, S0) == FP8_ERR_INVALID_ARGUMENT     # null q
    assert q(P, 4, 16, 16, Q, 16, 0, S0) == FP8_ERR_INVALID_ARGUMENT     # null scales
    assert q(P, -1, 16, 16, Q, 16, P, S0) == FP8_ERR_INVALID_ARGUMENT    # negative rows
    assert q(MIS, 4, 16, 16, Q, 16, P, S0) == FP8_ERR_UNSUPPORTED        # misaligned x
    assert q(P, 4, 16, 18, Q, 16, P, S0) == FP8_ERR_UNSUPPORTED          # x stride not 16 B
    assert q(P, 4, 16, 16, Q, 24, P, S0) == FP8_ERR_UNSUPPORTED          # q stride not 16 B
    assert q(P, 1 << 62, 16, 16, Q, 16, P, S0) == FP8_ERR_UNSUPPORTED    # beyond 32-bit rows
    assert q(P, 1 << 30, 1 << 30, 1 << 40, Q, 1 << 30, P, S0) == FP8_ERR_INVALID_ARGUMENT  # overflow
    assert q(0, 0, 16, 16, 0, 16, 0, S0) == FP8_OK                      # empty: no-op


def g(*a):
    return fp8.lib().fp8_gemm_scaled(*a)


def test_gemm_validation():
    # qa, lda, s_tok, qw, ldw, s_ch, y, ldy, M, N, K, ws, ws_bytes, stream
    ok = [P, 64, P, Q, 64, P, Q, 32, 4, 32, 64, 0, 0, S0]

    def with_(**kw):
        a = list(ok)
        idx = dict(qa=0, lda=1, s_tok=2, qw=3, ldw=4, s_ch=5, y=6, ldy=7, M=8, N=9, K=10, ws=11, wsb=12)
        for k, v in kw.items():
            a[idx[k]] = v
        return g(*a)

    assert with_(K=40, lda=48, ldw=48) == FP8_ERR_UNSUPPORTED
    assert with_(lda=32) == FP8_ERR_INVALID_ARGUMENT
    assert with_(ldw=48) == FP8_ERR_INVALID_ARGUMENT
    assert with_(ldy=16) == FP8_ERR_INVALID_ARGUMENT
    assert with_(ldw=72) == FP8_ERR_UNSUPPORTED          # weight stride not 16 B
    assert with_(lda=72) == FP8_ERR_UNSUPPORTED          # activation-code stride not 16 B
    assert with_(y=MIS) == FP8_ERR_UNSUPPORTED
    assert with_(qa=0) == FP8_ERR_INVALID_ARGUMENT
    assert with_(qw=0) == FP8_ERR_INVALID_ARGUMENT
    assert with_(s_tok=0) == FP8_ERR_INVALID_ARGUMENT
    assert with_(s_ch=0) == FP8_ERR_INVALID_ARGUMENT
    assert with_(y=0) == FP8_ERR_INVALID_ARGUMENT
    assert with_(s_ch=MIS) == FP8_ERR_UNSUPPORTED
    assert with_(M=-3) == FP8_ERR_INVALID_ARGUMENT
    # 2^23 x 2^23 output tiles of 128 x 128 do not fit a 32-bit launch grid
    assert with_(M=1 << 30, N=1 << 30, ldy=1 << 30) == FP8_ERR_UNSUPPORTED
    assert with_(M=0, qa=0, s_tok=0, y=0) == FP8_OK       # empty: no-op
    assert with_(N=0, qw=0, s_ch=0, y=0) == FP8_OK


def f(*a):
    return fp8.lib().fp8_quant_gemm_fused(*a)


def test_fused_validation():
    # x, ldx, qw, ldw, s_ch, y, ldy, M, N, K, qa_out, s_tok_out, ws, ws_bytes, stream
    need = fp8.fp8_workspace_bytes(4, 32, 64)
    base = [P, 64, Q, 64, P, Q, 32, 4, 32, 64, 0, 0, P, need, S0]

    def with_(**kw):
        a = list(base)
        idx = dict(x=0, ldx=1, qw=2, ldw=3, s_ch=4, y=5, ldy=6, M=7, N=8, K=9, qa=10, st=11, ws=12, wsb=13)
        for k, v in kw.items():
            a[idx[k]] = v
        return f(*a)

    assert with_(wsb=need - 1) == FP8_ERR_WORKSPACE
    assert with_(ws=0) == FP8_ERR_INVALID_ARGUMENT
    assert with_(ws=MIS) == FP8_ERR_UNSUPPORTED
    assert with_(x=0) == FP8_ERR_INVALID_ARGUMENT
    assert with_(ldx=60) == FP8_ERR_INVALID_ARGUMENT
    assert with_(K=24, ldx=32, ldw=32) == FP8_ERR_UNSUPPORTED
    assert with_(qa=MIS) == FP8_ERR_UNSUPPORTED
    assert with_(st=MIS) == FP8_ERR_UNSUPPORTED
    assert with_(M=0, x=0, y=0, ws=0, wsb=0) == FP8_OK


def gg(*a):
    return fp8.lib().fp8_gemm_grouped_scaled(*a)


def test_grouped_validation():
    # qa, s_tok, row_token, offsets, qw, s_ch, y, T, R, E, N, K, ws, ws_bytes, stream
    base = [P, P, P, P, Q, P, Q, 8, 16, 4, 32, 64, 0, 0, S0]

    def with_(**kw):
        a = list(base)
        idx = dict(qa=0, st=1, rt=2, off=3, qw=4, sc=5, y=6, T=7, R=8, E=9, N=10, K=11)
        for k, v in kw.items():
            a[idx[k]] = v
        return gg(*a)

    assert with_(K=8) == FP8_ERR_UNSUPPORTED
    assert with_(E=2000) == FP8_ERR_UNSUPPORTED
    assert with_(E=0) == FP8_ERR_INVALID_ARGUMENT
    assert with_(T=0, qa=0, st=0) == FP8_ERR_INVALID_ARGUMENT
    assert with_(rt=0) == FP8_ERR_INVALID_ARGUMENT
    assert with_(off=0) == FP8_ERR_INVALID_ARGUMENT
    assert with_(qw=0) == FP8_ERR_INVALID_ARGUMENT
    assert with_(sc=MIS) == FP8_ERR_UNSUPPORTED
    assert with_(R=-1) == FP8_ERR_INVALID_ARGUMENT
    assert with_(R=1 << 30, N=1 << 30) == FP8_ERR_UNSUPPORTED   # tile grid beyond 32 bits
    assert with_(R=0, rt=0, off=0, y=0) == FP8_OK


@pytest.mark.parametrize("name", ["fp8_quantize_per_token", "fp8_gemm_scaled", "fp8_quant_gemm_fused",
                                  "fp8_gemm_grouped_scaled"])
def test_python_binding_requires_cuda_tensors(name):
    import torch
    fn = getattr(fp8, name)
    with pytest.raises((TypeError, ValueError)):
        if name == "fp8_quantize_per_token":
            fn(torch.zeros(2, 16))
        elif name == "fp8_gemm_scaled":
            fn(torch.zeros(2, 16, dtype=torch.uint8), torch.ones(2), torch.zeros(2, 16, dtype=torch.uint8), torch.ones(2))
        elif name == "fp8_quant_gemm_fused":
            fn(torch.zeros(2, 16), torch.zeros(2, 16, dtype=torch.uint8), torch.ones(2))
        else:
            fn(torch.zeros(2, 16, dtype=torch.uint8), torch.ones(2), torch.zeros(2, dtype=torch.int32),
               torch.zeros(2, dtype=torch.int32), torch.zeros(1, 2, 16, dtype=torch.uint8), torch.ones(1, 2))


def test_static_clipped_and_calibration_validation():
    L = fp8.lib()
    # x, rows, K, ldx, scale, q, ldq, scales_out, stream
    assert L.fp8_quantize_static(P, 4, 15, 16, P, Q, 16, P, S0) == FP8_ERR_UNSUPPORTED       # K % 16
    assert L.fp8_quantize_static(P, 4, 16, 16, 0, Q, 16, P, S0) == FP8_ERR_INVALID_ARGUMENT  # no scale
    assert L.fp8_quantize_static(P, 4, 16, 16, P + 2, Q, 16, P, S0) == FP8_ERR_UNSUPPORTED   # misaligned scale
    assert L.fp8_quantize_static(P, 4, 16, 16, P, Q, 16, 0, S0) == FP8_ERR_INVALID_ARGUMENT  # no scales_out
    assert L.fp8_quantize_static(0, 0, 16, 16, 0, 0, 16, 0, S0) == FP8_OK                    # empty
    assert L.fp8_quantize_per_token_clipped(P, 4, 16, 16, 0, Q, 16, P, S0) == FP8_ERR_INVALID_ARGUMENT
    assert L.fp8_quantize_per_token_clipped(P, 4, 16, 12, P, Q, 16, P, S0) == FP8_ERR_INVALID_ARGUMENT
    # x, n, num, den, value_out, scale_out, ws, ws_bytes, stream
    wsb = L.fp8_calibrate_workspace_bytes()
    assert wsb >= 1040
    assert L.fp8_calibrate_percentile(P, 0, 999, 1000, P, P, Q, wsb, S0) == FP8_ERR_INVALID_ARGUMENT
    assert L.fp8_calibrate_percentile(P, 10, 0, 1000, P, P, Q, wsb, S0) == FP8_ERR_INVALID_ARGUMENT
    assert L.fp8_calibrate_percentile(P, 10, 1001, 1000, P, P, Q, wsb, S0) == FP8_ERR_INVALID_ARGUMENT
    assert L.fp8_calibrate_percentile(P, 10, 999, 1000, P, P, Q, wsb - 1, S0) == FP8_ERR_WORKSPACE
    assert L.fp8_calibrate_percentile(P, 10, 999, 1000, P, P, MIS, wsb, S0) == FP8_ERR_UNSUPPORTED
    assert L.fp8_calibrate_percentile(P, 1 << 33, 999, 1000, P, P, Q, wsb, S0) == FP8_ERR_UNSUPPORTED
    assert L.fp8_calibrate_percentile(0, 10, 999, 1000, P, P, Q, wsb, S0) == FP8_ERR_INVALID_ARGUMENT


def test_kv_validation():
    L = fp8.lib()
    E4, E5 = fp8.FP8_KV_E4M3, fp8.FP8_KV_E5M2
    # workspace: one fp32 partial maximum per channel and row chunk (about 256 workgroups in all)
    assert L.fp8_kv_scales_workspace_bytes(32768, 2048) == 256 * 2048 * 4   # 16-bit rows: 1 column block
    assert L.fp8_kv_scales_workspace_bytes(32768, 576) == 512 * 576 * 4
    assert L.fp8_kv_scales_workspace_bytes(0, 576) == 576 * 4          # one chunk; 2304 = 9 * 256
    assert L.fp8_kv_scales_workspace_bytes(0, 68) == 512              # rounded up to 256 bytes
    assert L.fp8_kv_scales_workspace_bytes(10, 6) == ctypes.c_size_t(-1).value     # C % 4
    assert L.fp8_kv_scales_workspace_bytes(-1, 8) == ctypes.c_size_t(-1).value
    wsb = L.fp8_kv_scales_workspace_bytes(64, 128)
    F32, BF16 = fp8.FP8_KV_F32, fp8.FP8_KV_BF16
    # kv, dtype, T, C, ldkv, fmt, scales, ws, ws_bytes, stream
    assert L.fp8_kv_channel_scales(P, F32, 64, 128, 128, E5, Q, P, wsb - 1, S0) == FP8_ERR_WORKSPACE
    assert L.fp8_kv_channel_scales(P, F32, 64, 128, 128, 2, Q, P, wsb, S0) == FP8_ERR_INVALID_ARGUMENT  # format
    assert L.fp8_kv_channel_scales(P, F32, 64, 130, 132, E5, Q, P, wsb, S0) == FP8_ERR_UNSUPPORTED      # C % 4
    assert L.fp8_kv_channel_scales(P, F32, 64, 128, 126, E5, Q, P, wsb, S0) == FP8_ERR_INVALID_ARGUMENT  # ldkv < C
    assert L.fp8_kv_channel_scales(P, F32, 64, 128, 130, E5, Q, P, wsb, S0) == FP8_ERR_UNSUPPORTED      # ldkv % 4
    assert L.fp8_kv_channel_scales(P, F32, 64, 128, 128, E5, MIS, P, wsb, S0) == FP8_ERR_UNSUPPORTED
    assert L.fp8_kv_channel_scales(P, F32, 64, 128, 128, E5, Q, 0, wsb, S0) == FP8_ERR_INVALID_ARGUMENT
    assert L.fp8_kv_channel_scales(P, F32, 64, 128, 128, E5, Q, MIS, wsb, S0) == FP8_ERR_UNSUPPORTED
    assert L.fp8_kv_channel_scales(0, F32, 0, 0, 0, E4, 0, 0, 0, S0) == FP8_OK                           # empty
    # kv, dtype, T, C, ldkv, scales, fmt, slot, cache, num_slots, stream
    assert L.fp8_kv_quantize_paged(P, F32, 8, 64, 64, Q, E5, P, Q, -1, S0) == FP8_ERR_INVALID_ARGUMENT
    assert L.fp8_kv_quantize_paged(P, F32, 8, 64, 64, Q, E5, 0, Q, 16, S0) == FP8_ERR_INVALID_ARGUMENT   # no slots
    assert L.fp8_kv_quantize_paged(P, F32, 8, 64, 64, Q, E5, P + 2, Q, 16, S0) == FP8_ERR_UNSUPPORTED
    assert L.fp8_kv_quantize_paged(P, F32, 8, 64, 64, Q, E5, P, MIS, 16, S0) == FP8_ERR_UNSUPPORTED      # cache
    assert L.fp8_kv_quantize_paged(P, F32, 8, 64, 64, Q, 7, P, Q, 16, S0) == FP8_ERR_INVALID_ARGUMENT
    assert L.fp8_kv_quantize_paged(P, F32, 8, 64, 64, Q, E5, P, Q, 1 << 31, S0) == FP8_ERR_UNSUPPORTED
    assert L.fp8_kv_quantize_paged(P, F32, 8, 64, 64, Q, E5, P, 0, 16, S0) == FP8_ERR_INVALID_ARGUMENT
    assert L.fp8_kv_quantize_paged(P, F32, 8, 64, 64, Q, E5, P, Q, 0, S0) == FP8_OK    # nothing to write into
    assert L.fp8_kv_quantize_paged(0, F32, 0, 64, 64, 0, E5, 0, Q, 16, S0) == FP8_OK
    # element types: 16-bit rows need 16-byte row strides (multiples of 8 elements); unknown types are rejected
    assert L.fp8_kv_channel_scales(P, BF16, 64, 128, 132, E5, Q, P, wsb, S0) == FP8_ERR_UNSUPPORTED   # 264 B rows
    assert L.fp8_kv_channel_scales(P, 3, 64, 128, 128, E5, Q, P, wsb, S0) == FP8_ERR_INVALID_ARGUMENT
    # 16-bit rows are read 8 channels at a time: C % 8 (C = 132 is fine for fp32 rows)
    assert L.fp8_kv_channel_scales(P, BF16, 64, 132, 136, E5, Q, P, wsb, S0) == FP8_ERR_UNSUPPORTED
    assert L.fp8_kv_quantize_paged(P, fp8.FP8_KV_F16, 8, 132, 136, Q, E5, P, Q, 16, S0) == FP8_ERR_UNSUPPORTED
    assert L.fp8_kv_dequantize_paged(Q, 16, P, 8, 132, Q, E5, P, BF16, 136, S0) == FP8_ERR_UNSUPPORTED
    assert L.fp8_kv_dequantize_paged(Q, 16, P, 8, 64, Q, E5, P, 5, 64, S0) == FP8_ERR_INVALID_ARGUMENT
    # cache, num_slots, slot, T, C, scales, fmt, out, out_dtype, ldo, stream
    assert L.fp8_kv_dequantize_paged(Q, 16, P, 8, 64, Q, E5, P, F32, 62, S0) == FP8_ERR_INVALID_ARGUMENT
    assert L.fp8_kv_dequantize_paged(Q, 16, P, 8, 64, Q, E5, P, F32, 66, S0) == FP8_ERR_UNSUPPORTED
    assert L.fp8_kv_dequantize_paged(Q, 16, P, 8, 64, Q, E5, MIS, F32, 64, S0) == FP8_ERR_UNSUPPORTED
    assert L.fp8_kv_dequantize_paged(Q, 16, 0, 8, 64, Q, E5, P, F32, 64, S0) == FP8_ERR_INVALID_ARGUMENT
    assert L.fp8_kv_dequantize_paged(0, 16, P, 8, 64, Q, E5, P, F32, 64, S0) == FP8_ERR_INVALID_ARGUMENT
    assert L.fp8_kv_dequantize_paged(Q, 16, 0, 0, 64, Q, E5, 0, F32, 64, S0) == FP8_OK


def test_mx_validation():
    L = fp8.lib()
    # x, rows, K, ldx, q, ldq, scales, stream
    assert L.fp8_quantize_mx(P, 4, 96, 96, Q, 96, P, S0) == FP8_ERR_UNSUPPORTED          # K % 128
    assert L.fp8_quantize_mx(P, 4, 128, 126, Q, 128, P, S0) == FP8_ERR_INVALID_ARGUMENT  # ldx < K
    assert L.fp8_quantize_mx(P, 4, 128, 128, Q, 128, 0, S0) == FP8_ERR_INVALID_ARGUMENT  # no scales
    assert L.fp8_quantize_mx(MIS, 4, 128, 128, Q, 128, P, S0) == FP8_ERR_UNSUPPORTED
    assert L.fp8_quantize_mx(0, 0, 128, 128, 0, 128, 0, S0) == FP8_OK
    assert L.fp8_mx_workspace_bytes(64, 8192, 28672) == 4 * 64 * 8192 * 4   # split-K partials
    assert L.fp8_mx_workspace_bytes(8192, 8192, 8192) == 0
    assert L.fp8_mx_workspace_bytes(8, 256, 96) == ctypes.c_size_t(-1).value  # K % 128
    # qa, lda, sa, qw, ldw, sw, y, ldy, M, N, K, ws, ws_bytes, stream
    assert L.fp8_gemm_mx(P, 96, P, Q, 96, P, P, 16, 8, 16, 96, 0, 0, S0) == FP8_ERR_UNSUPPORTED   # K % 128
    assert L.fp8_gemm_mx(P, 128, P + 2, Q, 128, P, P, 16, 8, 16, 128, 0, 0, S0) == FP8_ERR_UNSUPPORTED
    assert L.fp8_gemm_mx(P, 128, 0, Q, 128, P, P, 16, 8, 16, 128, 0, 0, S0) == FP8_ERR_INVALID_ARGUMENT
    assert L.fp8_gemm_mx(P, 28672, P, Q, 28672, P, P, 8192, 64, 8192, 28672, 0, 0, S0) == FP8_ERR_WORKSPACE
    assert L.fp8_gemm_mx(P, 128, P, Q, 128, P, P, 16, 0, 16, 128, 0, 0, S0) == FP8_OK


@pytest.mark.parametrize("call", ["quantize_static", "quantize_clipped", "calibrate", "fp8out", "quantize_mx",
                                  "gemm_mx", "kv_scales", "kv_quantize", "kv_dequantize", "kv_format"])
def test_python_bindings_reject_host_tensors_and_bad_arguments(call):
    """The bindings only marshal arguments: host tensors, wrong dtypes or shapes
    and unknown formats raise before anything reaches the library."""
    import torch
    x = torch.zeros(4, 128)
    u8 = torch.zeros(4, 128, dtype=torch.uint8)
    with pytest.raises((TypeError, ValueError)):
        if call == "quantize_static":
            fp8.fp8_quantize_static(x, torch.ones(1))
        elif call == "quantize_clipped":
            fp8.fp8_quantize_per_token_clipped(x, torch.ones(1))
        elif call == "calibrate":
            fp8.fp8_calibrate_percentile(x, 999, 1000)
        elif call == "fp8out":
            fp8.fp8_gemm_scaled_fp8out(u8, torch.ones(4), u8, torch.ones(4))
        elif call == "quantize_mx":
            fp8.fp8_quantize_mx(x)
        elif call == "gemm_mx":
            fp8.fp8_gemm_mx(u8, torch.zeros(1, 4, 4, dtype=torch.uint8), u8, torch.zeros(1, 4, 4, dtype=torch.uint8))
        elif call == "kv_scales":
            fp8.fp8_kv_channel_scales(x, "e5m2")
        elif call == "kv_quantize":
            fp8.fp8_kv_quantize_paged(x, torch.ones(128), torch.zeros(4, dtype=torch.int32), u8, "e5m2")
        elif call == "kv_dequantize":
            fp8.fp8_kv_dequantize_paged(u8, torch.zeros(4, dtype=torch.int32), torch.ones(128), "e5m2")
        else:
            fp8._kv_fmt("e4m2")


def test_gemm_workspace_bytes_is_the_gemm_alone():
    """fp8_gemm_workspace_bytes counts only the GEMM's split-K partial sums;
    fp8_workspace_bytes (the fused call) adds the staged codes and scales."""
    assert fp8.fp8_gemm_workspace_bytes(64, 8192, 28672) == 4 * 64 * 8192 * 4
    assert fp8.fp8_gemm_workspace_bytes(8, 14336, 4096) == 0
    assert fp8.fp8_gemm_workspace_bytes(8192, 8192, 8192) == 0
    assert fp8.fp8_gemm_workspace_bytes(-1, 5, 16) == ctypes.c_size_t(-1).value
    for M, N, K in [(64, 8192, 28672), (8, 14336, 4096), (8192, 8192, 8192), (300, 1024, 4096)]:
        stage = -(-M * K // 256) * 256 + -(-4 * M // 256) * 256
        assert fp8.fp8_workspace_bytes(M, N, K) == stage + fp8.fp8_gemm_workspace_bytes(M, N, K)
    # a workspace of exactly the GEMM's size is accepted (qa, lda, s_tok, qw, ldw, s_ch, y, ldy, M, N, K, ws, bytes)
    need = fp8.fp8_gemm_workspace_bytes(64, 8192, 28672)
    assert fp8.lib().fp8_gemm_scaled(P, 28672, P, Q, 28672, P, P, 8192, 64, 8192, 28672, P, need - 1, S0) \
        == FP8_ERR_WORKSPACE


class _GuardLib:
    """Stands in for the library: size queries and status names go to the real
    one, any other entry point raises (it must never be reached here)."""

    def __init__(self, real):
        self.real = real

    def __getattr__(self, name):
        if name.endswith("_bytes") or name == "fp8_status_string":
            return getattr(self.real, name)
        raise AssertionError(f"{name} reached the library")


def _stub_cls():
    import torch

    class DeviceStub(torch.Tensor):
        """A host tensor that reports itself as a cuda:0 tensor (no GPU here), so
        that one host tensor among them is the only thing a binding can reject."""

        @property
        def is_cuda(self):
            return True

        @property
        def device(self):
            return torch.device("cuda", 0)

    return DeviceStub


def _binding_case(call, host):
    """Run binding `call` with every tensor a device stub except the one named
    `host` (None: all stubs)."""
    import torch
    D = _stub_cls()

    def t(name, *shape, dtype=torch.float32):
        x = torch.zeros(*shape, dtype=dtype)
        return x if name == host else x.as_subclass(D)

    u8, f32, i32, bf = torch.uint8, torch.float32, torch.int32, torch.bfloat16
    M, N, K = 8, 32, 128
    ws = t("ws", 1 << 16, dtype=u8)
    if call == "fused":
        fp8.fp8_quant_gemm_fused(t("x", M, K), t("qw", N, K, dtype=u8), t("s_ch", N), y=t("y", M, N, dtype=bf),
                                 qa_out=t("qa_out", M, K, dtype=u8), s_tok_out=t("s_tok_out", M), ws=ws)
    elif call == "gemm":
        fp8.fp8_gemm_scaled(t("qa", M, K, dtype=u8), t("s_tok", M), t("qw", N, K, dtype=u8), t("s_ch", N),
                            y=t("y", M, N, dtype=bf), ws=ws)
    elif call == "fp8out":
        fp8.fp8_gemm_scaled_fp8out(t("qa", M, K, dtype=u8), t("s_tok", M), t("qw", N, K, dtype=u8), t("s_ch", N),
                                   q_out=t("q_out", M, N, dtype=u8), s_out=t("s_out", M),
                                   y32_out=t("y32_out", M, N), ws=ws)
    elif call == "grouped":
        E, T, R = 2, 4, 8
        fp8.fp8_gemm_grouped_scaled(t("qa", T, K, dtype=u8), t("s_tok", T), t("row_token", R, dtype=i32),
                                    t("expert_offsets", E + 1, dtype=i32), t("qw", E, N, K, dtype=u8),
                                    t("s_ch", E, N), y=t("y", R, N, dtype=bf), ws=ws)
    elif call == "quantize":
        fp8.fp8_quantize_per_token(t("x", M, K), q=t("q", M, K, dtype=u8), scales=t("scales", M))
    elif call == "gemm_mx":
        fp8.fp8_gemm_mx(t("qa", M, K, dtype=u8), t("sa", 1, M, 4, dtype=u8), t("qw", N, K, dtype=u8),
                        t("sw", 1, N, 4, dtype=u8), y=t("y", M, N, dtype=bf), ws=ws)
    elif call == "kv_scales":
        fp8.fp8_kv_channel_scales(t("kv", M, K), "e5m2", scales=t("scales", K), ws=ws)
    elif call == "calibrate":
        fp8.fp8_calibrate_percentile(t("x", M, K), 999, 1000, value=t("value", 1), scale=t("scale", 1), ws=ws)
    else:
        raise ValueError(call)


BINDING_TENSORS = {
    "fused": ["x", "qw", "s_ch", "y", "qa_out", "s_tok_out", "ws"],
    "gemm": ["qa", "s_tok", "qw", "s_ch", "y", "ws"],
    "fp8out": ["qa", "s_tok", "qw", "s_ch", "q_out", "s_out", "y32_out", "ws"],
    "grouped": ["qa", "s_tok", "row_token", "expert_offsets", "qw", "s_ch", "y", "ws"],
    "quantize": ["x", "q", "scales"],
    "gemm_mx": ["qa", "sa", "qw", "sw", "y", "ws"],
    "kv_scales": ["kv", "scales", "ws"],
    "calibrate": ["x", "value", "scale", "ws"],
}


@pytest.mark.parametrize("call,host", [(c, h) for c, hs in BINDING_TENSORS.items() for h in hs])
def test_every_tensor_argument_must_be_on_the_device(monkeypatch, call, host):
    """Each tensor argument of each binding, optional outputs and the
    workspace included, is rejected when it alone is a host tensor: the C ABI
    cannot tell a host pointer from a device pointer, and a kernel would fault
    on the host address.  With every tensor on the 'device' the call goes on to
    the library (the guard raises), so the rejection is the host tensor's."""
    monkeypatch.setattr(fp8, "lib", lambda real=fp8.lib(): _GuardLib(real))
    monkeypatch.setattr(fp8, "_stream", lambda stream: S0)
    with pytest.raises(AssertionError, match="reached the library"):
        _binding_case(call, None)
    with pytest.raises((TypeError, ValueError)):
        _binding_case(call, host)


def test_invalid_sizes_raise_instead_of_allocating(monkeypatch):
    """A size query answering SIZE_MAX (invalid sizes) raises the library's
    invalid-argument error instead of asking torch for SIZE_MAX bytes."""
    with pytest.raises(fp8.Fp8Error) as e:
        fp8._workspace(None, fp8.SIZE_MAX, "fp8_gemm_scaled", "cpu")
    assert e.value.code == FP8_ERR_INVALID_ARGUMENT


def test_noalloc_rejects_on_the_host():
    """The allocation-free fused call checks sizes before touching any device:
    beyond its static scratch array it returns FP8_ERR_WORKSPACE, invalid
    sizes FP8_ERR_INVALID_ARGUMENT."""
    L = fp8.lib()
    # x, ldx, qw, ldw, s_ch, y, ldy, M, N, K, qa_out, s_tok_out, stream
    big_m = fp8.FP8_NOALLOC_SCRATCH_BYTES // 4096 + 1024
    assert fp8.fp8_workspace_bytes(big_m, 256, 4096) > fp8.FP8_NOALLOC_SCRATCH_BYTES
    assert L.fp8_quant_gemm_fused_noalloc(P, 4096, Q, 4096, P, P, 256, big_m, 256, 4096, 0, 0, S0) \
        == FP8_ERR_WORKSPACE
    assert L.fp8_quant_gemm_fused_noalloc(P, 4096, Q, 4096, P, P, 256, -1, 256, 4096, 0, 0, S0) \
        == FP8_ERR_INVALID_ARGUMENT
    # the prefill shape fits
    assert fp8.fp8_workspace_bytes(8192, 8192, 8192) <= fp8.FP8_NOALLOC_SCRATCH_BYTES
    text = open(HEADER).read()
    assert re.search(r"#define FP8_NOALLOC_SCRATCH_BYTES \(72u << 20\)", text)
    assert fp8.FP8_NOALLOC_SCRATCH_BYTES == 72 << 20


def test_stream_read_validation():
    L = fp8.lib()
    # p, bytes, workgroups, nontemporal, sink, stream
    assert L.fp8_stream_read(P, 1000, 256, 0, Q, S0) == FP8_ERR_INVALID_ARGUMENT     # bytes % 16
    assert L.fp8_stream_read(P, 1024, 0, 0, Q, S0) == FP8_ERR_INVALID_ARGUMENT       # no workgroups
    assert L.fp8_stream_read(0, 1024, 256, 0, Q, S0) == FP8_ERR_INVALID_ARGUMENT
    assert L.fp8_stream_read(MIS, 1024, 256, 0, Q, S0) == FP8_ERR_UNSUPPORTED
    assert L.fp8_stream_read(P, 0, 256, 0, 0, S0) == FP8_OK
