"""MI355X-native unified-FP8 (W8A8) linear layer: Python binding.

A thin ctypes layer over libfp8w8a8.so (C ABI: include/fp8w8a8.h).  It only
marshals arguments -- torch tensors become device pointers, strides and the
current HIP stream -- and turns status codes into exceptions.  Every step of
the computation runs in the library's gfx950 kernels; there is no fallback:
if the library is missing, importing a function raises.

Entry points (same names as the C ABI):
  fp8_quantize_per_token(x)                -> (q uint8 [M,K], scales fp32 [M])
  fp8_quantize_static(x, scale)            -> (q, scales)   static per-tensor scale (device fp32 [1])
  fp8_quantize_per_token_clipped(x, clip)  -> (q, scales)   per-token scale, absmax clipped at *clip
  fp8_calibrate_percentile(x, num, den)    -> (value fp32 [1], scale fp32 [1])  nearest-rank |x| percentile
  fp8_gemm_scaled(qa, s_tok, qw, s_ch)     -> y bf16 [M,N]
  fp8_quant_gemm_fused(x, qw, s_ch)        -> y bf16 [M,N]  (optionally qa, s_tok)
  fp8_gemm_scaled_fp8out(qa, s_tok, qw, s_ch) -> (q_out uint8 [M,N], s_out fp32 [M])  (optionally y32)
  fp8_gemm_grouped_scaled(qa, s_tok, row_token, expert_offsets, qw, s_ch) -> y bf16 [R,N]
  fp8_workspace_bytes(M, N, K) (fused call), fp8_gemm_workspace_bytes(M, N, K),
  fp8_fp8out_workspace_bytes(M, N, K), fp8_grouped_workspace_bytes(T, R, E, N, K)
  fp8_status_string(code)
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8w8a8.so")

FP8_OK = 0
FP8_ERR_INVALID_ARGUMENT = 1
FP8_ERR_UNSUPPORTED = 2
FP8_ERR_WORKSPACE = 3
FP8_ERR_DEVICE = 4

# exported symbols, as declared in include/fp8w8a8.h
EXPORTS = ("fp8_quantize_per_token", "fp8_quantize_static", "fp8_quantize_per_token_clipped",
           "fp8_calibrate_percentile", "fp8_calibrate_workspace_bytes", "fp8_gemm_scaled", "fp8_quant_gemm_fused", "fp8_gemm_scaled_fp8out",
           "fp8_gemm_grouped_scaled", "fp8_workspace_bytes", "fp8_gemm_workspace_bytes", "fp8_fp8out_workspace_bytes",
           "fp8_grouped_workspace_bytes", "fp8_quantize_mx", "fp8_gemm_mx", "fp8_mx_workspace_bytes",
           "fp8_kv_channel_scales", "fp8_kv_scales_workspace_bytes",
           "fp8_kv_quantize_paged", "fp8_kv_dequantize_paged", "fp8_stream_read", "fp8_quant_gemm_fused_noalloc",
           "fp8_status_string")

_lib = None


class Fp8Error(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        super().__init__(f"{fn} failed: {status_name(code)}")


def lib():
    """Load libfp8w8a8.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run python fp8_w8a8_quantized_quantize_amd/_build.py")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, sz, st = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        L.fp8_quantize_per_token.restype = st
        L.fp8_quantize_per_token.argtypes = [vp, i64, i64, i64, vp, i64, vp, vp]
        L.fp8_quantize_static.restype = st
        L.fp8_quantize_static.argtypes = [vp, i64, i64, i64, vp, vp, i64, vp, vp]
        L.fp8_quantize_per_token_clipped.restype = st
        L.fp8_quantize_per_token_clipped.argtypes = [vp, i64, i64, i64, vp, vp, i64, vp, vp]
        L.fp8_calibrate_percentile.restype = st
        L.fp8_calibrate_percentile.argtypes = [vp, i64, i64, i64, vp, vp, vp, sz, vp]
        L.fp8_calibrate_workspace_bytes.restype = sz
        L.fp8_calibrate_workspace_bytes.argtypes = []
        L.fp8_gemm_scaled.restype = st
        L.fp8_gemm_scaled.argtypes = [vp, i64, vp, vp, i64, vp, vp, i64, i64, i64, i64, vp, sz, vp]
        L.fp8_quant_gemm_fused.restype = st
        L.fp8_quant_gemm_fused.argtypes = [vp, i64, vp, i64, vp, vp, i64, i64, i64, i64, vp, vp, vp, sz, vp]
        L.fp8_gemm_scaled_fp8out.restype = st
        L.fp8_gemm_scaled_fp8out.argtypes = [vp, i64, vp, vp, i64, vp, vp, i64, vp, vp, i64, i64, i64, vp, sz, vp]
        L.fp8_fp8out_workspace_bytes.restype = sz
        L.fp8_fp8out_workspace_bytes.argtypes = [i64, i64, i64]
        L.fp8_gemm_grouped_scaled.restype = st
        L.fp8_gemm_grouped_scaled.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, sz, vp]
        L.fp8_workspace_bytes.restype = sz
        L.fp8_workspace_bytes.argtypes = [i64, i64, i64]
        L.fp8_gemm_workspace_bytes.restype = sz
        L.fp8_gemm_workspace_bytes.argtypes = [i64, i64, i64]
        L.fp8_grouped_workspace_bytes.restype = sz
        L.fp8_grouped_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
        L.fp8_quantize_mx.restype = st
        L.fp8_quantize_mx.argtypes = [vp, i64, i64, i64, vp, i64, vp, vp]
        L.fp8_gemm_mx.restype = st
        L.fp8_gemm_mx.argtypes = [vp, i64, vp, vp, i64, vp, vp, i64, i64, i64, i64, vp, sz, vp]
        L.fp8_mx_workspace_bytes.restype = sz
        L.fp8_mx_workspace_bytes.argtypes = [i64, i64, i64]
        L.fp8_kv_channel_scales.restype = st
        L.fp8_kv_channel_scales.argtypes = [vp, st, i64, i64, i64, st, vp, vp, sz, vp]
        L.fp8_kv_scales_workspace_bytes.restype = sz
        L.fp8_kv_scales_workspace_bytes.argtypes = [i64, i64]
        L.fp8_kv_quantize_paged.restype = st
        L.fp8_kv_quantize_paged.argtypes = [vp, st, i64, i64, i64, vp, st, vp, vp, i64, vp]
        L.fp8_kv_dequantize_paged.restype = st
        L.fp8_kv_dequantize_paged.argtypes = [vp, i64, vp, i64, i64, vp, st, vp, st, i64, vp]
        L.fp8_quant_gemm_fused_noalloc.restype = st
        L.fp8_quant_gemm_fused_noalloc.argtypes = [vp, i64, vp, i64, vp, vp, i64, i64, i64, i64, vp, vp, vp]
        L.fp8_stream_read.restype = st
        L.fp8_stream_read.argtypes = [vp, sz, ctypes.c_int32, ctypes.c_int32, vp, vp]
        L.fp8_status_string.restype = ctypes.c_char_p
        L.fp8_status_string.argtypes = [st]
        _lib = L
    return _lib


def status_name(code):
    return lib().fp8_status_string(int(code)).decode()


def _check(fn, code):
    if code != FP8_OK:
        raise Fp8Error(fn, code)


def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


SIZE_MAX = (1 << 64) - 1


def _on_device(t, dtype, name, device=None):
    """t must be a torch tensor of `dtype` in GPU memory (on `device` when
    given): the library takes raw pointers and cannot tell a host address from
    a device one, so a host tensor is rejected here, before any call."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda:
        raise TypeError(f"{name}: expected a {dtype} CUDA tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")


def _rows(t, dtype, name, device=None):
    _on_device(t, dtype, name, device)
    if t.dim() != 2 or (t.shape[0] > 0 and t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name}: expected a 2-D row-major tensor (unit stride along the last dim)")
    return t.shape[0], t.shape[1], (t.stride(0) if t.shape[0] > 1 else t.shape[1])


def _vec(t, dtype, name, n, device=None):
    _on_device(t, dtype, name, device)
    if not t.is_contiguous():
        raise TypeError(f"{name}: expected a contiguous {dtype} CUDA tensor")
    if t.numel() != n:
        raise ValueError(f"{name}: expected {n} elements, got {t.numel()}")


def _dense(t, dtype, name, shape, device=None):
    """A contiguous device tensor of exactly `shape` (optional outputs)."""
    _on_device(t, dtype, name, device)
    if tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous {dtype} tensor of shape {tuple(shape)}")


def _workspace(ws, need, fn, device):
    """The caller's workspace (checked: a uint8 device tensor on `device` of at
    least `need` bytes), or a new one when ws is None; None when nothing is
    needed.  need == SIZE_MAX (the library's answer for invalid sizes) raises
    the library's FP8_ERR_INVALID_ARGUMENT."""
    torch = _torch()
    if need == SIZE_MAX:
        raise Fp8Error(fn, FP8_ERR_INVALID_ARGUMENT)
    if ws is None:
        return torch.empty(need, dtype=torch.uint8, device=device) if need > 0 else None
    _on_device(ws, torch.uint8, "ws", device)
    if not ws.is_contiguous():
        raise ValueError("ws: expected a contiguous uint8 tensor")
    return ws


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def fp8_workspace_bytes(M, N, K):
    """Workspace bytes of fp8_quant_gemm_fused (codes staged + the GEMM's)."""
    return int(lib().fp8_workspace_bytes(M, N, K))


def fp8_gemm_workspace_bytes(M, N, K):
    """Workspace bytes of fp8_gemm_scaled alone."""
    return int(lib().fp8_gemm_workspace_bytes(M, N, K))


def fp8_fp8out_workspace_bytes(M, N, K):
    return int(lib().fp8_fp8out_workspace_bytes(M, N, K))


def fp8_grouped_workspace_bytes(T, R, E, N, K):
    return int(lib().fp8_grouped_workspace_bytes(T, R, E, N, K))


def fp8_status_string(code):
    return status_name(code)


def fp8_quantize_per_token(x, q=None, scales=None, stream=None):
    """Per-row absmax E4M3 quantization of fp32 x [M, K] -> (q uint8 [M, K], scales fp32 [M])."""
    torch = _torch()
    M, K, ldx = _rows(x, torch.float32, "x")
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(M, dtype=torch.float32, device=x.device)
    Mq, Kq, ldq = _rows(q, torch.uint8, "q", x.device)
    if (Mq, Kq) != (M, K):
        raise ValueError("q: expected shape [M, K]")
    _vec(scales, torch.float32, "scales", M, x.device)
    _check("fp8_quantize_per_token",
           lib().fp8_quantize_per_token(_ptr(x), M, K, ldx, _ptr(q), ldq, _ptr(scales), _stream(stream)))
    return q, scales


def _scalar(t, name, device):
    torch = _torch()
    _on_device(t, torch.float32, name, device)
    if t.numel() < 1:
        raise TypeError(f"{name}: expected a float32 CUDA tensor holding one value")


def fp8_quantize_static(x, scale, q=None, scales_out=None, stream=None):
    """Static per-tensor quantization of fp32 x [M, K] with the device scalar
    `scale` -> (q uint8 [M, K], scales_out fp32 [M] filled with the scale)."""
    torch = _torch()
    M, K, ldx = _rows(x, torch.float32, "x")
    _scalar(scale, "scale", x.device)
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scales_out is None:
        scales_out = torch.empty(M, dtype=torch.float32, device=x.device)
    Mq, Kq, ldq = _rows(q, torch.uint8, "q", x.device)
    if (Mq, Kq) != (M, K):
        raise ValueError("q: expected shape [M, K]")
    _vec(scales_out, torch.float32, "scales_out", M, x.device)
    _check("fp8_quantize_static", lib().fp8_quantize_static(_ptr(x), M, K, ldx, _ptr(scale), _ptr(q), ldq,
                                                            _ptr(scales_out), _stream(stream)))
    return q, scales_out


def fp8_quantize_per_token_clipped(x, clip, q=None, scales=None, stream=None):
    """Per-token quantization with the row absmax clipped at the device scalar `clip`."""
    torch = _torch()
    M, K, ldx = _rows(x, torch.float32, "x")
    _scalar(clip, "clip", x.device)
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(M, dtype=torch.float32, device=x.device)
    Mq, Kq, ldq = _rows(q, torch.uint8, "q", x.device)
    if (Mq, Kq) != (M, K):
        raise ValueError("q: expected shape [M, K]")
    _vec(scales, torch.float32, "scales", M, x.device)
    _check("fp8_quantize_per_token_clipped",
           lib().fp8_quantize_per_token_clipped(_ptr(x), M, K, ldx, _ptr(clip), _ptr(q), ldq, _ptr(scales),
                                                _stream(stream)))
    return q, scales


def fp8_calibrate_percentile(x, num, den, value=None, scale=None, ws=None, stream=None):
    """Nearest-rank percentile num/den of |x| over all of x (fp32, contiguous)
    -> (value fp32 [1], static scale fp32 [1]) on the device."""
    torch = _torch()
    _on_device(x, torch.float32, "x")
    if not x.is_contiguous():
        raise TypeError("x: expected a contiguous float32 CUDA tensor")
    if value is None:
        value = torch.empty(1, dtype=torch.float32, device=x.device)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=x.device)
    _vec(value, torch.float32, "value", 1, x.device)
    _vec(scale, torch.float32, "scale", 1, x.device)
    ws = _workspace(ws, int(lib().fp8_calibrate_workspace_bytes()), "fp8_calibrate_percentile", x.device)
    _check("fp8_calibrate_percentile",
           lib().fp8_calibrate_percentile(_ptr(x), x.numel(), int(num), int(den), _ptr(value), _ptr(scale), _ptr(ws),
                                          _nbytes(ws), _stream(stream)))
    return value, scale


def fp8_mx_workspace_bytes(M, N, K):
    return int(lib().fp8_mx_workspace_bytes(M, N, K))


def _mx_scales(t, name, rows, K, device):
    _dense(t, _torch().uint8, name, (K // 128, rows, 4), device)


def fp8_quantize_mx(x, q=None, scales=None, stream=None):
    """Block-scaled E4M3 quantization of fp32 x [M, K] (K % 128 == 0) ->
    (q uint8 [M, K], scales uint8 [K/128, M, 4] chunk-major exponent bytes)."""
    torch = _torch()
    M, K, ldx = _rows(x, torch.float32, "x")
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((K // 128, M, 4), dtype=torch.uint8, device=x.device)
    Mq, Kq, ldq = _rows(q, torch.uint8, "q", x.device)
    if (Mq, Kq) != (M, K):
        raise ValueError("q: expected shape [M, K]")
    _mx_scales(scales, "scales", M, K, x.device)
    _check("fp8_quantize_mx", lib().fp8_quantize_mx(_ptr(x), M, K, ldx, _ptr(q), ldq, _ptr(scales), _stream(stream)))
    return q, scales


def fp8_gemm_mx(qa, sa, qw, sw, y=None, ws=None, stream=None):
    """y = bf16(sum over 32-blocks of 2^(ea + ew - 254) * block dot) for block-scaled
    E4M3 operands qa [M, K], qw [N, K] with chunk-major exponent bytes sa [K/128, M, 4],
    sw [K/128, N, 4]."""
    torch = _torch()
    M, K, lda = _rows(qa, torch.uint8, "qa")
    dev = qa.device
    N, K2, ldw = _rows(qw, torch.uint8, "qw", dev)
    if K2 != K:
        raise ValueError("qa and qw disagree on K")
    _mx_scales(sa, "sa", M, K, dev)
    _mx_scales(sw, "sw", N, K, dev)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    My, Ny, ldy = _rows(y, torch.bfloat16, "y", dev)
    if (My, Ny) != (M, N):
        raise ValueError("y: expected shape [M, N]")
    ws = _workspace(ws, fp8_mx_workspace_bytes(M, N, K), "fp8_gemm_mx", dev)
    _check("fp8_gemm_mx", lib().fp8_gemm_mx(_ptr(qa), lda, _ptr(sa), _ptr(qw), ldw, _ptr(sw), _ptr(y), ldy, M, N, K,
                                            _ptr(ws), _nbytes(ws), _stream(stream)))
    return y


FP8_KV_E4M3 = 0
FP8_KV_E5M2 = 1
FP8_KV_F32 = 0
FP8_KV_BF16 = 1
FP8_KV_F16 = 2
_KV_FORMATS = {"e4m3": FP8_KV_E4M3, "e5m2": FP8_KV_E5M2, FP8_KV_E4M3: FP8_KV_E4M3, FP8_KV_E5M2: FP8_KV_E5M2}


def _kv_fmt(fmt):
    if fmt not in _KV_FORMATS:
        raise ValueError(f"fmt: expected 'e4m3' or 'e5m2', got {fmt!r}")
    return _KV_FORMATS[fmt]


def fp8_kv_scales_workspace_bytes(T, C):
    return int(lib().fp8_kv_scales_workspace_bytes(T, C))


def _kv_dtype(t, name, device=None):
    torch = _torch()
    codes = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}
    if not isinstance(t, torch.Tensor) or t.dtype not in codes or not t.is_cuda:
        raise TypeError(f"{name}: expected a float32, bfloat16 or float16 CUDA tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    return codes[t.dtype]


def _kv_rows(t, name, device=None):
    dt = _kv_dtype(t, name, device)
    if t.dim() != 2 or (t.shape[0] > 0 and t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name}: expected a 2-D row-major tensor (unit stride along the last dim)")
    return t.shape[0], t.shape[1], (t.stride(0) if t.shape[0] > 1 else t.shape[1]), dt


def _kv_cache(cache, C=None, device=None):
    torch = _torch()
    _on_device(cache, torch.uint8, "cache", device)
    if not cache.is_contiguous() or cache.dim() != 2 or (C is not None and cache.shape[1] != C):
        raise TypeError("cache: expected a contiguous uint8 CUDA tensor [num_slots, C]")


def fp8_kv_channel_scales(kv, fmt="e5m2", scales=None, ws=None, stream=None):
    """Per-channel scales max(fl32(max_t |kv[t,c]| / fmt_max), 1e-12f) of kv [T, C]
    (float32, bfloat16 or float16) -> scales fp32 [C]."""
    torch = _torch()
    T, C, ldkv, dt = _kv_rows(kv, "kv")
    if scales is None:
        scales = torch.empty(C, dtype=torch.float32, device=kv.device)
    _vec(scales, torch.float32, "scales", C, kv.device)
    ws = _workspace(ws, fp8_kv_scales_workspace_bytes(T, C), "fp8_kv_channel_scales", kv.device)
    _check("fp8_kv_channel_scales",
           lib().fp8_kv_channel_scales(_ptr(kv), dt, T, C, ldkv, _kv_fmt(fmt), _ptr(scales), _ptr(ws),
                                       _nbytes(ws), _stream(stream)))
    return scales


def fp8_kv_quantize_paged(kv, scales, slot_mapping, cache, fmt="e5m2", stream=None):
    """Write kv [T, C] (float32, bfloat16 or float16) into the rows slot_mapping[t]
    of the uint8 cache [num_slots, C] (contiguous) as FP8 codes of kv / scales;
    returns cache."""
    torch = _torch()
    T, C, ldkv, dt = _kv_rows(kv, "kv")
    _vec(scales, torch.float32, "scales", C, kv.device)
    _vec(slot_mapping, torch.int32, "slot_mapping", T, kv.device)
    _kv_cache(cache, C, kv.device)
    _check("fp8_kv_quantize_paged",
           lib().fp8_kv_quantize_paged(_ptr(kv), dt, T, C, ldkv, _ptr(scales), _kv_fmt(fmt), _ptr(slot_mapping),
                                       _ptr(cache), cache.shape[0], _stream(stream)))
    return cache


def fp8_kv_dequantize_paged(cache, slot_mapping, scales, fmt="e5m2", out=None, out_dtype=None, stream=None):
    """Read cache rows slot_mapping[t] back -> out [T, C] (float32 by default, or
    bfloat16 / float16: out's dtype, else out_dtype)."""
    torch = _torch()
    _kv_cache(cache)
    dev = cache.device
    num_slots, C = cache.shape
    T = slot_mapping.numel() if isinstance(slot_mapping, torch.Tensor) else -1
    _vec(slot_mapping, torch.int32, "slot_mapping", T, dev)
    _vec(scales, torch.float32, "scales", C, dev)
    if out is None:
        out = torch.empty((T, C), dtype=out_dtype or torch.float32, device=dev)
    T2, C2, ldo, odt = _kv_rows(out, "out", dev)
    if (T2, C2) != (T, C):
        raise ValueError("out: expected shape [T, C]")
    _check("fp8_kv_dequantize_paged",
           lib().fp8_kv_dequantize_paged(_ptr(cache), num_slots, _ptr(slot_mapping), T, C, _ptr(scales),
                                         _kv_fmt(fmt), _ptr(out), odt, ldo, _stream(stream)))
    return out


def fp8_gemm_scaled(qa, s_tok, qw, s_ch, y=None, ws=None, stream=None):
    """y[m,n] = bf16(sum_k e4m3(qa[m,k]) e4m3(qw[n,k]) * s_tok[m] * s_ch[n]).

    ws: optional uint8 device workspace of at least fp8_gemm_workspace_bytes(M, N, K)
    bytes (scratch: its contents on entry do not matter); allocated per call
    when not given and the shape needs one."""
    torch = _torch()
    M, K, lda = _rows(qa, torch.uint8, "qa")
    dev = qa.device
    N, K2, ldw = _rows(qw, torch.uint8, "qw", dev)
    if K2 != K:
        raise ValueError("qa and qw disagree on K")
    _vec(s_tok, torch.float32, "s_tok", M, dev)
    _vec(s_ch, torch.float32, "s_ch", N, dev)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    My, Ny, ldy = _rows(y, torch.bfloat16, "y", dev)
    if (My, Ny) != (M, N):
        raise ValueError("y: expected shape [M, N]")
    ws = _workspace(ws, fp8_gemm_workspace_bytes(M, N, K), "fp8_gemm_scaled", dev)
    _check("fp8_gemm_scaled",
           lib().fp8_gemm_scaled(_ptr(qa), lda, _ptr(s_tok), _ptr(qw), ldw, _ptr(s_ch), _ptr(y), ldy, M, N, K,
                                 _ptr(ws), _nbytes(ws), _stream(stream)))
    return y


def fp8_quant_gemm_fused(x, qw, s_ch, y=None, qa_out=None, s_tok_out=None, ws=None, stream=None):
    """Quantize x per token, then the scaled FP8 GEMM, in one call -> y bf16 [M, N]."""
    torch = _torch()
    M, K, ldx = _rows(x, torch.float32, "x")
    dev = x.device
    N, K2, ldw = _rows(qw, torch.uint8, "qw", dev)
    if K2 != K:
        raise ValueError("x and qw disagree on K")
    _vec(s_ch, torch.float32, "s_ch", N, dev)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    My, Ny, ldy = _rows(y, torch.bfloat16, "y", dev)
    if (My, Ny) != (M, N):
        raise ValueError("y: expected shape [M, N]")
    if qa_out is not None:
        _dense(qa_out, torch.uint8, "qa_out", (M, K), dev)
    if s_tok_out is not None:
        _vec(s_tok_out, torch.float32, "s_tok_out", M, dev)
    ws = _workspace(ws, fp8_workspace_bytes(M, N, K), "fp8_quant_gemm_fused", dev)
    _check("fp8_quant_gemm_fused",
           lib().fp8_quant_gemm_fused(_ptr(x), ldx, _ptr(qw), ldw, _ptr(s_ch), _ptr(y), ldy, M, N, K,
                                      _ptr(qa_out), _ptr(s_tok_out), _ptr(ws), _nbytes(ws), _stream(stream)))
    return y


# size of the static device scratch array of fp8_quant_gemm_fused_noalloc
FP8_NOALLOC_SCRATCH_BYTES = 72 << 20


def fp8_quant_gemm_fused_noalloc(x, qw, s_ch, y, qa_out=None, s_tok_out=None, stream=None):
    """fp8_quant_gemm_fused without a workspace: the library's static device
    scratch array holds the staged codes and split-K partial sums, so the call
    allocates nothing (y, and qa_out / s_tok_out when wanted, are the caller's)."""
    torch = _torch()
    M, K, ldx = _rows(x, torch.float32, "x")
    dev = x.device
    N, K2, ldw = _rows(qw, torch.uint8, "qw", dev)
    if K2 != K:
        raise ValueError("x and qw disagree on K")
    _vec(s_ch, torch.float32, "s_ch", N, dev)
    My, Ny, ldy = _rows(y, torch.bfloat16, "y", dev)
    if (My, Ny) != (M, N):
        raise ValueError("y: expected shape [M, N]")
    if qa_out is not None:
        _dense(qa_out, torch.uint8, "qa_out", (M, K), dev)
    if s_tok_out is not None:
        _vec(s_tok_out, torch.float32, "s_tok_out", M, dev)
    _check("fp8_quant_gemm_fused_noalloc",
           lib().fp8_quant_gemm_fused_noalloc(_ptr(x), ldx, _ptr(qw), ldw, _ptr(s_ch), _ptr(y), ldy, M, N, K,
                                              _ptr(qa_out), _ptr(s_tok_out), _stream(stream)))
    return y


def fp8_gemm_scaled_fp8out(qa, s_tok, qw, s_ch, q_out=None, s_out=None, y32_out=None, ws=None, stream=None):
    """FP8-output GEMM: y32 = acc * s_tok * s_ch in fp32, re-quantized per token
    -> (q_out uint8 [M, N], s_out fp32 [M]); y32_out (fp32 [M, N]) optional."""
    torch = _torch()
    M, K, lda = _rows(qa, torch.uint8, "qa")
    dev = qa.device
    N, K2, ldw = _rows(qw, torch.uint8, "qw", dev)
    if K2 != K:
        raise ValueError("qa and qw disagree on K")
    _vec(s_tok, torch.float32, "s_tok", M, dev)
    _vec(s_ch, torch.float32, "s_ch", N, dev)
    if q_out is None:
        q_out = torch.empty((M, N), dtype=torch.uint8, device=dev)
    Mq, Nq, ldq = _rows(q_out, torch.uint8, "q_out", dev)
    if (Mq, Nq) != (M, N):
        raise ValueError("q_out: expected shape [M, N]")
    if s_out is None:
        s_out = torch.empty(M, dtype=torch.float32, device=dev)
    _vec(s_out, torch.float32, "s_out", M, dev)
    if y32_out is not None:
        _dense(y32_out, torch.float32, "y32_out", (M, N), dev)
    need = fp8_fp8out_workspace_bytes(M, N, K)
    if need != SIZE_MAX and y32_out is not None:
        need = int(lib().fp8_gemm_workspace_bytes(M, N, K))   # y32 lives in y32_out, not in ws
    ws = _workspace(ws, need, "fp8_gemm_scaled_fp8out", dev)
    _check("fp8_gemm_scaled_fp8out",
           lib().fp8_gemm_scaled_fp8out(_ptr(qa), lda, _ptr(s_tok), _ptr(qw), ldw, _ptr(s_ch), _ptr(q_out), ldq,
                                        _ptr(s_out), _ptr(y32_out), M, N, K, _ptr(ws), _nbytes(ws), _stream(stream)))
    return q_out, s_out


def fp8_gemm_grouped_scaled(qa, s_tok, row_token, expert_offsets, qw, s_ch, y=None, ws=None, stream=None):
    """Grouped MoE GEMM over expert-sorted routed rows -> y bf16 [R, N]."""
    torch = _torch()
    T, K, _ = _rows(qa, torch.uint8, "qa")
    dev = qa.device
    if not qa.is_contiguous():
        raise ValueError("qa: expected contiguous [T, K]")
    _on_device(qw, torch.uint8, "qw", dev)
    if qw.dim() != 3 or not qw.is_contiguous():
        raise ValueError("qw: expected a contiguous uint8 CUDA tensor [E, N, K]")
    E, N, K2 = qw.shape
    if K2 != K:
        raise ValueError("qa and qw disagree on K")
    _on_device(row_token, torch.int32, "row_token", dev)
    R = row_token.numel()
    _vec(s_tok, torch.float32, "s_tok", T, dev)
    _vec(row_token, torch.int32, "row_token", R, dev)
    _vec(expert_offsets, torch.int32, "expert_offsets", E + 1, dev)
    _dense(s_ch, torch.float32, "s_ch", (E, N), dev)
    if y is None:
        y = torch.empty((R, N), dtype=torch.bfloat16, device=dev)
    _dense(y, torch.bfloat16, "y", (R, N), dev)
    ws = _workspace(ws, fp8_grouped_workspace_bytes(T, R, E, N, K), "fp8_gemm_grouped_scaled", dev)
    _check("fp8_gemm_grouped_scaled",
           lib().fp8_gemm_grouped_scaled(_ptr(qa), _ptr(s_tok), _ptr(row_token), _ptr(expert_offsets), _ptr(qw),
                                         _ptr(s_ch), _ptr(y), T, R, E, N, K, _ptr(ws), _nbytes(ws), _stream(stream)))
    return y


def fp8_stream_read(buf, workgroups=256, nontemporal=False, sink=None, stream=None):
    """Read every byte of the contiguous device tensor `buf` once (the HBM read
    ceiling the decode kernels are measured against); returns the sink tensor."""
    torch = _torch()
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise TypeError("buf: expected a contiguous CUDA tensor")
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    _vec(sink, torch.int32, "sink", 1, buf.device)
    _check("fp8_stream_read", lib().fp8_stream_read(_ptr(buf), _nbytes(buf), int(workgroups), int(bool(nontemporal)),
                                                    _ptr(sink), _stream(stream)))
    return sink
