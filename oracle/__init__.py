"""CPU oracle for the unified-FP8 (W8A8) linear layer -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It is a ctypes wrapper over liboracle.so (fp8_oracle.c),
a plain C implementation written from the FP8 pages:
  - the OCP E4M3 codec (largest value 448 and smallest non-zero 2^-9, Llama 3
    FP8 page §1.1; +-448 clamp, FP8 deployment page §2.3);
  - the per-row absmax/448 quantizer (Llama 3 FP8 page §3.1 snippet, applied
    per output channel to weights and per token to activations as the DeepSeek
    V4 950 page §2.4 and §3.1 describe);
  - the FP8 x FP8 GEMM with wide accumulation and s_tok*s_ch rescale
    (DeepSeek V4 950 page §2.3), exact in binary64;
  - the grouped (MoE expert) variant of that GEMM;
  - the FP8-output form of the GEMM (the output converted back to FP8, DeepSeek
    V4 950 page §2.3), composed from the exact GEMM and the quantizer.
It shares no code with the HIP library.  Every function is pinned by the
`-m "not gpu"` tests against the pages' fixed points, PyTorch's float8_e4m3fn
cast, brute force and exact integer arithmetic.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

E4M3_MAX = 448.0
SCALE_FLOOR = np.float32(1e-12)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: run `python oracle/build.py`")
        L = ctypes.CDLL(_LIB_PATH)
        i64, vp, f64 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
        L.oracle_e4m3_decode.restype = f64
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode_array.restype = None
        L.oracle_e4m3_encode_array.argtypes = [vp, i64, vp]
        L.oracle_quantize_rows.restype = None
        L.oracle_quantize_rows.argtypes = [vp, i64, i64, i64, vp, i64, vp]
        L.oracle_quantize_static.restype = None
        L.oracle_quantize_static.argtypes = [vp, i64, i64, i64, ctypes.c_float, vp, i64]
        L.oracle_quantize_rows_clipped.restype = None
        L.oracle_quantize_rows_clipped.argtypes = [vp, i64, i64, i64, ctypes.c_float, vp, i64, vp]
        L.oracle_e5m2_decode.restype = ctypes.c_double
        L.oracle_e5m2_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e5m2_encode.restype = ctypes.c_uint8
        L.oracle_e5m2_encode.argtypes = [ctypes.c_float]
        L.oracle_e5m2_encode_array.restype = None
        L.oracle_e5m2_encode_array.argtypes = [vp, i64, vp]
        L.oracle_kv_channel_scales.restype = None
        L.oracle_kv_channel_scales.argtypes = [vp, i64, i64, i64, ctypes.c_int, vp]
        L.oracle_kv_quantize.restype = None
        L.oracle_kv_quantize.argtypes = [vp, i64, i64, i64, vp, ctypes.c_int, vp, vp, i64]
        L.oracle_kv_dequantize.restype = None
        L.oracle_kv_dequantize.argtypes = [vp, i64, vp, i64, i64, vp, ctypes.c_int, vp]
        L.oracle_mx_scale_code.restype = ctypes.c_uint8
        L.oracle_mx_scale_code.argtypes = [ctypes.c_float]
        L.oracle_quantize_mx.restype = None
        L.oracle_quantize_mx.argtypes = [vp, i64, i64, i64, vp, i64, vp]
        L.oracle_gemm_mx_ref_sampled.restype = None
        L.oracle_gemm_mx_ref_sampled.argtypes = [vp, i64, vp, vp, i64, vp, i64, vp, vp, i64, vp, vp]
        L.oracle_gemm_ref.restype = None
        L.oracle_gemm_ref.argtypes = [vp, i64, vp, vp, i64, vp, i64, i64, i64, vp, vp]
        L.oracle_gemm_ref_sampled.restype = None
        L.oracle_gemm_ref_sampled.argtypes = [vp, i64, vp, vp, i64, vp, i64, vp, vp, i64, vp, vp]
        L.oracle_grouped_ref_sampled.restype = ctypes.c_int
        L.oracle_grouped_ref_sampled.argtypes = [vp, vp, vp, vp, i64, vp, vp, i64, i64, vp, vp, i64, vp, vp]
        L.oracle_bf16_from_double.restype = ctypes.c_uint16
        L.oracle_bf16_from_double.argtypes = [f64]
        L.oracle_bf16_from_double_array.restype = None
        L.oracle_bf16_from_double_array.argtypes = [vp, i64, vp]
        L.oracle_fp16_from_double.restype = ctypes.c_uint16
        L.oracle_fp16_from_double.argtypes = [f64]
        L.oracle_fp16_from_double_array.restype = None
        L.oracle_fp16_from_double_array.argtypes = [vp, i64, vp]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_num_threads.argtypes = []
        L.oracle_set_num_threads.restype = None
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        L.oracle_init.restype = None
        L.oracle_init()
        _lib = L
    return _lib


def _p(a):
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def decode(codes):
    """E4M3 codes (uint8 array) -> float64 values (NaN for S.1111.111)."""
    codes = np.asarray(codes, dtype=np.uint8)
    L = lib()
    table = np.array([L.oracle_e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[codes]


def encode(values):
    """float32 array -> E4M3 codes (RNE, saturating)."""
    v = _c(values, np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().oracle_e4m3_encode_array(_p(v), v.size, _p(out))
    return out


def encode_fn_address():
    """Address of the C encoder (for the exhaustive pin, which runs in C)."""
    return ctypes.cast(lib().oracle_e4m3_encode, ctypes.c_void_p).value


def quantize_rows(x):
    """Per-row absmax quantization of a 2-D float32 array -> (codes uint8, scales float32)."""
    x = _c(x, np.float32)
    rows, K = x.shape
    q = np.empty((rows, K), dtype=np.uint8)
    s = np.empty(rows, dtype=np.float32)
    lib().oracle_quantize_rows(_p(x), rows, K, K, _p(q), K, _p(s))
    return q, s


E5M2 = 1
E4M3 = 0


def e5m2_decode(codes):
    """E5M2 codes (uint8 array) -> float64 values (+-inf, NaN for the specials)."""
    codes = np.asarray(codes, dtype=np.uint8)
    table = np.array([lib().oracle_e5m2_decode(c) for c in range(256)], dtype=np.float64)
    return table[codes]


def e5m2_encode(values):
    """float32 array -> E5M2 codes (RNE, saturating to +-57344)."""
    v = _c(values, np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().oracle_e5m2_encode_array(_p(v), v.size, _p(out))
    return out


def e5m2_encode_fn_address():
    return ctypes.cast(lib().oracle_e5m2_encode, ctypes.c_void_p).value


def kv_channel_scales(kv, fmt):
    """Per-channel KV scales of a [T, C] float32 batch: max(fl32(amax_c / fmt_max), 1e-12f)."""
    kv = _c(kv, np.float32)
    T, C = kv.shape
    s = np.empty(C, dtype=np.float32)
    lib().oracle_kv_channel_scales(_p(kv), T, C, C, int(fmt), _p(s))
    return s


def kv_quantize(kv, scales, fmt, slot, num_slots, cache=None):
    """Quantize [T, C] KV into a paged cache uint8 [num_slots, C].  Tokens whose
    slot is outside [0, num_slots) are skipped; rows no token maps to keep the
    contents of `cache` (zeros when it is not given)."""
    kv = _c(kv, np.float32)
    T, C = kv.shape
    cache = np.zeros((num_slots, C), dtype=np.uint8) if cache is None else _c(cache, np.uint8).copy()
    assert cache.shape == (num_slots, C)
    slot = _c(slot, np.int32)
    assert slot.size == T
    lib().oracle_kv_quantize(_p(kv), T, C, C, _p(_c(scales, np.float32)), int(fmt), _p(slot), _p(cache), num_slots)
    return cache


def kv_dequantize(cache, slot, scales, fmt):
    """[T, C] float32 read back of the cache rows slot[t] (zeros for a slot
    outside the cache)."""
    cache = _c(cache, np.uint8)
    slot = _c(slot, np.int32)
    num_slots, C = cache.shape
    out = np.empty((slot.size, C), dtype=np.float32)
    lib().oracle_kv_dequantize(_p(cache), num_slots, _p(slot), slot.size, C, _p(_c(scales, np.float32)), int(fmt),
                               _p(out))
    return out


MX_BLOCK = 32


def mx_scale_code(amax):
    """E8M0 code (exponent + 127) of the block scale for a block maximum amax."""
    return int(lib().oracle_mx_scale_code(float(np.float32(amax))))


def quantize_mx(x):
    """Block-scaled quantization of fp32 x [rows, K] (K % 32 == 0) ->
    (codes uint8 [rows, K], scale codes uint8 [rows, K/32])."""
    x = _c(x, np.float32)
    rows, K = x.shape
    assert K % MX_BLOCK == 0
    q = np.empty((rows, K), dtype=np.uint8)
    sc = np.empty((rows, K // MX_BLOCK), dtype=np.uint8)
    lib().oracle_quantize_mx(_p(x), rows, K, K, _p(q), K, _p(sc))
    return q, sc


def gemm_mx_ref_sampled(qa, sa, qw, sw, ms, ns):
    """Block-scaled GEMM reference at (ms[i], ns[i]) -> (ref, absref) float64."""
    qa, qw = _c(qa, np.uint8), _c(qw, np.uint8)
    sa, sw = _c(sa, np.uint8), _c(sw, np.uint8)
    ms, ns = _c(ms, np.int64), _c(ns, np.int64)
    M, K = qa.shape
    N = qw.shape[0]
    assert qw.shape[1] == K and sa.shape == (M, K // MX_BLOCK) and sw.shape == (N, K // MX_BLOCK)
    assert ms.shape == ns.shape
    assert ms.size == 0 or (ms.min() >= 0 and ms.max() < M and ns.min() >= 0 and ns.max() < N)
    ref = np.empty(ms.size, dtype=np.float64)
    ab = np.empty(ms.size, dtype=np.float64)
    lib().oracle_gemm_mx_ref_sampled(_p(qa), K, _p(sa), _p(qw), K, _p(sw), K, _p(ms), _p(ns), ms.size, _p(ref),
                                     _p(ab))
    return ref, ab


def gemm_mx_ref(qa, sa, qw, sw):
    """Full block-scaled GEMM reference -> (ref [M,N], absref [M,N]) float64."""
    M, N = qa.shape[0], qw.shape[0]
    mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    r, a = gemm_mx_ref_sampled(qa, sa, qw, sw, mm.ravel(), nn.ravel())
    return r.reshape(M, N), a.reshape(M, N)


def quantize_static(x, scale):
    """Static per-tensor quantization of a 2-D float32 array with one scale
    (saturating) -> codes uint8.  The scale is used as given."""
    x = _c(x, np.float32)
    rows, K = x.shape
    q = np.empty((rows, K), dtype=np.uint8)
    lib().oracle_quantize_static(_p(x), rows, K, K, np.float32(scale), _p(q), K)
    return q


def quantize_rows_clipped(x, clip):
    """Per-row absmax quantization with the absmax clipped at `clip` -> (codes, scales)."""
    x = _c(x, np.float32)
    rows, K = x.shape
    q = np.empty((rows, K), dtype=np.uint8)
    s = np.empty(rows, dtype=np.float32)
    lib().oracle_quantize_rows_clipped(_p(x), rows, K, K, np.float32(clip), _p(q), K, _p(s))
    return q, s


def percentile_nearest_rank(x, num, den):
    """Nearest-rank percentile num/den of |x| (DeepSeek V4 950 page, §3.1): the
    r-th smallest |x| with r = ceil(num * n / den), clamped to [1, n]."""
    a = np.sort(np.abs(np.asarray(x, dtype=np.float32)).ravel())
    n = a.size
    r = -(-(int(num) * n) // int(den))
    r = min(max(r, 1), n)
    return np.float32(a[r - 1])


def static_scale(value):
    """The static scale of a calibrated magnitude: max(fl32(value / 448), 1e-12f)."""
    s = np.float32(value) / np.float32(E4M3_MAX)
    return np.float32(max(s, SCALE_FLOOR))


def gemm_ref(qa, s_tok, qw, s_ch):
    """Exact scaled FP8 GEMM: (ref [M,N] float64, absref [M,N] float64)."""
    qa, qw = _c(qa, np.uint8), _c(qw, np.uint8)
    s_tok, s_ch = _c(s_tok, np.float32), _c(s_ch, np.float32)
    M, K = qa.shape
    N, K2 = qw.shape
    assert K == K2 and s_tok.shape == (M,) and s_ch.shape == (N,)
    ref = np.empty((M, N), dtype=np.float64)
    ab = np.empty((M, N), dtype=np.float64)
    lib().oracle_gemm_ref(_p(qa), K, _p(s_tok), _p(qw), K, _p(s_ch), M, N, K, _p(ref), _p(ab))
    return ref, ab


def gemm_ref_sampled(qa, s_tok, qw, s_ch, ms, ns):
    qa, qw = _c(qa, np.uint8), _c(qw, np.uint8)
    s_tok, s_ch = _c(s_tok, np.float32), _c(s_ch, np.float32)
    ms, ns = _c(ms, np.int64), _c(ns, np.int64)
    M, K = qa.shape
    N = qw.shape[0]
    assert qw.shape[1] == K and ms.shape == ns.shape
    assert ms.size == 0 or (ms.min() >= 0 and ms.max() < M and ns.min() >= 0 and ns.max() < N)
    ref = np.empty(ms.size, dtype=np.float64)
    ab = np.empty(ms.size, dtype=np.float64)
    lib().oracle_gemm_ref_sampled(_p(qa), K, _p(s_tok), _p(qw), K, _p(s_ch), K, _p(ms), _p(ns), ms.size,
                                  _p(ref), _p(ab))
    return ref, ab


def grouped_ref_sampled(qa, s_tok, row_token, offsets, qw, s_ch, rs, ns):
    """Grouped MoE reference at routed rows rs, columns ns.  qw [E,N,K], s_ch [E,N]."""
    qa, qw = _c(qa, np.uint8), _c(qw, np.uint8)
    s_tok, s_ch = _c(s_tok, np.float32), _c(s_ch, np.float32)
    row_token, offsets = _c(row_token, np.int32), _c(offsets, np.int32)
    rs, ns = _c(rs, np.int64), _c(ns, np.int64)
    E, N, K = qw.shape
    assert qa.shape[1] == K and s_ch.shape == (E, N) and offsets.shape == (E + 1,)
    ref = np.empty(rs.size, dtype=np.float64)
    ab = np.empty(rs.size, dtype=np.float64)
    rc = lib().oracle_grouped_ref_sampled(_p(qa), _p(s_tok), _p(row_token), _p(offsets), E, _p(qw), _p(s_ch),
                                          N, K, _p(rs), _p(ns), rs.size, _p(ref), _p(ab))
    if rc != 0:
        raise ValueError("a sampled row lies outside every expert's range")
    return ref, ab


def fp8out_ref(qa, s_tok, qw, s_ch):
    """FP8-output GEMM from the definition (DeepSeek V4 950 page, §2.3: the FP32
    result converted back to FP8; per-token scales as for the activations,
    §2.4 and §3.1): y = the exact scaled product rounded once to fp32, then the
    per-row absmax quantizer on y.  Returns (y32 float32 [M,N], codes, scales)."""
    ref, _ = gemm_ref(qa, s_tok, qw, s_ch)
    y32 = ref.astype(np.float32)
    q, s = quantize_rows(y32)
    return y32, q, s


def bf16_from_double(v):
    v = _c(v, np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().oracle_bf16_from_double_array(_p(v), v.size, _p(out))
    return out


def fp16_from_double(v):
    """Nearest IEEE binary16 of each double, ties to even, as uint16 bits
    (the rounding of the 16-bit KV read back)."""
    v = _c(v, np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().oracle_fp16_from_double_array(_p(v), v.size, _p(out))
    return out


def bf16_bits_to_f64(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def tolerance_check(y_bits, ref, absref, rel_abs=1e-3, rel_ref=2.0 ** -8):
    """The pass criterion |y - ref| <= 1e-3 * sum|a*w| * s_tok*s_ch + 2^-8 * |ref|.

    Returns a dict: ok, worst normalised error (error / bound), fraction of
    outputs equal to the correctly rounded bf16 of ref, count checked."""
    y = bf16_bits_to_f64(y_bits)
    ref = np.asarray(ref, dtype=np.float64)
    absref = np.asarray(absref, dtype=np.float64)
    err = np.abs(y - ref)
    bound = rel_abs * absref + rel_ref * np.abs(ref)
    finite = np.isfinite(y)
    with np.errstate(divide="ignore", invalid="ignore"):
        norm = np.where(bound > 0, err / bound, np.where(err == 0, 0.0, np.inf))
    ok = bool(np.all(finite) and np.all(err <= bound))
    exact = bf16_from_double(ref)
    return dict(ok=ok, worst=float(norm.max()) if norm.size else 0.0,
                frac_rne=float(np.mean(exact == np.asarray(y_bits, dtype=np.uint16))) if norm.size else 1.0,
                n=int(norm.size), n_bad=int(np.sum(~(err <= bound)) + np.sum(~finite)))


def num_threads():
    return int(lib().oracle_num_threads())


def set_num_threads(n):
    lib().oracle_set_num_threads(int(n))
