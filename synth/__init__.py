"""Seeded synthetic inputs shared by the oracle and the HIP path.

Only random draws and layouts live here (see synth.c for the generator and the
distributions); no quantization or GEMM arithmetic.  The workload table below
gives the shapes of the linear layers the FP8 pages discuss: a tiny case,
Llama-3-8B and -70B decode FFN projections, a 70B prefill square GEMM, and a
DeepSeek-style MoE expert batch.
"""
import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

# sub-stream ids: one per tensor family so draws never overlap
STREAM_X = 10
STREAM_W = 20
STREAM_ROUTE = 30
STREAM_KV = 40
STREAM_KV_SLOTS = 50
STREAM_EXPERT_W = 1000  # expert e uses streams 1000 + 2e, 1000 + 2e + 1


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: run `python synth/build.py`")
        L = ctypes.CDLL(_LIB_PATH)
        u64, i64, f32, f64 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_float, ctypes.c_double
        vp = ctypes.c_void_p
        L.synth_stream_key.restype = u64
        L.synth_stream_key.argtypes = [u64, u64]
        L.synth_u64.restype = u64
        L.synth_u64.argtypes = [u64, u64]
        L.synth_uniform.restype = f64
        L.synth_uniform.argtypes = [u64, u64]
        L.synth_normal.restype = f64
        L.synth_normal.argtypes = [u64, u64]
        L.synth_normal_f32.restype = None
        L.synth_normal_f32.argtypes = [u64, u64, i64, f32, vp]
        L.synth_choose.restype = None
        L.synth_choose.argtypes = [u64, i64, i64, vp]
        L.synth_activations.restype = None
        L.synth_activations.argtypes = [u64, u64, i64, i64, i64, i64, f32, vp, vp]
        L.synth_weights.restype = None
        L.synth_weights.argtypes = [u64, u64, i64, i64, i64, i64, vp]
        L.synth_kv.restype = None
        L.synth_kv.argtypes = [u64, u64, i64, i64, i64, i64, f32, vp]
        L.synth_permutation.restype = None
        L.synth_permutation.argtypes = [u64, i64, vp]
        L.synth_routing.restype = ctypes.c_int
        L.synth_routing.argtypes = [u64, u64, i64, i64, i64, f64, vp, vp, vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def activations(M, K, n_outliers, outlier_mult, seed=0, stream=STREAM_X, out=None):
    """X [M, K] fp32 ~ N(0,1) with `n_outliers` columns scaled by `outlier_mult`.

    Returns (X, outlier_columns)."""
    x = np.empty((M, K), dtype=np.float32) if out is None else out
    assert x.dtype == np.float32 and x.shape == (M, K) and x.flags.c_contiguous
    cols = np.empty(max(n_outliers, 1), dtype=np.int64)
    lib().synth_activations(seed, stream, M, K, K, n_outliers, outlier_mult, _ptr(x), _ptr(cols))
    return x, cols[:n_outliers]


def weights(N, K, seed=0, stream=STREAM_W, n0=0, out=None):
    """W [N, K] fp32: 0.02 * N(0,1) * exp(0.5 * N(0,1) per output row)."""
    w = np.empty((N, K), dtype=np.float32) if out is None else out
    assert w.dtype == np.float32 and w.shape == (N, K) and w.flags.c_contiguous
    lib().synth_weights(seed, stream, n0, N, K, K, _ptr(w))
    return w


def normals(n, seed=0, stream=0, offset=0, mul=1.0):
    a = np.empty(n, dtype=np.float32)
    lib().synth_normal_f32(lib().synth_stream_key(seed, stream), offset, n, mul, _ptr(a))
    return a


def routing(T, E, topk, zipf_s, seed=0, stream=STREAM_ROUTE):
    """Top-k distinct experts per token, Zipf(s) over expert rank.

    Returns (token_expert [T, topk], row_token [T*topk], expert_offsets [E+1]),
    int32, routed rows sorted by expert and by token within an expert."""
    te = np.empty(T * topk, dtype=np.int32)
    rt = np.empty(T * topk, dtype=np.int32)
    off = np.empty(E + 1, dtype=np.int32)
    rc = lib().synth_routing(seed, stream, T, E, topk, zipf_s, _ptr(te), _ptr(rt), _ptr(off))
    if rc != 0:
        raise ValueError("routing: need 0 <= topk <= min(E, 64)")
    return te.reshape(T, topk), rt, off


def kv_activations(T, C, seed=0, n_outliers=None, outlier_mult=20.0, stream=STREAM_KV, out=None):
    """KV rows [T, C] fp32: N(0,1) times a per-channel gain exp(0.5 N(0,1)),
    1% of the channels (by default) with a further `outlier_mult` gain."""
    kv = np.empty((T, C), dtype=np.float32) if out is None else out
    assert kv.dtype == np.float32 and kv.shape == (T, C) and kv.flags.c_contiguous
    n_out = n_outlier_channels(C) if n_outliers is None else n_outliers
    lib().synth_kv(seed, stream, T, C, C, n_out, outlier_mult, _ptr(kv))
    return kv


def kv_slot_mapping(T, block_size, num_blocks, seed=0, stream=STREAM_KV_SLOTS):
    """Cache slots of T tokens of one sequence in a paged cache: the sequence's
    logical block i sits in physical block perm[i] of a random permutation of
    num_blocks blocks, so token t goes to perm[t // B] * B + t % B.  int32."""
    nb_used = -(-T // block_size)
    if nb_used > num_blocks:
        raise ValueError("kv_slot_mapping: the cache has too few blocks")
    perm = np.empty(max(num_blocks, 1), dtype=np.int64)
    lib().synth_permutation(lib().synth_stream_key(seed, stream), num_blocks, _ptr(perm))
    t = np.arange(T, dtype=np.int64)
    return (perm[t // block_size] * block_size + t % block_size).astype(np.int32)


def n_outlier_channels(K):
    """1% of the channels (rounded), the outlier share of the decode/prefill workloads."""
    return int(math.floor(0.01 * K + 0.5))


# Workloads: the shapes of the linear layers on the FP8 pages.
#   dense: X [M, K] activations, W [N, K] weights (nn.Linear [out, in] layout)
#   moe:   X [T, K] token activations, W [E, N, K] expert weights, top-k routing
WORKLOADS = {
    "tiny": dict(kind="dense", M=16, K=256, N=256, n_out=2, mult=30.0,
                 desc="tiny W8A8 GEMM M=16 K=256 N=256"),
    "llama3-8b-decode-up": dict(kind="dense", M=8, K=4096, N=14336, n_out=None, mult=50.0,
                                desc="Llama-3-8B FFN up-proj decode M=8 K=4096 N=14336"),
    "llama3-70b-decode-gateup": dict(kind="dense", M=64, K=8192, N=28672, n_out=None, mult=50.0,
                                     desc="Llama-3-70B gate/up decode M=64 K=8192 N=28672"),
    "llama3-70b-decode-down": dict(kind="dense", M=64, K=28672, N=8192, n_out=None, mult=50.0,
                                   desc="Llama-3-70B down decode M=64 K=28672 N=8192"),
    # one GPU's shard of the 70B decode layer at tensor-parallel degree 4 (the
    # FFN split along the intermediate size): gate/up column-parallel (N / 4),
    # down row-parallel (K / 4)
    "llama3-70b-tp4-gateup": dict(kind="dense", M=64, K=8192, N=7168, n_out=None, mult=50.0,
                                  desc="Llama-3-70B gate/up decode, TP=4 shard, M=64 K=8192 N=7168"),
    "llama3-70b-tp4-down": dict(kind="dense", M=64, K=7168, N=8192, n_out=None, mult=50.0,
                                desc="Llama-3-70B down decode, TP=4 shard, M=64 K=7168 N=8192"),
    "llama3-70b-prefill": dict(kind="dense", M=8192, K=8192, N=8192, n_out=None, mult=50.0,
                               desc="Llama-3-70B prefill square GEMM M=N=K=8192 with fused quantize"),
    "moe-64x2048x7168": dict(kind="moe", T=4096, E=64, topk=8, zipf=1.1, K=7168, N=2048, n_out=None,
                             mult=50.0, desc="MoE 64 experts K=7168 N=2048, 4096 tokens top-8 Zipf(1.1)"),
    "kv-llama3-70b-32k": dict(kind="kv", T=32768, C=2048, block=16, fmt="e5m2", dtype="bf16",
                              desc="Llama-3-70B KV cache, one layer (8 KV heads x 128, K and V), "
                                   "32768-token prefill of bf16 rows into 16-token pages, E5M2"),
}


def workload_outliers(w):
    return w["n_out"] if w["n_out"] is not None else n_outlier_channels(w["K"])


def make_dense(name, seed=0):
    """(X fp32 [M,K], W fp32 [N,K]) of a dense workload."""
    w = WORKLOADS[name]
    assert w["kind"] == "dense"
    x, _ = activations(w["M"], w["K"], workload_outliers(w), w["mult"], seed=seed)
    wt = weights(w["N"], w["K"], seed=seed)
    return x, wt


def expert_weights(E, N, K, seed=0, experts=None, out=None):
    """W [E, N, K] fp32 (or just the listed experts, stacked)."""
    ids = list(range(E)) if experts is None else list(experts)
    w = np.empty((len(ids), N, K), dtype=np.float32) if out is None else out
    for i, e in enumerate(ids):
        weights(N, K, seed=seed, stream=STREAM_EXPERT_W + 2 * e, out=w[i])
    return w
