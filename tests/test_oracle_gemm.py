"""Pins of the oracle's scaled FP8 GEMM, grouped GEMM, BF16 rounding and the
tolerance check (CPU only).

The GEMM is pinned against:
  - an int64 GEMM in units of 2^-18 (every E4M3 value is an integer multiple
    of 2^-9), with the integer values taken from PyTorch's decode: the oracle's
    binary64 sum must equal it exactly;
  - PyTorch float64 matmul of the PyTorch-decoded operands (exact here too);
  - exact rational brute force (fractions.Fraction) on tiny inputs;
  - special cases with closed forms: one-hot weight rows, and codes of
    +-1, +-2, +-4 with unit scales (integer results).
The grouped GEMM is pinned against the dense products of each expert's rows,
gathered by numpy and multiplied by PyTorch.  The BF16 rounding is pinned to
PyTorch's float32 -> bfloat16 cast.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from tests._helpers import torch_e4m3_values

TV = torch_e4m3_values()
FINITE_CODES = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def _random_codes(shape, rng):
    return rng.choice(FINITE_CODES, size=shape).astype(np.uint8)


def _ints(codes):
    return np.rint(TV[codes] * 512).astype(np.int64)


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (7, 13, 48), (33, 17, 256), (64, 40, 1024)])
def test_exact_against_int64_gemm(M, N, K):
    rng = np.random.default_rng(M * 1000 + N)
    qa, qw = _random_codes((M, K), rng), _random_codes((N, K), rng)
    ones_m, ones_n = np.ones(M, np.float32), np.ones(N, np.float32)
    ref, ab = oracle.gemm_ref(qa, ones_m, qw, ones_n)
    iref = _ints(qa) @ _ints(qw).T                     # units of 2^-18
    assert np.array_equal(ref * 2.0 ** 18, iref.astype(np.float64))
    iab = np.abs(_ints(qa))[:, None, :] * np.abs(_ints(qw))[None, :, :]
    assert np.array_equal(ab * 2.0 ** 18, iab.sum(-1).astype(np.float64))


def test_worst_case_magnitude_stays_exact():
    # all codes +-448 at K = 28672 (the largest K of the workloads): |sum| = K * 448^2
    K = 28672
    qa = np.full((2, K), 0x7E, np.uint8)
    qw = np.full((2, K), 0x7E, np.uint8)
    qw[1, ::2] = 0xFE
    qw[1, 1] = 0x01
    ref, _ = oracle.gemm_ref(qa, np.ones(2, np.float32), qw, np.ones(2, np.float32))
    exact0 = K * 448 * 448
    exact1 = (K // 2 - 1) * 448 * 448 - (K // 2) * 448 * 448 + 448 * 2 ** -9
    assert ref[0, 0] == exact0 and ref[0, 1] == exact1


def test_matches_torch_float64_matmul_with_scales():
    rng = np.random.default_rng(3)
    x, _ = synth.activations(24, 512, 5, 50.0, seed=2)
    w = synth.weights(40, 512, seed=2)
    qa, st = oracle.quantize_rows(x)
    qw, sc = oracle.quantize_rows(w)
    ref, _ = oracle.gemm_ref(qa, st, qw, sc)
    a = torch.from_numpy(TV[qa])
    b = torch.from_numpy(TV[qw])
    d = (a @ b.T).numpy()
    want = d * (st.astype(np.float64)[:, None] * sc.astype(np.float64)[None, :])
    assert np.array_equal(ref, want)
    # sampled evaluation agrees with the full one
    ms, ns = rng.integers(0, 24, 100), rng.integers(0, 40, 100)
    r2, a2 = oracle.gemm_ref_sampled(qa, st, qw, sc, ms, ns)
    full_ref, full_ab = oracle.gemm_ref(qa, st, qw, sc)
    assert np.array_equal(r2, full_ref[ms, ns]) and np.array_equal(a2, full_ab[ms, ns])


def test_rational_brute_force_tiny():
    rng = np.random.default_rng(9)
    M, N, K = 3, 4, 16
    qa, qw = _random_codes((M, K), rng), _random_codes((N, K), rng)
    st = np.array([0.5, 3.0, 1e-3], np.float32)
    sc = np.array([2.0, 0.25, 7.0, 1e-2], np.float32)
    ref, _ = oracle.gemm_ref(qa, st, qw, sc)
    for m in range(M):
        for n in range(N):
            d = sum(Fraction(TV[qa[m, k]]) * Fraction(TV[qw[n, k]]) for k in range(K))
            exact = d * Fraction(float(st[m])) * Fraction(float(sc[n]))
            # oracle: exact D, exact scale product, one rounding of the final product
            assert ref[m, n] == float(exact) or abs(Fraction(ref[m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 53)


def test_one_hot_weight_rows():
    rng = np.random.default_rng(4)
    M, N, K = 8, 32, 64
    qa = _random_codes((M, K), rng)
    cols = rng.integers(0, K, N)
    qw = np.zeros((N, K), np.uint8)
    qw[np.arange(N), cols] = 0x38  # 1.0
    st = rng.uniform(0.1, 2, M).astype(np.float32)
    sc = rng.uniform(0.1, 2, N).astype(np.float32)
    ref, _ = oracle.gemm_ref(qa, st, qw, sc)
    want = TV[qa][:, cols] * (st.astype(np.float64)[:, None] * sc.astype(np.float64)[None, :])
    assert np.array_equal(ref, want)


def test_small_integer_codes_unit_scales():
    # codes of +-1, +-2, +-4 (0x38, 0x40, 0x48 and negatives), K = 16: integer results
    rng = np.random.default_rng(5)
    pool = np.array([0x38, 0x40, 0x48, 0xB8, 0xC0, 0xC8], np.uint8)
    vals = {0x38: 1, 0x40: 2, 0x48: 4, 0xB8: -1, 0xC0: -2, 0xC8: -4}
    qa, qw = rng.choice(pool, (16, 16)), rng.choice(pool, (16, 16))
    ref, _ = oracle.gemm_ref(qa, np.ones(16, np.float32), qw, np.ones(16, np.float32))
    ia = np.vectorize(vals.get)(qa)
    iw = np.vectorize(vals.get)(qw)
    assert np.array_equal(ref, (ia @ iw.T).astype(np.float64))
    assert np.all(np.abs(ref) <= 256)


def test_grouped_matches_gathered_dense_products():
    T, E, topk, N, K = 40, 6, 2, 24, 128
    rng = np.random.default_rng(6)
    te, rt, off = synth.routing(T, E, topk, 1.1, seed=1)
    qa, st = _random_codes((T, K), rng), rng.uniform(0.01, 1, T).astype(np.float32)
    qw, sc = _random_codes((E, N, K), rng), rng.uniform(0.01, 1, (E, N)).astype(np.float32)
    R = T * topk
    rs = np.repeat(np.arange(R), N)
    ns = np.tile(np.arange(N), R)
    ref, ab = oracle.grouped_ref_sampled(qa, st, rt, off, qw, sc, rs, ns)
    ref = ref.reshape(R, N)
    for e in range(E):
        rows = np.arange(off[e], off[e + 1])
        toks = rt[rows]
        d = (torch.from_numpy(TV[qa[toks]]) @ torch.from_numpy(TV[qw[e]]).T).numpy()
        want = d * (st.astype(np.float64)[toks][:, None] * sc[e].astype(np.float64)[None, :])
        assert np.array_equal(ref[rows], want), e


def test_grouped_rejects_rows_outside_all_experts():
    qa = np.zeros((2, 16), np.uint8)
    with pytest.raises(ValueError):
        oracle.grouped_ref_sampled(qa, np.ones(2, np.float32), np.zeros(2, np.int32), np.array([0, 1], np.int32),
                                   np.zeros((1, 4, 16), np.uint8), np.ones((1, 4), np.float32), [1], [0])


def test_bf16_rounding_matches_torch_on_fp32_values():
    rng = np.random.default_rng(8)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    # add exact ties (8 significant bits + a half) and their neighbours
    base = (rng.integers(128, 256, 2000) * 2.0 ** rng.integers(-130, 120, 2000)).astype(np.float64)
    ties = (base + base / 256.0).astype(np.float32)
    v = np.concatenate([v, ties, np.nextafter(ties, 0), np.nextafter(ties, np.inf)])
    v = v[np.isfinite(v) & (np.abs(v) < 3.38e38)]
    ours = oracle.bf16_from_double(v.astype(np.float64))
    theirs = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_tolerance_check_accepts_rounded_ref_and_catches_planted_mistakes():
    x, _ = synth.activations(32, 1024, 10, 50.0, seed=12)
    w = synth.weights(32, 1024, seed=12)
    qa, st = oracle.quantize_rows(x)
    qw, sc = oracle.quantize_rows(w)
    ref, ab = oracle.gemm_ref(qa, st, qw, sc)
    good = oracle.tolerance_check(oracle.bf16_from_double(ref), ref, ab)
    assert good["ok"] and good["frac_rne"] == 1.0
    # planted in the oracle's inputs: a dropped 16-wide K block, a transposed
    # operand, a wrong scale index -- each must fail the check
    qw_drop = qw.copy()
    qw_drop[:, 512:528] = 0
    bad1, _ = oracle.gemm_ref(qa, st, qw_drop, sc)
    bad2, _ = oracle.gemm_ref(qw, st, qa, sc)
    bad3, _ = oracle.gemm_ref(qa, st[::-1].copy(), qw, sc)
    for bad in (bad1, bad2, bad3):
        assert not oracle.tolerance_check(oracle.bf16_from_double(bad), ref, ab)["ok"]
