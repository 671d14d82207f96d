"""Pins of the oracle's block-scaled ("MX") quantizer and GEMM (CPU only).

  - the scale code against its closed form: v = max(fl32(amax / 448), 1e-12f)
    and 2^(e-1) < v <= 2^e, checked with exact float comparisons, plus hand
    values (448 -> 2^0, 449 -> 2^1, 224 -> 2^-1, 0 -> 2^-39);
  - the codes against PyTorch's float8_e4m3fn cast of x / 2^e, block by block;
  - no element is clipped: every block's largest |x| lands on a code in
    (224, 448];
  - the GEMM against a PyTorch float64 matmul of the dequantized operands and
    an exact rational brute force on a tiny case; a reference that takes the
    wrong block for the scales is caught.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from tests._helpers import torch_e4m3_values, torch_encode


def _closed_form_code(amax):
    v = np.float32(np.float32(amax) / np.float32(448.0))
    v = max(v, np.float32(1e-12))
    e = int(np.ceil(np.log2(np.float64(v))))
    # fix up the float64 log2 near powers of two with exact comparisons
    while np.ldexp(1.0, e) < v:
        e += 1
    while np.ldexp(1.0, e - 1) >= v:
        e -= 1
    return e + 127


@pytest.mark.parametrize("amax,code", [(448.0, 127), (449.0, 128), (224.0, 126), (224.0001, 127), (0.0, 88),
                                       (896.0, 128), (1e-10, 88), (1e-9, 89), (3e38, 127 + 120)])
def test_scale_code_hand_values(amax, code):
    assert oracle.mx_scale_code(amax) == code


def test_scale_code_closed_form_on_random_and_boundary_maxima():
    rng = np.random.default_rng(1)
    bits = rng.integers(0x00800000, 0x7F000000, 20000, dtype=np.uint32)
    vals = list(bits.view(np.float32))
    for k in range(-60, 100):
        b = np.float32(448.0 * 2.0 ** k)
        vals += [b, np.nextafter(b, np.float32(0)), np.nextafter(b, np.float32(np.inf))]
    for a in vals:
        assert oracle.mx_scale_code(a) == _closed_form_code(a), a


def _blocks(rows, K, seed):
    x, _ = synth.activations(rows, K, max(1, K // 100), 50.0, seed=seed)
    x[0, :32] = 0.0                 # an all-zero block
    x[0, 32:64] *= 1e-20            # a tiny block
    x[1, :32] = 448.0 * 4           # a block whose maximum is exactly 448 * 2^2
    return x


def test_codes_equal_pytorch_cast_of_the_scaled_block():
    x = _blocks(24, 512, seed=2)
    q, sc = oracle.quantize_mx(x)
    for r in range(x.shape[0]):
        for b in range(x.shape[1] // 32):
            e = int(sc[r, b]) - 127
            scaled = (x[r, 32 * b:32 * b + 32].astype(np.float64) / 2.0 ** e).astype(np.float32)
            assert np.array_equal(q[r, 32 * b:32 * b + 32], torch_encode(scaled)), (r, b)


def test_no_block_is_clipped_and_the_maximum_uses_the_top_binade():
    x = _blocks(24, 512, seed=3)
    q, sc = oracle.quantize_mx(x)
    vals = torch_e4m3_values()
    deq = np.abs(vals[q]) * np.ldexp(1.0, sc.astype(np.int64) - 127).repeat(32, axis=1)
    for r in range(x.shape[0]):
        for b in range(x.shape[1] // 32):
            blk = np.abs(x[r, 32 * b:32 * b + 32])
            if blk.max() == 0:
                assert np.all(q[r, 32 * b:32 * b + 32] & 0x7F == 0) and sc[r, b] == 88
                continue
            top = np.abs(vals[q[r, 32 * b:32 * b + 32]]).max()
            assert 224.0 <= top <= 448.0 or sc[r, b] == 88, (r, b, top)
    assert q[1, 0] == 0x7E and sc[1, 0] == 129
    # every element within half a quantum of its block
    err = np.abs(deq - np.abs(x))
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * np.ldexp(1.0, sc.astype(np.int64) - 127).repeat(32, axis=1)) * (1 + 1e-12))


def _deq(q, sc):
    return torch_e4m3_values()[q] * np.ldexp(1.0, sc.astype(np.int64) - 127).repeat(32, axis=1)


def test_gemm_against_float64_matmul_of_dequantized_operands():
    x = _blocks(20, 256, seed=4)
    w = synth.weights(36, 256, seed=4)
    qa, sa = oracle.quantize_mx(x)
    qw, sw = oracle.quantize_mx(w)
    ref, absref = oracle.gemm_mx_ref(qa, sa, qw, sw)
    A, W = torch.from_numpy(_deq(qa, sa)), torch.from_numpy(_deq(qw, sw))
    want = (A @ W.T).numpy()
    assert np.all(np.abs(ref - want) <= 1e-12 * absref + 1e-300)
    assert np.allclose(absref, (A.abs() @ W.abs().T).numpy(), rtol=1e-12, atol=0)


def test_gemm_exact_rational_brute_force_tiny():
    rng = np.random.default_rng(5)
    qa = rng.integers(0, 256, (2, 64), dtype=np.uint8)
    qw = rng.integers(0, 256, (3, 64), dtype=np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x11
    qw[(qw & 0x7F) == 0x7F] = 0x22
    sa = rng.integers(110, 140, (2, 2), dtype=np.uint8)
    sw = rng.integers(110, 140, (3, 2), dtype=np.uint8)
    vals = torch_e4m3_values()
    ref, _ = oracle.gemm_mx_ref(qa, sa, qw, sw)
    for m in range(2):
        for n in range(3):
            tot = Fraction(0)
            for k in range(64):
                b = k // 32
                tot += (Fraction(vals[qa[m, k]]) * Fraction(vals[qw[n, k]]) *
                        Fraction(2) ** (int(sa[m, b]) - 127) * Fraction(2) ** (int(sw[n, b]) - 127))
            assert abs(Fraction(ref[m, n]) - tot) <= abs(tot) * Fraction(1, 2 ** 50)


def test_a_reference_with_the_wrong_block_index_is_caught():
    x = _blocks(8, 128, seed=6)
    w = synth.weights(8, 128, seed=6)
    qa, sa = oracle.quantize_mx(x)
    qw, sw = oracle.quantize_mx(w)
    ref, _ = oracle.gemm_mx_ref(qa, sa, qw, sw)
    # plant: scale blocks of 16 instead of 32 (reads block k // 16, clamped)
    vals = torch_e4m3_values()
    bad = np.zeros_like(ref)
    for m in range(8):
        for n in range(8):
            for k in range(128):
                b = min(k // 16, 3)
                bad[m, n] += vals[qa[m, k]] * vals[qw[n, k]] * 2.0 ** (int(sa[m, b]) + int(sw[n, b]) - 254)
    assert not np.allclose(ref, bad, rtol=1e-6)
