"""Pins of the oracle's FP8-output GEMM (DeepSeek V4 950 page, §2.3: FP8 in,
FP32 accumulate, FP8 out; per-token output scales as for the activations)."""
import numpy as np
import torch

import oracle
from tests._helpers import torch_e4m3_values


def test_one_hot_worked_example():
    """qa all 1.0 (code 0x38), qw row n one-hot at k = n with code 0x38, unit
    token scales except row 1 (2.0), s_ch[n] = n + 1: y[m, n] = s_tok[m] (n+1).
    Row m's output scale is fl32(16 s_tok[m] / 448); the codes are PyTorch's
    float8_e4m3fn cast of the float32 quotients y / s."""
    M, N, K = 2, 16, 16
    qa = np.full((M, K), 0x38, np.uint8)
    qw = np.zeros((N, K), np.uint8)
    qw[np.arange(N), np.arange(N)] = 0x38
    s_tok = np.array([1.0, 2.0], np.float32)
    s_ch = np.arange(1, N + 1, dtype=np.float32)
    y32, q, s = oracle.fp8out_ref(qa, s_tok, qw, s_ch)
    want_y = (s_tok[:, None] * s_ch[None, :]).astype(np.float32)
    assert np.array_equal(y32, want_y)
    want_s = np.float32(16.0) * s_tok / np.float32(448.0)
    assert np.array_equal(s, want_s.astype(np.float32))
    quot = (want_y / want_s[:, None]).astype(np.float32)
    want_q = torch.from_numpy(quot).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, want_q)
    assert np.all(q[:, -1] == 0x7E)   # each row's largest output maps to 448


def test_decoded_output_tracks_the_exact_product():
    """On random operands the decoded output dec(q) * s stays within E4M3's
    half-ulp (2^-4 relative for normals, s * 2^-10 absolute in the subnormal
    range) of the exact scaled product."""
    rng = np.random.default_rng(3)
    vals = torch_e4m3_values()
    finite = np.array([c for c in range(256) if np.isfinite(vals[c])], np.uint8)
    M, N, K = 5, 64, 96
    qa = rng.choice(finite, (M, K))
    qw = rng.choice(finite, (N, K))
    s_tok = rng.uniform(0.01, 2.0, M).astype(np.float32)
    s_ch = rng.uniform(0.001, 0.1, N).astype(np.float32)
    ref, _ = oracle.gemm_ref(qa, s_tok, qw, s_ch)
    y32, q, s = oracle.fp8out_ref(qa, s_tok, qw, s_ch)
    dec = oracle.decode(q) * s[:, None].astype(np.float64)
    bound = 2.0 ** -4 * np.abs(ref) + s[:, None].astype(np.float64) * 2.0 ** -10 + np.abs(ref) * 2.0 ** -23
    assert np.all(np.abs(dec - ref) <= bound)
    assert np.all(np.abs(y32.astype(np.float64) - ref) <= np.abs(ref) * 2.0 ** -24)


def test_planted_wrong_row_scale_is_caught():
    """A reference that took the absmax over columns instead of rows fails the
    worked example's scale check."""
    M, N, K = 2, 16, 16
    qa = np.full((M, K), 0x38, np.uint8)
    qw = np.zeros((N, K), np.uint8)
    qw[np.arange(N), np.arange(N)] = 0x38
    s_tok = np.array([1.0, 2.0], np.float32)
    s_ch = np.arange(1, N + 1, dtype=np.float32)
    y32, _, s = oracle.fp8out_ref(qa, s_tok, qw, s_ch)
    wrong = np.abs(y32).max(axis=0)[:M] / np.float32(448.0)
    assert not np.array_equal(s, wrong.astype(np.float32))


def _fp8out_case(M=12, N=256, K=512, seed=5):
    import synth
    x, _ = synth.activations(M, K, 5, 50.0, seed=seed)
    w = synth.weights(N, K, seed=seed)
    qa, st = oracle.quantize_rows(x)
    qw, sc = oracle.quantize_rows(w)
    ref, ab = oracle.gemm_ref(qa, st, qw, sc)
    return qa, st, qw, sc, ref, ab


def test_admissibility_rule_accepts_every_y32_within_the_bound():
    """The rule the GPU FP8-output test applies (tests/_helpers.py
    fp8out_admissible) accepts the oracle's own codes and scales, and the
    quantization of any fp32 output pushed to +-0.99 of the GEMM bound."""
    from tests._helpers import fp8out_admissible
    qa, st, qw, sc, ref, ab = _fp8out_case()
    _, q, s = oracle.fp8out_ref(qa, st, qw, sc)
    r = fp8out_admissible(q, s, ref, ab)
    assert r["scale_ok"].all() and r["code_ok"].all()
    b = 1e-3 * ab + 2.0 ** -22 * np.abs(ref)
    rng = np.random.default_rng(1)
    for sign in (+1.0, -1.0, None):
        d = rng.choice([-1.0, 1.0], ref.shape) if sign is None else sign
        y = (ref + 0.99 * d * b).astype(np.float32)
        q2, s2 = oracle.quantize_rows(y)
        r2 = fp8out_admissible(q2, s2, ref, ab)
        assert r2["scale_ok"].all() and r2["code_ok"].all()
        # every code that moved sits where the interval holds a rounding boundary
        assert not np.any((q2 != q) & (s2 == s)[:, None] & ~r2["code_ambiguous"])


def test_admissibility_rule_catches_planted_mistakes():
    """A code moved one step where no rounding boundary is in reach, a doubled
    row scale and a sign flip are rejected."""
    from tests._helpers import fp8out_admissible
    qa, st, qw, sc, ref, ab = _fp8out_case()
    _, q, s = oracle.fp8out_ref(qa, st, qw, sc)
    r = fp8out_admissible(q, s, ref, ab)
    i, j = np.argwhere(~r["code_ambiguous"] & ((q & 0x7F) > 8) & ((q & 0x7F) < 0x7E))[0]
    bad = q.copy()
    bad[i, j] += 1
    assert not fp8out_admissible(bad, s, ref, ab)["code_ok"][i, j]
    s2 = s.copy()
    s2[3] *= np.float32(2.0)
    assert not fp8out_admissible(q, s2, ref, ab)["scale_ok"][3]
    flip = q.copy()
    k = np.argwhere(np.abs(ref) > 100 * (1e-3 * ab))
    i, j = k[0]
    flip[i, j] ^= 0x80
    assert not fp8out_admissible(flip, s, ref, ab)["code_ok"][i, j]
