"""Helpers of the GPU parity tests: device buffers, oracle comparisons."""
import sys

import numpy as np
import torch

import oracle

DEV = "cuda:0"


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def to_host(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def assert_codes_equal(got, want, what):
    got, want = np.asarray(got), np.asarray(want)
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {bad.shape[0]} mismatches; first at {i}: gpu 0x{int(got[i]):x} "
                             f"oracle 0x{int(want[i]):x}")


def assert_scales_equal(got, want, what):
    gb, wb = np.asarray(got, np.float32).view(np.uint32), np.asarray(want, np.float32).view(np.uint32)
    if not np.array_equal(gb, wb):
        i = int(np.argwhere(gb != wb)[0][0])
        raise AssertionError(f"{what}: scale bits differ at {i}: gpu 0x{gb[i]:08x} oracle 0x{wb[i]:08x}")


def assert_within_tolerance(y_bits, ref, absref, what):
    """|y - ref| <= 1e-3 * sum|a*w| * s_tok*s_ch + 2^-8 |ref| on every element."""
    r = oracle.tolerance_check(y_bits, ref, absref)
    log(f"  {what}: n={r['n']} worst/bound={r['worst']:.3g} exact-bf16 fraction={r['frac_rne']:.4f}")
    assert r["ok"], f"{what}: {r['n_bad']} of {r['n']} outside tolerance (worst {r['worst']:.3g} x bound)"
    return r
