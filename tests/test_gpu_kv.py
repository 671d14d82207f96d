"""GPU parity of the FP8 KV-cache codec (through the C ABI): per-channel
scales, paged quantize and read back equal the oracle bit for bit, in E4M3
and E5M2, for ragged shapes, strided batches, permuted block tables, padding
and out-of-range slots, and the full 32768-token prefill of one Llama-3-70B
layer in the launch configuration the benchmark times."""
import numpy as np
import pytest
import torch

import fp8_w8a8_quantized_quantize_amd as fp8
import oracle
import synth
from tests._gpu import DEV, assert_codes_equal, assert_scales_equal, log, to_dev, to_host

pytestmark = pytest.mark.gpu

FMTS = [("e4m3", oracle.E4M3), ("e5m2", oracle.E5M2)]


def _codec_sample(fmt_id, seed):
    """fp32 values covering every rounding decision of the format: random bit
    patterns up to past its range, every midpoint of neighbouring codes and
    the fp32 values next to it, the codes' own values, and specials."""
    rng = np.random.default_rng(seed)
    top = 0x47800000 if fmt_id == oracle.E5M2 else 0x44000000  # 65536.0f, 512.0f
    bits = rng.integers(0, top, size=1 << 20, dtype=np.uint32)
    dec = oracle.e5m2_decode if fmt_id == oracle.E5M2 else oracle.decode
    nfin = 124 if fmt_id == oracle.E5M2 else 127
    mags = dec(np.arange(nfin, dtype=np.uint8))
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    extra = np.array([1e30, 3e38, 57344.0, 59392.0, 61440.0, 448.0, 464.0, 480.0, 1e-45, 1e-40, 0.0], np.float32)
    v = np.concatenate([bits.view(np.float32), mids, np.nextafter(mids, np.float32(0)),
                        np.nextafter(mids, np.float32(1e9)), mags.astype(np.float32), extra])
    v = np.concatenate([v, -v])
    C = 256
    v = np.concatenate([v, np.zeros((-v.size) % C, np.float32)])
    return v.reshape(-1, C)


@pytest.mark.parametrize("fmt,fid", FMTS)
def test_codec_matches_oracle_with_unit_scales(fmt, fid):
    kv = _codec_sample(fid, seed=fid + 7)
    T, C = kv.shape
    ones = torch.ones(C, dtype=torch.float32, device=DEV)
    slot = torch.arange(T, dtype=torch.int32, device=DEV)
    cache = torch.zeros((T, C), dtype=torch.uint8, device=DEV)
    fp8.fp8_kv_quantize_paged(to_dev(kv), ones, slot, cache, fmt)
    want = oracle.kv_quantize(kv, np.ones(C, np.float32), fid, np.arange(T, dtype=np.int32), T)
    assert_codes_equal(to_host(cache), want, f"{fmt} codes of {kv.size} values")


@pytest.mark.parametrize("fmt,fid", FMTS)
def test_decode_of_all_256_codes(fmt, fid):
    codes = np.arange(256, dtype=np.uint8).reshape(1, 256)
    for s in [np.ones(256, np.float32), synth.normals(256, seed=fid, mul=0.37)]:
        s = np.abs(s).astype(np.float32)
        out = fp8.fp8_kv_dequantize_paged(to_dev(codes), to_dev(np.array([0], np.int32)), to_dev(s), fmt)
        got, want = to_host(out), oracle.kv_dequantize(codes, np.array([0], np.int32), s, fid)
        assert np.array_equal(np.isnan(got), np.isnan(want))
        fin = ~np.isnan(want)
        assert np.array_equal(got[fin].view(np.uint32), want[fin].view(np.uint32)), fmt


SCALE_SHAPES = [(0, 64), (1, 4), (7, 576), (100, 2048), (1000, 1028), (4099, 512), (33, 4100)]


@pytest.mark.parametrize("fmt,fid", FMTS)
@pytest.mark.parametrize("T,C", SCALE_SHAPES)
def test_channel_scales_exact(fmt, fid, T, C):
    kv = synth.kv_activations(T, C, seed=T + C)
    if T > 2:
        kv[:, 1] = 0.0       # floor
        kv[T // 2, 2] = -kv[T // 2, 2] * 1e4   # one huge value in a channel
    s = fp8.fp8_kv_channel_scales(to_dev(kv), fmt)
    assert_scales_equal(to_host(s), oracle.kv_channel_scales(kv, fid), f"{fmt} T={T} C={C}")


def test_channel_scales_strided_batch_and_stale_workspace():
    T, C, ld = 777, 576, 640
    big = synth.kv_activations(T, ld, seed=11)
    view = to_dev(big)[:, :C]
    ws = torch.full((fp8.fp8_kv_scales_workspace_bytes(T, C),), 0xFF, dtype=torch.uint8, device=DEV)
    s = fp8.fp8_kv_channel_scales(view, "e5m2", ws=ws)
    assert_scales_equal(to_host(s), oracle.kv_channel_scales(big[:, :C], oracle.E5M2), "strided")


PAGED = [(37, 24, 8, 9), (1000, 576, 16, 80), (4096, 2048, 16, 300), (3, 4, 1, 5)]


@pytest.mark.parametrize("fmt,fid", FMTS)
@pytest.mark.parametrize("T,C,B,nb", PAGED)
def test_paged_quantize_and_read_back(fmt, fid, T, C, B, nb):
    kv = synth.kv_activations(T, C, seed=T * 3 + C)
    s = oracle.kv_channel_scales(kv, fid)
    s[0] = np.float32(s[0] / 3)         # a stale scale for channel 0: its values saturate
    s[-1] = np.float32(0.0)             # below the floor: the 1e-12 floor applies
    slot = synth.kv_slot_mapping(T, B, nb, seed=T)
    if T > 4:
        slot[[1, T - 2]] = -1           # padding tokens
        slot[T // 2] = nb * B + 3       # outside the cache: skipped
    ns = nb * B
    prior = np.full((ns, C), 0x11, dtype=np.uint8)
    cache = to_dev(prior)
    fp8.fp8_kv_quantize_paged(to_dev(kv), to_dev(s), to_dev(slot), cache, fmt)
    want = oracle.kv_quantize(kv, s, fid, slot, ns, cache=prior)
    assert_codes_equal(to_host(cache), want, f"{fmt} cache T={T} C={C}")
    out = fp8.fp8_kv_dequantize_paged(cache, to_dev(slot), to_dev(s), fmt)
    back = oracle.kv_dequantize(want, slot, s, fid)
    got = to_host(out)
    assert np.array_equal(got.view(np.uint32), back.view(np.uint32)), f"{fmt} read back T={T} C={C}"


def test_decode_append_and_strided_read_back():
    """Decode steps append one token per sequence to an existing cache with the
    prefill's scales; reading back writes into a strided output."""
    C, B, nb = 2048, 16, 64
    ns = nb * B
    pre = synth.kv_activations(512, C, seed=21)
    s = oracle.kv_channel_scales(pre, oracle.E5M2)
    slot_pre = synth.kv_slot_mapping(512, B, nb, seed=21)
    cache = torch.zeros((ns, C), dtype=torch.uint8, device=DEV)
    fp8.fp8_kv_quantize_paged(to_dev(pre), to_dev(s), to_dev(slot_pre), cache, "e5m2")
    want = oracle.kv_quantize(pre, s, oracle.E5M2, slot_pre, ns)
    used = set(slot_pre.tolist())
    free = np.array([i for i in range(ns) if i not in used][:64], dtype=np.int32)
    new = synth.kv_activations(64, C, seed=22) * np.float32(2.0)   # beyond the prefill range: saturates
    fp8.fp8_kv_quantize_paged(to_dev(new), to_dev(s), to_dev(free), cache, "e5m2")
    want = oracle.kv_quantize(new, s, oracle.E5M2, free, ns, cache=want)
    assert_codes_equal(to_host(cache), want, "append")
    allslots = np.concatenate([slot_pre, free])
    out = torch.full((allslots.size, C + 12), -1.0, dtype=torch.float32, device=DEV)
    fp8.fp8_kv_dequantize_paged(cache, to_dev(allslots), to_dev(s), "e5m2", out=out[:, :C])
    got = to_host(out)
    back = oracle.kv_dequantize(want, allslots, s, oracle.E5M2)
    assert np.array_equal(got[:, :C].view(np.uint32), back.view(np.uint32))
    assert np.all(got[:, C:] == -1.0)


def test_full_size_prefill_of_one_layer():
    """The benchmark's workload at full size: 32768 tokens x 2048 channels,
    16-token pages, E5M2; every scale, code and read-back value compared."""
    w = synth.WORKLOADS["kv-llama3-70b-32k"]
    T, C, B = w["T"], w["C"], w["block"]
    nb = T // B + 256
    log(f"  kv full size: T={T} C={C} B={B} blocks={nb}")
    kv = synth.kv_activations(T, C, seed=0)
    slot = synth.kv_slot_mapping(T, B, nb, seed=0)
    kv_d, slot_d = to_dev(kv), to_dev(slot)
    cache = torch.zeros((nb * B, C), dtype=torch.uint8, device=DEV)
    s = fp8.fp8_kv_channel_scales(kv_d, "e5m2")
    fp8.fp8_kv_quantize_paged(kv_d, s, slot_d, cache, "e5m2")
    out = fp8.fp8_kv_dequantize_paged(cache, slot_d, s, "e5m2")
    s_want = oracle.kv_channel_scales(kv, oracle.E5M2)
    assert_scales_equal(to_host(s), s_want, "full-size scales")
    c_want = oracle.kv_quantize(kv, s_want, oracle.E5M2, slot, nb * B)
    assert_codes_equal(to_host(cache), c_want, "full-size cache")
    back = oracle.kv_dequantize(c_want, slot, s_want, oracle.E5M2)
    assert np.array_equal(to_host(out).view(np.uint32), back.view(np.uint32))
    rel = np.abs(back - kv).max() / np.abs(kv).max()
    log(f"  kv full size: max |read back - kv| / max |kv| = {rel:.3g}")


@pytest.mark.parametrize("fmt,fid", FMTS)
def test_overflowing_quotients_saturate(fmt, fid):
    """x / s beyond fp32 (huge x, scale at the 1e-12 floor) gives the largest code, not NaN."""
    C = 16
    kv = np.array([[3e38, -3e38, 1e30, -1e27, 1e26, 1.0, -2.5e-7, 0.0] * 2], np.float32)
    s = np.full(C, 1e-12, np.float32)
    s[8:] = 0.0
    cache = torch.zeros((2, C), dtype=torch.uint8, device=DEV)
    fp8.fp8_kv_quantize_paged(to_dev(kv), to_dev(s), to_dev(np.array([1], np.int32)), cache, fmt)
    want = oracle.kv_quantize(kv, s, fid, np.array([1], np.int32), 2)
    top = 0x7B if fid == oracle.E5M2 else 0x7E
    assert (want[1, :5] & 0x7F).tolist() == [top] * 5
    assert_codes_equal(to_host(cache), want, f"{fmt} overflow")


@pytest.mark.parametrize("fmt,fid", FMTS)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_16bit_kv_rows_in_and_read_back_out(fmt, fid, dtype):
    """KV rows in bf16 / fp16 (the converted fp32 value decides everything) and the
    read back rounded to bf16 / fp16: scales, codes and output bits against the
    oracle run on the same values."""
    T, C, B, nb = 1500, 576, 16, 100
    kv32 = synth.kv_activations(T, C, seed=41)
    kv_d = torch.from_numpy(kv32).to(DEV).to(dtype)
    kv_vals = kv_d.float().cpu().numpy()            # the exact values of the 16-bit rows
    slot = synth.kv_slot_mapping(T, B, nb, seed=41)
    slot[5] = -1
    s = fp8.fp8_kv_channel_scales(kv_d, fmt)
    s_want = oracle.kv_channel_scales(kv_vals, fid)
    assert_scales_equal(to_host(s), s_want, f"{fmt} {dtype} scales")
    cache = torch.zeros((nb * B, C), dtype=torch.uint8, device=DEV)
    fp8.fp8_kv_quantize_paged(kv_d, s, to_dev(slot), cache, fmt)
    c_want = oracle.kv_quantize(kv_vals, s_want, fid, slot, nb * B)
    assert_codes_equal(to_host(cache), c_want, f"{fmt} {dtype} cache")
    back32 = oracle.kv_dequantize(c_want, slot, s_want, fid)
    out = fp8.fp8_kv_dequantize_paged(cache, to_dev(slot), s, fmt, out_dtype=dtype)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    if dtype == torch.bfloat16:
        want = oracle.bf16_from_double(back32.astype(np.float64))
    else:
        want = oracle.fp16_from_double(back32.astype(np.float64))
    assert np.array_equal(got, want), f"{fmt} {dtype} read back"


def test_16bit_strided_rows():
    T, C, ld = 300, 512, 520
    big = torch.from_numpy(synth.kv_activations(T, ld, seed=43)).to(DEV).to(torch.bfloat16)
    view = big[:, :C]
    s = fp8.fp8_kv_channel_scales(view, "e5m2")
    vals = view.float().cpu().numpy()
    assert_scales_equal(to_host(s), oracle.kv_channel_scales(vals, oracle.E5M2), "strided bf16")
