#!/usr/bin/env python3
"""Benchmark of the unified-FP8 (W8A8) linear layer on one MI355X.

One step = one pass of the hot path over one batch of synthetic input:
  dense workloads: fp8_quant_gemm_fused (per-token E4M3 quantization of the
                   activations + FP8 GEMM with the s_tok*s_ch BF16 epilogue)
                   against pre-quantized weights;
  MoE workload:    per-token quantization of the token activations +
                   fp8_gemm_grouped_scaled over the expert-sorted routed rows.
Weight quantization is the offline step and is not timed.

Default: the Llama-3-70B prefill GEMM M = N = K = 8192 with the fused
activation quantization, reported as TFLOP/s (2*M*N*K per step); its `roofline`
rates the MFMA GEMM kernel alone against the 5.0 PFLOP/s dense FP8 peak.
`detail` carries the other configurations of the metric, each timed on its
own: the decode shapes (8B up-projection, 70B gate/up and down, and the 70B
TP=4 shards) as HBM GB/s against 8 TB/s and against the measured streaming-read
ceiling of the same byte count, and the grouped MoE GEMM.  Decode workloads
rotate several weight copies (>= 512 MB in total) so that the 256 MB Infinity
Cache cannot serve the weights across steps.

Timing: every workload is first run back to back for --prewarm seconds (the
GPU clock takes about 20 ms of sustained load to settle).  Short steps (decode)
are then timed as replays of a HIP graph holding 10 consecutive steps, each
replay bracketed by HIP events on the launch stream (torch's current stream,
which the library launches on); long steps (prefill, MoE: hundreds of
microseconds, which the host launches far ahead of the GPU) as eager launches
with an event after each step.  ms_per_step is the total over all timed steps;
the per-step median / p10 / p90 come from the replays (or steps).

The JSON line adds
  roofline:     the dominant kernel timed alone, algorithmic FLOPs (or bytes)
                per launch over its average duration, against the MI355X peak;
                traffic from the committed rocprofv3 counter summary
                (profiles/hbm_traffic.txt) when it was taken on the current
                kernel source, else null;
  cpu_baseline: the CPU oracle (exact binary64 reference) timed on the host on
                a bounded sample of the same workload, single-threaded and on
                all host threads, with the CPU model.
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 W8A8 GEMM TFLOPS (prefill) & HBM GB/s (decode M≤64), % of roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA
ROTATE_BYTES = 512 << 20       # weight copies rotated per decode workload
DEFAULT_WORKLOAD = "llama3-70b-prefill"
DETAIL_DENSE = ["llama3-8b-decode-up", "llama3-70b-decode-gateup", "llama3-70b-decode-down",
                "llama3-70b-tp4-gateup", "llama3-70b-tp4-down"]
DETAIL_MOE = "moe-64x2048x7168"
DETAIL_STEPS = 200             # steps per detail workload (decode: graphs of 10 steps)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
KERNEL_SOURCES = {
    "skinny": ["gemm_skinny.hip", "device_common.hpp"],
    "mfma": ["gemm_mfma.hip", "device_common.hpp"],
    "kv": ["kv_cache.hip", "device_common.hpp"],
    "stream": ["stream_read.hip", "device_common.hpp"],
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--prewarm", type=float, default=0.5,
                    help="seconds of back-to-back steps before each timed region (GPU clock settling)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU-oracle sample time (split between the single-thread and the all-thread run)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-detail", action="store_true", help="time only --workload (no other configurations)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches instead of HIP-graph replays of the steps")
    ap.add_argument("--out", choices=("bf16", "fp8"), default="bf16",
                    help="bf16: the fused quantize+GEMM step (default); fp8: the FP8-output GEMM "
                         "(fp8_gemm_scaled_fp8out on FP8 activations, dense workloads)")
    ap.add_argument("--act", choices=("dynamic", "static", "clipped"), default="dynamic",
                    help="activation scales: per-token absmax (default, the fused call), a static per-tensor "
                         "scale calibrated as the P99.9 of |x|, or per-token scales clipped at the P99.99 of |x|")
    ap.add_argument("--scales", choices=("token", "mx"), default="token",
                    help="token: per-token x per-channel scales (default); mx: 32-element block scales "
                         "(fp8_quantize_mx + fp8_gemm_mx, dense workloads)")
    ap.add_argument("--kv-dtype", choices=("bf16", "f16", "f32"), default=None,
                    help="element type of the KV rows and of the read back (KV workloads; default: the workload's)")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="only measure the streaming-read ceiling (fp8_stream_read) at the decode weight sizes")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run 5 plain device copies of 512 MiB (reference for rocprofv3 FETCH/WRITE_SIZE)")
    ap.add_argument("--profile", action="store_true",
                    help="one workload, no detail and no CPU baseline: for runs under rocprofv3 (the usual "
                         "warm-up and pre-warm are kept, so the clock has settled)")
    return ap.parse_args()


log = lambda *a: print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ helpers --

def kernel_source_hash(kind):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "fp8_w8a8_quantized_quantize_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(workload, kind, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 PMC
    summary, if it was taken on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    src = kernel_source_hash(kind)
    with open(TRAFFIC_FILE) as f:
        for line in f:
            m = re.match(r"^TRAFFIC\s+(\{.*\})\s*$", line.strip())
            if not m:
                continue
            rec = json.loads(m.group(1))
            if rec.get("workload") == workload and rec.get("kernel") == kernel and rec.get("source") == src:
                return rec.get("hbm_bytes_per_launch")
    return None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def pct(v, q):
    v = sorted(v)
    return v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]


def group_for(steps, target):
    """The largest divisor of steps that is <= target (steps per graph)."""
    return max(d for d in range(1, max(1, min(target, steps)) + 1) if steps % d == 0)


def prewarm(fn, seconds):
    """Run fn back to back for about `seconds` (lets the GPU clock settle)."""
    import torch
    t0, i = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn(i)
            i += 1
        torch.cuda.synchronize()
    return i


def timed(fn, steps, warmup, graph, group, prewarm_s):
    """warmup untimed calls of fn(i), the pre-warm, then `steps` timed steps:
    with graph=True as steps/group replays of a HIP graph holding `group`
    consecutive steps (so host launch cost is not measured; the kernels and
    their on-GPU dispatch gaps are), each replay bracketed by HIP events on
    the launch stream; else eager launches with an event after every step.
    group <= 1 (steps of a few hundred microseconds, which the host launches
    far ahead of the GPU) also takes eager launches: replays of a one-step
    graph measured about 2 % slower than both a long graph and eager launches
    on the 8192^3 GEMM, which agree within 0.5 %.
    Returns dict(total_ms, steps, per_step_ms: one value per replay or step)."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    if prewarm_s > 0:
        prewarm(fn, prewarm_s)
    torch.cuda.synchronize()
    if not graph or group <= 1:
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        evs[0].record()
        for i in range(steps):
            fn(i)
            evs[i + 1].record()
        torch.cuda.synchronize()
        per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
        return dict(total_ms=evs[0].elapsed_time(evs[steps]), steps=steps, per_step_ms=per)
    group = group_for(steps, group)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(0)  # warm the capture stream
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        for i in range(group):
            fn(i)
    g.replay()  # untimed first replay
    torch.cuda.synchronize()
    reps = steps // group
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    evs[0].record()
    for r in range(reps):
        g.replay()
        evs[r + 1].record()
    torch.cuda.synchronize()
    per = [evs[r].elapsed_time(evs[r + 1]) / group for r in range(reps)]
    return dict(total_ms=evs[0].elapsed_time(evs[reps]), steps=reps * group, per_step_ms=per, group=group)


def stats_us(t):
    """Per-step mean / median / p10 / p90 in microseconds."""
    per = t["per_step_ms"]
    return dict(mean_us=round(t["total_ms"] / t["steps"] * 1e3, 3), median_us=round(pct(per, 0.5) * 1e3, 3),
                p10_us=round(pct(per, 0.1) * 1e3, 3), p90_us=round(pct(per, 0.9) * 1e3, 3),
                steps=t["steps"], steps_per_replay=t.get("group", 1))


def gen_dense(w, seed):
    import synth
    x, _ = synth.activations(w["M"], w["K"], synth.workload_outliers(w), w["mult"], seed=seed)
    wt = synth.weights(w["N"], w["K"], seed=seed)
    return x, wt


def weight_copies(t, nbytes):
    copies = max(1, math.ceil(ROTATE_BYTES / nbytes))
    return [t] + [t.clone() for _ in range(copies - 1)]


def free_gpu():
    import gc
    import torch
    gc.collect()
    torch.cuda.empty_cache()


# ------------------------------------------------------------- CPU baseline --

def cpu_time_oracle(work, units_per_call, target_s, threads):
    """Time work(n) (n sample units) with the oracle on `threads` threads:
    a short probe picks n so that one call takes about target_s, then that
    call is timed.  Returns (units, seconds)."""
    import oracle
    oracle.set_num_threads(threads)
    n = max(1, units_per_call)
    t0 = time.perf_counter()
    work(n)
    dt = max(time.perf_counter() - t0, 1e-6)
    n = max(1, int(n * target_s / dt))
    t0 = time.perf_counter()
    done = work(n)
    return done, time.perf_counter() - t0


def cpu_baseline(work, unit_value, unit, sample_desc, target_s, probe_units):
    """The oracle's rate single-threaded and on all host threads (OpenMP's
    default team size); work(n) runs n sample units and returns the units done;
    unit_value converts units to the metric's quantity."""
    import oracle
    all_threads = oracle.num_threads()
    u1, s1 = cpu_time_oracle(work, probe_units, target_s / 2, 1)
    un, sn = cpu_time_oracle(work, probe_units, target_s / 2, all_threads)
    oracle.set_num_threads(all_threads)
    return dict(value=round(unit_value(un) / sn, 6), unit=unit, cores=all_threads, kind="oracle",
                sample=sample_desc(un), seconds=round(sn, 2),
                single_thread=dict(value=round(unit_value(u1) / s1, 6), unit=unit, cores=1, sample=sample_desc(u1),
                                   seconds=round(s1, 2)),
                cpu_model=cpu_model())


def cpu_baseline_dense(w, x, wq_h, sc_h, target_s):
    """Per-token quantization + exact binary64 GEMM of sampled activation rows
    against all weight rows (the fused step on those rows)."""
    import oracle
    M, N, K = w["M"], w["N"], w["K"]

    def work(n):
        done = 0
        while done < n:
            rows = min(M, n - done)
            qa, st = oracle.quantize_rows(x[:rows])
            oracle.gemm_ref(qa, st, wq_h, sc_h)
            done += rows
        return done

    decode = M <= 64
    if decode:
        unit, val = "GB/s", (lambda r: r * (4 * K + 2 * N) / 1e9 + (r / M) * (N * K + 4 * N) / 1e9)
    else:
        unit, val = "TFLOP/s", (lambda r: 2.0 * r * N * K / 1e12)
    desc = lambda r: (f"per-token quantization + exact binary64 GEMM of {r} activation rows "
                      f"({'passes over all ' + str(M) if decode else 'the first rows of ' + str(M)}) "
                      f"against all {N} weight rows")
    return cpu_baseline(work, val, unit, desc, target_s, probe_units=min(M, 4))


# ------------------------------------------------------------ dense workload --

def run_dense(name, steps, warmup, graph, prewarm_s, seed, group, want_cpu, cpu_s, act="dynamic"):
    """Time one dense workload: the step (fused quantize + GEMM, or the static /
    clipped quantizer + GEMM) and the GEMM kernel alone on pre-quantized
    activations.  Returns a dict with the step and GEMM statistics, the
    roofline of the dominant kernel and (want_cpu) the CPU baseline."""
    import numpy as np
    import torch
    import fp8_w8a8_quantized_quantize_amd as fp8
    import synth

    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[name]
    M, N, K = w["M"], w["N"], w["K"]
    log(f"[bench] {name}: generating inputs M={M} N={N} K={K}")
    x, wt = gen_dense(w, seed)
    wq, sc = fp8.fp8_quantize_per_token(torch.from_numpy(wt).to(dev))  # offline weight conversion
    del wt
    wcopies = weight_copies(wq, N * K)
    copies = len(wcopies)
    xd = torch.from_numpy(x).to(dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, fp8.fp8_workspace_bytes(M, N, K)), dtype=torch.uint8, device=dev)
    gws = fp8.fp8_gemm_workspace_bytes(M, N, K)
    gws = torch.empty(gws, dtype=torch.uint8, device=dev) if gws > 0 else None
    qa = torch.empty((M, K), dtype=torch.uint8, device=dev)
    st = torch.empty(M, dtype=torch.float32, device=dev)

    def step(i):
        fp8.fp8_quant_gemm_fused(xd, wcopies[i % copies], sc, y=y, ws=ws)

    calib = None
    if act != "dynamic":
        # offline calibration on the same activations, timed once on its own
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        num, den = (999, 1000) if act == "static" else (9999, 10000)
        fp8.fp8_calibrate_percentile(xd, num, den)
        c0.record()
        value, sscale = fp8.fp8_calibrate_percentile(xd, num, den)
        c1.record()
        torch.cuda.synchronize()
        cal_ms = c0.elapsed_time(c1)
        calib = dict(percentile=f"{num}/{den}", value=float(value.cpu()[0]), scale=float(sscale.cpu()[0]),
                     calibrate_us=round(cal_ms * 1e3, 3), calibrate_gbs=round(4 * M * K / (cal_ms * 1e-3) / 1e9, 1))
        qs = torch.empty((M, K), dtype=torch.uint8, device=dev)
        ss = torch.empty(M, dtype=torch.float32, device=dev)

        def step(i):
            if act == "static":
                fp8.fp8_quantize_static(xd, sscale, q=qs, scales_out=ss)
            else:
                fp8.fp8_quantize_per_token_clipped(xd, value, q=qs, scales=ss)
            fp8.fp8_gemm_scaled(qs, ss, wcopies[i % copies], sc, y=y, ws=gws)

    # the dominant kernel alone: the GEMM on pre-quantized activations
    fp8.fp8_quantize_per_token(xd, q=qa, scales=st)

    def gemm(i):
        fp8.fp8_gemm_scaled(qa, st, wcopies[i % copies], sc, y=y, ws=gws)

    log(f"[bench] {name}: {copies} weight copies; warmup {warmup}, pre-warm {prewarm_s} s, {steps} steps")
    t_step = timed(step, steps, warmup, graph, group, prewarm_s)
    t_gemm = timed(gemm, steps, warmup, graph, group, prewarm_s)
    ms = t_step["total_ms"] / t_step["steps"]
    gemm_ms = t_gemm["total_ms"] / t_gemm["steps"]
    decode = M <= 64
    flops = 2.0 * M * N * K
    step_bytes = 4 * M * K + N * K + 4 * N + 2 * M * N           # fused: fp32 x in, codes W, s_ch, bf16 y out
    gemm_bytes = M * K + 4 * M + N * K + 4 * N + 2 * M * N       # GEMM kernel: codes x, s_tok, W, s_ch, y
    kind = "skinny" if decode else "mfma"
    # The library runs the fused call as one kernel (quantization in the
    # GEMM's prologue) for M <= 16 rows whose codes fit in LDS, whose fp32
    # values fit in 16 float4 registers per lane, and N <= 8192
    # (include/fp8w8a8.h); then that kernel is the whole step and is the
    # one the roofline rates.
    one_kernel = (act == "dynamic" and M <= 16 and M * (K + 16) <= 64 * 1024 + 256
                  and -(-K // 256) <= (16 if M <= 8 else 8) and 0 < N <= 8192)
    splits = decode and fp8.fp8_gemm_workspace_bytes(M, N, K) > 0
    if decode:
        value, unit = step_bytes / (ms * 1e-3) / 1e9, "GB/s"
        g_ach = gemm_bytes / (gemm_ms * 1e-3) / 1e9
        if one_kernel:
            roof = dict(bound="hbm", achieved=round(value, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                        frac=round(value / HBM_PEAK_GBS, 4), kernel="gemm_skinny_fused_kernel",
                        per_launch=f"{step_bytes} algorithmic bytes (fp32 x in, E4M3 W, scales, bf16 y out)",
                        avg_launch_us=round(ms * 1e3, 3),
                        gemm_only=dict(kernel="gemm_skinny_kernel (fp8_gemm_scaled on pre-quantized codes)",
                                       avg_launch_us=round(gemm_ms * 1e3, 3), achieved=round(g_ach, 1),
                                       frac=round(g_ach / HBM_PEAK_GBS, 4)))
        else:
            roof = dict(bound="hbm", achieved=round(g_ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                        frac=round(g_ach / HBM_PEAK_GBS, 4),
                        kernel="gemm_skinny_kernel" + (" + skinny_splitk_reduce" if splits else ""),
                        per_launch=f"{gemm_bytes} algorithmic bytes (E4M3 x and W, scales, bf16 y out)",
                        avg_launch_us=round(gemm_ms * 1e3, 3))
    else:
        value, unit = flops / (ms * 1e-3) / 1e12, "TFLOP/s"
        achieved = flops / (gemm_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=FP8_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / FP8_PEAK_TFLOPS, 4), kernel="gemm_mfma_kernel",
                    per_launch=f"{flops:.6g} FLOP", avg_launch_us=round(gemm_ms * 1e3, 3))
    roof["traffic"] = read_traffic(name, kind, roof["kernel"].split(" ")[0] if not one_kernel else roof["kernel"])
    roof["gemm_us"] = stats_us(t_gemm)
    cfg = dict(workload=name, M=M, N=N, K=K, seed=seed, weight_copies=copies,
               step=("fp8_quant_gemm_fused" if act == "dynamic" else
                     ("fp8_quantize_static" if act == "static" else "fp8_quantize_per_token_clipped")
                     + " + fp8_gemm_scaled"), act_scales=act, out="bf16")
    res = dict(name=name, decode=decode, value=value, unit=unit, ms=ms, steps=t_step["steps"], roofline=roof,
               config=cfg, step_us=stats_us(t_step), step_tflops=round(flops / (ms * 1e-3) / 1e12, 2),
               step_gbs=round(step_bytes / (ms * 1e-3) / 1e9, 1), gemm_bytes=gemm_bytes, calibration=calib)
    if want_cpu:
        log(f"[bench] {name}: timing the CPU oracle")
        res["cpu"] = cpu_baseline_dense(w, x, wq.cpu().numpy(), sc.cpu().numpy(), cpu_s)
    del wcopies, wq, xd, y, ws, gws, qa, st
    free_gpu()
    return res


# --------------------------------------------------------------- MoE workload --

def run_moe(name, steps, warmup, graph, prewarm_s, seed, group, want_cpu, cpu_s):
    import numpy as np
    import torch
    import fp8_w8a8_quantized_quantize_amd as fp8
    import synth

    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[name]
    T, E, k, N, K = w["T"], w["E"], w["topk"], w["N"], w["K"]
    log(f"[bench] {name}: generating inputs T={T} E={E} top-{k} N={N} K={K}")
    te, rt, off = synth.routing(T, E, k, w["zipf"], seed=seed)
    x, _ = synth.activations(T, K, synth.workload_outliers(w), w["mult"], seed=seed)
    xd = torch.from_numpy(x).to(dev)
    qw = torch.empty((E, N, K), dtype=torch.uint8, device=dev)
    sc = torch.empty((E, N), dtype=torch.float32, device=dev)
    for e0 in range(0, E, 8):
        we = synth.expert_weights(E, N, K, seed=seed, experts=range(e0, e0 + 8)).reshape(8 * N, K)
        fp8.fp8_quantize_per_token(torch.from_numpy(we).to(dev), q=qw[e0:e0 + 8].view(8 * N, K),
                                   scales=sc[e0:e0 + 8].view(-1))
    rtd, offd = torch.from_numpy(rt).to(dev), torch.from_numpy(off).to(dev)
    R = rt.size
    qa = torch.empty((T, K), dtype=torch.uint8, device=dev)
    st = torch.empty(T, dtype=torch.float32, device=dev)
    y = torch.empty((R, N), dtype=torch.bfloat16, device=dev)

    def step(i):
        fp8.fp8_quantize_per_token(xd, q=qa, scales=st)
        fp8.fp8_gemm_grouped_scaled(qa, st, rtd, offd, qw, sc, y=y)

    def gemm(i):
        fp8.fp8_gemm_grouped_scaled(qa, st, rtd, offd, qw, sc, y=y)

    log(f"[bench] {name}: warmup {warmup}, pre-warm {prewarm_s} s, {steps} steps")
    t_step = timed(step, steps, warmup, graph, group, prewarm_s)
    t_gemm = timed(gemm, steps, warmup, graph, group, prewarm_s)
    ms = t_step["total_ms"] / t_step["steps"]
    gemm_ms = t_gemm["total_ms"] / t_gemm["steps"]
    flops = 2.0 * R * N * K
    gemm_bytes = E * N * K + 4 * E * N + T * K + 4 * T + 4 * R + 4 * (E + 1) + 2 * R * N
    value, unit = flops / (ms * 1e-3) / 1e12, "TFLOP/s"
    achieved = flops / (gemm_ms * 1e-3) / 1e12
    t_roof = max(flops / (FP8_PEAK_TFLOPS * 1e12), gemm_bytes / (HBM_PEAK_GBS * 1e9))
    roof = dict(bound="mfma", achieved=round(achieved, 1), peak=FP8_PEAK_TFLOPS, unit="TFLOP/s",
                frac=round(achieved / FP8_PEAK_TFLOPS, 4), traffic=read_traffic(name, "mfma", "gemm_mfma_kernel"),
                kernel="gemm_mfma_kernel (grouped)", per_launch=f"{flops:.6g} FLOP",
                avg_launch_us=round(gemm_ms * 1e3, 3), gemm_us=stats_us(t_gemm),
                roofline_time_us=round(t_roof * 1e6, 1),
                roofline_time_frac=round(t_roof / (gemm_ms * 1e-3), 4),
                achieved_gbs=round(gemm_bytes / (gemm_ms * 1e-3) / 1e9, 1))
    cfg = dict(workload=name, T=T, E=E, topk=k, N=N, K=K, R=R, zipf=w["zipf"], seed=seed,
               step="fp8_quantize_per_token + fp8_gemm_grouped_scaled", out="bf16")
    res = dict(name=name, value=value, unit=unit, ms=ms, steps=t_step["steps"], roofline=roof, config=cfg,
               step_us=stats_us(t_step), expert_rows_max=int(np.diff(off).max()),
               expert_rows_min=int(np.diff(off).min()))
    if want_cpu:
        import oracle
        log(f"[bench] {name}: timing the CPU oracle")
        qw_h, sc_h = qw.cpu().numpy(), sc.cpu().numpy()
        qa_h, st_h = oracle.quantize_rows(x)
        rng = np.random.default_rng(0)

        def work(n):
            rs, ns = rng.integers(0, R, n), rng.integers(0, N, n)
            oracle.grouped_ref_sampled(qa_h, st_h, rt, off, qw_h, sc_h, rs, ns)
            return n

        res["cpu"] = cpu_baseline(work, lambda n: 2.0 * n * K / 1e12, "TFLOP/s",
                                  lambda n: f"{n} random routed outputs (exact binary64 dots of K={K})",
                                  cpu_s, probe_units=4096)
    del qw, sc, xd, qa, st, y, rtd, offd
    free_gpu()
    return res


# ------------------------------------------------------ read ceiling (HBM) --

def read_ceiling(sizes, log_each=False):
    """Best plain streaming-read rate (fp8_stream_read) for each byte count in
    `sizes`, over a few grid sizes and both load kinds, rotating buffer copies
    (>= 512 MB) past the Infinity Cache.  Returns {bytes: dict}."""
    import torch
    import fp8_w8a8_quantized_quantize_amd as fp8
    dev = torch.device("cuda:0")
    out = {}
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for nbytes in sizes:
        nbytes = (nbytes + 15) // 16 * 16
        copies = max(2, math.ceil(ROTATE_BYTES / nbytes))
        bufs = [torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device=dev) for _ in range(copies)]
        best = None
        for wgs in (256, 512, 1024, 2048):
            for nt in (False, True):
                def fn(i, wgs=wgs, nt=nt):
                    fp8.fp8_stream_read(bufs[i % copies], workgroups=wgs, nontemporal=nt, sink=sink)
                t = timed(fn, 100, 5, True, 10, 0.1)
                us = t["total_ms"] / t["steps"] * 1e3
                gbs = nbytes / (us * 1e-6) / 1e9
                if log_each:
                    log(f"[read] {nbytes} B wgs={wgs} nt={nt}: {us:.2f} us {gbs:.0f} GB/s")
                if best is None or gbs > best["gbs"]:
                    best = dict(bytes=nbytes, us=round(us, 3), gbs=round(gbs, 1), frac=round(gbs / HBM_PEAK_GBS, 4),
                                workgroups=wgs, nontemporal=nt, copies=copies)
        out[nbytes] = best
        del bufs
        free_gpu()
    return out


# ---------------------------------------------------------------------- main --

def emit(value, unit, steps, warmup, ms, cfg, roof, cpu, detail, dtype="fp8e4m3 (fp32 accumulate, bf16 out)"):
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype, "data": "synthetic (seeded; no dataset, no trained weights)",
        "config": cfg, "roofline": roof, "cpu_baseline": cpu, "detail": detail,
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path; run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import fp8_w8a8_quantized_quantize_amd as fp8
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X (no GPU visible)", file=sys.stderr)
        sys.exit(3)
    fp8.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        src = torch.ones(512 << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": 512 << 20, "bytes_written": 512 << 20}))
        return
    if args.read_ceiling:
        sizes = sorted({synth.WORKLOADS[n]["N"] * synth.WORKLOADS[n]["K"] for n in DETAIL_DENSE}
                       | {939524096, 1 << 30})
        rc = read_ceiling(sizes, log_each=True)
        print(json.dumps({"read_ceiling": list(rc.values()), "kernel": "stream_read_kernel",
                          "source": kernel_source_hash("stream")}), flush=True)
        return
    w = synth.WORKLOADS[args.workload]
    steps, warmup, graph = args.steps, args.warmup, not args.no_graph
    if args.profile:
        steps = min(steps, 50)
    want_cpu = not args.no_cpu_baseline and not args.profile
    detail_on = not args.no_detail and not args.profile and args.workload == DEFAULT_WORKLOAD

    if args.out == "fp8":
        if w["kind"] != "dense":
            print("--out fp8 is for the dense workloads", file=sys.stderr)
            sys.exit(2)
        return bench_fp8out(args, w, dev, steps, warmup, graph, want_cpu)
    if w["kind"] == "kv":
        return bench_kv(args, w, dev, steps, warmup, graph, want_cpu)
    if args.scales == "mx":
        if w["kind"] != "dense":
            print("--scales mx is for the dense workloads", file=sys.stderr)
            sys.exit(2)
        return bench_mx(args, w, dev, steps, warmup, graph, want_cpu)

    if w["kind"] == "dense":
        group = 10 if w["M"] <= 64 else 1
        r = run_dense(args.workload, steps, warmup, graph, args.prewarm, args.seed, group, want_cpu,
                      args.cpu_seconds, act=args.act)
    else:
        r = run_moe(args.workload, steps, warmup, graph, args.prewarm, args.seed, 1, want_cpu, args.cpu_seconds)
    detail = dict(timing=("hip-graph replays of 10 steps (decode) or eager launches with an event per step "
                          "(prefill, MoE), after a pre-warm" if graph else "eager launches after a pre-warm"),
                  prewarm_s=args.prewarm, step_us=r["step_us"])
    if "step_tflops" in r:
        detail.update(step_tflops=r["step_tflops"], step_gbs=r["step_gbs"])
    if r.get("calibration"):
        detail["calibration"] = r["calibration"]
    if w["kind"] == "moe":
        detail.update(expert_rows_max=r["expert_rows_max"], expert_rows_min=r["expert_rows_min"])
    if detail_on:
        # the decode side of the metric (HBM GB/s) and the grouped MoE GEMM,
        # each timed on its own after its own pre-warm
        ceil = read_ceiling(sorted({synth.WORKLOADS[n]["N"] * synth.WORKLOADS[n]["K"] for n in DETAIL_DENSE}))
        dec = {}
        for name in DETAIL_DENSE:
            d = run_dense(name, DETAIL_STEPS, 20, graph, args.prewarm, args.seed, 10, False, 0)
            wn = synth.WORKLOADS[name]
            c = ceil[(wn["N"] * wn["K"] + 15) // 16 * 16]
            rf = dict(d["roofline"])
            rf["frac_of_read_ceiling"] = round(rf["achieved"] / c["gbs"], 4)
            dec[name] = dict(M=wn["M"], N=wn["N"], K=wn["K"], weight_copies=d["config"]["weight_copies"],
                             step_us=d["step_us"], step_gbs=d["step_gbs"], roofline=rf)
        detail["decode"] = dec
        detail["read_ceiling"] = dict(kernel="stream_read_kernel (fp8_stream_read: plain 16-byte loads, "
                                             "8 in flight per thread, best of 4 grid sizes x 2 load kinds)",
                                      sizes=list(ceil.values()))
        m = run_moe(DETAIL_MOE, 50, 5, graph, args.prewarm, args.seed, 1, False, 0)
        detail["moe"] = dict(config=m["config"], step_us=m["step_us"], step_tflops=round(m["value"], 1),
                             roofline=m["roofline"], expert_rows_max=m["expert_rows_max"],
                             expert_rows_min=m["expert_rows_min"])
    emit(r["value"], r["unit"], r["steps"], warmup, r["ms"], r["config"], r["roofline"], r.get("cpu"), detail)


def bench_fp8out(args, w, dev, steps, warmup, graph, want_cpu):
    """One step = fp8_gemm_scaled_fp8out: FP8 activation codes and scales in
    (as a previous FP8-output layer leaves them), FP32 accumulation, the output
    re-quantized per token to E4M3 codes and scales."""
    import numpy as np
    import torch
    import fp8_w8a8_quantized_quantize_amd as fp8
    M, N, K = w["M"], w["N"], w["K"]
    log(f"[bench] {args.workload} (FP8 output): generating inputs M={M} N={N} K={K}")
    x, wt = gen_dense(w, args.seed)
    wq, sc = fp8.fp8_quantize_per_token(torch.from_numpy(wt).to(dev))
    del wt
    wcopies = weight_copies(wq, N * K)
    copies = len(wcopies)
    qa, st = fp8.fp8_quantize_per_token(torch.from_numpy(x).to(dev))
    q_out = torch.empty((M, N), dtype=torch.uint8, device=dev)
    s_out = torch.empty(M, dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, fp8.fp8_fp8out_workspace_bytes(M, N, K)), dtype=torch.uint8, device=dev)

    def step(i):
        fp8.fp8_gemm_scaled_fp8out(qa, st, wcopies[i % copies], sc, q_out=q_out, s_out=s_out, ws=ws)

    t = timed(step, steps, warmup, graph, 10 if M <= 64 else 1, args.prewarm)
    ms = t["total_ms"] / t["steps"]
    flops = 2.0 * M * N * K
    step_bytes = M * K + 4 * M + N * K + 4 * N + M * N + 4 * M   # codes+scales in, W, s_ch, codes+scales out
    decode = M <= 64
    if decode:
        value, unit = step_bytes / (ms * 1e-3) / 1e9, "GB/s"
        roof = dict(bound="hbm", achieved=round(value, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(value / HBM_PEAK_GBS, 4))
        per_launch = f"{step_bytes} algorithmic bytes"
    else:
        value, unit = flops / (ms * 1e-3) / 1e12, "TFLOP/s"
        roof = dict(bound="mfma", achieved=round(value, 1), peak=FP8_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(value / FP8_PEAK_TFLOPS, 4))
        per_launch = f"{flops:.6g} FLOP"
    roof.update(kernel="fp8_gemm_scaled_fp8out (GEMM with fp32 output, then the per-token output quantizer; "
                       "rated as one step)",
                per_launch=per_launch, avg_launch_us=round(ms * 1e3, 3),
                traffic=read_traffic(f"{args.workload}@fp8out", "skinny" if decode else "mfma",
                                     "fp8_gemm_scaled_fp8out"))
    cfg = dict(workload=args.workload, M=M, N=N, K=K, seed=args.seed, weight_copies=copies,
               step="fp8_gemm_scaled_fp8out", out="e4m3 codes + fp32 per-token scales")
    detail = dict(timing="hip-graph replays after a pre-warm" if graph else "eager launches", prewarm_s=args.prewarm,
                  step_us=stats_us(t))
    cpu = None
    if want_cpu:
        import oracle
        log("[bench] timing the CPU oracle")
        qa_h, st_h, wq_h, sc_h = qa.cpu().numpy(), st.cpu().numpy(), wq.cpu().numpy(), sc.cpu().numpy()

        def work(n):
            done = 0
            while done < n:
                rows = min(M, n - done)
                oracle.fp8out_ref(qa_h[:rows], st_h[:rows], wq_h, sc_h)
                done += rows
            return done

        if decode:
            val = lambda r: r * (K + 4 + N + 4) / 1e9 + (r / M) * (N * K + 4 * N) / 1e9
        else:
            val = lambda r: 2.0 * r * N * K / 1e12
        cpu = cpu_baseline(work, val, unit,
                           lambda r: f"oracle.fp8out_ref (exact GEMM rounded once to fp32, then the per-token "
                                     f"quantizer) on {r} activation rows against all {N} weight rows",
                           args.cpu_seconds, probe_units=min(M, 4))
    emit(value, unit, t["steps"], warmup, ms, cfg, roof, cpu, detail, dtype="fp8e4m3 (fp32 accumulate, e4m3 out)")


def bench_mx(args, w, dev, steps, warmup, graph, want_cpu):
    """One step = fp8_quantize_mx of the activations + fp8_gemm_mx against
    block-scaled weights (quantized once, untimed): 32-element blocks along K
    with power-of-two scales applied inside the K loop by the block-scaled
    MFMA."""
    import numpy as np
    import torch
    import fp8_w8a8_quantized_quantize_amd as fp8
    M, N, K = w["M"], w["N"], w["K"]
    log(f"[bench] {args.workload} (block scales): generating inputs M={M} N={N} K={K}")
    x, wt = gen_dense(w, args.seed)
    wq, ws_ = fp8.fp8_quantize_mx(torch.from_numpy(wt).to(dev))
    del wt
    copies = max(1, math.ceil(ROTATE_BYTES / (N * K)))
    wcopies = [(wq, ws_)] + [(wq.clone(), ws_.clone()) for _ in range(copies - 1)]
    xd = torch.from_numpy(x).to(dev)
    qa = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sa = torch.empty((K // 128, M, 4), dtype=torch.uint8, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = fp8.fp8_mx_workspace_bytes(M, N, K)
    ws = torch.empty(ws, dtype=torch.uint8, device=dev) if ws > 0 else None

    def step(i):
        fp8.fp8_quantize_mx(xd, q=qa, scales=sa)
        fp8.fp8_gemm_mx(qa, sa, wcopies[i % copies][0], wcopies[i % copies][1], y=y, ws=ws)

    def gemm(i):
        fp8.fp8_gemm_mx(qa, sa, wcopies[i % copies][0], wcopies[i % copies][1], y=y, ws=ws)

    grp = 10 if M <= 64 else 1
    t = timed(step, steps, warmup, graph, grp, args.prewarm)
    tg = timed(gemm, steps, warmup, graph, grp, args.prewarm)
    ms, g_ms = t["total_ms"] / t["steps"], tg["total_ms"] / tg["steps"]
    flops = 2.0 * M * N * K
    gemm_bytes = N * K + N * K // 32 + M * K + M * K // 32 + 2 * M * N
    step_bytes = 4 * M * K + N * K + N * K // 32 + 2 * M * N
    decode = M <= 64
    if decode:
        value, unit = step_bytes / (ms * 1e-3) / 1e9, "GB/s"
        ach = gemm_bytes / (g_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s", frac=round(ach / HBM_PEAK_GBS, 4),
                    per_launch=f"{gemm_bytes} algorithmic bytes (codes + exponent bytes of both operands, bf16 y)")
        kernel = "gemm_skinny_kernel (block-scaled)"
    else:
        value, unit = flops / (ms * 1e-3) / 1e12, "TFLOP/s"
        ach = flops / (g_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(ach, 1), peak=FP8_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(ach / FP8_PEAK_TFLOPS, 4), per_launch=f"{flops:.6g} FLOP")
        kernel = "gemm_mfma_kernel (block-scaled)"
    roof.update(kernel=kernel, avg_launch_us=round(g_ms * 1e3, 3), gemm_us=stats_us(tg),
                traffic=read_traffic(f"{args.workload}@mx", "skinny" if decode else "mfma",
                                     "gemm_skinny_kernel" if decode else "gemm_mfma_kernel"))
    cfg = dict(workload=args.workload, M=M, N=N, K=K, seed=args.seed, weight_copies=copies,
               step="fp8_quantize_mx + fp8_gemm_mx", scales="32-element blocks, power-of-two (E8M0)", out="bf16")
    detail = dict(timing="hip-graph replays after a pre-warm" if graph else "eager launches", prewarm_s=args.prewarm,
                  step_us=stats_us(t), step_tflops=round(flops / (ms * 1e-3) / 1e12, 2))
    cpu = None
    if want_cpu:
        import oracle
        log("[bench] timing the CPU oracle")
        wq_h = wq.cpu().numpy()
        # the exponent bytes back in [rows][K/32] order for the oracle
        sw_h = ws_.cpu().numpy().transpose(1, 0, 2).reshape(N, K // 32)
        rng = np.random.default_rng(0)

        def work(n):
            rows = rng.integers(0, M, max(1, n // 64))
            xs = x[rows]
            qa_h, sa_h = oracle.quantize_mx(xs)
            ms_ = np.repeat(np.arange(rows.size), 64)[:n]
            ns_ = rng.integers(0, N, ms_.size)
            oracle.gemm_mx_ref_sampled(qa_h, sa_h, wq_h, sw_h, ms_, ns_)
            return ms_.size

        cpu = cpu_baseline(work, lambda n: 2.0 * n * K / 1e12, "TFLOP/s",
                           lambda n: f"block-scaled quantization of sampled activation rows + {n} exact binary64 "
                                     f"block-scaled dots of K={K} against random weight rows",
                           args.cpu_seconds, probe_units=256)
    emit(value, unit, t["steps"], warmup, ms, cfg, roof, cpu, detail,
         dtype="fp8e4m3 with e8m0 block scales (fp32 accumulate, bf16 out)")


def bench_kv(args, w, dev, steps, warmup, graph, want_cpu):
    """One step = writing one layer's prefill KV into the paged FP8 cache:
    fp8_kv_channel_scales (per-channel scales of the batch) then
    fp8_kv_quantize_paged (codes into the slots the block table names).  The
    read back (fp8_kv_dequantize_paged, what attention would consume) is timed
    on its own.  Several copies of the batch are rotated so the 256 MB
    Infinity Cache cannot carry a step's input into the next step."""
    import numpy as np
    import torch
    import fp8_w8a8_quantized_quantize_amd as fp8
    import synth
    T, C, B, fmt = w["T"], w["C"], w["block"], w["fmt"]
    kvdt = args.kv_dtype or w["dtype"]
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[kvdt]
    eb = 4 if kvdt == "f32" else 2
    nb = T // B + 256
    log(f"[bench] {args.workload}: generating inputs T={T} C={C} block={B} blocks={nb} fmt={fmt} rows={kvdt}")
    kv = synth.kv_activations(T, C, seed=args.seed)
    slot = synth.kv_slot_mapping(T, B, nb, seed=args.seed)
    copies = 2 if eb == 4 else 3   # >= 400 MB of rows rotated past the Infinity Cache
    kvd = [torch.from_numpy(kv).to(dev).to(tdt)]
    kvd += [kvd[0].clone() for _ in range(copies - 1)]
    slotd = torch.from_numpy(slot).to(dev)
    cache = torch.zeros((nb * B, C), dtype=torch.uint8, device=dev)
    scales = torch.empty(C, dtype=torch.float32, device=dev)
    ws = torch.empty(fp8.fp8_kv_scales_workspace_bytes(T, C), dtype=torch.uint8, device=dev)
    out = torch.empty((T, C), dtype=tdt, device=dev)

    def step(i):
        fp8.fp8_kv_channel_scales(kvd[i % copies], fmt, scales=scales, ws=ws)
        fp8.fp8_kv_quantize_paged(kvd[i % copies], scales, slotd, cache, fmt)

    def scales_only(i):
        fp8.fp8_kv_channel_scales(kvd[i % copies], fmt, scales=scales, ws=ws)

    def quant_only(i):
        fp8.fp8_kv_quantize_paged(kvd[i % copies], scales, slotd, cache, fmt)

    def read_back(i):
        fp8.fp8_kv_dequantize_paged(cache, slotd, scales, fmt, out=out)

    log(f"[bench] warmup {warmup}, pre-warm {args.prewarm} s, timing {steps} steps")
    t = timed(step, steps, warmup, graph, 10, args.prewarm)
    t_sc = timed(scales_only, steps, warmup, graph, 10, args.prewarm)
    t_q = timed(quant_only, steps, warmup, graph, 10, args.prewarm)
    t_dq = timed(read_back, steps, warmup, graph, 10, args.prewarm)
    avg = lambda tt: tt["total_ms"] / tt["steps"]
    ms, sc_ms, q_ms, dq_ms = avg(t), avg(t_sc), avg(t_q), avg(t_dq)
    # algorithmic bytes: the batch read once, codes written once, scales and slots
    step_bytes = eb * T * C + T * C + 4 * C + 4 * T
    scale_bytes = eb * T * C + 4 * C
    quant_bytes = eb * T * C + 4 * C + 4 * T + T * C
    dq_bytes = T * C + 4 * T + 4 * C + eb * T * C
    gbs = lambda b, tm: b / (tm * 1e-3) / 1e9
    value = gbs(step_bytes, ms)
    q_ach = gbs(quant_bytes, q_ms)
    roof = dict(bound="hbm", achieved=round(q_ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(q_ach / HBM_PEAK_GBS, 4), kernel="kv_quantize_paged",
                per_launch=f"{quant_bytes} algorithmic bytes ({kvdt} kv in, slots, scales, FP8 codes out)",
                avg_launch_us=round(q_ms * 1e3, 3), traffic=read_traffic(args.workload, "kv", "kv_quantize_paged"),
                others=dict(channel_scales=dict(kernels="kv_amax_partial + kv_scale_finish",
                                                avg_us=round(sc_ms * 1e3, 3), achieved=round(gbs(scale_bytes, sc_ms), 1),
                                                frac=round(gbs(scale_bytes, sc_ms) / HBM_PEAK_GBS, 4),
                                                per_launch=f"{scale_bytes} algorithmic bytes"),
                            read_back=dict(kernel="kv_dequantize_paged", avg_us=round(dq_ms * 1e3, 3),
                                           achieved=round(gbs(dq_bytes, dq_ms), 1),
                                           frac=round(gbs(dq_bytes, dq_ms) / HBM_PEAK_GBS, 4),
                                           per_launch=f"{dq_bytes} algorithmic bytes")))
    cfg = dict(workload=args.workload, T=T, C=C, block=B, blocks=nb, fmt=fmt, rows=kvdt, seed=args.seed,
               kv_copies=copies, step="fp8_kv_channel_scales + fp8_kv_quantize_paged")
    detail = dict(timing="hip-graph replays after a pre-warm" if graph else "eager launches", prewarm_s=args.prewarm,
                  step_us=stats_us(t), step_gbs_counting_both_reads=round(gbs(step_bytes + eb * T * C, ms), 1))
    cpu = None
    if want_cpu:
        import oracle
        log("[bench] timing the CPU oracle")
        fid = oracle.E5M2 if fmt == "e5m2" else oracle.E4M3
        kv_h = kvd[0][:8192].float().cpu().numpy()   # the values the rows hold

        def work(n):
            rows = min(n, kv_h.shape[0])
            # the sample's slots, renumbered into a cache of `rows` rows (same scatter order)
            compact = np.empty(rows, dtype=np.int32)
            compact[np.argsort(slot[:rows], kind="stable")] = np.arange(rows, dtype=np.int32)
            s_h = oracle.kv_channel_scales(kv_h[:rows], fid)
            oracle.kv_quantize(kv_h[:rows], s_h, fid, compact, rows)
            return rows

        def work_reps(n):
            done = 0
            while done < n:
                done += work(min(4096, n - done))
            return done

        cpu = cpu_baseline(work_reps, lambda r: r * (eb * C + C + 4) / 1e9, "GB/s",
                           lambda r: f"channel scales + paged quantize over {r} token rows in batches of up to "
                                     f"4096 (their slots renumbered into a cache of the batch's size)",
                           args.cpu_seconds, probe_units=1024)
    emit(value, "GB/s", t["steps"], warmup, ms, cfg, roof, cpu, detail, dtype=f"{kvdt} in, {fmt} codes")


if __name__ == "__main__":
    main()
