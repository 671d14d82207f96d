#!/usr/bin/env python3
"""Benchmark of the unified-FP8 (W8A8) linear layer on one MI355X.

One step = one pass of the hot path over one batch of synthetic input:
  dense workloads: fp8_quant_gemm_fused (per-token E4M3 quantization of the
                   activations + FP8 GEMM with the s_tok*s_ch BF16 epilogue)
                   against pre-quantized weights;
  MoE workload:    per-token quantization of the token activations +
                   fp8_gemm_grouped_scaled over the expert-sorted routed rows.
Weight quantization is the offline step and is not timed.

Default workload: the Llama-3-8B FFN up-projection decode (M=8, K=4096,
N=14336), reported as algorithmic HBM GB/s.  Decode workloads rotate several
weight copies (>= 512 MB in total) so that the 256 MB Infinity Cache cannot
serve the weights across steps.

The JSON line adds
  roofline:     the dominant kernel (the GEMM) timed alone with HIP events on
                the launch stream, algorithmic bytes (or FLOPs) per launch over
                its average duration, against the MI355X peak;
  cpu_baseline: the CPU oracle timed on the host on a bounded sample of the
                same workload.
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
DEFAULT_WORKLOAD = "llama3-8b-decode-up"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
KERNEL_SOURCES = {
    "skinny": ["gemm_skinny.hip", "device_common.hpp"],
    "mfma": ["gemm_mfma.hip", "device_common.hpp"],
    "kv": ["kv_cache.hip", "device_common.hpp"],
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU-oracle sample time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches instead of one HIP-graph replay of the steps")
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
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run 5 plain device copies of 512 MiB (reference for rocprofv3 FETCH/WRITE_SIZE)")
    ap.add_argument("--profile", action="store_true",
                    help="at most 50 timed steps after the usual warm-up, no CPU baseline: for runs under "
                         "rocprofv3 (the GPU clock needs the warm-up to settle)")
    return ap.parse_args()


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


def gen_dense(w, seed):
    import synth
    x, _ = synth.activations(w["M"], w["K"], synth.workload_outliers(w), w["mult"], seed=seed)
    wt = synth.weights(w["N"], w["K"], seed=seed)
    return x, wt


def time_loop(fn, n, warmup, graph):
    """Run fn(i) warmup times, then time n calls with HIP events on the stream
    the library launches on (torch's current stream).  With graph=True the n
    calls are captured once into a HIP graph and the timed region is one
    replay, so host launch overhead is not part of the measurement (the
    kernels and their on-GPU dispatch gaps are).  Returns (total ms,
    per-step ms list or None)."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    if graph:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn(0)  # warm the capture stream
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        g.replay()  # untimed first replay
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1), None
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    evs[0].record()
    for i in range(n):
        fn(i)
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(n)]
    return evs[0].elapsed_time(evs[n]), per


def pct(v, q):
    v = sorted(v)
    return v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]


def cpu_baseline_dense(w, x, wt_q, sc, target_s):
    """The CPU oracle (per-token quantization + exact binary64 GEMM against all
    weight rows) on the step's activation rows: every row, repeated for about
    target_s seconds when a pass is short (decode); otherwise the first rows
    that take about target_s seconds (prefill)."""
    import oracle
    M, N, K = w["M"], w["N"], w["K"]
    rows = min(M, 8)
    t0 = time.perf_counter()
    qa, st = oracle.quantize_rows(x[:rows])
    oracle.gemm_ref(qa, st, wt_q, sc)
    dt = max(time.perf_counter() - t0, 1e-6)
    if rows < M:
        rows = int(min(M, max(rows, rows * target_s / dt)))
    reps = 0
    t0 = time.perf_counter()
    while True:
        qa, st = oracle.quantize_rows(x[:rows])
        oracle.gemm_ref(qa, st, wt_q, sc)
        reps += 1
        elapsed = time.perf_counter() - t0
        if rows < M or elapsed >= target_s:
            break
    flops = 2.0 * reps * rows * N * K
    bytes_ = reps * (rows * (4 * K + 2 * N) + N * K + 4 * N)
    sample = (f"{reps} pass(es) over {rows} of {M} activation rows: per-token quantization + exact binary64 "
              f"GEMM against all {N} weight rows")
    return dict(elapsed=elapsed, flops=flops, bytes=bytes_, cores=oracle.num_threads(), sample=sample)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path; run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
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
    w = synth.WORKLOADS[args.workload]
    steps, warmup = args.steps, args.warmup
    if args.profile:
        steps = min(steps, 50)
    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    graph = not args.no_graph

    if args.out == "fp8":
        if w["kind"] != "dense":
            print("--out fp8 is for the dense workloads", file=sys.stderr)
            sys.exit(2)
        return bench_fp8out(args, w, dev, steps, warmup, graph, log)
    if w["kind"] == "kv":
        return bench_kv(args, w, dev, steps, warmup, graph, log)
    if args.scales == "mx":
        if w["kind"] != "dense":
            print("--scales mx is for the dense workloads", file=sys.stderr)
            sys.exit(2)
        return bench_mx(args, w, dev, steps, warmup, graph, log)
    if w["kind"] == "dense":
        M, N, K = w["M"], w["N"], w["K"]
        log(f"[bench] {args.workload}: generating inputs M={M} N={N} K={K}")
        x, wt = gen_dense(w, args.seed)
        wq, sc = fp8.fp8_quantize_per_token(torch.from_numpy(wt).to(dev))  # offline weight conversion
        wbytes = N * K
        copies = max(1, math.ceil(ROTATE_BYTES / wbytes))
        wcopies = [wq] + [wq.clone() for _ in range(copies - 1)]
        xd = torch.from_numpy(x).to(dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        # library scratch (activation codes staged by the fused call, split-k partial sums)
        ws = torch.empty(max(1, fp8.fp8_workspace_bytes(M, N, K)), dtype=torch.uint8, device=dev)
        qa = torch.empty((M, K), dtype=torch.uint8, device=dev)
        st = torch.empty(M, dtype=torch.float32, device=dev)

        def step(i):
            fp8.fp8_quant_gemm_fused(xd, wcopies[i % copies], sc, y=y, ws=ws)

        calib = None
        if args.act != "dynamic":
            # offline calibration on the same activations, timed once on its own
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            num, den = (999, 1000) if args.act == "static" else (9999, 10000)
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
                if args.act == "static":
                    fp8.fp8_quantize_static(xd, sscale, q=qs, scales_out=ss)
                else:
                    fp8.fp8_quantize_per_token_clipped(xd, value, q=qs, scales=ss)
                fp8.fp8_gemm_scaled(qs, ss, wcopies[i % copies], sc, y=y, ws=ws)

        # the dominant kernel alone: the GEMM on pre-quantized activations
        fp8.fp8_quantize_per_token(xd, q=qa, scales=st)

        def gemm(i):
            fp8.fp8_gemm_scaled(qa, st, wcopies[i % copies], sc, y=y, ws=ws)

        log(f"[bench] {copies} weight copies; warmup {warmup}, timing {steps} steps")
        total_ms, per = time_loop(step, steps, warmup, graph)
        gemm_ms, gemm_per = time_loop(gemm, steps, warmup, graph)
        ms = total_ms / steps
        decode = M <= 64
        flops = 2.0 * M * N * K
        step_bytes = 4 * M * K + N * K + 4 * N + 2 * M * N           # fused: fp32 x in, codes W, s_ch, bf16 y out
        gemm_bytes = M * K + 4 * M + N * K + 4 * N + 2 * M * N       # GEMM kernel: codes x, s_tok, W, s_ch, y
        gemm_avg_ms = gemm_ms / steps
        kind = "skinny" if decode else "mfma"
        # The library runs the fused call as one kernel (quantization in the
        # GEMM's prologue) for M <= 16 rows whose codes fit in LDS, whose fp32
        # values fit in 16 float4 registers per lane, and N <= 8192
        # (include/fp8w8a8.h); then that kernel is the whole step and is the
        # one the roofline rates.
        one_kernel = (args.act == "dynamic" and M <= 16 and M * (K + 16) <= 64 * 1024 + 256
                      and -(-K // 256) <= (16 if M <= 8 else 8) and 0 < N <= 8192)
        gemm_only = None
        if decode:
            value, unit = step_bytes / (ms * 1e-3) / 1e9, "GB/s"
            g_ach = gemm_bytes / (gemm_avg_ms * 1e-3) / 1e9
            if one_kernel:
                achieved, rated_bytes, rated_ms = value, step_bytes, ms
                gemm_only = dict(kernel="gemm_skinny_kernel (fp8_gemm_scaled on pre-quantized codes)",
                                 avg_launch_us=round(gemm_avg_ms * 1e3, 3), achieved=round(g_ach, 1),
                                 frac=round(g_ach / HBM_PEAK_GBS, 4), per_launch=f"{gemm_bytes} algorithmic bytes")
            else:
                achieved, rated_bytes, rated_ms = g_ach, gemm_bytes, gemm_avg_ms
            roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                        frac=round(achieved / HBM_PEAK_GBS, 4))
        else:
            value, unit = flops / (ms * 1e-3) / 1e12, "TFLOP/s"
            achieved = flops / (gemm_avg_ms * 1e-3) / 1e12
            roof = dict(bound="mfma", achieved=round(achieved, 1), peak=FP8_PEAK_TFLOPS, unit="TFLOP/s",
                        frac=round(achieved / FP8_PEAK_TFLOPS, 4))
        if decode and one_kernel:
            roof["kernel"] = "gemm_skinny_fused_kernel"
            roof["per_launch"] = f"{rated_bytes} algorithmic bytes (fp32 x in, E4M3 W, scales, bf16 y out)"
            roof["avg_launch_us"] = round(rated_ms * 1e3, 3)
            roof["gemm_only"] = gemm_only
        else:
            roof["kernel"] = f"gemm_{kind}_kernel"
            roof["per_launch"] = (f"{gemm_bytes} algorithmic bytes" if decode else f"{flops:.6g} FLOP")
            roof["avg_launch_us"] = round(gemm_avg_ms * 1e3, 3)
        roof["traffic"] = read_traffic(args.workload, kind, roof["kernel"])
        cfg = dict(workload=args.workload, M=M, N=N, K=K, seed=args.seed, weight_copies=copies,
                   step=("fp8_quant_gemm_fused" if args.act == "dynamic" else
                         ("fp8_quantize_static" if args.act == "static" else "fp8_quantize_per_token_clipped")
                         + " + fp8_gemm_scaled"), act_scales=args.act, out="bf16")
        extra = dict(timing="hip-graph replay of the steps" if graph else "eager launches",
                     step_us=round(ms * 1e3, 3), step_tflops=round(flops / (ms * 1e-3) / 1e12, 2),
                     step_gbs=round(step_bytes / (ms * 1e-3) / 1e9, 1))
        if calib:
            extra["calibration"] = calib
        if per:
            extra.update(step_us_median=round(pct(per, 0.5) * 1e3, 3), step_us_p10=round(pct(per, 0.1) * 1e3, 3),
                         step_us_p90=round(pct(per, 0.9) * 1e3, 3), gemm_us_median=round(pct(gemm_per, 0.5) * 1e3, 3))
        cpu = None
        if not args.no_cpu_baseline and not args.profile:
            log("[bench] timing the CPU oracle")
            wq_h = wq.cpu().numpy()
            sc_h = sc.cpu().numpy()
            r = cpu_baseline_dense(w, x, wq_h, sc_h, args.cpu_seconds)
            cv = (r["bytes"] / r["elapsed"] / 1e9) if decode else (r["flops"] / r["elapsed"] / 1e12)
            cpu = dict(value=round(cv, 6), unit=unit, cores=r["cores"], kind="oracle", sample=r["sample"],
                       seconds=round(r["elapsed"], 2))
    else:
        T, E, k, N, K = w["T"], w["E"], w["topk"], w["N"], w["K"]
        log(f"[bench] {args.workload}: generating inputs T={T} E={E} top-{k} N={N} K={K}")
        te, rt, off = synth.routing(T, E, k, w["zipf"], seed=args.seed)
        x, _ = synth.activations(T, K, synth.workload_outliers(w), w["mult"], seed=args.seed)
        xd = torch.from_numpy(x).to(dev)
        qw = torch.empty((E, N, K), dtype=torch.uint8, device=dev)
        sc = torch.empty((E, N), dtype=torch.float32, device=dev)
        for e0 in range(0, E, 8):
            we = synth.expert_weights(E, N, K, seed=args.seed, experts=range(e0, e0 + 8)).reshape(8 * N, K)
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

        total_ms, per = time_loop(step, steps, warmup, graph)
        gemm_ms, gemm_per = time_loop(gemm, steps, warmup, graph)
        ms = total_ms / steps
        flops = 2.0 * R * N * K
        gemm_bytes = E * N * K + 4 * E * N + T * K + 4 * T + 4 * R + 4 * (E + 1) + 2 * R * N
        gemm_avg_ms = gemm_ms / steps
        value, unit = flops / (ms * 1e-3) / 1e12, "TFLOP/s"
        achieved = flops / (gemm_avg_ms * 1e-3) / 1e12
        t_roof = max(flops / (FP8_PEAK_TFLOPS * 1e12), gemm_bytes / (HBM_PEAK_GBS * 1e9))
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=FP8_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / FP8_PEAK_TFLOPS, 4), traffic=read_traffic(args.workload, "mfma", "gemm_mfma_kernel"),
                    kernel="gemm_mfma_kernel (grouped)", per_launch=f"{flops:.6g} FLOP",
                    avg_launch_us=round(gemm_avg_ms * 1e3, 3),
                    roofline_time_frac=round(t_roof / (gemm_avg_ms * 1e-3), 4),
                    achieved_gbs=round(gemm_bytes / (gemm_avg_ms * 1e-3) / 1e9, 1))
        cfg = dict(workload=args.workload, T=T, E=E, topk=k, N=N, K=K, R=R, zipf=w["zipf"], seed=args.seed,
                   step="fp8_quantize_per_token + fp8_gemm_grouped_scaled", out="bf16")
        extra = dict(timing="hip-graph replay of the steps" if graph else "eager launches", step_us=round(ms * 1e3, 3),
                     expert_rows_max=int(np.diff(off).max()), expert_rows_min=int(np.diff(off).min()))
        if per:
            extra.update(step_us_median=round(pct(per, 0.5) * 1e3, 3), step_us_p10=round(pct(per, 0.1) * 1e3, 3),
                         step_us_p90=round(pct(per, 0.9) * 1e3, 3), gemm_us_median=round(pct(gemm_per, 0.5) * 1e3, 3))
        cpu = None
        if not args.no_cpu_baseline and not args.profile:
            import oracle
            log("[bench] timing the CPU oracle")
            qw_h, sc_h = qw.cpu().numpy(), sc.cpu().numpy()
            rng = np.random.default_rng(0)
            t0 = time.perf_counter()
            qa_h, st_h = oracle.quantize_rows(x)
            n_el, elapsed = 0, 0.0
            while elapsed < args.cpu_seconds:
                rs = rng.integers(0, R, 1 << 14)
                ns = rng.integers(0, N, 1 << 14)
                oracle.grouped_ref_sampled(qa_h, st_h, rt, off, qw_h, sc_h, rs, ns)
                n_el += rs.size
                elapsed = time.perf_counter() - t0
            cpu = dict(value=round(2.0 * n_el * K / elapsed / 1e12, 6), unit="TFLOP/s", cores=oracle.num_threads(),
                       kind="oracle", seconds=round(elapsed, 2),
                       sample=f"quantize all {T} token rows + {n_el} random routed outputs (exact binary64 dots)")

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8e4m3 (fp32 accumulate, bf16 out)", "data": "synthetic (seeded; no dataset, no trained weights)",
        "config": cfg, "roofline": roof, "cpu_baseline": cpu, "detail": extra,
    }
    print(json.dumps(out), flush=True)


def bench_fp8out(args, w, dev, steps, warmup, graph, log):
    """One step = fp8_gemm_scaled_fp8out: FP8 activation codes and scales in
    (as a previous FP8-output layer leaves them), FP32 accumulation, the output
    re-quantized per token to E4M3 codes and scales."""
    import torch
    import fp8_w8a8_quantized_quantize_amd as fp8
    M, N, K = w["M"], w["N"], w["K"]
    log(f"[bench] {args.workload} (FP8 output): generating inputs M={M} N={N} K={K}")
    x, wt = gen_dense(w, args.seed)
    wq, sc = fp8.fp8_quantize_per_token(torch.from_numpy(wt).to(dev))
    copies = max(1, math.ceil(ROTATE_BYTES / (N * K)))
    wcopies = [wq] + [wq.clone() for _ in range(copies - 1)]
    qa, st = fp8.fp8_quantize_per_token(torch.from_numpy(x).to(dev))
    q_out = torch.empty((M, N), dtype=torch.uint8, device=dev)
    s_out = torch.empty(M, dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, fp8.fp8_fp8out_workspace_bytes(M, N, K)), dtype=torch.uint8, device=dev)

    def step(i):
        fp8.fp8_gemm_scaled_fp8out(qa, st, wcopies[i % copies], sc, q_out=q_out, s_out=s_out, ws=ws)

    total_ms, per = time_loop(step, steps, warmup, graph)
    ms = total_ms / steps
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
    roof.update(kernel="fp8_gemm_scaled_fp8out (GEMM with fp32 output, then the per-token output quantizer)",
                per_launch=per_launch, avg_launch_us=round(ms * 1e3, 3), traffic=None)
    cfg = dict(workload=args.workload, M=M, N=N, K=K, seed=args.seed, weight_copies=copies,
               step="fp8_gemm_scaled_fp8out", out="e4m3 codes + fp32 per-token scales")
    extra = dict(timing="hip-graph replay of the steps" if graph else "eager launches", step_us=round(ms * 1e3, 3))
    if per:
        extra.update(step_us_median=round(pct(per, 0.5) * 1e3, 3))
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8e4m3 (fp32 accumulate, e4m3 out)", "data": "synthetic (seeded; no dataset, no trained weights)",
        "config": cfg, "roofline": roof, "cpu_baseline": None, "detail": extra,
    }
    print(json.dumps(out), flush=True)


def bench_mx(args, w, dev, steps, warmup, graph, log):
    """One step = fp8_quantize_mx of the activations + fp8_gemm_mx against
    block-scaled weights (quantized once, untimed): 32-element blocks along K
    with power-of-two scales applied inside the K loop by the block-scaled
    MFMA."""
    import torch
    import fp8_w8a8_quantized_quantize_amd as fp8
    M, N, K = w["M"], w["N"], w["K"]
    log(f"[bench] {args.workload} (block scales): generating inputs M={M} N={N} K={K}")
    x, wt = gen_dense(w, args.seed)
    wq, ws_ = fp8.fp8_quantize_mx(torch.from_numpy(wt).to(dev))
    copies = max(1, math.ceil(ROTATE_BYTES / (N * K)))
    wcopies = [(wq, ws_)] + [(wq.clone(), ws_.clone()) for _ in range(copies - 1)]
    xd = torch.from_numpy(x).to(dev)
    qa = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sa = torch.empty((K // 128, M, 4), dtype=torch.uint8, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, fp8.fp8_mx_workspace_bytes(M, N, K)), dtype=torch.uint8, device=dev)

    def step(i):
        fp8.fp8_quantize_mx(xd, q=qa, scales=sa)
        fp8.fp8_gemm_mx(qa, sa, wcopies[i % copies][0], wcopies[i % copies][1], y=y, ws=ws)

    def gemm(i):
        fp8.fp8_gemm_mx(qa, sa, wcopies[i % copies][0], wcopies[i % copies][1], y=y, ws=ws)

    total_ms, per = time_loop(step, steps, warmup, graph)
    gemm_ms, _ = time_loop(gemm, steps, warmup, graph)
    ms, g_ms = total_ms / steps, gemm_ms / steps
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
    roof.update(kernel=kernel, avg_launch_us=round(g_ms * 1e3, 3),
                traffic=read_traffic(f"{args.workload}@mx", "skinny" if decode else "mfma",
                                     "gemm_skinny_kernel" if decode else "gemm_mfma_kernel"))
    cfg = dict(workload=args.workload, M=M, N=N, K=K, seed=args.seed, weight_copies=copies,
               step="fp8_quantize_mx + fp8_gemm_mx", scales="32-element blocks, power-of-two (E8M0)", out="bf16")
    extra = dict(timing="hip-graph replay of the steps" if graph else "eager launches", step_us=round(ms * 1e3, 3),
                 step_tflops=round(flops / (ms * 1e-3) / 1e12, 2))
    if per:
        extra.update(step_us_median=round(pct(per, 0.5) * 1e3, 3))
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8e4m3 with e8m0 block scales (fp32 accumulate, bf16 out)",
        "data": "synthetic (seeded; no dataset, no trained weights)",
        "config": cfg, "roofline": roof, "cpu_baseline": None, "detail": extra,
    }
    print(json.dumps(out), flush=True)


def bench_kv(args, w, dev, steps, warmup, graph, log):
    """One step = writing one layer's prefill KV into the paged FP8 cache:
    fp8_kv_channel_scales (per-channel scales of the batch) then
    fp8_kv_quantize_paged (codes into the slots the block table names).  The
    read back (fp8_kv_dequantize_paged, what attention would consume) is timed
    on its own.  Two copies of the batch are rotated so the 256 MB Infinity
    Cache cannot carry a step's input into the next step."""
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

    log(f"[bench] warmup {warmup}, timing {steps} steps")
    total_ms, per = time_loop(step, steps, warmup, graph)
    sc_ms, _ = time_loop(scales_only, steps, warmup, graph)
    q_ms, _ = time_loop(quant_only, steps, warmup, graph)
    dq_ms, _ = time_loop(read_back, steps, warmup, graph)
    ms, sc_ms, q_ms, dq_ms = total_ms / steps, sc_ms / steps, q_ms / steps, dq_ms / steps
    # algorithmic bytes: the batch read once, codes written once, scales and slots
    step_bytes = eb * T * C + T * C + 4 * C + 4 * T
    scale_bytes = eb * T * C + 4 * C
    quant_bytes = eb * T * C + 4 * C + 4 * T + T * C
    dq_bytes = T * C + 4 * T + 4 * C + eb * T * C
    gbs = lambda b, t: b / (t * 1e-3) / 1e9
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
               kv_copies=copies,
               step="fp8_kv_channel_scales + fp8_kv_quantize_paged")
    extra = dict(timing="hip-graph replay of the steps" if graph else "eager launches", step_us=round(ms * 1e3, 3),
                 step_gbs_counting_both_reads=round(gbs(step_bytes + eb * T * C, ms), 1))
    if per:
        extra.update(step_us_median=round(pct(per, 0.5) * 1e3, 3))
    cpu = None
    if not args.no_cpu_baseline and not args.profile:
        import oracle
        log("[bench] timing the CPU oracle")
        rows = min(T, 4096)
        fid = oracle.E5M2 if fmt == "e5m2" else oracle.E4M3
        kv = kvd[0][:rows].float().cpu().numpy()   # the values the rows hold
        # the sample's slots, renumbered into a cache of `rows` rows (same scatter order)
        compact = np.empty(rows, dtype=np.int32)
        compact[np.argsort(slot[:rows], kind="stable")] = np.arange(rows, dtype=np.int32)
        t0 = time.perf_counter()
        reps = 0
        while True:
            s_h = oracle.kv_channel_scales(kv[:rows], fid)
            oracle.kv_quantize(kv[:rows], s_h, fid, compact, rows)
            reps += 1
            elapsed = time.perf_counter() - t0
            if elapsed >= args.cpu_seconds:
                break
        b = reps * (eb * rows * C + rows * C + 4 * C + 4 * rows)
        cpu = dict(value=round(b / elapsed / 1e9, 6), unit="GB/s", cores=oracle.num_threads(), kind="oracle",
                   seconds=round(elapsed, 2),
                   sample=f"{reps} pass(es) of channel scales + paged quantize over the first {rows} of {T} tokens "
                          f"(their slots renumbered into a {rows}-row cache)")
    res = {
        "metric": METRIC, "value": round(value, 3), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"{kvdt} in, {fmt} codes", "data": "synthetic (seeded; no dataset, no trained weights)",
        "config": cfg, "roofline": roof, "cpu_baseline": cpu, "detail": extra,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
