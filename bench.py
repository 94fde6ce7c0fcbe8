"""Benchmark of the MI355X sparse-MoE layer (one GPU).

Default workload (the headline metric): one Qwen3.8-Flash-Next-shaped MoE
layer decoding a 4-token verify window -- hidden 2560, 512 experts, top-10,
expert FF 640, q2b32 experts, Zipf(1.1) router bias.  A step is one
moe_forward call through the whole hot path (router, top-k, weights, counting
sort, dequant + gate/up + SwiGLU, down + weighted combine) on one layer and
one window of 4 tokens.  Steps cycle over 48 resident layers of that shape
(every layer has its own router, Zipf permutation and 512 experts) and 16
distinct input windows, so that successive steps read different expert
weights and the 256 MB Infinity Cache does not serve repeated reads.

Other workloads (--workload): C3 (the 48-layer chain with residual adds at
window 1/4/8) and C4 (the 43-layer DeepSeek-shaped chain, 256+1 experts,
q4b32); a step is then one full chain pass, with the per-token RMS pre-norm
of every layer input (without it the stream of random experts overflows).  C5 is the DeepSeek-shaped
prefill chunk (4096 tokens x hidden 4096, 256+1 experts, top-6, FF 2048,
q4b32, Zipf-skewed routing): a step is one moe_forward of the whole chunk,
and the roofline is that of the gate/up grouped GEMM on bf16 MFMA.

C2_q2b64 and C3_q2b64 are C2 and C3 with q2b64 experts (one fp16 scale per
64 2-bit codes: 2.25 bits per weight, 1,382,400 bytes per expert).

Single decode layers (C2): the timed steps replay a HIP graph captured here, of
one input cycle when the step count is a multiple of it and of exactly the
timed steps otherwise; the eager time of the same steps is reported as
ms_per_step_eager, and the spread (ms_per_step_p10_p50_p90) comes from further
replays, each timed on its own.  Chains (C3, C4): each step is one
moe_forward call, which replays the library's own HIP graph of the chain; the
spread comes from every step between events of its own, as for the prefill
chunk.

Printed: one JSON line with tokens/s, HBM GB/s on expert bytes, the roofline
of the dominant kernel (gate/up, measured with HIP events recorded around
each launch on the launch stream) and the fp64 oracle's throughput on the
host cores as a CPU baseline.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "MoE-layer tokens/s + achieved HBM GB/s on expert weights (decode, window 4)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=960)
    p.add_argument("--warmup", type=int, default=96)
    p.add_argument("--workload", default="C2", choices=["C2", "C3", "C4", "C5", "C2_q2b64", "C3_q2b64"])
    p.add_argument("--T", type=int, default=4, help="tokens per window")
    p.add_argument("--layers", type=int, default=0, help="resident layers (default: 48 for C2/C3, 43 for C4)")
    p.add_argument("--windows", type=int, default=16)
    p.add_argument("--seed", type=int, default=1)
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle CPU-baseline leg")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                   help="after the timed work, copy an MB-sized device buffer 8 times (a known-size stream for "
                        "calibrating rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    p.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "MB"),
                   help="no GPU: turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) of a run made with "
                        "--copy-calibration MB into profiles/gateup_traffic.json (C2: the decode gate/up kernel) "
                        "or profiles/gemm1_traffic.json (--workload C5: the gate/up grouped GEMM)")
    return p.parse_args()


def main():
    args = parse()
    if args.summarize_pmc:
        return summarize_pmc(args)
    if args.gpus != 1:
        print(json.dumps({"error": "the layer runs on one GPU: --gpus above 1 is not supported (no collectives, no sharding)"}))
        sys.exit(2)
    if args.workload == "C5":
        return run_prefill(args)
    import torch

    import moe_inputs as mi
    from moe_inputs.configs import C2, C2_Q2B64, C3, C3_Q2B64, C4
    from quantized_expert_ffn_softmax_amd import MoEContext

    cfg = {"C2": C2, "C3": C3, "C4": C4, "C2_q2b64": C2_Q2B64, "C3_q2b64": C3_Q2B64}[args.workload]
    L = args.layers or (43 if args.workload == "C4" else 48)
    T = args.T
    chain = args.workload in ("C3", "C4", "C3_q2b64")
    torch.cuda.init()
    dev = torch.device("cuda:0")

    log(f"[bench] workload {args.workload}: H={cfg.H} F={cfg.F} E={cfg.E}+{cfg.S} k={cfg.k} layers={L} T={T}")
    t0 = time.time()
    ctx = MoEContext(cfg.H, cfg.F, cfg.E, cfg.S, cfg.k, L, cfg.fmt, 8)
    for layer in range(L):
        W, b, ex = mi.layer_inputs(cfg, args.seed, layer)
        ctx.load(layer, router_w=W, router_bias=b, experts=ex)
        del ex
        if layer % 8 == 7 or layer == L - 1:
            log(f"[bench] loaded {layer + 1}/{L} layers ({time.time() - t0:.0f}s)")
    xs = [torch.from_numpy(mi.gen_x(args.seed, w, T, cfg.H).view(np.int16)).view(torch.bfloat16).to(dev)
          for w in range(args.windows)]
    y = torch.empty_like(xs[0])

    def step(i, profile=False, trace_ids=None):
        if chain:
            return ctx.forward(xs[i % len(xs)], 0, L, residual=True, y=y, profile=profile, prenorm=True)
        layer = i % L
        from quantized_expert_ffn_softmax_amd import moe_forward, MOE_FWD_PROFILE
        moe_forward(ctx.handle, xs[i % len(xs)], y, T, layer, 1, MOE_FWD_PROFILE if profile else 0,
                    None, trace_ids, None)

    # ---- warmup, then the same steps eagerly (reported beside) and as HIP graph replays (the timed value).
    #      Decode steps are launch-bound, so the timed steps replay a HIP graph: of one full input cycle
    #      (every resident layer and window once) when the step count is a multiple of it, else of exactly
    #      the timed steps.  The spread after the timed region comes from further replays of the same graph.
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    cycle = len(xs) if chain else int(np.lcm(L, len(xs)))
    gsteps = cycle if args.steps % cycle == 0 else args.steps
    replays = args.steps // gsteps

    def timed_eager():
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for i in range(args.steps):
            step(i)
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1)

    if chain:
        # a chain step is one moe_forward of every layer: the library replays its own HIP graph of the
        # whole chain (captured on the first call with these buffers), nothing is captured here
        for i in range(len(xs)):
            step(i)
        torch.cuda.synchronize()
        ms_total = timed_eager()
        ms_eager = ms_total
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        evs[0].record()
        for i in range(args.steps):
            step(i)
            evs[i + 1].record()
        torch.cuda.synchronize()
        spread = np.percentile([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)], [10, 50, 90])
        launch_desc = f"one moe_forward per step, replaying the library's HIP graph of the {L}-layer chain"
    else:
        ms_eager = timed_eager()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            graph.capture_begin()
            for i in range(gsteps):
                step(i)
            graph.capture_end()
        torch.cuda.current_stream().wait_stream(side)
        graph.replay()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(replays):
            graph.replay()
        ev1.record()
        torch.cuda.synchronize()
        ms_total = ev0.elapsed_time(ev1)
        # spread: further replays of the same graph, each timed on its own, per step
        n_rep = max(5, replays)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_rep + 1)]
        evs[0].record()
        for r in range(n_rep):
            graph.replay()
            evs[r + 1].record()
        torch.cuda.synchronize()
        spread = np.percentile([evs[r].elapsed_time(evs[r + 1]) / gsteps for r in range(n_rep)], [10, 50, 90])
        launch_desc = f"{replays} replay(s) of a HIP graph of {gsteps} steps (captured by the caller)"
    ms_per_step = ms_total / args.steps
    tokens_per_s = T * args.steps / (ms_total / 1e3)
    log(f"[bench] timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step ({launch_desc}), "
        f"{ms_eager / args.steps * 1e3:.1f} us/step eager")

    # ---- routing of every (layer, window) pair used: distinct experts -> algorithmic bytes
    n_pairs = L if chain else int(np.lcm(L, len(xs)))
    n_steps_acct = len(xs) if chain else n_pairs
    U = {}
    for i in range(n_steps_acct):
        if chain:
            _, _, tid, _ = ctx.forward(xs[i % len(xs)], 0, L, residual=True, trace=True, prenorm=True)
            for layer in range(L):
                U[(layer, i % len(xs))] = len(np.unique(tid[layer].cpu().numpy()))
        else:
            layer = i % L
            ids, _, _, _ = ctx.route(layer, xs[i % len(xs)])
            U[(layer, i % len(xs))] = len(np.unique(ids.cpu().numpy()))
    expert_bytes = cfg.expert_bytes
    gu_bytes = 2 * expert_bytes // 3  # G and U of one expert
    dn_bytes = expert_bytes // 3

    def step_bytes(i):
        w = i % len(xs)
        if chain:
            return sum((U[(l, w)] + cfg.S) * expert_bytes + cfg.router_bytes for l in range(L))
        layer = i % L
        return (U[(layer, w)] + cfg.S) * expert_bytes + cfg.router_bytes

    total_bytes = sum(step_bytes(i) for i in range(args.steps))
    hbm_gbps = total_bytes / (ms_total / 1e3) / 1e9

    # ---- profiled pass: a HIP event pair bound to each kernel dispatch (hipExtLaunchKernelGGL), on the
    #      stream the kernels run on
    nprof = min(args.steps, 4 * n_pairs if not chain else len(xs))
    ctx.profile_read()
    for i in range(nprof):
        step(i, profile=True)
    torch.cuda.synchronize()
    recs = ctx.profile_read()
    per_kernel = {}
    for name, layer, ms in recs:
        per_kernel.setdefault(name, []).append(ms)
    # algorithmic bytes of the gate/up launches of the profiled steps, in launch order
    gu_launch_bytes, dn_launch_bytes = [], []
    for i in range(nprof):
        w = i % len(xs)
        layers = range(L) if chain else [i % L]
        for layer in layers:
            gu_launch_bytes.append((U[(layer, w)] + cfg.S) * gu_bytes)
            dn_launch_bytes.append((U[(layer, w)] + cfg.S) * dn_bytes)
    gu_ms = per_kernel.get("gateup", [])
    dn_ms = per_kernel.get("down", [])
    assert len(gu_ms) == len(gu_launch_bytes), (len(gu_ms), len(gu_launch_bytes))
    gu_avg_us = 1e3 * float(np.mean(gu_ms))
    gu_achieved = float(np.sum(gu_launch_bytes)) / (float(np.sum(gu_ms)) / 1e3) / 1e9
    dn_achieved = float(np.sum(dn_launch_bytes)) / (float(np.sum(dn_ms)) / 1e3) / 1e9
    kernels_us = {k: round(1e3 * float(np.mean(v)), 2) for k, v in per_kernel.items()}
    log(f"[bench] per-kernel mean us (events): {kernels_us}")
    log(f"[bench] gate/up {gu_achieved:.0f} GB/s, down {dn_achieved:.0f} GB/s, layer {hbm_gbps:.0f} GB/s")

    if args.copy_calibration:
        calibration_copy(torch, args.copy_calibration, dev)

    traffic = None
    tpath = os.path.join(ROOT, "profiles", "gateup_traffic.json")
    if os.path.exists(tpath) and not chain:
        with open(tpath) as f:
            tr = json.load(f)
        if tr.get("workload") == args.workload and tr.get("kernel_sha") == kernel_sha():
            traffic = tr.get("bytes_per_launch")

    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_eager": round(ms_eager / args.steps, 5),
        "ms_per_step_p10_p50_p90": [round(float(v), 5) for v in spread],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"{args.workload}: " + ("one Qwen-shaped MoE decode layer per step, cycling "
                                                  f"{L} resident layers and {len(xs)} windows" if not chain else
                                                  f"{L}-layer MoE-only decode chain with residual per step")),
            "T": T, "H": cfg.H, "F": cfg.F, "E": cfg.E, "S": cfg.S, "k": cfg.k, "layers_resident": L,
            "quant": {1: "q4b32", 2: "q2b32", 3: "q2b64"}[cfg.fmt], "seed": args.seed,
            "launch": launch_desc,
        },
        "hbm_GBps": round(hbm_gbps, 1),
        "hbm_frac": round(hbm_gbps / HBM_PEAK_GBPS, 4),
        "kernels_us": kernels_us,
        "roofline": {
            "kernel": "k_gateup_decode",
            "bound": "hbm",
            "achieved": round(gu_achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(gu_achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "avg_launch_us": round(gu_avg_us, 3),
            "bytes_per_launch": round(float(np.mean(gu_launch_bytes)), 1),
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, args, L, chain, T)
    ctx.close()
    print(json.dumps(result), flush=True)


def run_prefill(args):
    """C5: one 4096-token prefill chunk through one resident layer per step."""
    import torch

    import moe_inputs as mi
    from moe_inputs.configs import C5
    from quantized_expert_ffn_softmax_amd import MoEContext

    cfg = C5
    T = cfg.T[0]
    # the GEMMs' clock settles over the first dozen chunks after the upload
    # (1.5 ms falling to 1.1 ms per gate/up launch), so the default warmup covers them
    steps = args.steps if args.steps != 960 else 40
    warmup = args.warmup if args.warmup != 96 else 20
    torch.cuda.init()
    dev = torch.device("cuda:0")
    log(f"[bench] workload C5: T={T} H={cfg.H} F={cfg.F} E={cfg.E}+{cfg.S} k={cfg.k}")
    ctx = MoEContext(cfg.H, cfg.F, cfg.E, cfg.S, cfg.k, 1, cfg.fmt, T)
    W, b, ex = mi.layer_inputs(cfg, args.seed, 0)
    ctx.load(0, router_w=W, router_bias=b, experts=ex)
    del ex
    x = torch.from_numpy(mi.gen_x(args.seed, 0, T, cfg.H).view(np.int16)).view(torch.bfloat16).to(dev)
    y = torch.empty_like(x)
    log("[bench] loaded")
    for _ in range(warmup):
        ctx.forward(x, y=y)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        ctx.forward(x, y=y)
    ev1.record()
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / steps
    log(f"[bench] timed {steps} steps: {ms_per_step:.3f} ms/step")
    # spread: every step between events of its own (after the timed region)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        ctx.forward(x, y=y)
        evs[i + 1].record()
    torch.cuda.synchronize()
    spread = np.percentile([evs[i].elapsed_time(evs[i + 1]) for i in range(steps)], [10, 50, 90])
    # profiled pass: HIP event pairs bound to each dispatch, on the launch stream
    ctx.profile_read()
    for _ in range(steps):
        ctx.forward(x, y=y, profile=True)
    torch.cuda.synchronize()
    per_kernel = {}
    for name, _, ms in ctx.profile_read():
        per_kernel.setdefault(name, []).append(ms)
    n_sort = 3  # histogram, scan, scatter launches per step
    kernels_us = {k: round(1e3 * float(np.mean(v)) * (n_sort if k == "pf_sort" else 1), 2)
                  for k, v in per_kernel.items()}
    log(f"[bench] per-kernel mean us (events): {kernels_us}")
    rows = T * cfg.k + cfg.S * T
    gemm1_flops = 2.0 * rows * cfg.H * 2 * cfg.F
    gemm2_flops = 2.0 * rows * cfg.F * cfg.H
    g1_s = float(np.mean(per_kernel["pf_gemm1"])) / 1e3
    g2_s = float(np.mean(per_kernel["pf_gemm2"])) / 1e3
    g1_tflops = gemm1_flops / g1_s / 1e12
    g2_tflops = gemm2_flops / g2_s / 1e12
    layer_tflops = (gemm1_flops + gemm2_flops + 2.0 * T * cfg.E * cfg.H) / (ms_per_step / 1e3) / 1e12
    weight_bytes = (cfg.E + cfg.S) * cfg.expert_bytes
    log(f"[bench] gemm1 {g1_tflops:.0f} TFLOP/s, gemm2 {g2_tflops:.0f} TFLOP/s, layer {layer_tflops:.0f} TFLOP/s")
    if args.copy_calibration:
        calibration_copy(torch, args.copy_calibration, dev)
    # HBM bytes per gate/up GEMM launch from the committed counter summary, if
    # it was taken on the current prefill source
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "gemm1_traffic.json")
    if os.path.exists(tpath):
        with open(tpath) as f:
            tr = json.load(f)
        if tr.get("workload") == "C5" and tr.get("kernel_sha") == kernel_sha("moe_prefill.hip"):
            traffic = tr.get("bytes_per_launch")
    result = {
        "metric": "MoE-layer tokens/s (prefill chunk) + MFMA TFLOP/s of the grouped GEMMs",
        "value": round(T * steps / (ms_total / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_p10_p50_p90": [round(float(v), 4) for v in spread],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "C5: one DeepSeek-shaped 4096-token prefill chunk through one layer per step",
                   "T": T, "H": cfg.H, "F": cfg.F, "E": cfg.E, "S": cfg.S, "k": cfg.k, "quant": "q4b32",
                   "zipf_s": cfg.bias_param, "seed": args.seed},
        "layer_TFLOPs": round(layer_tflops, 1),
        "weight_GBps": round(weight_bytes / (ms_per_step / 1e3) / 1e9, 1),
        "kernels_us": kernels_us,
        "gemm2_TFLOPs": round(g2_tflops, 1),
        "roofline": {
            "kernel": "k_pf_gemm<q4,gate/up>",
            "bound": "mfma",
            "achieved": round(g1_tflops, 1),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(g1_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "avg_launch_us": round(g1_s * 1e6, 2),
            "flops_per_launch": gemm1_flops,
        },
    }
    if not args.no_cpu_baseline:
        import oracle
        W, b, ex = mi.layer_inputs(cfg, args.seed, 0)
        xs = mi.gen_x(args.seed, 0, T, cfg.H)
        n = 0
        t1 = time.perf_counter()
        while time.perf_counter() - t1 < args.cpu_seconds and n < T:
            oracle.moe_layer(np.ascontiguousarray(xs[n:n + 8]), cfg.H, cfg.F, cfg.E, cfg.S, cfg.k, cfg.fmt, W, b, ex,
                             cfg.expert_bytes)
            n += 8
        dt = time.perf_counter() - t1
        result["cpu_baseline"] = {"value": round(n / dt, 3), "unit": "tokens/s", "cores": oracle.num_threads(),
                                  "kind": "oracle", "sample": f"first {n} tokens of the chunk, 8 per oracle call",
                                  "seconds": round(dt, 2), **host_cpu()}
    ctx.close()
    print(json.dumps(result), flush=True)


def calibration_copy(torch, mb, dev):
    """8 device copies of an MB-sized buffer: a stream of known size for the counters."""
    src = torch.empty(mb << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(8):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def summarize_pmc(args):
    """HBM traffic of the dominant kernel from two counter runs of the same command.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are each scaled by what the
    same counter reads for the calibration copy (the 8 largest copy dispatches,
    MB read and MB written each).  C2: the decode gate/up kernel; C5: the
    gate/up grouped GEMM."""
    import csv
    fetch_csv, write_csv, mb = args.summarize_pmc
    calib_kib = int(mb) * 1024
    prefill = args.workload == "C5"
    pattern = "k_pf_gemm<1, 1>" if prefill else "k_gateup_decode"

    def load(path, counter):
        per = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                per.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
        gu = [v for k, vs in per.items() if pattern in k for v in vs]
        cp = sorted((v for k, vs in per.items() if "copyBuffer" in k for v in vs), reverse=True)[:8]
        if not gu or len(cp) < 8:
            raise SystemExit(f"{path}: {len(gu)} {pattern} and {len(cp)} calibration dispatches found")
        return float(np.mean(gu)), float(np.mean(cp)), len(gu)

    f_gu, f_cp, n_f = load(fetch_csv, "FETCH_SIZE")
    w_gu, w_cp, n_w = load(write_csv, "WRITE_SIZE")
    kf, kw = calib_kib / f_cp, calib_kib / w_cp
    out = {
        "workload": "C5" if prefill else "C2",
        "kernel": pattern,
        "kernel_sha": kernel_sha("moe_prefill.hip" if prefill else "moe_kernels.hip"),
        "fetch_kib_per_dispatch": round(f_gu, 1), "write_kib_per_dispatch": round(w_gu, 1),
        "dispatches": [n_f, n_w],
        "calibration_copy_MiB": int(mb),
        "calibration_fetch_kib": round(f_cp, 1), "calibration_write_kib": round(w_cp, 1),
        "scale_fetch": round(kf, 4), "scale_write": round(kw, 4),
        "bytes_per_launch": round((f_gu * kf + w_gu * kw) * 1024, 1),
    }
    path = os.path.join(ROOT, "profiles", "gemm1_traffic.json" if prefill else "gateup_traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def kernel_sha(source="moe_kernels.hip"):
    """Hash of the code a kernel is built from: the source and the two device headers it includes, with
    comments, blank lines and trailing spaces removed, so that a comment edit keeps counters valid while
    any change to the code drops them."""
    import hashlib
    import re
    h = hashlib.sha256()
    for name in (source, "moe_device.h", "moe_internal.h"):
        with open(os.path.join(ROOT, "quantized_expert_ffn_softmax_amd", "csrc", name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())
        h.update(name.encode() + b"\0" + code.encode() + b"\0")
    return h.hexdigest()[:16]


def host_cpu():
    """The host the oracle ran on: CPU model, logical CPUs visible to the process, and the physical cores
    among them (distinct (physical id, core id) pairs of /proc/cpuinfo)."""
    model = ""
    cores = set()
    visible = os.sched_getaffinity(0)
    try:
        with open("/proc/cpuinfo") as f:
            proc = phys = None
            for line in f:
                key, _, val = line.partition(":")
                key, val = key.strip(), val.strip()
                if key == "processor":
                    proc, phys = int(val), None
                elif key == "model name" and not model:
                    model = val
                elif key == "physical id":
                    phys = val
                elif key == "core id" and proc in visible:
                    cores.add((phys, val))
    except OSError:
        pass
    return {"cpu_model": model, "nproc": len(visible), "physical_cores": len(cores) or None}


def _time_layer_calls(cfg, W, b, ex, xs, budget_s, max_calls):
    """Oracle layer calls on pre-generated windows (input generation outside the timed calls)."""
    import oracle
    calls = 0
    t = 0.0
    while t < budget_s and calls < max_calls:
        x = xs[calls % len(xs)]
        t1 = time.perf_counter()
        oracle.moe_layer(x, cfg.H, cfg.F, cfg.E, cfg.S, cfg.k, cfg.fmt, W, b, ex, cfg.expert_bytes)
        t += time.perf_counter() - t1
        calls += 1
    return calls, t


def cpu_baseline(cfg, args, L, chain, T):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload; single-layer workloads are
    also timed on one thread (and the tiny 4-token layer beside them)."""
    import moe_inputs as mi
    import oracle
    from moe_inputs.configs import C1
    threads = oracle.num_threads()
    extra = {}
    if not chain:
        W, b, ex = mi.layer_inputs(cfg, args.seed, 0)
        xs = [mi.gen_x(args.seed, w, T, cfg.H) for w in range(args.windows)]
        calls, dt = _time_layer_calls(cfg, W, b, ex, xs, args.cpu_seconds, 256)
        n_tokens = T * calls
        sample = f"{calls} calls of layer 0 on {T}-token windows (inputs generated before timing)"
        # one thread: the same layer, and the tiny layer (hidden 256, 16 experts, top-2, 4 tokens)
        oracle.set_num_threads(1)
        try:
            c1, d1 = _time_layer_calls(cfg, W, b, ex, xs, min(4.0, args.cpu_seconds / 3), 64)
            W1, b1, ex1 = mi.layer_inputs(C1, 1, 0)
            x1 = [mi.gen_x(1, w, 4, C1.H) for w in range(4)]
            cc1, dd1 = _time_layer_calls(C1, W1, b1, ex1, x1, 1.0, 4096)
        finally:
            oracle.set_num_threads(threads)
        extra = {"single_thread": {"value": round(T * c1 / d1, 3), "unit": "tokens/s", "calls": c1,
                                   "seconds": round(d1, 2)},
                 "tiny_layer_C1": {"tokens_per_s_all_threads": None, "tokens_per_s_single_thread":
                                   round(4 * cc1 / dd1, 1), "calls": cc1}}
        cA, dA = _time_layer_calls(C1, W1, b1, ex1, x1, 1.0, 4096)
        extra["tiny_layer_C1"]["tokens_per_s_all_threads"] = round(4 * cA / dA, 1)
    else:
        # a chain step needs every layer; time the layers one by one and extrapolate nothing:
        # the sample is the first layers of one chain step
        x = mi.gen_x(args.seed, 0, T, cfg.H)
        dt = 0.0
        calls = 0
        for layer in range(L):
            W, b, ex = mi.layer_inputs(cfg, args.seed, layer)
            t1 = time.perf_counter()
            y, *_ = oracle.moe_layer(oracle.rmsnorm_bf16(x), cfg.H, cfg.F, cfg.E, cfg.S, cfg.k, cfg.fmt, W, b, ex,
                                     cfg.expert_bytes)
            x = oracle.residual_bf16(x, y)
            dt += time.perf_counter() - t1
            calls += 1
            if dt > args.cpu_seconds:
                break
        n_tokens = T * calls / L  # fraction of one chain step
        sample = f"first {calls} of {L} layers of one chain step, T={T} (input generation excluded)"
    return {"value": round(n_tokens / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": sample, "seconds": round(dt, 2), **host_cpu(), **extra}


if __name__ == "__main__":
    main()
