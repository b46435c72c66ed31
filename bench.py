#!/usr/bin/env python3
"""Benchmark of the block-scaled FP8 GEMM path on one MI355X.

Default workload: the dense FP8 NT GEMM sweep m in {64, 128, 4096} x (n, k) in
{(4096, 7168), (7168, 2048), (24576, 1536), (7168, 16384)}, 1x128 LHS and
128x128 RHS FP32 block scales, BF16 output.  One step is one pass of the whole
hot path over every shape: the per-token-group cast of the fp32 activations
(x -> E4M3 codes + scales) followed by the GEMM.  Weights are quantised once,
before timing, by the 128x128 block cast.  Inputs are seeded synthetic
N(0, 1) data, resident in HBM before the timed region; every shape keeps
enough rotated copies of its buffers that at least 1 GiB is touched between
two uses of the same copy (4x the 256 MB Infinity Cache).

Prints one JSON line.  `value` is the sweep's total GEMM FLOP divided by the
measured step time (cast included; the steps are bracketed by two events
only).  Each timed step is a replay of a HIP graph holding that step's
launches (one graph per rotation index), so the kernels run back to back;
the same steps launched one call at a time from Python are timed as well
(`ms_per_step_host_launched`).  Per-kernel durations come from a second
phase that captures many launches of one kernel into a HIP graph and times
its replays between two events on the same stream.  `roofline` describes
the kernel that takes the most time: algorithmic FLOP (or bytes) per launch
divided by its mean launch duration.  `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 GEMM TFLOPS (large M) and HBM GB/s (M<=256) at 1 MI355X, % of roofline"
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
RIDGE = PEAK_FP8_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # FLOP per byte
ROTATE_BYTES = 1 << 30

SWEEP_NK = [(4096, 7168), (7168, 2048), (24576, 1536), (7168, 16384)]
WORKLOADS = {
    "sweep": [(m, n, k) for m in (64, 128, 4096) for (n, k) in SWEEP_NK],
    "cfg0": [(64, 2112, 7168)],
    "large": [(8192, 8192, 8192), (16384, 7168, 16384)],
}
DESCRIPTION = {
    "sweep": ("dense FP8 E4M3 NT GEMM sweep m in {64,128,4096} x (n,k) in {(4096,7168),(7168,2048),"
              "(24576,1536),(7168,16384)}; 1x128 LHS / 128x128 RHS FP32 block scales; BF16 out; "
              "step = per-token-group cast of fp32 activations + GEMM for every shape"),
    "cfg0": "dense FP8 E4M3 NT GEMM m=64 n=2112 k=7168; step = activation cast + GEMM",
    "large": ("dense FP8 E4M3 NT GEMM m=n=k=8192 and m=16384 n=7168 k=16384, 1% x50 outliers; "
              "step = activation cast + GEMM"),
}


def algorithmic(m, n, k):
    """FLOP and HBM bytes the GEMM must move: A, B, both scale tensors, the
    BF16 output (padding, LDS traffic and split-K scratch not counted)."""
    kg, nb = math.ceil(k / 128), math.ceil(n / 128)
    flop = 2.0 * m * n * k
    nbytes = m * k + n * k + m * kg * 4 + nb * kg * 4 + m * n * 2
    return flop, nbytes


def cast_bytes(m, k):
    kg = math.ceil(k / 128)
    return m * k * 4 + m * k + m * kg * 4


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="sweep", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target duration of the oracle sample")
    ap.add_argument("--shape", action="append", default=[],
                    help="m,n,k to time instead of the workload's shapes (repeatable)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="run only a plain device copy of this many bytes (counter calibration)")
    ap.add_argument("--digest", action="store_true", help="print the GEMM kernel source digest and exit")
    ap.add_argument("--no-jit", action="store_true", help="skip the runtime-specialised kernels' timings")
    ap.add_argument("--no-extra", action="store_true", help="skip the MoE layout and E5M2 timings")
    ap.add_argument("--no-graph", action="store_true",
                    help="time host-launched steps only (no HIP graph replay of the step)")
    ap.add_argument("--no-grouped", action="store_true",
                    help="skip the grouped-GEMM measurements (MoE prefill and decode configurations)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other dense workloads (m=64 n=2112 k=7168; the large outlier shapes)")
    args = ap.parse_args()
    if args.digest:
        print(kernel_source_digest())
        return
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              f"(across GPUs the GEMM shards by N, by M or by expert, with no exchange inside it)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from fp8_block_scaled_04_amd import binding, synth

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    torch.cuda.set_device(0)
    if args.copy_bytes:
        copy_calibration(args.copy_bytes, args.steps)
        return
    binding.lib()
    shapes = WORKLOADS[args.workload]
    if args.shape:
        shapes = [tuple(int(v) for v in sh.split(",")) for sh in args.shape]
        DESCRIPTION[args.workload] = "custom shapes (not the default workload); step = activation cast + GEMM"
    outliers = args.workload == "large"
    stream = torch.cuda.current_stream()

    # ---- inputs: generate, upload, quantise weights, rotate ----------------
    t0 = time.time()
    host, cases = build_cases(shapes, outliers)
    print(f"[bench] inputs ready in {time.time() - t0:.1f}s ({torch.cuda.memory_allocated() / 2**30:.1f} GiB "
          f"on the device)", file=sys.stderr, flush=True)

    def cast(c, b, st=stream):
        binding.fp8_cast_per_token_group(b["x"], b["q"], b["s"], stream=st)

    def gemm(c, b, st=stream):
        binding.fp8_gemm_nt(b["q"], b["s"], b["qb"], b["sb"], b["out"], workspace=c["ws"], stream=st)

    def run_step(step, st=stream):
        for c in cases:
            b = c["sets"][step % len(c["sets"])]
            cast(c, b, st)
            gemm(c, b, st)

    for s in range(args.warmup):
        run_step(s)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    def timed_steps(launch):
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        start.record(stream)
        for s in range(args.steps):
            launch(args.warmup + s)
        stop.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(stop), time.perf_counter() - wall0

    # ---- the timed region: K whole steps, bracketed by two events ----------
    # Each step is replayed from a HIP graph (one per rotation index; every
    # library call is graph-capturable), so the kernels of a step run back to
    # back: launched one by one from Python, the host's per-call cost is
    # longer than the GPU time of the small shapes.  The host-launched step
    # is timed as well and reported beside it.
    graphs = {}
    if not args.no_graph:
        for s in range(args.warmup, args.warmup + args.steps):
            key = s % max(len(c["sets"]) for c in cases)   # the step's rotation index
            if key in graphs:
                continue
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run_step(s, None)     # None: the capture stream
            graphs[key] = g
        for g in graphs.values():
            g.replay()
        torch.cuda.synchronize()
    nrot = max(len(c["sets"]) for c in cases)
    host_ms, _ = timed_steps(run_step)
    if graphs:
        total_ms, wall = timed_steps(lambda s: graphs[s % nrot].replay())
    else:
        total_ms, wall = host_ms, None
    ms_per_step = total_ms / args.steps
    print(f"[bench] timed {args.steps} steps: {total_ms:.2f} ms on the GPU clock "
          f"({'graph replays' if graphs else 'host launches'}); host-launched steps {host_ms:.2f} ms",
          file=sys.stderr, flush=True)

    # ---- per-kernel launch durations -------------------------------------
    total_flop = sum(c["flop"] for c in cases)
    by_shape = [time_gemm_case(torch, stream, c) for c in cases]
    dom = max(cases, key=lambda c: c["gemm_ms"])
    dom_bound = "mfma" if dom["flop"] / dom["bytes"] >= RIDGE else "hbm"
    # mean launch duration (HIP events on the launch stream), as rocprofv3 averages
    if dom_bound == "mfma":
        achieved = dom["flop"] / (dom["gemm_mean_ms"] * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=PEAK_FP8_TFLOPS, unit="TFLOP/s")
    else:
        achieved = dom["bytes"] / (dom["gemm_mean_ms"] * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBS, unit="GB/s")
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(dom["m"], dom["n"], dom["k"])
    roof["kernel"] = f"fp8_gemm_nt m={dom['m']} n={dom['n']} k={dom['k']}"
    roof["per_launch"] = (f"{dom['flop']:.4g} FLOP (2*m*n*k)" if dom_bound == "mfma"
                          else f"{dom['bytes']:.4g} B (A + B + scales + bf16 out)")
    roof["mean_launch_us"] = round(dom["gemm_mean_ms"] * 1e3, 2)

    small = [c for c in cases if c["m"] <= 256]
    large = [c for c in cases if c["m"] > 256]
    summary = {}
    if small:
        summary["small_m_gemm_gbs"] = round(sum(c["bytes"] for c in small) /
                                            (sum(c["gemm_ms"] for c in small) * 1e-3) / 1e9, 1)
    if large:
        summary["large_m_gemm_tflops"] = round(sum(c["flop"] for c in large) /
                                               (sum(c["gemm_ms"] for c in large) * 1e-3) / 1e12, 1)

    result = {
        "metric": METRIC,
        "value": round(total_flop / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_host_launched": round(host_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": DESCRIPTION[args.workload], "shapes": [list(s) for s in shapes],
                   "seed": 0, "rotated_sets": {f"{c['m']}x{c['n']}x{c['k']}": len(c["sets"]) for c in cases}},
        "roofline": roof,
        "summary": summary,
        "by_shape": by_shape,
    }

    if not args.no_jit:
        result["jit"] = jit_measurements(torch, stream, cases)
    sweep_shapes = list(shapes)
    del cases, graphs
    torch.cuda.empty_cache()
    if not args.no_grouped and not args.shape:
        result["grouped"] = grouped_measurements(stream)
    if not args.no_configs and not args.shape:
        torch.cuda.empty_cache()
        result["dense_configs"] = dense_config_measurements(torch, stream)
    if not args.no_extra and not args.shape:
        torch.cuda.empty_cache()
        result["moe_layout"] = moe_measurements(stream)
        torch.cuda.empty_cache()
        result["formats"] = format_measurements(stream)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(sweep_shapes, host, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def build_cases(shapes, outliers):
    """Seeded N(0, 1) fp32 activations and weights for every shape (1% of
    the elements of both operands x50 when `outliers`), uploaded; weights
    quantised once by the 128x128 block cast; every buffer rotated over
    enough copies that >= 1 GiB is touched between two uses of one copy."""
    import torch
    from fp8_block_scaled_04_amd import binding, synth
    host = {}
    for (m, n, k) in shapes:
        if (m, k) not in host:
            x = synth.normal_f32(0, synth.S_LHS, (m, k))
            if outliers:
                x = synth.with_outliers(x, 0, synth.S_OUT_LHS)
            host[(m, k)] = x
        if (n, k) not in host:
            w = synth.normal_f32(0, synth.S_RHS, (n, k))
            if outliers:
                w = synth.with_outliers(w, 0, synth.S_OUT_RHS)
            host[(n, k)] = w
    cases = []
    for (m, n, k) in shapes:
        kg, nb = math.ceil(k / 128), math.ceil(n / 128)
        ld = max(4, (m + 3) // 4 * 4)
        x_d = torch.from_numpy(host[(m, k)]).cuda()
        w_d = torch.from_numpy(host[(n, k)]).cuda()
        qb0 = torch.empty((n, k), dtype=torch.uint8, device="cuda")
        sb0 = torch.empty((nb, kg), dtype=torch.float32, device="cuda")
        binding.fp8_cast_per_block(w_d, qb0, sb0)
        del w_d
        foot = 4 * m * k + m * k + kg * ld * 4 + n * k + nb * kg * 4 + 2 * m * n
        reps = int(min(64, max(1, math.ceil(ROTATE_BYTES / foot))))
        ws_bytes = binding.fp8_gemm_workspace_bytes(m, n, k)
        ws = torch.empty(max(1, ws_bytes // 4), dtype=torch.float32, device="cuda") if ws_bytes else None
        sets = []
        for r in range(reps):
            sets.append(dict(
                x=x_d if r == 0 else x_d.clone(),
                q=torch.empty((m, k), dtype=torch.uint8, device="cuda"),
                s=torch.empty((kg, ld), dtype=torch.float32, device="cuda"),
                qb=qb0 if r == 0 else qb0.clone(),
                sb=sb0 if r == 0 else sb0.clone(),
                out=torch.empty((m, n), dtype=torch.bfloat16, device="cuda"),
            ))
        flop, nbytes = algorithmic(m, n, k)
        cases.append(dict(m=m, n=n, k=k, sets=sets, ws=ws, flop=flop, bytes=nbytes,
                          cast_bytes=cast_bytes(m, k)))
    torch.cuda.synchronize()
    return host, cases


def time_gemm_case(torch, stream, c):
    """Median and mean launch duration of the case's GEMM (graph replays of
    rotated launches), its cast's median, and the roofline record."""
    from fp8_block_scaled_04_amd import binding

    def gemm(b, st):
        binding.fp8_gemm_nt(b["q"], b["s"], b["qb"], b["sb"], b["out"], workspace=c["ws"], stream=st)

    def cast(b, st):
        binding.fp8_cast_per_token_group(b["x"], b["q"], b["s"], stream=st)

    reps = max(10, min(200, int(2e4 / max(1.0, c["flop"] / 1e9))))
    batches = replay_mean_ms(torch, stream, gemm, c["sets"], reps, 3)
    gemm_ms = float(np.median(batches))
    cast_ms = float(np.median(replay_mean_ms(torch, stream, cast, c["sets"], reps, 1)))
    c["gemm_ms"], c["cast_ms"], c["gemm_mean_ms"] = gemm_ms, cast_ms, float(np.mean(batches))
    tflops = c["flop"] / (gemm_ms * 1e-3) / 1e12
    gbs = c["bytes"] / (gemm_ms * 1e-3) / 1e9
    bound = "mfma" if c["flop"] / c["bytes"] >= RIDGE else "hbm"
    frac = tflops / PEAK_FP8_TFLOPS if bound == "mfma" else gbs / PEAK_HBM_GBS
    return dict(m=c["m"], n=c["n"], k=c["k"], gemm_us=round(gemm_ms * 1e3, 2),
                mean_launch_us=round(c["gemm_mean_ms"] * 1e3, 2),
                gemm_us_min_max=[round(min(batches) * 1e3, 2), round(max(batches) * 1e3, 2)],
                cast_us=round(cast_ms * 1e3, 2), tflops=round(tflops, 1), gbs=round(gbs, 1),
                bound=bound, frac=round(frac, 4), cast_gbs=round(c["cast_bytes"] / (cast_ms * 1e-3) / 1e9, 1))


# The other dense workloads, measured beside the metric's sweep: the small
# case (m=64, n=2112, k=7168) and the large compute-bound shapes with 1% of
# the elements of both operands scaled by 50.
DENSE_CONFIGS = [
    ("config0", "dense m=64 n=2112 k=7168, N(0,1), seed 0", [(64, 2112, 7168)], False),
    ("config4", "dense m=n=k=8192 and m=16384 n=7168 k=16384, N(0,1) with 1% of elements x50, seed 0",
     [(8192, 8192, 8192), (16384, 7168, 16384)], True),
]


def dense_config_measurements(torch, stream):
    out = {}
    for name, desc, shapes, outliers in DENSE_CONFIGS:
        t0 = time.time()
        _, cases = build_cases(shapes, outliers)
        recs = []
        for c in cases:
            rec = time_gemm_case(torch, stream, c)
            rec["rotated_sets"] = len(c["sets"])
            recs.append(rec)
            print(f"[bench] {name} {c['m']}x{c['n']}x{c['k']}: {rec['gemm_us']} us, {rec['tflops']} TFLOP/s, "
                  f"{rec['gbs']} GB/s ({rec['bound']} {rec['frac']})", file=sys.stderr, flush=True)
        out[name] = dict(workload=desc, shapes=recs, seconds=round(time.time() - t0, 1))
        del cases
        torch.cuda.empty_cache()
    return out


def jit_measurements(torch, stream, cases):
    """Runtime shape specialisation per sweep shape: the ahead-of-time tile
    configuration rebuilt with n and k compiled in (compile time on a cold
    cache, then timed like the ahead-of-time kernel)."""
    from fp8_block_scaled_04_amd import binding

    out = []
    for c in cases:
        m, n, k = c["m"], c["n"], c["k"]
        cfg = binding._config(binding.fp8_jit_default_config(binding.FP8G_JIT_DENSE, m, n, k), specialize=1)
        t0 = time.perf_counter()
        try:
            binding.fp8_jit_warmup(binding.FP8G_JIT_DENSE, n, k, config=cfg)
        except binding.Fp8GemmError as e:   # e.g. the build would spill registers: refused
            out.append(dict(m=m, n=n, k=k, refused=binding.status_string(e.status)))
            continue
        compile_s = time.perf_counter() - t0

        def jit(b, st, c=c, cfg=cfg):
            binding.fp8_jit_gemm_nt(b["q"], binding.FP8G_E4M3, b["s"], b["qb"], binding.FP8G_E4M3, b["sb"], b["out"],
                                    config=cfg, workspace=c["ws"], stream=st)

        reps = max(10, min(200, int(2e4 / max(1.0, c["flop"] / 1e9))))
        ms = float(np.median(replay_mean_ms(torch, stream, jit, c["sets"], reps, 3)))
        out.append(dict(m=m, n=n, k=k, jit_us=round(ms * 1e3, 2), aot_us=round(c["gemm_ms"] * 1e3, 2),
                        aot_over_jit=round(c["gemm_ms"] / ms, 3), first_call_s=round(compile_s, 2)))
        print(f"[bench] jit {m}x{n}x{k}: {ms * 1e3:.2f} us (ahead of time {c['gemm_ms'] * 1e3:.2f} us)",
              file=sys.stderr, flush=True)
    return dict(config="ahead-of-time tile configuration, n and k compiled in", cache=binding.fp8_jit_get_cache_dir(),
                stats=binding.fp8_jit_stats(), by_shape=out)


MOE = {
    "prefill": dict(tokens=16384, groups=8, n=4096, k=7168),
    "decode": dict(tokens=2048, groups=16, max_m=256, n=4096, k=7168),
}


def moe_measurements(stream):
    """The MoE layout steps around the grouped GEMMs, each timed on its own
    like the GEMMs (graph replay, rotated buffers): routing layout (expert
    counts, stable ranks, destinations), scatter of the quantised rows and
    their scales to the laid-out operand, gather of the BF16 outputs back to
    token order.  Tokens are routed uniformly at random over the experts
    (seed 0).  Algorithmic bytes: scatter moves each token's k codes and k/128
    scales once each way, gather its n BF16 outputs once each way."""
    import torch
    from fp8_block_scaled_04_amd import binding, synth
    out = {}
    for name, c in MOE.items():
        T, G, n, k = c["tokens"], c["groups"], c["n"], c["k"]
        kg = math.ceil(k / 128)
        e = np.minimum((synth.uniform(0, synth.S_GROUP_SIZES, T) * G).astype(np.int64), G - 1).astype(np.int32)
        ed = torch.from_numpy(e).cuda()
        ws = torch.empty(binding.fp8_moe_layout_workspace_bytes(T, G) // 4 + 1, dtype=torch.int32, device="cuda")
        if name == "prefill":
            rows = binding.fp8_moe_contiguous_rows(T, G)
            rpg = rows
            layout = lambda st: binding.fp8_moe_layout_contiguous(ed, G, rows, workspace=ws, stream=st)
        else:
            rows = G * c["max_m"]
            rpg = c["max_m"]
            layout = lambda st: binding.fp8_moe_layout_masked(ed, G, c["max_m"], workspace=ws, stream=st)
        dst = layout(None)[2 if name == "prefill" else 1]
        torch.cuda.synchronize()
        ld_in, ld_out = max(4, (T + 3) // 4 * 4), max(4, (rpg + 3) // 4 * 4)
        nsets = max(1, math.ceil(ROTATE_BYTES / (T * (k + 2 * n) + rows * (k + 2 * n))))
        sets = []
        for _ in range(nsets):
            sets.append(dict(
                q=torch.randint(0, 255, (T, k), dtype=torch.uint8, device="cuda"),
                s=torch.rand((kg, ld_in), dtype=torch.float32, device="cuda"),
                q_out=torch.empty((rows, k), dtype=torch.uint8, device="cuda"),
                s_out=torch.empty((rows // rpg, kg, ld_out), dtype=torch.float32, device="cuda"),
                y=torch.randn((rows, n), device="cuda").to(torch.bfloat16),
                back=torch.empty((T, n), dtype=torch.bfloat16, device="cuda")))
        torch.cuda.synchronize()
        layout_ms = float(np.median(replay_mean_ms(torch, stream, lambda b, st: layout(st), sets, 50, 3)))
        scatter_ms = float(np.median(replay_mean_ms(
            torch, stream, lambda b, st: binding.fp8_moe_scatter_rows(b["q"], b["s"], dst, b["q_out"], b["s_out"],
                                                                      rows_per_group=rpg, stream=st), sets, 50, 3)))
        gather_ms = float(np.median(replay_mean_ms(
            torch, stream, lambda b, st: binding.fp8_moe_gather_rows(b["y"], dst, b["back"], stream=st), sets, 50, 3)))
        placed = int((dst >= 0).sum().item())
        scatter_bytes = 2 * placed * (k + 4 * kg) + 4 * T
        gather_bytes = 2 * T * n * 2 + 4 * T
        out[name] = dict(tokens=T, groups=G, k=k, n=n, placed_rows=placed, laid_out_rows=rows,
                         layout_us=round(layout_ms * 1e3, 2), scatter_us=round(scatter_ms * 1e3, 2),
                         gather_us=round(gather_ms * 1e3, 2),
                         scatter_gbs=round(scatter_bytes / (scatter_ms * 1e-3) / 1e9, 1),
                         gather_gbs=round(gather_bytes / (gather_ms * 1e-3) / 1e9, 1),
                         scatter_frac=round(scatter_bytes / (scatter_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                         gather_frac=round(gather_bytes / (gather_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4))
        print(f"[bench] moe {name}: layout {layout_ms * 1e3:.1f} us, scatter {scatter_ms * 1e3:.1f} us, "
              f"gather {gather_ms * 1e3:.1f} us", file=sys.stderr, flush=True)
        del sets
        torch.cuda.empty_cache()
    return out


def format_measurements(stream):
    """E5M2 operands (either side) against E4M3 on the dominant shape and a
    small-M shape, with operands cast from the same N(0, 1) data in each
    format; and the per-token-group cast to each format."""
    import torch
    from fp8_block_scaled_04_amd import binding
    E4, E5 = binding.FP8G_E4M3, binding.FP8G_E5M2
    out = []
    for (m, n, k) in [(4096, 7168, 16384), (64, 7168, 16384)]:
        kg, nb = math.ceil(k / 128), math.ceil(n / 128)
        g = torch.Generator("cuda").manual_seed(0)
        x = torch.randn((m, k), device="cuda", generator=g)
        w = torch.randn((n, k), device="cuda", generator=g)
        ops = {}
        for f in (E4, E5):
            qa = torch.empty((m, k), dtype=torch.uint8, device="cuda")
            sa = torch.empty((kg, max(4, (m + 3) // 4 * 4)), dtype=torch.float32, device="cuda")
            binding.fp8_cast_per_token_group_fmt(x, f, qa, sa)
            qb = torch.empty((n, k), dtype=torch.uint8, device="cuda")
            sb = torch.empty((nb, kg), dtype=torch.float32, device="cuda")
            binding.fp8_cast_per_block_fmt(w, f, qb, sb)
            ops[f] = (qa, sa, qb, sb)
        del w
        ws_bytes = binding.fp8_gemm_workspace_bytes(m, n, k)
        ws = torch.empty(max(1, ws_bytes // 4), dtype=torch.float32, device="cuda") if ws_bytes else None
        o = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        flop, nbytes = algorithmic(m, n, k)
        reps = max(5, min(100, int(2e4 / max(1.0, flop / 1e9))))
        rec = dict(m=m, n=n, k=k)
        for fa, fb, tag in [(E4, E4, "e4m3_e4m3"), (E4, E5, "e4m3_e5m2"), (E5, E5, "e5m2_e5m2")]:
            qa, sa, _, _ = ops[fa]
            _, _, qb, sb = ops[fb]
            fn = lambda b, st, qa=qa, sa=sa, qb=qb, sb=sb, fa=fa, fb=fb: binding.fp8_gemm_nt_fmt(
                qa, fa, sa, qb, fb, sb, o, workspace=ws, stream=st)
            ms = float(np.median(replay_mean_ms(torch, stream, fn, [None], reps, 3)))
            rec[tag + "_us"] = round(ms * 1e3, 2)
            rec[tag + "_tflops"] = round(flop / (ms * 1e-3) / 1e12, 1)
        if m == 4096:
            for f, tag in [(E4, "e4m3"), (E5, "e5m2")]:
                qa, sa, _, _ = ops[f]
                fn = lambda b, st, f=f, qa=qa, sa=sa: binding.fp8_cast_per_token_group_fmt(x, f, qa, sa, stream=st)
                ms = float(np.median(replay_mean_ms(torch, stream, fn, [None], 20, 3)))
                rec["cast_" + tag + "_us"] = round(ms * 1e3, 2)
        out.append(rec)
        print(f"[bench] formats {m}x{n}x{k}: {rec}", file=sys.stderr, flush=True)
        del ops, x
        torch.cuda.empty_cache()
    return out


GROUPED = {
    "contiguous": dict(groups=8, n=4096, k=7168),
    "masked": dict(groups=16, max_m=256, n=4096, k=7168),
}


def replay_mean_ms(torch, stream, fn, sets, reps, batches):
    """Mean duration of one launch: `reps` launches of fn (rotating the input
    sets) are captured into one HIP graph, which is replayed `batches` times
    on `stream` between two events each.  Replaying a graph issues the
    kernels back to back on the GPU, so kernels shorter than the host's
    per-call launch cost are timed by the GPU, not by the host."""
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for r in range(2):
            fn(sets[r % len(sets)], None)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for r in range(reps):
            fn(sets[r % len(sets)], None)
    graph.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(batches):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / reps)
    del graph
    return out


def grouped_measurements(stream):
    """The two grouped GEMMs at their MoE shapes, timed like the dense shapes
    (launches back to back between two events, rotated input sets):
      contiguous (prefill): G=8 experts, n=4096, k=7168, expert rows 128*U{4..32}
        concatenated in expert order, m_indices per row;
      masked (decode): G=16 slots of max_m=256 rows, n=4096, k=7168, valid rows
        per group U{0..256} in a device tensor.
    Seeded N(0,1) activations and weights, quantised on the GPU (1x128 and
    128x128 casts).  FLOP and bytes count valid rows only."""
    import torch
    from fp8_block_scaled_04_amd import binding, synth
    out = []

    def timed(fn, sets, reps):
        batches = replay_mean_ms(torch, stream, fn, sets, reps, 3)
        return float(np.median(batches)), float(np.mean(batches)), batches

    def weights(G, n, k):
        kg, nb = math.ceil(k / 128), math.ceil(n / 128)
        w = synth.normal_f32(0, synth.S_RHS, (G, n, k))
        qb = torch.empty((G, n, k), dtype=torch.uint8, device="cuda")
        sb = torch.empty((G, nb, kg), dtype=torch.float32, device="cuda")
        for g in range(G):
            wd = torch.from_numpy(w[g]).cuda()
            binding.fp8_cast_per_block(wd, qb[g], sb[g])
        del w
        return qb, sb

    def record(name, desc, flop, nbytes, med, mean, batches, extra):
        tflops = flop / (med * 1e-3) / 1e12
        gbs = nbytes / (med * 1e-3) / 1e9
        bound = "mfma" if flop / nbytes >= RIDGE else "hbm"
        frac = tflops / PEAK_FP8_TFLOPS if bound == "mfma" else gbs / PEAK_HBM_GBS
        rec = dict(kernel=name, workload=desc, gemm_us=round(med * 1e3, 2), mean_launch_us=round(mean * 1e3, 2),
                   gemm_us_min_max=[round(min(batches) * 1e3, 2), round(max(batches) * 1e3, 2)],
                   tflops=round(tflops, 1), gbs=round(gbs, 1), bound=bound, frac=round(frac, 4),
                   flop=flop, alg_bytes=nbytes)
        rec.update(extra)
        out.append(rec)
        print(f"[bench] {name}: {med * 1e3:.1f} us, {tflops:.0f} TFLOP/s, {gbs:.0f} GB/s", file=sys.stderr,
              flush=True)

    # ---- contiguous layout ---------------------------------------------------
    c = GROUPED["contiguous"]
    G, n, k = c["groups"], c["n"], c["k"]
    kg, nb = math.ceil(k / 128), math.ceil(n / 128)
    sizes = synth.contiguous_group_sizes(G, 0)
    M = int(sizes.sum())
    x = synth.normal_f32(0, synth.S_LHS, (M, k))
    m_idx = np.repeat(np.arange(G, dtype=np.int32), sizes)
    xd = torch.from_numpy(x).cuda()
    del x
    qa = torch.empty((M, k), dtype=torch.uint8, device="cuda")
    sa = torch.empty((kg, M), dtype=torch.float32, device="cuda")
    binding.fp8_cast_per_token_group(xd, qa, sa)
    del xd
    qb, sb = weights(G, n, k)
    mi = torch.from_numpy(m_idx).cuda()
    foot = M * k + G * n * k + M * n * 2
    nsets = max(1, math.ceil(ROTATE_BYTES / foot))
    sets = [(qa, sa, qb, sb, torch.empty((M, n), dtype=torch.bfloat16, device="cuda"))]
    for _ in range(1, nsets):
        sets.append((qa.clone(), sa.clone(), qb.clone(), sb.clone(),
                     torch.empty((M, n), dtype=torch.bfloat16, device="cuda")))
    torch.cuda.synchronize()

    def run_c(bufs, st):
        a, s_, b, t, o = bufs
        binding.fp8_grouped_gemm_contiguous(a, s_, b, t, o, mi, stream=st)

    med, mean, batches = timed(run_c, sets, 20)
    flop = 2.0 * M * n * k
    nbytes = M * k + G * n * k + M * kg * 4 + G * nb * kg * 4 + M * n * 2 + M * 4
    record("fp8_grouped_gemm_contiguous",
           f"MoE prefill: G={G} experts, n={n}, k={k}, rows per expert 128*U{{4..32}} (seed 0), M={M}",
           flop, nbytes, med, mean, batches, dict(m_total=M, group_rows=[int(v) for v in sizes], rotated_sets=nsets))
    del sets, qa, sa, qb, sb, mi
    torch.cuda.empty_cache()

    # ---- masked layout ---------------------------------------------------------
    c = GROUPED["masked"]
    G, max_m, n, k = c["groups"], c["max_m"], c["n"], c["k"]
    kg, nb = math.ceil(k / 128), math.ceil(n / 128)
    counts = synth.masked_counts(G, max_m, 0)
    x = synth.normal_f32(0, synth.S_LHS, (G, max_m, k))
    qa = torch.empty((G, max_m, k), dtype=torch.uint8, device="cuda")
    sa = torch.empty((G, kg, max_m), dtype=torch.float32, device="cuda")
    for g in range(G):
        binding.fp8_cast_per_token_group(torch.from_numpy(x[g]).cuda(), qa[g], sa[g])
    del x
    qb, sb = weights(G, n, k)
    mm = torch.from_numpy(counts).cuda()
    foot = G * max_m * k + G * n * k + G * max_m * n * 2
    nsets = max(1, math.ceil(ROTATE_BYTES / foot))
    sets = [(qa, sa, qb, sb, torch.empty((G, max_m, n), dtype=torch.bfloat16, device="cuda"))]
    for _ in range(1, nsets):
        sets.append((qa.clone(), sa.clone(), qb.clone(), sb.clone(),
                     torch.empty((G, max_m, n), dtype=torch.bfloat16, device="cuda")))
    torch.cuda.synchronize()

    def run_m(bufs, st):
        a, s_, b, t, o = bufs
        binding.fp8_grouped_gemm_masked(a, s_, b, t, o, mm, stream=st)

    med, mean, batches = timed(run_m, sets, 20)
    valid = int(counts.sum())
    active = int((counts > 0).sum())
    flop = 2.0 * valid * n * k
    nbytes = valid * k + active * n * k + valid * kg * 4 + active * nb * kg * 4 + valid * n * 2 + G * 4
    record("fp8_grouped_gemm_masked",
           f"MoE decode: G={G} slots of max_m={max_m} rows, n={n}, k={k}, valid rows per group U{{0..{max_m}}} "
           f"(seed 0), {valid} valid rows",
           flop, nbytes, med, mean, batches, dict(valid_rows=valid, masked_m=[int(v) for v in counts],
                                                  rotated_sets=nsets))
    del sets, qa, sa, qb, sb, mm
    torch.cuda.empty_cache()
    return out


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "fp8_block_scaled_04_amd", "csrc", f)
                  for f in ("gemm_kernel.hpp", "device_common.hpp", "host_common.hpp", "dense_launch.hip", "fp8gemm.hip")]


def kernel_source_digest():
    import hashlib
    h = hashlib.sha1()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(m, n, k):
    """HBM bytes per launch of the GEMM for this shape, from the committed
    rocprofv3 FETCH_SIZE/WRITE_SIZE summary (scaled by the copy-kernel
    calibration recorded with it); None when no summary matches this shape
    and the current kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    digest = kernel_source_digest()
    for line in text.splitlines():
        if line.startswith("traffic:"):
            rec = json.loads(line[len("traffic:"):])
            if rec.get("shape") == [m, n, k] and rec.get("kernel_sources") == digest:
                return rec["hbm_bytes_per_launch"]
    return None


def copy_calibration(nbytes, steps):
    """A plain device-to-device copy of nbytes, repeated: the reference that
    scales the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "launches": steps}), flush=True)


def host_description():
    """Threads, nproc and CPU model of the machine the oracle runs on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return dict(nproc=os.cpu_count(), affinity=affinity, cpu_model=model)


def cpu_baseline(shapes, host, target_s):
    """The CPU oracle (as it stands) on the metric's workload: every row of
    every shape (cast of the fp32 activations + GEMM), on all the threads the
    oracle uses, scaled to the metric's unit (TFLOP/s of GEMM work).  Only
    if a short calibration predicts more than 3 x `target_s` seconds is the
    first r rows of every shape timed instead, r sized to about `target_s`
    seconds (and the sample says so)."""
    import oracle
    threads = oracle.hardware_threads()
    wq = {}
    for (m, n, k) in shapes:
        if (n, k) not in wq:
            wq[(n, k)] = oracle.cast_128x128(host[(n, k)], nthreads=threads)  # offline weights: not timed

    def run(rows):
        flop, t = 0.0, 0.0
        for (m, n, k) in shapes:
            r = min(m, rows)
            x = np.ascontiguousarray(host[(m, k)][:r])
            qb, sb = wq[(n, k)]
            t0 = time.perf_counter()
            qa, sa = oracle.cast_1x128(x, nthreads=threads)
            oracle.gemm_nt(qa, sa, qb, sb, nthreads=threads)
            t += time.perf_counter() - t0
            flop += 2.0 * r * n * k
        return flop, t

    mmax = max(m for m, _, _ in shapes)
    total_flop = sum(2.0 * m * n * k for m, n, k in shapes)
    cal_flop, cal_t = run(32)                      # calibration: 32 rows of every shape
    predicted = cal_t * total_flop / cal_flop
    if predicted <= 3 * target_s:
        rows, what = mmax, "the whole workload: every row of every shape"
    else:
        rows = int(max(32, min(mmax, 32 * target_s / max(cal_t, 1e-3))))
        what = f"a sample: the first {rows} rows (all rows if fewer) of every shape"
    flop, t = run(rows)
    rec = {"value": round(flop / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": f"{what}, cast + GEMM: {flop / 2e9:.1f} G MAC in {t:.1f} s",
           "threads": threads}
    rec.update(host_description())
    return rec


if __name__ == "__main__":
    main()
