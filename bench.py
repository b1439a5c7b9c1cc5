#!/usr/bin/env python3
"""Benchmark of the local W4A16 MoE forward on one MI355X.

One step = one forward at every token count of the sweep (route preparation,
gather, gate/up GEMM, activation, down GEMM, FP32 combine: the whole path) on
seeded synthetic inputs already resident in HBM.  Each forward is captured in
a HIP graph and replayed; before every timed replay a read-only pass over a
512 MiB buffer evicts the L2 caches and the 256 MB Infinity Cache, so weights
stream from HBM ("cold").  The evicting pass only reads, so no dirty lines are
left to be written back while the timed forward runs.
Warm numbers (10 back-to-back replays, the caches holding whatever fits) are
reported beside them as context.

Prints ONE JSON line.  `value` is the geometric mean over the token sweep of
the cold per-forward latency in microseconds (lower is better).  The
`roofline` object covers the dominant kernel (the stage with the largest
share of the sweep's time), timed with HIP events recorded by the library
around each stage on the stream it launches on; `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "local MoE latency (us) at 1-2048 tokens, 384e H7168 I256 top8; HBM GB/s & MFMA %"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2516.6, "fp16": 2516.6}
STAGES = ("route_prep", "gate_up_gemm", "down_gemm", "combine")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def workload_bytes_flops(wl, ids, T):
    """Algorithmic bytes per stage and for the whole forward, and flops."""
    import torch

    E, H, I, K, N1 = wl.num_experts, wl.hidden, wl.inter, wl.top_k, wl.n1
    loc = ids.long() - wl.expert_offset
    valid = (loc >= 0) & (loc < E)
    Rv = int(valid.sum())
    D = int(torch.unique(loc[valid]).numel()) if Rv else 0
    if wl.per_channel:
        w13 = N1 * H // 2 + N1 * 2
        w2 = H * I // 2 + H * 2
    else:
        w13 = N1 * H // 2 + N1 * (H // 32) * 2
        w2 = H * I // 2 + H * (I // 32) * 2
    R = T * K
    stage = {
        "route_prep": 4 * R + 4 * R + 4 * (E + 1) * 2,
        "gate_up_gemm": D * w13 + T * H * 2 + Rv * I * 2,
        "down_gemm_fused": D * w2 + Rv * I * 2 + T * H * 2 + 8 * R,
        "down_gemm": D * w2 + Rv * I * 2 + Rv * H * 2,
        "combine": Rv * H * 2 + T * H * 2 + 8 * R,
    }
    total = D * (w13 + w2) + 2 * T * H * 2 + 8 * R
    flops = {"gate_up_gemm": 2.0 * Rv * N1 * H, "down_gemm": 2.0 * Rv * H * I}
    flops["down_gemm_fused"] = flops["down_gemm"]
    return stage, total, flops["gate_up_gemm"] + flops["down_gemm"], flops, D, Rv


def cpu_baseline(wl, Wg, budget_s):
    """The CPU oracle (as it stands) on a bounded sample of the same sweep."""
    import numpy as np
    import torch

    import oracle
    from w4a16_mixture_experts_amd import synth

    def b(t):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)

    Wc = Wg.to("cpu")
    args = (Wc.w13_packed.numpy(), b(Wc.w13_scales), Wc.w2_packed.numpy(), b(Wc.w2_scales))
    res, spent = {}, 0.0
    for T in sorted(wl.tokens):
        tok = synth.make_tokens(wl, T)
        t0 = time.perf_counter()
        oracle.moe_forward(b(tok.x), *args, tok.topk_ids.numpy(), tok.topk_weights.numpy(),
                           hidden=wl.hidden, inter=wl.inter, num_experts=wl.num_experts,
                           expert_offset=wl.expert_offset,
                           act=oracle.ACT_SILU_GATED if wl.gated else oracle.ACT_RELU2,
                           layout=oracle.Q_PER_CHANNEL if wl.per_channel else oracle.Q_GROUP_K,
                           dtype=oracle.DT_FP16 if wl.dtype == torch.float16 else oracle.DT_BF16)
        dt = time.perf_counter() - t0
        spent += dt
        res[T] = dt * 1e6
        log(f"[cpu baseline] T={T}: {dt * 1e3:.1f} ms (total {spent:.1f} s)")
        if spent > budget_s:
            break
    return res, oracle.max_threads()


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="kimi_tp8")
    ap.add_argument("--tokens", default="", help="comma list (default: the workload's sweep)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--no-graph", action="store_true", help="time eager calls instead")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU; --gpus {args.gpus} is not supported "
              "(the local MoE path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)

    import torch

    from w4a16_mixture_experts_amd import binding, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    binding.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.WORKLOADS[args.workload]
    sweep = [int(t) for t in args.tokens.split(",")] if args.tokens else list(wl.tokens)
    dtype_name = "fp16" if wl.dtype == torch.float16 else "bf16"

    log(f"[bench] generating {wl.name} weights on the GPU")
    Wg = synth.make_weights(wl, device=dev)
    flush_buf = torch.ones(128 * 1024 * 1024, dtype=torch.int32, device=dev)   # 512 MiB

    def flush():
        flush_buf.max()     # reads the whole buffer, writes one value

    torch.cuda.synchronize()

    cases = []
    for T in sweep:
        tok = synth.make_tokens(wl, T).to(dev)
        desc = binding.desc_for(wl, T)
        plan = binding.get_plan(desc)
        ws = torch.empty(max(1, binding.workspace_size(desc)), dtype=torch.uint8, device=dev)
        out = torch.empty(T, wl.hidden, dtype=wl.dtype, device=dev)

        def fwd(tok=tok, ws=ws, out=out, **kw):
            return binding.forward_workload(wl, Wg, tok, out=out, workspace=ws, **kw)

        fwd()
        torch.cuda.synchronize()
        graph = None
        if not args.no_graph:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                fwd()
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                fwd()
            torch.cuda.synchronize()
        stage_b, total_b, total_f, stage_f, D, Rv = workload_bytes_flops(wl, tok.topk_ids.cpu(), T)
        cases.append(dict(T=T, tok=tok, fwd=fwd, graph=graph, plan=plan, stage_bytes=stage_b,
                          bytes=total_b, flops=total_f, stage_flops=stage_f, D=D, Rv=Rv,
                          cold=[], warm=[], stages={s: [] for s in STAGES}))
        log(f"[bench] T={T}: plan path={plan.path} block_m={plan.block_m} "
            f"k_slice={plan.k_slice} touched experts={D}")

    def replay(c):
        if c["graph"] is not None:
            c["graph"].replay()
        else:
            c["fwd"]()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)

    def step(record):
        for c in cases:
            flush()
            ev0.record()
            replay(c)
            ev1.record()
            ev1.synchronize()
            if record:
                c["cold"].append(ev0.elapsed_time(ev1) * 1e3)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"[bench] timed {args.steps} steps in {wall:.2f} s")

    # warm context: 10 back-to-back replays
    for c in cases:
        for _ in range(3):
            ev0.record()
            for _ in range(10):
                replay(c)
            ev1.record()
            ev1.synchronize()
            c["warm"].append(ev0.elapsed_time(ev1) * 1e3 / 10)

    # per-stage durations (eager calls, library-recorded events, cold caches)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
    for c in cases:
        for _ in range(max(5, args.steps // 2)):
            flush()
            c["fwd"](stage_events=evs)
            torch.cuda.synchronize()
            for si, name in enumerate(STAGES):
                a, b = evs[2 * si], evs[2 * si + 1]
                if name in ("route_prep", "combine") and c["plan"].path == 2:
                    continue
                c["stages"][name].append(a.elapsed_time(b) * 1e3)

    lat_cold = {c["T"]: statistics.median(c["cold"]) for c in cases}
    lat_warm = {c["T"]: statistics.median(c["warm"]) for c in cases}
    geo = math.exp(sum(math.log(v) for v in lat_cold.values()) / len(lat_cold))
    table = {}
    best = None
    for c in cases:
        T = c["T"]
        st = {k: statistics.median(v) for k, v in c["stages"].items() if v}
        down_key = "down_gemm_fused" if c["plan"].path == 2 else "down_gemm"
        row = {
            "latency_us_cold": round(lat_cold[T], 3),
            "latency_us_warm": round(lat_warm[T], 3),
            "hbm_gbps_cold": round(c["bytes"] / lat_cold[T] / 1e3, 1),
            "hbm_frac_cold": round(c["bytes"] / lat_cold[T] / 1e3 / HBM_PEAK_GBS, 4),
            "tflops_cold": round(c["flops"] / lat_cold[T] / 1e6, 2),
            "mfma_frac_cold": round(c["flops"] / lat_cold[T] / 1e6 / MFMA_PEAK_TFLOPS[dtype_name], 4),
            "algorithmic_bytes": int(c["bytes"]),
            "touched_experts": c["D"],
            "valid_routes": c["Rv"],
            "plan": {"path": "small-batch" if c["plan"].path == 2 else "grouped",
                     "block_m": c["plan"].block_m, "k_slice": c["plan"].k_slice},
            "stage_us": {k: round(v, 3) for k, v in st.items()},
        }
        for k, v in st.items():
            key = down_key if k == "down_gemm" else k
            if key in c["stage_bytes"] and v > 0:
                row.setdefault("stage_gbps", {})[k] = round(c["stage_bytes"][key] / v / 1e3, 1)
            if best is None or v > best[0]:
                best = (v, T, k, key, c)
        table[str(T)] = row

    v, Tb, kname, key, cb = best
    bts = cb["stage_bytes"].get(key, 0)
    achieved = bts / v / 1e3
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": kname, "tokens": Tb, "avg_launch_us": round(v, 3),
                "algorithmic_bytes_per_launch": int(bts)}

    cpu = None
    if not args.no_cpu_baseline:
        res, cores = cpu_baseline(wl, Wg, args.cpu_budget_s)
        done = sorted(res)
        gpu_same = math.exp(sum(math.log(lat_cold[t]) for t in done) / len(done))
        cpu_geo = math.exp(sum(math.log(res[t]) for t in done) / len(done))
        cpu = {"value": round(cpu_geo, 1), "unit": "us", "cores": cores, "kind": "oracle",
               "sample": f"{wl.name}, one oracle forward at each T in {done} (geometric mean of "
                         f"the per-forward latency); GPU geomean over the same T: "
                         f"{gpu_same:.2f} us",
               "per_tokens_us": {str(t): round(res[t], 1) for t in done}}

    line = {
        "metric": METRIC,
        "value": round(geo, 3),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sum(lat_cold.values()) / 1e3, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_name,
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: {wl.num_experts} local experts (of {wl.num_global_experts}), "
                        f"hidden {wl.hidden}, intermediate {wl.inter}, top-{wl.top_k}, "
                        f"INT4 {'per-channel' if wl.per_channel else 'group-32'}, "
                        f"{'SiLU-gated' if wl.gated else 'ReLU^2'}",
            "tokens": sweep,
            "value_definition": "geometric mean over the token sweep of the cold-cache "
                                "latency of one forward (HIP graph replay)",
            "parallelism": "single GPU",
            "per_tokens": table,
            "wall_s_timed_region": round(wall, 3),
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
