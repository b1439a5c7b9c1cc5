#!/usr/bin/env python3
"""Benchmark of the local W4A16 MoE forward on one MI355X.

A forward is the whole path (route preparation, gather, gate/up GEMM,
activation, down GEMM, FP32 combine) on seeded synthetic inputs already
resident in HBM.  One step measures, at every token count of the sweep:
  1. a read-only pass over a 512 MiB buffer evicts the L2 caches and the
     256 MB Infinity Cache (it only reads, so no dirty lines are left to be
     written back while the forward runs);
  2. cold latency: a HIP graph holding G copies of (eviction pass, forward)
     and a graph holding G eviction passes alone are replayed back to back
     between HIP events; the difference divided by G is the device time of
     one forward on cold caches, without the submission latency of a launch
     (the pages time graph replays the same way);
  3. the cache is evicted again and the forward runs once more as direct
     calls, with HIP events that the library records around each stage on the
     stream it launches on: per-stage kernel durations in the same timed
     region (the `roofline` kernel's average launch duration).
Warm numbers (a graph of G back-to-back forwards, caches holding whatever
fits) are reported afterwards as context.

Prints ONE JSON line.  `value` is the geometric mean over the token sweep of
the mean cold per-forward latency in microseconds (lower is better).
`roofline` covers the dominant kernel (the one with the largest share of the
sweep's time); `cpu_baseline` times the CPU oracle on a bounded sample of the
same workload.
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


KERNEL_PREFIX = "w4moe::"


def kernel_name(wl, plan, stage):
    """Kernel(s) a stage launches, spelled as the profiler prints them (w/o arguments)."""
    import torch

    dt = 1 if wl.dtype == torch.float16 else 0
    lay = 1 if wl.per_channel else 0
    if plan.path == 2:
        return {"gate_up_gemm": f"small_h_kernel<{dt}, {lay}, ...>",
                "down_gemm": f"decode_down_kernel<{dt}, {lay}, ...>"}[stage]
    if stage == "route_prep":
        return "route_prep_kernel"
    if stage == "combine":
        return f"combine_kernel<{dt}>"
    if plan.block_m != 64:
        return f"block_m {plan.block_m} {stage}"
    if stage == "gate_up_gemm":
        if plan.splitk_chunks:
            return (f"up_splitk_kernel<{dt}, {lay}, 2> + "
                    f"splitk_act_kernel<{dt}, {'true' if wl.gated else 'false'}>")
        return f"tile_gemm_kernel<{dt}, {lay}, {0 if wl.gated else 1}>"
    if wl.inter <= 256:   # the reduction fits the resident down kernel
        return f"down_resident_kernel<{dt}, {lay}, {1 if wl.inter <= 128 else 2}>"
    return f"tile_gemm_kernel<{dt}, {lay}, 2>"


def measured_traffic(kname, tokens):
    """HBM bytes per launch from the committed counter summary, if it covers this
    kernel as it is now built (same kernel source hash, same token sweep)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    ent = rec.get("kernels", {}).get(kname)
    if ent is None or ent.get("tokens") != tokens:
        return None
    src = os.path.join(ROOT, "w4a16_mixture_experts_amd", "csrc", ent["source"])
    if not os.path.exists(src) or source_hash(src) != ent.get("source_sha256"):
        return None
    return ent["hbm_bytes_per_launch"]


def source_hash(path):
    import hashlib

    h = hashlib.sha256()
    for p in (path, os.path.join(os.path.dirname(path), "device.h")):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_pass(args, wl, sweep, dev):
    """Inputs built on the host and copied over, then only library launches
    (and device-to-device copies), for rocprofv3 counter runs that must not
    see other device kernels.  The packed weights are random bytes and the
    scales 1: the memory traffic of the kernels depends on the shapes and the
    routing, which is the timed run's (same generator, same seeds), not on
    the weight values.  With --copy-calibration-mib, three plain copies of
    that size come first (the calibration for the byte counters)."""
    import numpy as np
    import torch

    from w4a16_mixture_experts_amd import binding, synth

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * 1024 * 1024 // 4
        src = torch.ones(n, dtype=torch.float32).to(dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[counters] copy calibration: 3 x {args.copy_calibration_mib} MiB copied")
        del src, dst
    rng = np.random.default_rng(0)
    E, H, I, N1 = wl.num_experts, wl.hidden, wl.inter, wl.n1
    if wl.per_channel:
        shapes = [(E, N1 // 2, H), (E, N1), (E, H // 2, I), (E, H)]
    else:
        shapes = [(E, N1, H // 2), (E, N1, H // 32), (E, H, I // 2), (E, H, I // 32)]
    ts = []
    for i, sh in enumerate(shapes):
        if i % 2 == 0:
            ts.append(torch.from_numpy(rng.integers(0, 256, size=sh, dtype=np.uint8)).to(dev))
        else:
            ts.append(torch.ones(sh, dtype=wl.dtype).to(dev))
    W = synth.Weights(*ts)
    for T in sweep:
        tok = synth.make_tokens(wl, T).to(dev)
        for _ in range(args.steps):
            binding.forward_workload(wl, W, tok)
        torch.cuda.synchronize()
        log(f"[counters] T={T}: {args.steps} forwards")


# kernel whose HBM traffic the counter pass measures: the gate/up tile kernel
# (group layout, bf16, LDS scales; per-group or fp16 route), as a prefix of
# the names the profiler prints and as this script prints it
COUNTED = ("tile_gemm_kernel<0, 0, 0, true,", "tile_gemm_kernel<0, 0, 0>", "tile.hip")


def summarize_counters(args, sweep):
    """profiles/traffic.json from two --counter-pass runs (FETCH_SIZE, then
    WRITE_SIZE, KiB per dispatch).  Each counter is scaled by known bytes /
    counted bytes of the run's plain copies (--copy-calibration-mib each);
    the counted kernel's launches come in sweep order, --steps per T."""
    import csv

    known = args.copy_calibration_mib * 1024 * 1024
    if known <= 0:
        raise SystemExit("--summarize-counters needs --copy-calibration-mib (the copies' size)")
    per = {}
    factors = {}
    for name, path in zip(("FETCH_SIZE", "WRITE_SIZE"), args.summarize_counters):
        with open(path) as f:
            rows = [r for r in csv.DictReader(f) if r["Counter_Name"] == name]
        # the calibration copies: the largest copy dispatches of the run
        cb = [r for r in rows if "copyBuffer" in r["Kernel_Name"]]
        big = max((int(r["Grid_Size"]) for r in cb), default=0)
        copies = [float(r["Counter_Value"]) * 1024 for r in cb if int(r["Grid_Size"]) == big]
        if not copies:
            raise SystemExit(f"{path}: no calibration copies")
        factors[name] = known / statistics.fmean(copies)
        ks = [float(r["Counter_Value"]) * 1024 for r in rows if COUNTED[0] in r["Kernel_Name"]]
        if len(ks) != args.steps * len(sweep):
            raise SystemExit(f"{path}: {len(ks)} launches of {COUNTED[0]}, expected "
                             f"{args.steps} x {len(sweep)}")
        per[name] = {T: statistics.fmean(ks[i * args.steps:(i + 1) * args.steps]) * factors[name]
                     for i, T in enumerate(sweep)}
    by_t = {T: per["FETCH_SIZE"][T] + per["WRITE_SIZE"][T] for T in sweep}
    src = os.path.join(ROOT, "w4a16_mixture_experts_amd", "csrc", COUNTED[2])
    rec = {"kernels": {COUNTED[1]: {
        "tokens": sweep,
        "source": COUNTED[2],
        "source_sha256": source_hash(src),
        "hbm_bytes_per_launch": int(statistics.fmean(by_t.values())),
        "hbm_bytes_by_tokens": {str(T): int(v) for T, v in by_t.items()},
        "fetch_bytes_by_tokens": {str(T): int(v) for T, v in per["FETCH_SIZE"].items()},
        "write_bytes_by_tokens": {str(T): int(v) for T, v in per["WRITE_SIZE"].items()},
        "calibration": {"copy_bytes": known, "fetch_factor": round(factors["FETCH_SIZE"], 4),
                        "write_factor": round(factors["WRITE_SIZE"], 4)},
    }}}
    out = os.path.join(ROOT, "profiles", "traffic.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def cpu_baseline(wl, Wg, budget_s, min_s):
    """The CPU oracle (as it stands) on a bounded sample of the same sweep."""
    import numpy as np
    import torch

    import oracle
    from w4a16_mixture_experts_amd import synth

    def b(t):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)

    Wc = Wg.to("cpu")
    args = (Wc.w13_packed.numpy(), b(Wc.w13_scales), Wc.w2_packed.numpy(), b(Wc.w2_scales))
    # whole passes over the sweep until min_s of CPU work is spent (at least
    # one pass), stopping early once budget_s is exceeded; mean per T
    times, spent, passes = {}, 0.0, 0
    while spent < min_s and spent <= budget_s:
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
            times.setdefault(T, []).append(dt * 1e6)
            log(f"[cpu baseline] pass {passes} T={T}: {dt * 1e3:.1f} ms (total {spent:.1f} s)")
            if spent > budget_s:
                break
        passes += 1
    res = {T: sum(v) / len(v) for T, v in times.items()}
    return res, oracle.max_threads(), passes


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="kimi_tp8")
    ap.add_argument("--tokens", default="", help="comma list (default: the workload's sweep)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0,
                    help="stop the CPU oracle baseline once this much CPU time is spent")
    ap.add_argument("--cpu-min-s", type=float, default=10.0,
                    help="repeat whole sweeps of the CPU oracle until this much time is spent")
    ap.add_argument("--no-graph", action="store_true", help="time eager calls instead")
    ap.add_argument("--graph-reps", type=int, default=10,
                    help="forwards per captured graph (G); per-forward time = graph time / G")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from the counter_collection.csv files of "
                         "a --counter-pass run under rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE")
    ap.add_argument("--counter-pass", action="store_true",
                    help="host-built inputs and library calls only (for counter runs)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run three plain copies of this many MiB: the known-size "
                         "kernel that scales the HBM counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU; --gpus {args.gpus} is not supported "
              "(the local MoE path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)

    import torch

    from w4a16_mixture_experts_amd import binding, synth

    if args.summarize_counters:
        sweep = [int(t) for t in args.tokens.split(",")] if args.tokens else \
            list(synth.WORKLOADS[args.workload].tokens)
        summarize_counters(args, sweep)
        return
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    binding.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.WORKLOADS[args.workload]
    sweep = [int(t) for t in args.tokens.split(",")] if args.tokens else list(wl.tokens)
    dtype_name = "fp16" if wl.dtype == torch.float16 else "bf16"

    if args.counter_pass:
        counter_pass(args, wl, sweep, dev)
        return

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * 1024 * 1024 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: 3 x {args.copy_calibration_mib} MiB read + written")
        del src, dst

    log(f"[bench] generating {wl.name} weights on the GPU")
    Wg = synth.make_weights(wl, device=dev)
    flush_rows = torch.ones(16384, 8192, dtype=torch.int32, device=dev)   # 512 MiB
    flush_out = torch.empty(16384, dtype=torch.int32, device=dev)

    def flush():
        # reads the whole buffer, writes 64 KiB; a row-wise reduction needs no
        # cross-block semaphores (no memset node when captured)
        torch.amax(flush_rows, dim=1, out=flush_out)

    G = args.graph_reps

    def capture(fn):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    graph_flush = None if args.no_graph else capture(lambda: [flush() for _ in range(G)])

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
        g_cold = g_warm = None
        if not args.no_graph:
            def cold_body(fwd=fwd):
                for _ in range(G):
                    flush()
                    fwd()

            def warm_body(fwd=fwd):
                for _ in range(G):
                    fwd()

            g_cold = capture(cold_body)
            g_warm = capture(warm_body)
        # router scoring + top-k on the same token batch (context: the step
        # before the timed forward), timed the same way
        ids_r = torch.empty(T, wl.top_k, dtype=torch.int32, device=dev)
        w_r = torch.empty(T, wl.top_k, dtype=torch.float32, device=dev)

        def route(tok=tok, ids_r=ids_r, w_r=w_r):
            return binding.route_topk(tok.logits, wl.top_k, out=(ids_r, w_r))

        route()
        g_route = None
        if not args.no_graph:
            def route_body(route=route):
                for _ in range(G):
                    flush()
                    route()

            g_route = capture(route_body)
        stage_b, total_b, total_f, stage_f, D, Rv = workload_bytes_flops(wl, tok.topk_ids.cpu(), T)
        cases.append(dict(T=T, tok=tok, fwd=fwd, g_cold=g_cold, g_warm=g_warm, plan=plan,
                          route=route, g_route=g_route, router=[],
                          stage_bytes=stage_b,
                          bytes=total_b, flops=total_f, stage_flops=stage_f, D=D, Rv=Rv,
                          cold=[], warm=[], stages={s: [] for s in STAGES}))
        log(f"[bench] T={T}: plan path={plan.path} block_m={plan.block_m} "
            f"k_slice={plan.k_slice} touched experts={D}")

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev2 = torch.cuda.Event(enable_timing=True)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(8)]

    def step(record):
        for c in cases:
            if c["g_cold"] is not None:
                # G x (evict, forward) minus G x (evict): per-forward device time
                # without the per-launch submission latency
                ev0.record()
                graph_flush.replay()
                ev1.record()
                c["g_cold"].replay()
                ev2.record()
            else:
                flush()
                ev0.record()
                c["fwd"]()
                ev1.record()
            flush()
            c["fwd"](stage_events=evs)
            evs[7 if c["plan"].path == 1 else 5].synchronize()
            if record:
                if c["g_cold"] is not None:
                    c["cold"].append((ev1.elapsed_time(ev2) - ev0.elapsed_time(ev1)) * 1e3 / G)
                else:
                    c["cold"].append(ev0.elapsed_time(ev1) * 1e3)
                for si, name in enumerate(STAGES):
                    if name in ("route_prep", "combine") and c["plan"].path == 2:
                        continue
                    c["stages"][name].append(evs[2 * si].elapsed_time(evs[2 * si + 1]) * 1e3)
            # router, cold, outside the forward's timing
            if c["g_route"] is not None:
                ev0.record()
                graph_flush.replay()
                ev1.record()
                c["g_route"].replay()
                ev2.record()
            else:
                flush()
                ev0.record()
                c["route"]()
                ev1.record()
                ev2.record()
            ev2.synchronize()
            if record:
                c["router"].append(((ev1.elapsed_time(ev2) - ev0.elapsed_time(ev1)) / G
                                    if c["g_route"] is not None else ev0.elapsed_time(ev1)) * 1e3)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"[bench] timed {args.steps} steps in {wall:.2f} s")

    # warm context: G back-to-back forwards in one graph (caches hold what fits)
    for c in cases:
        for _ in range(3):
            ev0.record()
            if c["g_warm"] is not None:
                c["g_warm"].replay()
            else:
                for _ in range(G):
                    c["fwd"]()
            ev1.record()
            ev1.synchronize()
            c["warm"].append(ev0.elapsed_time(ev1) * 1e3 / G)

    lat_cold = {c["T"]: statistics.fmean(c["cold"]) for c in cases}
    lat_warm = {c["T"]: statistics.median(c["warm"]) for c in cases}
    geo = math.exp(sum(math.log(v) for v in lat_cold.values()) / len(lat_cold))
    table = {}
    per_kernel = {}   # kernel -> list of (duration us, algorithmic bytes, flops) per launch
    for c in cases:
        T = c["T"]
        st = {k: statistics.fmean(v) for k, v in c["stages"].items() if v}
        down_key = "down_gemm_fused" if c["plan"].path == 2 else "down_gemm"
        row = {
            "latency_us_cold": round(lat_cold[T], 3),
            "latency_us_cold_median": round(statistics.median(c["cold"]), 3),
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
            "router_us_cold": round(statistics.fmean(c["router"]), 3) if c["router"] else None,
            "stage_kernel": {k: kernel_name(wl, c["plan"], k) for k in st},
        }
        for k, v in st.items():
            key = down_key if k == "down_gemm" else k
            if key in c["stage_bytes"] and v > 0:
                row.setdefault("stage_gbps", {})[k] = round(c["stage_bytes"][key] / v / 1e3, 1)
                per_kernel.setdefault(kernel_name(wl, c["plan"], k), []).append(
                    (v, c["stage_bytes"][key], c["stage_flops"].get(key, 0.0), T))
        table[str(T)] = row

    # dominant kernel: largest summed duration over the sweep; achieved = mean
    # algorithmic bytes per launch / mean launch duration
    kname, launches = max(per_kernel.items(), key=lambda kv: sum(x[0] for x in kv[1]))
    dur = statistics.fmean(x[0] for x in launches)
    bts = statistics.fmean(x[1] for x in launches)
    fl = statistics.fmean(x[2] for x in launches)
    achieved = bts / dur / 1e3
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(kname, [x[3] for x in launches]),
                "kernel": kname, "tokens": [x[3] for x in launches],
                "avg_launch_us": round(dur, 3),
                "algorithmic_bytes_per_launch": int(bts),
                "mfma_frac": round(fl / dur / 1e6 / MFMA_PEAK_TFLOPS[dtype_name], 4)}

    cpu = None
    if not args.no_cpu_baseline:
        res, cores, passes = cpu_baseline(wl, Wg, args.cpu_budget_s, args.cpu_min_s)
        done = sorted(res)
        gpu_same = math.exp(sum(math.log(lat_cold[t]) for t in done) / len(done))
        cpu_geo = math.exp(sum(math.log(res[t]) for t in done) / len(done))
        cpu = {"value": round(cpu_geo, 1), "unit": "us", "cores": cores, "kind": "oracle",
               "sample": f"{wl.name}, {passes} pass(es) of one oracle forward at each T in {done} "
                         f"(geometric mean over T of the mean per-forward latency); GPU geomean "
                         f"over the same T: "
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
                                "device time of one forward: (graph of G x (cache eviction, "
                                "forward) - graph of G x eviction) / G, mean over the timed "
                                "steps",
            "graph_reps": G,
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
