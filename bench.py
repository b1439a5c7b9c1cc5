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
import dataclasses
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
        if plan.splitk_chunks and plan.act_in_down:
            return f"up_splitk_kernel<{dt}, {lay}, 2>"
        if plan.splitk_chunks:
            return (f"up_splitk_kernel<{dt}, {lay}, 2> + "
                    f"splitk_act_kernel<{dt}, {'true' if wl.gated else 'false'}>")
        return f"tile_gemm_kernel<{dt}, {lay}, {0 if wl.gated else 1}>"
    if wl.inter <= 256:   # the reduction fits the resident down kernel
        nkb = 1 if wl.inter <= 128 else 2
        if plan.act_in_down:   # activations formed from the split-K partials
            return f"down_resident_kernel<{dt}, {lay}, {nkb}, true>"
        return f"down_resident_kernel<{dt}, {lay}, {nkb}, false>"
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
                               layout=(oracle.Q_PER_CHANNEL if wl.per_channel else
                                       oracle.Q_FP4_GROUP_K if wl.fp4 else oracle.Q_GROUP_K),
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



# SQ counters of one --counter-pass run under rocprofv3 --pmc (one pass: 8 SQ
# counters and GRBM_GUI_ACTIVE).  MFMA busy % = SQ_VALU_MFMA_BUSY_CYCLES (summed
# over the 1024 SIMDs) / (GRBM_GUI_ACTIVE of one XCD * 1024), the form of
# rocprofv3's derived MfmaUtil; the CSV holds GRBM_GUI_ACTIVE summed over the
# 8 XCDs.  Counted MFMA flops are the MOPS counters times 512 (their unit).
SQ_SET = ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
          "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS",
          "SQ_LDS_BANK_CONFLICT", "SQ_WAVES")
SIMDS = 256 * 4
XCDS = 8
GPU_CLOCK_GHZ = 2.4


def counter_agg(path, args, sweep):
    """{(T, kernel): {"n", "ns", "c": {counter: sum}}} from the counter CSV of a
    --counter-pass run (launches in sweep order, --steps per T)."""
    import csv
    import re

    with open(path) as f:
        rows = list(csv.DictReader(f))
    by_disp = {}
    for r in rows:
        d = by_disp.setdefault(r["Dispatch_Id"], {"kernel": r["Kernel_Name"], "c": {},
                                                  "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d["c"][r["Counter_Name"]] = d["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    disp = [by_disp[k] for k in sorted(by_disp, key=int)]
    # dispatches come in sweep order: each forward launches the same kernel
    # sequence for a T, --steps times
    def short(k):
        k = k.replace("void w4moe::", "").replace("w4moe::", "")
        return re.sub(r"\([\w ,:*&]*\)$", "", k)

    # split into forwards: the first kernel of a forward is route preparation
    # (grouped path) or small_h_kernel (small batch); a chunked preparation
    # is two launches, rank then scatter
    starts = [j for j, d in enumerate(disp)
              if "rp_one" in d["kernel"] or "rp_rank" in d["kernel"]
              or "small_h_kernel" in d["kernel"]]
    fwd = [disp[a:b] for a, b in zip(starts, starts[1:] + [len(disp)])]
    if len(fwd) != args.steps * len(sweep):
        raise SystemExit(f"{len(fwd)} forwards in the counter file, expected {args.steps} x {len(sweep)}")
    agg = {}
    for ti, T in enumerate(sweep):
        for f in fwd[ti * args.steps:(ti + 1) * args.steps]:
            for d in f:
                a = agg.setdefault((T, short(d["kernel"])), {"n": 0, "ns": 0.0, "c": {}})
                a["n"] += 1
                a["ns"] += d["ns"]
                for k, v in d["c"].items():
                    a["c"][k] = a["c"].get(k, 0.0) + v
    return agg


def summarize_sq(args, sweep):
    """A text table per kernel and token count from the counter CSV of a
    --counter-pass run (launches in sweep order, --steps per T)."""
    agg = counter_agg(args.summarize_sq, args, sweep)
    lines = []
    hdr = ("T", "kernel", "us/launch", "MFMA busy %", "MFMA TFLOP/s counted", "frac of 2.5 PF",
           "VALU insts", "MFMA insts", "VALU:MFMA", "LDS insts", "LDS bank-conflict cycles")
    lines.append(" | ".join(hdr))
    for (T, k), a in agg.items():
        n = a["n"]
        c = {kk: v / n for kk, v in a["c"].items()}
        us = a["ns"] / n / 1e3
        gui = c.get("GRBM_GUI_ACTIVE", 0.0)
        # GRBM_GUI_ACTIVE comes summed over the XCDs' GRBM instances
        util = 100.0 * c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (gui / XCDS * SIMDS) if gui else 0.0
        flops = 512.0 * (c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + c.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0))
        tf = flops / (us * 1e-6) / 1e12 if us > 0 else 0.0
        valu, mfma = c.get("SQ_INSTS_VALU", 0.0), c.get("SQ_INSTS_MFMA", 0.0)
        lines.append(" | ".join([str(T), k, f"{us:.1f}", f"{util:.1f}", f"{tf:.1f}",
                                 f"{tf / MFMA_PEAK_TFLOPS['bf16']:.3f}", f"{valu:.3e}",
                                 f"{mfma:.3e}", f"{valu / mfma:.2f}" if mfma else "-",
                                 f"{c.get('SQ_INSTS_LDS', 0.0):.3e}",
                                 f"{c.get('SQ_LDS_BANK_CONFLICT', 0.0):.3e}"]))
    print("\n".join(lines))


# Stall and latency counters, one rocprofv3 --pmc pass each (STALL_PASSES).
# VmemLatency and LdsLatency are rocprofv3's derived cycles per vector-memory
# (LDS) instruction in flight; the SQ_WAIT_* / SQ_ACTIVE_* counters are
# wave-cycles, divided here by SQ_WAVE_CYCLES (the share of a wave's life).
STALL_PASSES = (
    ("VmemLatency",),
    ("LdsLatency",),
    ("SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY",
     "SQ_ACTIVE_INST_VMEM", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS"),
    ("MemUnitStalled", "TCP_TCC_READ_REQ_LATENCY_sum", "TCP_TCC_READ_REQ_sum"),
)


def summarize_stalls(args, sweep):
    """A text table of STALL_PASSES per kernel and token count from the
    counter CSVs of one --counter-pass run per pass (comma list, pass order)."""
    merged = {}
    for path in args.summarize_stalls.split(","):
        for key, a in counter_agg(path, args, sweep).items():
            m = merged.setdefault(key, {"n": a["n"], "ns": a["ns"], "c": {}})
            for k, v in a["c"].items():
                m["c"][k] = v / a["n"]
    lines = [" | ".join(("T", "kernel", "us/launch", "VMEM latency cyc", "LDS latency cyc",
                         "TA stalled %", "L1->L2 read latency cyc", "waiting %", "waiting to issue %",
                         "issuing %", "VALU issuing %"))]
    for (T, k), m in merged.items():
        c = m["c"]
        wc = c.get("SQ_WAVE_CYCLES", 0.0)
        pct = (lambda x: f"{100.0 * c.get(x, 0.0) / wc:.0f}") if wc else (lambda x: "-")
        rq = c.get("TCP_TCC_READ_REQ_sum", 0.0)
        lat = f"{c.get('TCP_TCC_READ_REQ_LATENCY_sum', 0.0) / rq:.0f}" if rq else "-"
        lines.append(" | ".join([str(T), k, f"{m['ns'] / m['n'] / 1e3:.1f}",
                                 f"{c.get('VmemLatency', 0.0):.0f}", f"{c.get('LdsLatency', 0.0):.0f}",
                                 f"{c.get('MemUnitStalled', 0.0):.1f}", lat, pct("SQ_WAIT_ANY"),
                                 pct("SQ_WAIT_INST_ANY"), pct("SQ_ACTIVE_INST_ANY"),
                                 pct("SQ_ACTIVE_INST_VALU")]))
    print("\n".join(lines))


def summarize_trace(args):
    """A markdown table of the library's kernels from the kernel_stats.csv of a
    rocprofv3 --kernel-trace --stats run (all launches of the run)."""
    import csv
    import re

    with open(args.summarize_trace) as f:
        rows = list(csv.DictReader(f))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = ["| kernel | calls | avg us | min us | max us | share of GPU time % |",
             "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"]
        if "w4moe" not in name:
            continue
        short = re.sub(r"\(w4moe::\w+\)$", "", name.replace("void w4moe::", "").replace("w4moe::", ""))
        short = re.sub(r"\([\w ,:*&]*\)$", "", short).replace("(anonymous namespace)::", "")
        lines.append(f"| {short} | {int(r['Calls'])} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{100.0 * float(r['TotalDurationNs']) / total:.2f} |")
    print("\n".join(lines))


def sweep_of(wl, args, headline):
    if headline and args.tokens:
        return [int(t) for t in args.tokens.split(",")]
    return list(wl.tokens)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workloads", default="kimi_tp8,deepseek_local,per_channel,relu2_skew,tiny,"
                                           "kimi_tp8_fp4,deepseek_local_fp4",
                    help="comma list; the first is the headline (value, roofline, cpu_baseline), "
                         "the others are reported under other_workloads")
    ap.add_argument("--workload", default="kimi_tp8",
                    help="workload of --counter-pass / --summarize-* runs")
    ap.add_argument("--tokens", default="", help="comma list for the headline workload "
                                                 "(default: its sweep)")
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
    ap.add_argument("--summarize-sq", metavar="CSV",
                    help="print a table of the SQ counters (SQ_SET) of a --counter-pass run")
    ap.add_argument("--summarize-stalls", metavar="CSVS",
                    help="print a table of the stall counters (STALL_PASSES) from one "
                         "--counter-pass run per pass (comma list of their CSVs, in pass order)")
    ap.add_argument("--summarize-trace", metavar="CSV",
                    help="print a table of the library's kernels from a rocprofv3 "
                         "--kernel-trace --stats kernel_stats.csv")
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

    if args.summarize_trace:
        summarize_trace(args)
        return

    import torch

    from w4a16_mixture_experts_amd import binding, synth

    if args.summarize_counters or args.summarize_sq or args.summarize_stalls:
        sweep = [int(t) for t in args.tokens.split(",")] if args.tokens else \
            list(synth.WORKLOADS[args.workload].tokens)
        if args.summarize_counters:
            summarize_counters(args, sweep)
        elif args.summarize_sq:
            summarize_sq(args, sweep)
        else:
            summarize_stalls(args, sweep)
        return
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    binding.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.counter_pass:
        wl = synth.WORKLOADS[args.workload]
        sweep = [int(t) for t in args.tokens.split(",")] if args.tokens else list(wl.tokens)
        counter_pass(args, wl, sweep, dev)
        return

    names = [n for n in args.workloads.split(",") if n]
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

    def cold_graph(fn):
        def body(fn=fn):
            for _ in range(G):
                flush()
                fn()
        return None if args.no_graph else capture(body)

    # the streaming-read probe reads a buffer of the weight bytes a forward
    # streams; one buffer as large as the largest such count
    weights, cases = {}, []
    for wi, name in enumerate(names):
        wl = synth.WORKLOADS[name]
        log(f"[bench] generating {wl.name} weights on the GPU")
        Wg = synth.make_weights(wl, device=dev)
        weights[name] = Wg
        for T in sweep_of(wl, args, wi == 0):
            tok = synth.make_tokens(wl, T).to(dev)
            desc = binding.desc_for(wl, T)
            plan = binding.get_plan(desc)
            ws = torch.empty(max(1, binding.workspace_size(desc)), dtype=torch.uint8, device=dev)
            out = torch.empty(T, wl.hidden, dtype=wl.dtype, device=dev)

            def fwd(tok=tok, ws=ws, out=out, Wg=Wg, wl=wl, **kw):
                return binding.forward_workload(wl, Wg, tok, out=out, workspace=ws, **kw)

            fwd()
            torch.cuda.synchronize()
            g_cold = cold_graph(fwd)
            g_warm = None
            if not args.no_graph:
                def warm_body(fwd=fwd):
                    for _ in range(G):
                        fwd()
                g_warm = capture(warm_body)
            # router scoring + top-k on the same token batch (context: the step
            # before the timed forward), timed the same way
            ids_r = torch.empty(T, wl.top_k, dtype=torch.int32, device=dev)
            w_r = torch.empty(T, wl.top_k, dtype=torch.float32, device=dev)

            def route(tok=tok, ids_r=ids_r, w_r=w_r, k=wl.top_k):
                return binding.route_topk(tok.logits, k, out=(ids_r, w_r))

            route()
            g_route = cold_graph(route)
            # the forward with the router fused in (same token batch, from its logits)
            out_r = torch.empty(T, wl.hidden, dtype=wl.dtype, device=dev)
            ids_f = torch.empty(T, wl.top_k, dtype=torch.int32, device=dev)
            w_f = torch.empty(T, wl.top_k, dtype=torch.float32, device=dev)
            ws_r = torch.empty(max(1, binding.workspace_size(desc)), dtype=torch.uint8,
                               device=dev)

            def routed(tok=tok, out_r=out_r, ids_f=ids_f, w_f=w_f, ws_r=ws_r, Wg=Wg, wl=wl, **kw):
                return binding.forward_workload_routed(wl, Wg, tok, out=out_r, ids_out=(ids_f, w_f),
                                                       workspace=ws_r, **kw)

            routed()
            g_routed = cold_graph(routed)
            # the fused finalize mode (grouped path): the combine inside the
            # down launch, reported beside the default non-fused mode
            fused = None
            g_fused = None
            if plan.path == 1:
                ws_f = torch.empty(max(1, binding.workspace_size(binding.desc_for(
                    wl, T, fused_finalize=1))), dtype=torch.uint8, device=dev)
                out_f = torch.empty(T, wl.hidden, dtype=wl.dtype, device=dev)

                def fused(tok=tok, ws_f=ws_f, out_f=out_f, Wg=Wg, wl=wl):
                    return binding.forward_workload(wl, Wg, tok, out=out_f, workspace=ws_f,
                                                    fused_finalize=1)

                fused()
                g_fused = cold_graph(fused)
            # per-channel weights re-laid once into the group layout (setup,
            # outside the timed region): the forward then takes the group
            # layout's kernels; reported beside the per-channel forward
            rep = None
            g_rep = None
            if wl.per_channel:
                if name + "/group" not in weights:
                    p13, s13 = binding.repack_per_channel(Wg.w13_packed, Wg.w13_scales)
                    p2, s2 = binding.repack_per_channel(Wg.w2_packed, Wg.w2_scales)
                    weights[name + "/group"] = synth.Weights(p13, s13, p2, s2)
                Wr = weights[name + "/group"]
                wlr = dataclasses.replace(wl, per_channel=False)
                ws_g = torch.empty(max(1, binding.workspace_size(binding.desc_for(wlr, T))),
                                   dtype=torch.uint8, device=dev)
                out_g = torch.empty(T, wl.hidden, dtype=wl.dtype, device=dev)

                def rep(tok=tok, ws_g=ws_g, out_g=out_g, Wr=Wr, wlr=wlr):
                    return binding.forward_workload(wlr, Wr, tok, out=out_g, workspace=ws_g)

                rep()
                g_rep = cold_graph(rep)
            stage_b, total_b, total_f, stage_f, D, Rv = workload_bytes_flops(
                wl, tok.topk_ids.cpu(), T)
            cases.append(dict(wl=wl, head=wi == 0, T=T, tok=tok, fwd=fwd, g_cold=g_cold,
                              g_warm=g_warm, plan=plan, route=route, g_route=g_route, router=[],
                              routed=routed, g_routed=g_routed, routed_cold=[], routed_stage=[],
                              fused=fused, g_fused=g_fused, fused_cold=[],
                              rep=rep, g_rep=g_rep, rep_cold=[],
                              stage_bytes=stage_b, bytes=total_b, flops=total_f,
                              stage_flops=stage_f, D=D, Rv=Rv,
                              wbytes=D * weight_bytes_per_expert(wl),
                              cold=[], warm=[], probe=[], stages={s: [] for s in STAGES}))
            log(f"[bench] {wl.name} T={T}: plan path={plan.path} splitk={plan.splitk_chunks} "
                f"k_slice={plan.k_slice} touched experts={D}")

    pbytes = max(c["wbytes"] for c in cases)
    probe_buf = torch.zeros(pbytes + 8192, dtype=torch.uint8, device=dev)
    probe_sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for c in cases:
        row = probe_row_bytes(c["wl"])
        nb = c["wbytes"] // row * row

        def probe(nb=nb, row=row):
            binding.stream_probe(probe_buf, nb, row, probe_sink)

        probe()
        c["g_probe"] = cold_graph(probe)
        c["probe_fn"] = probe
        c["probe_bytes"] = nb
    torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev2 = torch.cuda.Event(enable_timing=True)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
    evs_r = [torch.cuda.Event(enable_timing=True) for _ in range(8)]

    def time_cold(g, fn):
        """Device time of fn on cold caches: graph difference, or eager."""
        if g is not None:
            ev0.record()
            graph_flush.replay()
            ev1.record()
            g.replay()
            ev2.record()
            ev2.synchronize()
            return (ev1.elapsed_time(ev2) - ev0.elapsed_time(ev1)) * 1e3 / G
        flush()
        ev0.record()
        fn()
        ev1.record()
        ev1.synchronize()
        return ev0.elapsed_time(ev1) * 1e3

    def step(record):
        for c in cases:
            t_cold = time_cold(c["g_cold"], c["fwd"])
            flush()
            c["fwd"](stage_events=evs)
            evs[7 if c["plan"].path == 1 else 5].synchronize()
            t_route = time_cold(c["g_route"], c["route"])
            t_probe = time_cold(c["g_probe"], c["probe_fn"])
            t_routed = time_cold(c["g_routed"], c["routed"])
            t_fused = time_cold(c["g_fused"], c["fused"]) if c["fused"] is not None else None
            t_rep = time_cold(c["g_rep"], c["rep"]) if c["rep"] is not None else None
            # first stage of the routed forward: routing fused with route
            # preparation (grouped path) or with the gate/up GEMM (small batch)
            si = 0 if c["plan"].path == 1 else 1
            flush()
            c["routed"](stage_events=evs_r)
            evs_r[7 if c["plan"].path == 1 else 5].synchronize()
            t_rstage = evs_r[2 * si].elapsed_time(evs_r[2 * si + 1]) * 1e3
            if record:
                c["cold"].append(t_cold)
                c["router"].append(t_route)
                c["probe"].append(t_probe)
                c["routed_cold"].append(t_routed)
                c["routed_stage"].append(t_rstage)
                if t_fused is not None:
                    c["fused_cold"].append(t_fused)
                if t_rep is not None:
                    c["rep_cold"].append(t_rep)
                for si, name in enumerate(STAGES):
                    if name in ("route_prep", "combine") and c["plan"].path == 2:
                        continue
                    c["stages"][name].append(evs[2 * si].elapsed_time(evs[2 * si + 1]) * 1e3)

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

    def report(wcases):
        wl = wcases[0]["wl"]
        dtype_name = "fp16" if wl.dtype == torch.float16 else "bf16"
        lat_cold = {c["T"]: statistics.fmean(c["cold"]) for c in wcases}
        lat_warm = {c["T"]: statistics.median(c["warm"]) for c in wcases}
        geo = math.exp(sum(math.log(v) for v in lat_cold.values()) / len(lat_cold))
        table = {}
        per_kernel = {}   # kernel -> list of (duration us, algorithmic bytes, flops, T) per launch
        for c in wcases:
            T = c["T"]
            st = {k: statistics.fmean(v) for k, v in c["stages"].items() if v}
            down_key = "down_gemm_fused" if c["plan"].path == 2 else "down_gemm"
            pr = statistics.fmean(c["probe"])
            row = {
                "latency_us_cold": round(lat_cold[T], 3),
                "latency_us_cold_median": round(statistics.median(c["cold"]), 3),
                "latency_us_warm": round(lat_warm[T], 3),
                "hbm_gbps_cold": round(c["bytes"] / lat_cold[T] / 1e3, 1),
                "hbm_frac_cold": round(c["bytes"] / lat_cold[T] / 1e3 / HBM_PEAK_GBS, 4),
                "tflops_cold": round(c["flops"] / lat_cold[T] / 1e6, 2),
                "mfma_frac_cold": round(c["flops"] / lat_cold[T] / 1e6 /
                                        MFMA_PEAK_TFLOPS[dtype_name], 4),
                "algorithmic_bytes": int(c["bytes"]),
                "touched_experts": c["D"],
                "valid_routes": c["Rv"],
                "plan": {"path": "small-batch" if c["plan"].path == 2 else "grouped",
                         "splitk_chunks": c["plan"].splitk_chunks,
                         "fp16_route": c["plan"].fp16_route},
                "stage_us": {k: round(v, 3) for k, v in st.items()},
                "router_us_cold": round(statistics.fmean(c["router"]), 3),
                "fused_finalize_us_cold": (round(statistics.fmean(c["fused_cold"]), 3)
                                           if c["fused_cold"] else None),
                "group_layout_repacked_us_cold": (round(statistics.fmean(c["rep_cold"]), 3)
                                                  if c["rep_cold"] else None),
                "routed": {
                    "latency_us_cold": round(statistics.fmean(c["routed_cold"]), 3),
                    "fused_stage": ("routing + route preparation (one launch up to 16 tokens)"
                                    if c["plan"].path == 1 else
                                    "routing + gate/up GEMM (one launch up to 16 routes and "
                                    "512 gate/up workgroups)"),
                    "fused_stage_us": round(statistics.fmean(c["routed_stage"]), 3),
                    "unfused_us": round(statistics.fmean(c["router"]) + st.get(
                        "route_prep" if c["plan"].path == 1 else "gate_up_gemm", 0.0), 3),
                },
                "stream_probe": {"bytes": c["probe_bytes"], "us_cold": round(pr, 3),
                                 "gbps": round(c["probe_bytes"] / pr / 1e3, 1),
                                 "frac": round(c["probe_bytes"] / pr / 1e3 / HBM_PEAK_GBS, 4),
                                 "forward_over_probe": round(lat_cold[T] / pr, 3)},
                "stage_kernel": {k: kernel_name(wl, c["plan"], k) for k in st},
            }
            for k, v in st.items():
                key = down_key if k == "down_gemm" else k
                if key in c["stage_bytes"] and v > 0:
                    row.setdefault("stage_gbps", {})[k] = round(c["stage_bytes"][key] / v / 1e3, 1)
                    per_kernel.setdefault(kernel_name(wl, c["plan"], k), []).append(
                        (v, c["stage_bytes"][key], c["stage_flops"].get(key, 0.0), T))
            table[str(T)] = row
        # dominant kernel: largest summed duration over the sweep; achieved =
        # mean algorithmic bytes per launch / mean launch duration
        kname, launches = max(per_kernel.items(), key=lambda kv: sum(x[0] for x in kv[1]))
        dur = statistics.fmean(x[0] for x in launches)
        bts = statistics.fmean(x[1] for x in launches)
        fl = statistics.fmean(x[2] for x in launches)
        achieved = bts / dur / 1e3
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(kname, [x[3] for x in launches]),
                "kernel": kname, "tokens": [x[3] for x in launches],
                "avg_launch_us": round(dur, 3),
                "algorithmic_bytes_per_launch": int(bts),
                "mfma_frac": round(fl / dur / 1e6 / MFMA_PEAK_TFLOPS[dtype_name], 4)}
        return wl, dtype_name, lat_cold, geo, table, roof

    head_cases = [c for c in cases if c["head"]]
    wl, dtype_name, lat_cold, geo, table, roofline = report(head_cases)
    others = {}
    for name in names[1:]:
        wc = [c for c in cases if c["wl"].name == name]
        owl, odt, olat, ogeo, otable, oroof = report(wc)
        others[name] = {"workload": describe(owl), "dtype": odt, "tokens": list(olat),
                        "geomean_us_cold": round(ogeo, 3), "per_tokens": otable,
                        "dominant_kernel": oroof}

    cpu = None
    if not args.no_cpu_baseline:
        res, cores, passes = cpu_baseline(wl, weights[wl.name], args.cpu_budget_s, args.cpu_min_s)
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
        "ms_per_step": round(sum(statistics.fmean(c["cold"]) for c in cases) / 1e3, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_name,
        "data": "synthetic",
        "config": {
            "workload": describe(wl),
            "tokens": list(lat_cold),
            "value_definition": "geometric mean over the token sweep of the cold-cache "
                                "device time of one forward: (graph of G x (cache eviction, "
                                "forward) - graph of G x eviction) / G, mean over the timed "
                                "steps",
            "graph_reps": G,
            "parallelism": "single GPU",
            "per_tokens": table,
            "wall_s_timed_region": round(wall, 3),
            "step": "one cold forward at every token count of every listed workload "
                    "(the headline and other_workloads), plus the router, the forward "
                    "with the router fused in, and the streaming-read probe at the same "
                    "token counts",
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "other_workloads": others,
    }
    print(json.dumps(line), flush=True)


def describe(wl):
    return (f"{wl.name}: {wl.num_experts} local experts (of {wl.num_global_experts}), "
            f"hidden {wl.hidden}, intermediate {wl.inter}, top-{wl.top_k}, "
            f"{'FP4 (MXFP4) group-32' if wl.fp4 else 'INT4 per-channel' if wl.per_channel else 'INT4 group-32'}, "
            f"{'SiLU-gated' if wl.gated else 'ReLU^2'}")


def weight_bytes_per_expert(wl):
    E, H, I, N1 = wl.num_experts, wl.hidden, wl.inter, wl.n1
    if wl.per_channel:
        return N1 * H // 2 + N1 * 2 + H * I // 2 + H * 2
    return N1 * H // 2 + N1 * (H // 32) * 2 + H * I // 2 + H * (I // 32) * 2


def probe_row_bytes(wl):
    """Row length of the probe: a packed gate/up weight row (H/2 bytes in the
    group layout, H bytes per channel pair), rounded down to 64 bytes."""
    r = wl.hidden if wl.per_channel else wl.hidden // 2
    return max(64, min(8192, r // 64 * 64))


if __name__ == "__main__":
    main()
