#!/usr/bin/env python3
"""Benchmark of one GPU's share of the MoE expert-parallel layer (MI355X).

One step = the 1F1B two-micro-batch step of the expert-parallel overlap pages
(1F1B note page 2, "MoE 1F1B overlap"): the forward of one micro-batch and the
backward (dgrad, then wgrad deferred past the other's expert GEMMs) of the other,
on two streams, so that every step passes T tokens through the whole layer
forward and backward.  Throughput = T / step time (tokens/s).  Inputs are
synthetic (seeded), resident in HBM before the timed region.

Prints ONE JSON line on stdout; diagnostics go to stderr.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "MoE layer fwd+bwd tokens/s on 1 MI355X; grouped-GEMM MFMA util %; dispatch HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 (and fp16) matrix-core peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak

GEMM_KERNELS = ("ffn_gate_up", "ffn_down", "dgrad_act", "dgrad_in", "wgrad")
COPY_PROBE_BYTES = 1 << 30
TRAFFIC_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")


def err(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(w, N, T_loc):
    """Algorithmic work per step (one launch of each, plus the shared expert's
    launches of the same GEMMs over all T tokens when the workload has one):
    flops for the GEMMs, HBM bytes for the permute kernels (one pass over each
    operand, no re-reads)."""
    d, F, T, K, E = w.d, w.F, w.T, w.K, w.E
    b = 4 if w.dtype == "f32" else 2
    Fs = w.F_s
    return {
        "ffn_gate_up": ("flop", 2.0 * N * d * 2 * F + 2.0 * T * d * 2 * Fs),
        "ffn_down": ("flop", 2.0 * N * F * d + 2.0 * T * Fs * d),
        "dgrad_act": ("flop", 2.0 * N * d * F + 2.0 * T * d * Fs),
        "dgrad_in": ("flop", 2.0 * N * 2 * F * d + 2.0 * T * 2 * Fs * d),
        "wgrad": ("flop", 6.0 * N * d * F + 6.0 * T * d * Fs),
        "router": ("flop", 2.0 * T * d * E),
        # router weight gradient x^T dlogits on the matrix cores (bf16 data);
        # the two-term split of dlogits forms it twice, counted once here
        "dwr_mfma": ("flop", 2.0 * T * d * E),
        # x rows of tokens with a local expert + row map -> N rows
        "permute": ("byte", T_loc * d * b + 4.0 * T * K + N * d * b),
        # y_p rows + gates + row map -> out
        "combine": ("byte", N * d * b + 8.0 * T * K + T * d * b),
        # dout + y_p rows + gates + map -> dy_p rows + dgates
        "combine_bwd": ("byte", T * d * b + 2.0 * N * d * b + 12.0 * T * K),
        # dx_p rows + map -> dx
        "dispatch_bwd": ("byte", N * d * b + 4.0 * T * K + T * d * b),
    }


KERNEL_SOURCE = {k: "gemm_mfma.hip" for k in GEMM_KERNELS}
KERNEL_SOURCE.update({k: "dispatch.hip" for k in ("permute", "combine", "combine_bwd",
                                                  "dispatch_bwd")})


def kernel_source_hash(name):
    """sha256 of the source that defines kernel `name` and the shared header."""
    import hashlib
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "combine_expert_ffn_amd",
                        "csrc")
    h = hashlib.sha256()
    for f in (KERNEL_SOURCE[name], "moe_internal.h"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic(workload):
    """Per-launch HBM bytes of each kernel from the committed counter summary
    (rocprofv3 FETCH_SIZE and WRITE_SIZE, scaled by the copy probe), keeping
    only kernels whose source is unchanged since the counters were taken."""
    import re
    path = os.path.join(TRAFFIC_DIR, f"traffic_{workload}.md")
    if not os.path.exists(path):
        return {}
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), flags=re.S)
    if not m:
        return {}
    rec = json.loads(m.group(1))
    out = {}
    for name, ent in rec.get("kernels", {}).items():
        if name in KERNEL_SOURCE and ent.get("source_sha256") == kernel_source_hash(name):
            out[name] = ent["hbm_bytes_per_launch"]
    return out


def cpu_oracle_baseline(w, inp, target_s=10.0):
    """The oracle as it stands, timed on this host on the first Ts tokens of the
    workload (full weights), one forward + backward; Ts grown until the run
    takes about target_s seconds."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    fb = w.route == "force_balance"
    X = {k: (None if v is None else np.asarray(v, np.float64)) for k, v in inp.items()}

    def run(Ts):
        t0 = time.perf_counter()
        f = O.layer_forward(X["x"][:Ts], w.K, w.e_lo, w.E_l, X["W_gu"], X["W_down"],
                            W_r=X["W_r"], bias=X["bias"], E=w.E, force_balance=fb,
                            gates=None if X["gates"] is None else X["gates"][:Ts],
                            prec=w.dtype)
        O.layer_backward(f, X["x"][:Ts], X["dout"][:Ts], X["W_gu"], X["W_down"], W_r=X["W_r"],
                         differentiate_router=not fb, prec=w.dtype)
        return time.perf_counter() - t0

    Ts = min(w.T, 64)
    el = run(Ts)
    while el < target_s / 4 and Ts < w.T:
        Ts = min(w.T, max(Ts * 2, int(Ts * target_s / max(el, 1e-3))))
        el = run(Ts)
    # the whole workload is shorter than the target: repeat it until the
    # sample holds about target_s seconds of CPU work
    reps, total = 1, el
    while total < target_s:
        total += run(Ts)
        reps += 1
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return {"value": reps * Ts / total, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": cpu_model,
            "sample": f"first {Ts} of {w.T} tokens of {w.name}, full weights, {reps} x one "
                      f"forward+backward (float64 numpy, {w.dtype} rounding points), "
                      f"{total:.1f} s"}


def group_plan(K, G0):
    """Steps per captured graph for K timed steps: (G, rem) with G even and
    G * reps + rem == K, rem in {0, 1} (one eager step when K is odd); G0 when
    it divides K, else the largest even divisor of K (or of K - 1) up to 2 G0;
    (None, K) when K is too small for a graph."""
    def best(n):
        if n >= 2 and n % G0 == 0:
            return G0
        c = [g for g in range(2, min(n, 2 * G0) + 1, 2) if n % g == 0]
        return max(c) if c else None

    g = best(K)
    if g:
        return g, 0
    g = best(K - 1) if K > 1 else None
    return (g, 1) if g else (None, K)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="ep16_rank_bf16")
    ap.add_argument("--tokens", type=int, default=None, help="override T of the workload")
    ap.add_argument("--cpu-baseline", choices=("on", "off"), default="on")
    ap.add_argument("--graph", choices=("on", "off"), default="on",
                    help="time the overlapped steps as replays of a HIP graph that holds two "
                         "steps (on) or as eager launches (off)")
    ap.add_argument("--fused-permute", choices=("on", "off"), default="off",
                    help="fuse the permute into the expert GEMMs (MOE_STEP_FUSED_PERMUTE): GEMM1 "
                         "and wgrad read the token rows of x through the dispatch plan, no xp")
    ap.add_argument("--wgrad-order", choices=("mid", "last"), default="mid",
                    help="where the backward micro-batch's wgrad runs on its stream: between the "
                         "two dgrad GEMMs (mid, MOE_STEP_MID_WGRAD) or after the dispatch "
                         "backward (last); the same order is used for the serialized steps")
    ap.add_argument("--pipeline", choices=("on", "off"), default="on",
                    help="run the overlapped steps G at a time through moe_overlap_steps, the "
                         "streams' roles alternating so consecutive steps overlap (on), or one "
                         "moe_overlap_step call per step, joined at every step boundary (off)")
    ap.add_argument("--group", type=int, default=10,
                    help="steps per moe_overlap_steps call and per captured graph (even; "
                         "--steps must be a multiple of it)")
    ap.add_argument("--overlapped-only", action="store_true",
                    help="run only the warm-up and the overlapped steps and print no JSON line: "
                         "the program to trace with rocprofv3 --kernel-trace for the overlap of "
                         "the two streams' kernels")
    ap.add_argument("--serialized-only", action="store_true",
                    help="skip the overlapped steps and print no JSON line: the program to trace "
                         "with rocprofv3 --kernel-trace for per-kernel durations comparable to the "
                         "bench's event timings (taken on the serialized steps)")
    ap.add_argument("--counter-pass", action="store_true",
                    help="run a few serialized steps and a copy probe of known size, print no "
                         "JSON line: the program to run under rocprofv3 --pmc FETCH_SIZE / "
                         "WRITE_SIZE for the per-kernel HBM traffic")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        err("bench.py: measures one GPU's share of the expert-parallel layer; runs on more "
            "than one GPU are not supported.")
        sys.exit(2)

    import torch
    import combine_expert_ffn_amd as M
    from combine_expert_ffn_amd.inputs import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        err("bench.py: no GPU visible")
        sys.exit(1)
    M.lib()  # fails loudly if libmoe.so is not built
    w = WORKLOADS[args.workload]
    if args.tokens:
        w = w.with_tokens(args.tokens)
    err(f"[bench] workload {w.name}: T={w.T} d={w.d} F={w.F} E={w.E} E_l={w.E_l} K={w.K} "
        f"{w.dtype} route={w.route}")
    inp = make_inputs(w, seed=0, microbatches=2)
    s = M.shape_of(w)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}.get(w.dtype, torch.float32)
    D = lambda a: torch.from_numpy(a).to("cuda", tdt)
    F32 = lambda a: torch.from_numpy(a).to("cuda")
    topk = w.route == "topk"
    mode = M.MOE_ROUTE_TOPK if topk else M.MOE_ROUTE_FORCE_BALANCE
    W_gu, W_down = D(inp["W_gu"]), D(inp["W_down"])
    W_r = D(inp["W_r"]) if topk else None
    bias = F32(inp["bias"]) if inp["bias"] is not None else None
    dW_gu = torch.zeros(w.E_l, 2 * w.F, w.d, dtype=torch.float32, device="cuda")
    dW_down = torch.zeros(w.E_l, w.d, w.F, dtype=torch.float32, device="cuda")
    dW_r = torch.zeros(w.d, w.E, dtype=torch.float32, device="cuda") if topk else None
    ws = torch.empty(M.moe_step_workspace_bytes_shared(s, w.F_s), dtype=torch.uint8,
                     device="cuda")
    fused = args.fused_permute == "on"
    pipelined = args.pipeline == "on"
    G = args.group
    if G < 2 or G % 2:
        err("bench.py: --group must be even")
        sys.exit(2)
    # flags of every step: the fused permute and the wgrad's place in the
    # backward stream's order (both leave the results unchanged)
    FUSED = ((M.MOE_STEP_FUSED_PERMUTE if fused else 0) |
             (M.MOE_STEP_MID_WGRAD if args.wgrad_order == "mid" else 0))
    shared = None
    if w.F_s:  # a shared expert beside the routed ones
        shared = (D(inp["W_gu_s"]), D(inp["W_down_s"]),
                  torch.zeros(2 * w.F_s, w.d, dtype=torch.float32, device="cuda"),
                  torch.zeros(w.d, w.F_s, dtype=torch.float32, device="cuda"))
    mbs = [M.MicroBatch(s, x=D(inp["x"]), dout=D(inp["dout"]),
                        gates=None if topk else F32(inp["gates"]), fused=fused, F_s=w.F_s),
           M.MicroBatch(s, x=D(inp["x_b"]), dout=D(inp["dout_b"]),
                        gates=None if topk else F32(inp["gates_b"]), fused=fused, F_s=w.F_s)]
    s0 = torch.cuda.current_stream()
    s1 = torch.cuda.Stream()

    def step(fwd, bwd, flags):
        st = M.make_step(s, mode, W_gu, W_down, dW_gu, dW_down, ws, fwd=fwd, bwd=bwd, W_r=W_r,
                         bias=bias, dW_r=dW_r, accumulate=M.MOE_ACCUM_DW, shared=shared)
        M.moe_overlap_step(st, s0, s1, flags | FUSED)

    def make(i):  # step i forwards one micro-batch and back-propagates the other
        return M.make_step(s, mode, W_gu, W_down, dW_gu, dW_down, ws, fwd=mbs[(i + 1) % 2],
                           bwd=mbs[i % 2], W_r=W_r, bias=bias, dW_r=dW_r,
                           accumulate=M.MOE_ACCUM_DW, shared=shared)

    def issue(i0, n, flags, q):
        """Issue steps i0 .. i0+n-1 on q (and s1): one pipelined moe_overlap_steps
        call per group of G steps for overlapped steps with --pipeline on, else one
        moe_overlap_step call per step."""
        if pipelined and not flags & M.MOE_STEP_SERIALIZE:
            for g0 in range(i0, i0 + n, G):
                M.moe_overlap_steps([make(j) for j in range(g0, min(g0 + G, i0 + n))], q, s1,
                                    flags | FUSED)
        else:
            for j in range(i0, i0 + n):
                M.moe_overlap_step(make(j), q, s1, flags | FUSED)
        return i0 + n

    def run_loop(n, flags, i0):
        return issue(i0, n, flags, s0)

    step(mbs[0], None, 0)  # prime: micro-batch 0 forwarded
    if args.counter_pass:
        run_loop(args.steps, M.MOE_STEP_SERIALIZE, 0)
        # copy probe: a plain elementwise pass (negation) that reads and writes
        # COPY_PROBE_BYTES each, larger than the last-level cache, so the
        # counters' reading for it calibrates bytes per counted KiB
        src = torch.ones(COPY_PROBE_BYTES // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        err(f"[bench] counter pass done: {args.steps} serialized steps, 3 copy probes of "
            f"{COPY_PROBE_BYTES} bytes")
        return
    i = run_loop(args.warmup, 0, 0)
    torch.cuda.synchronize()
    counts = [mbs[k].counts.cpu() for k in range(2)]
    N = int(counts[0].sum())
    T_loc = int((mbs[0].row_of_pair >= 0).any(dim=1).sum())

    if args.serialized_only:
        i = run_loop(args.warmup + args.steps, M.MOE_STEP_SERIALIZE, i)
        torch.cuda.synchronize()
        err(f"[bench] serialized-only pass done: {args.warmup + args.steps} steps")
        return
    # ---- timed region 1: overlapped 1F1B steps (the product schedule) -> value
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(s0)
    i = run_loop(args.steps, 0, i)
    ev1.record(s0)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    err(f"[bench] overlapped: {ms_step:.4f} ms/step (wall {1e3 * wall / args.steps:.4f})")
    if args.overlapped_only:
        return
    ms_eager = ms_step

    # ---- timed region 1b: the same overlapped steps replayed from a HIP graph
    # holding two consecutive steps (the micro-batches swap roles each step)
    # -> value.  The library records only kernels and events into the graph.
    Gk, rem = group_plan(args.steps, G)
    medians = {}  # median per-step time over the graph replays, by serialize flag

    def graph_ms(i, flags):
        """Capture Gk consecutive steps with `flags` into one HIP graph (Gk even,
        so the micro-batches' roles at the end match the start), replay it
        (warm-up, then timed), and time exactly --steps steps: the replays plus
        `rem` (0 or 1) eager steps inside the same timed region; returns (ms per
        step, wall ms per step, i)."""
        K = args.steps
        if Gk is None:  # too few steps for a graph: all eager
            i = issue(i, max(2, args.warmup), flags, s0)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            ev0.record(s0)
            i = issue(i, K, flags, s0)
            ev1.record(s0)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
            return ev0.elapsed_time(ev1) / K, 1e3 * wall / K, i
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(s0)
        with torch.cuda.graph(g, stream=cap, capture_error_mode="thread_local"):
            issue(i, Gk, flags, torch.cuda.current_stream())
        i += Gk
        warm = max(1, args.warmup // Gk)
        for _ in range(warm):
            g.replay()
        torch.cuda.synchronize()
        reps = (K - rem) // Gk
        i += Gk * warm
        # an event after every replay as well: per-replay times for the median
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
        t0 = time.perf_counter()
        ev0.record(s0)
        for r in range(reps):
            g.replay()
            marks[r].record(s0)
        i += Gk * reps
        i = issue(i, rem, flags, s0)
        ev1.record(s0)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = [ev0.elapsed_time(marks[0]) / Gk] + [marks[r - 1].elapsed_time(marks[r]) / Gk
                                                  for r in range(1, reps)]
        medians[flags & M.MOE_STEP_SERIALIZE] = sorted(per)[len(per) // 2]
        return ev0.elapsed_time(ev1) / K, 1e3 * wall / K, i

    launch = "eager launches"
    ms_serial_graph = None
    if args.graph == "on":
        ms_step, wall_ms, i = graph_ms(i, 0)
        launch = (f"hipGraph replay ({Gk} steps per graph)" if Gk else "eager launches") + \
            (" + 1 eager step" if Gk and rem else "")
        err(f"[bench] overlapped, graph replay: {ms_step:.4f} ms/step (wall {wall_ms:.4f})")
        ms_serial_graph, wall_ms, i = graph_ms(i, M.MOE_STEP_SERIALIZE)
        err(f"[bench] serialized, graph replay: {ms_serial_graph:.4f} ms/step "
            f"(wall {wall_ms:.4f})")

    # ---- timed region 1c: the same steps serialized on one stream, eager
    i = run_loop(args.warmup, M.MOE_STEP_SERIALIZE, i)
    torch.cuda.synchronize()
    ev0.record(s0)
    i = run_loop(args.steps, M.MOE_STEP_SERIALIZE, i)
    ev1.record(s0)
    torch.cuda.synchronize()
    ms_serial_eager = ev0.elapsed_time(ev1) / args.steps
    err(f"[bench] serialized, eager: {ms_serial_eager:.4f} ms/step -> overlap "
        f"x{ms_serial_eager / ms_eager:.3f} (eager vs eager)")

    # ---- timed region 2: the same steps serialized on one stream, with every
    # kernel bracketed by HIP events on its stream (no concurrency, so each
    # kernel's interval is its own execution); per-kernel times only, the
    # events' own cost makes this step time no baseline
    i = run_loop(args.warmup, M.MOE_STEP_SERIALIZE, i)
    M.moe_timing_reset()
    M.moe_timing_enable(64 * args.steps)
    torch.cuda.synchronize()
    ev0.record(s0)
    i = run_loop(args.steps, M.MOE_STEP_SERIALIZE, i)
    ev1.record(s0)
    torch.cuda.synchronize()
    M.moe_timing_disable()
    ms_serial_events = ev0.elapsed_time(ev1) / args.steps
    kern = M.moe_timing_report()
    err(f"[bench] serialized (kernel events on): {ms_serial_events:.4f} ms/step")
    ms_serial = ms_serial_graph if ms_serial_graph is not None else ms_serial_eager

    nonfinite = int(sum((~torch.isfinite(t.float())).sum().item()
                        for mb in mbs for t in (mb.out, mb.dx)))

    # ---- per-kernel achieved rates from the live kernel events
    work = algorithmic(w, N, T_loc)
    traffic = stored_traffic(w.name) if args.tokens is None else {}
    kernels = {}
    for name, (tot_ms, n) in sorted(kern.items(), key=lambda kv: -kv[1][0]):
        avg_s = tot_ms / 1e3 / max(n, 1)
        ent = {"avg_us": round(avg_s * 1e6, 2), "launches_per_step": round(n / args.steps, 3),
               "ms_per_step": round(tot_ms / args.steps, 4)}
        step_s = tot_ms / 1e3 / args.steps   # this kernel's time per step
        if name in work:
            kind, amount = work[name]      # per step
            if kind == "flop":
                ach = amount / step_s / 1e12
                ent.update(achieved=round(ach, 1), unit="TFLOP/s",
                           frac=round(ach / PEAK_BF16_TFLOPS, 4))
            else:
                ach = amount / step_s / 1e9
                ent.update(achieved=round(ach, 1), unit="GB/s", frac=round(ach / PEAK_HBM_GBS, 4))
        if name in traffic:
            ent["traffic"] = traffic[name]
        kernels[name] = ent
        err(f"  {name:14s} {ent}")

    gemm = [k for k in GEMM_KERNELS if k in kern]
    dom = max(gemm, key=lambda k: kern[k][0])
    dom_avg_s = kern[dom][0] / 1e3 / kern[dom][1]
    dom_per_step = kern[dom][1] / args.steps
    dom_ach = work[dom][1] / (dom_avg_s * dom_per_step) / 1e12
    gemm_flops = sum(work[k][1] * args.steps for k in gemm)
    gemm_s = sum(kern[k][0] / 1e3 for k in gemm)
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(dom_ach, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(dom_ach / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic.get(dom),
                "algorithmic_per_launch": f"{work[dom][1] / dom_per_step:.4g} flop",
                "launches_per_step": round(dom_per_step, 3),
                "avg_launch_us": round(dom_avg_s * 1e6, 2)}
    # the dispatch kernel; with the fused permute there is none (GEMM1 gathers x),
    # and the forward's remaining permute-class kernel, combine, is reported
    disp_kernel = "combine" if fused else "permute"
    disp = kernels.get(disp_kernel, {})

    tokens_per_s = w.T / (ms_step / 1e3)
    cpu = None
    if args.cpu_baseline == "on":
        cpu = cpu_oracle_baseline(w, inp)
        err(f"[bench] cpu oracle: {cpu}")

    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "F": w.F, "E": w.E, "e_lo": w.e_lo,
                   "E_l": w.E_l, "K": w.K, "routing": w.route, "N_rows": N,
                   "step": "1F1B: forward of one micro-batch + backward of the other, "
                           "two streams, " + ("wgrad between the two dgrad GEMMs"
                                              if args.wgrad_order == "mid" else
                                              "wgrad deferred to the end"),
                   "launch": launch,
                   "pipeline": (f"moe_overlap_steps, {G} steps per call, stream roles "
                                "alternating" if pipelined else
                                "one moe_overlap_step per step, joined at each boundary"),
                   "permute": "fused into GEMM1 and wgrad" if fused else "separate kernel",
                   "shared_expert_F": w.F_s},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "grouped_gemm_mfma_util": round(gemm_flops / gemm_s / 1e12 / PEAK_BF16_TFLOPS, 4),
        "dispatch_hbm_gbs": disp.get("achieved"),
        "dispatch_hbm_kernel": disp_kernel,
        # serialized = the same steps on one stream, launched the same way
        # (graph replay or eager) as the overlapped value, no kernel events
        "serialized_ms_per_step": round(ms_serial, 4),
        # median over the timed graph replays of their per-step time
        "median_replay_ms_per_step": (round(medians[0], 4) if 0 in medians else None),
        "median_replay_serialized_ms_per_step": (
            round(medians[M.MOE_STEP_SERIALIZE], 4) if M.MOE_STEP_SERIALIZE in medians
            else None),
        "overlap_speedup": round(ms_serial / ms_step, 4),
        "eager_overlapped_ms_per_step": round(ms_eager, 4),
        "eager_serialized_ms_per_step": round(ms_serial_eager, 4),
        "eager_overlap_speedup": round(ms_serial_eager / ms_eager, 4),
        "kernels": kernels,
        "nonfinite_outputs": nonfinite,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
