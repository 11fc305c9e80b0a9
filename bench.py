#!/usr/bin/env python3
"""Benchmark of one GPU's share of the MoE expert-parallel layer (MI355X).

One step = the 1F1B two-micro-batch step of the expert-parallel overlap pages
(1F1B note page 2, "MoE 1F1B overlap"): the forward of one micro-batch and the
backward (dgrad, then wgrad deferred past the other's expert GEMMs) of the
other, on two streams, so that every step passes T tokens through the whole
layer forward and backward.  Throughput = T / step time (tokens/s).  Inputs are
synthetic (seeded), resident in HBM before the timed region.  The default
workload is the whole 128-expert layer on one GPU (T = 16384, d = 2048,
F = 768, top-8, bf16), the largest configuration that fits one GPU.

Prints ONE JSON line on stdout; diagnostics go to stderr.

``--summarize KIND`` turns rocprofv3 output into the summaries kept under
profiles/ (kernel trace, HBM traffic, MFMA counters, stream overlap); it needs
no GPU.
"""

from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import statistics
import sys
import time

METRIC = "MoE layer fwd+bwd tokens/s on 1 MI355X; grouped-GEMM MFMA util %; dispatch HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 (and fp16) matrix-core peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak
DEFAULT_WORKLOAD = "ep1_128exp_bf16"
OVERLAP_WORKLOAD = "two_microbatch_bf16"

GEMM_KERNELS = ("ffn_gate_up", "ffn_down", "dgrad_act", "dgrad_in", "wgrad", "wgrad_multi")
# kernels whose algorithmic work is given per launch (the others' per step)
PER_LAUNCH = ("wgrad_multi",)
COPY_PROBE_BYTES = 1 << 30
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_DIR = os.path.join(ROOT, "profiles")


def err(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(w, N, T_loc, accumulate=True, fused=False, fcb=False, group=2):
    """Algorithmic work per step of each kernel (one launch of each, plus the
    shared expert's launches of the same GEMMs over all T tokens when the
    workload has one): {name: {"flop": F, "byte": B}}.  Bytes count one pass
    over every operand and result (no re-reads); the GEMMs' bytes include the
    expert weights, and wgrad's the float32 weight gradients (read and written
    with accumulate, written without).  fused: the permute fused into GEMM1
    and wgrad (x rows instead of xp); fcb: the fused combine backward (dout
    rows instead of dy_p, ag written by dgrad_act).  `wgrad_multi` (the grouped
    weight gradient, one launch per `group` steps) is given per launch: the
    group's micro-batches' operands and one pass over the float32 weight
    gradients."""
    d, F, T, K, E, E_l = w.d, w.F, w.T, w.K, w.E, w.E_l
    b = 4 if w.dtype == "f32" else 2
    Fs = w.F_s
    wgu, wdn = E_l * 2 * F * d * b, E_l * d * F * b          # expert weights
    sgu, sdn = 2 * Fs * d * b, d * Fs * b                    # shared expert weights
    dW = 4.0 * (E_l * 3 * F * d + 3 * Fs * d)                # float32 dW_gu + dW_down
    xin = (T_loc if fused else N) * d * b                    # GEMM1 A operand rows
    dyin = (T_loc if fcb else N) * d * b                     # dgrad / wgrad dy operand rows
    agout = N * F * b if fcb else 0                          # ag written by dgrad_act
    out = {
        "ffn_gate_up": {"flop": 2.0 * N * d * 2 * F + 2.0 * T * d * 2 * Fs,
                        "byte": xin + wgu + N * 3 * F * b + T * d * b * (Fs > 0) + sgu
                        + T * 3 * Fs * b},
        "ffn_down": {"flop": 2.0 * N * F * d + 2.0 * T * Fs * d,
                     "byte": N * F * b + wdn + N * d * b + T * Fs * b + sdn + T * d * b * (Fs > 0)},
        "dgrad_act": {"flop": 2.0 * N * d * F + 2.0 * T * d * Fs,
                      "byte": dyin + wdn + N * 2 * F * b * 2 + agout
                      + (T * d * b + sdn + T * 2 * Fs * b * 2) * (Fs > 0)},
        "dgrad_in": {"flop": 2.0 * N * 2 * F * d + 2.0 * T * 2 * Fs * d,
                     "byte": N * 2 * F * b + wgu + N * d * b
                     + (T * 2 * Fs * b + sgu + T * d * b) * (Fs > 0)},
        "wgrad": {"flop": 6.0 * N * d * F + 6.0 * T * d * Fs,
                  "byte": dyin + N * (F + 2 * F) * b + xin + T * (2 * d + 3 * Fs) * b * (Fs > 0)
                  + dW * (2 if accumulate else 1)},
        "wgrad_multi": {"flop": group * (6.0 * N * d * F),
                        "byte": group * (dyin + N * (F + 2 * F) * b + xin)
                       + 4.0 * E_l * 3 * F * d * (2 if accumulate else 1)},
        "router": {"flop": 2.0 * T * d * E, "byte": T * d * b + d * E * b + 4.0 * T * E},
        # router weight gradient x^T dlogits on the matrix cores (bf16 data);
        # the two-term split of dlogits forms it twice, counted once here
        "dwr_mfma": {"flop": 2.0 * T * d * E, "byte": T * d * b + 4.0 * T * E},
        # x rows of tokens with a local expert + row map -> N rows
        "permute": {"byte": T_loc * d * b + 4.0 * T * K + N * d * b},
        # y_p rows + gates + row map -> out
        "combine": {"byte": N * d * b + 8.0 * T * K + T * d * b},
        # dout + y_p rows + gates + map -> dy_p rows (not with fcb) + dgates
        "combine_bwd": {"byte": T * d * b + (1 if fcb else 2) * N * d * b + 12.0 * T * K},
        # dx_p rows + map -> dx
        "dispatch_bwd": {"byte": N * d * b + 4.0 * T * K + T * d * b},
    }
    return out


def rate(work, seconds):
    """(bound, achieved, peak, unit, frac) of one launch: the kernel is bound
    by whichever of its flops at the matrix-core peak and its bytes at the HBM
    peak takes longer, and is rated against that peak."""
    t_f = work.get("flop", 0.0) / (PEAK_BF16_TFLOPS * 1e12)
    t_b = work.get("byte", 0.0) / (PEAK_HBM_GBS * 1e9)
    if t_f >= t_b:
        ach = work["flop"] / seconds / 1e12
        return "mfma", ach, PEAK_BF16_TFLOPS, "TFLOP/s", ach / PEAK_BF16_TFLOPS
    ach = work["byte"] / seconds / 1e9
    return "hbm", ach, PEAK_HBM_GBS, "GB/s", ach / PEAK_HBM_GBS


KERNEL_SOURCE = {k: "gemm_mfma.hip" for k in GEMM_KERNELS}
KERNEL_SOURCE.update({k: "dispatch.hip" for k in ("permute", "combine", "combine_bwd",
                                                  "dispatch_bwd")})


def kernel_source_hash(name):
    """sha256 of the source that defines kernel `name` and the shared header."""
    import hashlib
    csrc = os.path.join(ROOT, "combine_expert_ffn_amd", "csrc")
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


def group_plan(K, G0, unit=2):
    """Steps per captured graph for K timed steps: (G, rem) with G a multiple
    of `unit` (the steps after which the micro-batch buffer sets are back in
    their roles) and
    G * reps + rem == K, rem < unit eager steps; G0 when it divides K - rem,
    else the largest such divisor of K - rem up to 2 G0; (None, K) when K is
    too small for a graph."""
    def best(n):
        if n >= unit and n % G0 == 0:
            return G0
        c = [g for g in range(unit, min(n, 2 * G0) + 1, unit) if n % g == 0]
        return max(c) if c else None

    for rem in range(unit):
        g = best(K - rem) if K - rem >= unit else None
        if g:
            return g, rem
    return None, K


# ---------------------------------------------------------------------------
# one workload's device state and step issue
# ---------------------------------------------------------------------------
class Layer:
    """Weights, gradient buffers, workspace and two micro-batches of one
    workload on the GPU, and the issue of 1F1B steps on two streams."""

    def __init__(self, w, args, s0, s1):
        import numpy as np
        import torch
        import combine_expert_ffn_amd as M
        from combine_expert_ffn_amd.inputs import make_inputs

        self.M, self.w, self.s0, self.s1 = M, w, s0, s1
        self.inp = inp = make_inputs(w, seed=0, microbatches=2)
        s = self.s = M.shape_of(w)
        tdt = {"bf16": torch.bfloat16, "f16": torch.float16}.get(w.dtype, torch.float32)
        D = lambda a: torch.from_numpy(a).to("cuda", tdt)
        F32 = lambda a: torch.from_numpy(a).to("cuda")
        self.topk = topk = w.route == "topk"
        self.mode = M.MOE_ROUTE_TOPK if topk else M.MOE_ROUTE_FORCE_BALANCE
        self.W_gu, self.W_down = D(inp["W_gu"]), D(inp["W_down"])
        self.W_r = D(inp["W_r"]) if topk else None
        self.bias = F32(inp["bias"]) if inp["bias"] is not None else None
        z = lambda *sh: torch.zeros(*sh, dtype=torch.float32, device="cuda")
        self.dW_gu, self.dW_down = z(w.E_l, 2 * w.F, w.d), z(w.E_l, w.d, w.F)
        self.dW_r = z(w.d, w.E) if topk else None
        self.ws = torch.empty(M.moe_step_workspace_bytes_shared(s, w.F_s), dtype=torch.uint8,
                              device="cuda")
        self.fused = args.fused_permute == "on"
        self.fcb = args.fused_combine_bwd == "on"
        self.scatter = args.fused_scatter == "on"
        # the grouped weight gradient keeps the micro-batches back-propagated
        # in a group's steps until its last step: group + 1 buffer sets rotate
        self.pair = (args.wgrad_group > 1 and args.pipeline == "on" and
                     not (self.fused or self.fcb))
        self.group = args.wgrad_group if self.pair else 1
        self.R = self.group + 1 if self.pair else 2
        self.pipelined = args.pipeline == "on"
        self.G = args.group
        # flags of every step: the fused permute and the wgrad's place in the
        # backward stream's order (both leave the results unchanged)
        self.FLAGS = ((M.MOE_STEP_FUSED_PERMUTE if self.fused else 0) |
                      (M.MOE_STEP_FUSED_COMBINE_BWD if self.fcb else 0) |
                      (M.MOE_STEP_FUSED_SCATTER if self.scatter else 0) |
                      (M.MOE_STEP_MID_WGRAD if args.wgrad_order == "mid" else 0) |
                      ({2: M.MOE_STEP_PAIR_WGRAD, 4: M.MOE_STEP_GROUP4_WGRAD}.get(self.group, 0)))
        self.shared = None
        if w.F_s:  # a shared expert beside the routed ones
            self.shared = (D(inp["W_gu_s"]), D(inp["W_down_s"]), z(2 * w.F_s, w.d),
                           z(w.d, w.F_s))
        mk = lambda x, dout, g: M.MicroBatch(s, x=D(x), dout=D(dout),
                                             gates=None if topk else F32(g), fused=self.fused,
                                             F_s=w.F_s, fused_bwd=self.fcb)
        self.mbs = [mk(inp["x"], inp["dout"], inp["gates"]),
                    mk(inp["x_b"], inp["dout_b"], inp.get("gates_b"))]
        # more sets: the two draws' tokens in reverse order, then the first
        # draw's rolled by a few tokens
        for k in range(2, self.R):
            src = "" if k % 2 == 0 else "_b"
            g = inp.get("gates" + src)
            if k < 4:
                fx = lambda a: a[::-1].copy()
            else:
                fx = lambda a: np.roll(a, 7 * k, axis=0)
            self.mbs.append(mk(fx(inp["x" + src]), fx(inp["dout" + src]),
                               None if g is None else fx(g)))
        self.i = 0  # steps issued so far (after the priming forward)
        M.moe_overlap_step(self.make_step(self.mbs[0], None), s0, s1,
                           self.FLAGS & ~(M.MOE_STEP_PAIR_WGRAD | M.MOE_STEP_GROUP4_WGRAD))

    def make_step(self, fwd, bwd):
        M = self.M
        return M.make_step(self.s, self.mode, self.W_gu, self.W_down, self.dW_gu, self.dW_down,
                           self.ws, fwd=fwd, bwd=bwd, W_r=self.W_r, bias=self.bias,
                           dW_r=self.dW_r, accumulate=M.MOE_ACCUM_DW, shared=self.shared)

    def make(self, i):  # step i forwards one micro-batch and back-propagates another
        return self.make_step(self.mbs[(i + 1) % self.R], self.mbs[i % self.R])

    def issue(self, n, flags, q=None):
        """Issue the next n steps on q (and s1): one pipelined moe_overlap_steps
        call per group of G steps for overlapped steps with --pipeline on, else
        one moe_overlap_step call per step (serialized steps run the same
        groups through moe_overlap_steps with MOE_STEP_SERIALIZE)."""
        M = self.M
        q = q or self.s0
        i0 = self.i
        if self.pipelined:
            for g0 in range(i0, i0 + n, self.G):
                M.moe_overlap_steps([self.make(j) for j in range(g0, min(g0 + self.G, i0 + n))],
                                    q, self.s1, flags | self.FLAGS)
        else:
            for j in range(i0, i0 + n):
                M.moe_overlap_step(self.make(j), q, self.s1, flags | self.FLAGS)
        self.i += n

    def capture(self, n, flags):
        """A HIP graph of the next n steps (n even: the micro-batches' roles at
        its end match its start, so it can be replayed)."""
        import torch
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(self.s0)
        with torch.cuda.graph(g, stream=cap, capture_error_mode="thread_local"):
            self.issue(n, flags, torch.cuda.current_stream())
        torch.cuda.synchronize()
        return g


def ab_medians(runs, rounds, s0):
    """Alternate the timed callables of `runs` ({name: (fn, steps)}) for
    `rounds` rounds, each run bracketed by events on s0; returns
    {name: median ms per step}.  Alternating keeps the two schedules under the
    same clock and thermal state."""
    import torch
    per = {k: [] for k in runs}
    for _ in range(rounds):
        for k, (fn, n) in runs.items():
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(s0)
            fn()
            b.record(s0)
            torch.cuda.synchronize()
            per[k].append(a.elapsed_time(b) / n)
    return {k: statistics.median(v) for k, v in per.items()}


def overlap_ab(L, G, rounds, graph):
    """Overlapped against serialized steps of layer L, alternated (A/B), as
    replays of two captured G-step graphs (graph=True) or as eager groups of G
    steps; returns (overlapped ms, serialized ms) medians per step."""
    M = L.M
    if graph:
        go = L.capture(G, 0)
        gs = L.capture(G, M.MOE_STEP_SERIALIZE)
        for _ in range(2):
            go.replay()
            gs.replay()
        runs = {"o": (go.replay, G), "s": (gs.replay, G)}
    else:
        runs = {"o": (lambda: L.issue(G, 0), G),
                "s": (lambda: L.issue(G, M.MOE_STEP_SERIALIZE), G)}
        for f, _ in runs.values():
            f()
    med = ab_medians(runs, rounds, L.s0)
    return med["o"], med["s"]


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=48,
                    help="timed steps (default 48: whole groups of four steps in calls of 12)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--tokens", type=int, default=None, help="override T of the workload")
    ap.add_argument("--cpu-baseline", choices=("on", "off"), default="on")
    ap.add_argument("--graph", choices=("on", "off"), default=None,
                    help="time the overlapped steps as replays of a HIP graph of --group steps "
                         "(on) or as eager launches (off); default: off with grouped weight "
                         "gradients (the library does not capture them), else on")
    ap.add_argument("--fused-permute", choices=("on", "off"), default="off",
                    help="fuse the permute into the expert GEMMs (MOE_STEP_FUSED_PERMUTE): GEMM1 "
                         "and wgrad read the token rows of x through the dispatch plan, no xp")
    ap.add_argument("--fused-combine-bwd", choices=("on", "off"), default="off",
                    help="fuse the combine backward into the expert GEMMs "
                         "(MOE_STEP_FUSED_COMBINE_BWD): no dy_p; dgrad and wgrad read the dout "
                         "rows through the dispatch plan and apply the gates")
    ap.add_argument("--fused-scatter", choices=("on", "off"), default="off",
                    help="fuse the unpermute into GEMM2 (MOE_STEP_FUSED_SCATTER): its epilogue "
                         "writes y by (token, slot) pair, so the combine and its backward read "
                         "each token's rows as one run (bit-identical results)")
    ap.add_argument("--wgrad-order", choices=("mid", "last"), default="mid",
                    help="where the backward micro-batch's wgrad runs on its stream: between the "
                         "two dgrad GEMMs (mid, MOE_STEP_MID_WGRAD) or after the dispatch "
                         "backward (last); the same order is used for the serialized steps")
    ap.add_argument("--pipeline", choices=("on", "off"), default="on",
                    help="run the overlapped steps G at a time through moe_overlap_steps, the "
                         "streams' roles alternating so consecutive steps overlap (on), or one "
                         "moe_overlap_step call per step, joined at every step boundary (off)")
    ap.add_argument("--wgrad-group", type=int, choices=(1, 2, 4), default=4,
                    help="steps whose routed experts' weight gradients run as one launch "
                         "(2: MOE_STEP_PAIR_WGRAD, 4: MOE_STEP_GROUP4_WGRAD; dW read and "
                         "written once per group; group + 1 micro-batch buffer sets); not "
                         "with the fused paths, and with --graph off only (the library "
                         "rejects grouped steps under stream capture: a captured run of "
                         "paired steps ended in a host crash whose cause is not found)")
    ap.add_argument("--group", type=int, default=None,
                    help="steps per moe_overlap_steps call and per captured graph: a "
                         "multiple of 2, and of the weight-gradient group (default 10, or "
                         "12 with grouped weight gradients)")
    ap.add_argument("--ab-rounds", type=int, default=6,
                    help="rounds of the alternating overlapped / serialized comparison")
    ap.add_argument("--overlap-workload", default=OVERLAP_WORKLOAD,
                    help="second workload whose overlapped / serialized ratio is reported too "
                         "(the two-micro-batch top-8 configuration); 'none' to skip")
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
                         "JSON line: the program to run under rocprofv3 --pmc for the per-kernel "
                         "HBM traffic (FETCH_SIZE / WRITE_SIZE) and MFMA counters")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="time the vendor library's dense bf16 GEMM (torch.matmul) on the "
                         "shapes of the five expert GEMMs with the workload's dispatched rows "
                         "as one matrix, print one line per shape and exit (no JSON line): "
                         "a reference rate for the grouped kernels on the same chip")
    ap.add_argument("--roctx", action="store_true",
                    help="bracket every phase of the step with a roctx range (MOE_ROCTX=1): "
                         "run eagerly (--graph off) under rocprofv3 --marker-trace")
    ap.add_argument("--summarize", choices=("kernels", "traffic", "mfma", "overlap", "phases"),
                    help="write profiles/<kind>_<workload>.md from rocprofv3 output (no GPU)")
    ap.add_argument("--inputs", nargs="+", help="rocprofv3 files for --summarize: a kernel "
                    "trace (kernels, overlap), FETCH_SIZE then WRITE_SIZE counter csv "
                    "(traffic), the MFMA counter csv (mfma), or a kernel trace, a HIP API "
                    "trace and a marker trace of one --roctx run (phases)")
    ap.add_argument("--profile-cmd", action="append", default=[],
                    help="the command(s) that made the --inputs, quoted in the summary")
    ap.add_argument("--out", default=None, help="summary file (default profiles/<kind>_<wl>.md)")
    ap.add_argument("--n-rows", type=int, default=None,
                    help="--summarize with a local expert window: the rows dispatched to it")
    ap.add_argument("--t-loc", type=int, default=None,
                    help="--summarize with a local expert window: tokens with a local expert")
    args = ap.parse_args()

    if args.summarize:
        return summarize(args)
    if args.roctx:  # read by the library at its first phase
        os.environ["MOE_ROCTX"] = "1"

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        err("bench.py: measures one GPU's share of the expert-parallel layer; runs on more "
            "than one GPU are not supported.")
        sys.exit(2)

    import torch
    import combine_expert_ffn_amd as M
    from combine_expert_ffn_amd.inputs import WORKLOADS

    if not torch.cuda.is_available():
        err("bench.py: no GPU visible")
        sys.exit(1)
    M.lib()  # fails loudly if libmoe.so is not built
    pairing = args.wgrad_group > 1 and args.pipeline == "on" and \
        args.fused_permute == "off" and args.fused_combine_bwd == "off"
    # steps after which a captured graph's buffer sets are back in their roles
    # (graphs hold ungrouped steps only: two sets)
    unit = args.wgrad_group if pairing else 2
    if args.group is None:
        args.group = 12 if pairing else 10
    if args.graph is None:
        args.graph = "off" if pairing else "on"
    if pairing and args.graph == "on":
        err("bench.py: grouped weight gradients need --graph off (they are not captured)")
        sys.exit(2)
    if args.group < unit or args.group % unit:
        err(f"bench.py: --group must be a multiple of {unit}")
        sys.exit(2)
    w = WORKLOADS[args.workload]
    if args.tokens:
        w = w.with_tokens(args.tokens)
    err(f"[bench] workload {w.name}: T={w.T} d={w.d} F={w.F} E={w.E} E_l={w.E_l} K={w.K} "
        f"{w.dtype} route={w.route}")
    if args.vendor_gemm:
        return vendor_gemm(w)
    s0 = torch.cuda.current_stream()
    s1 = torch.cuda.Stream()
    L = Layer(w, args, s0, s1)
    SER = M.MOE_STEP_SERIALIZE

    if args.counter_pass:
        L.issue(args.steps, SER)
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
    L.issue(args.warmup, 0)
    torch.cuda.synchronize()
    counts = L.mbs[0].counts.cpu()
    N = int(counts.sum())
    T_loc = int((L.mbs[0].row_of_pair >= 0).any(dim=1).sum())
    err(f"[bench] dispatched rows N = {N}, tokens with a local expert T_loc = {T_loc}")

    if args.serialized_only:
        L.issue(args.warmup + args.steps, SER)
        torch.cuda.synchronize()
        err(f"[bench] serialized-only pass done: {args.warmup + args.steps} steps")
        return
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if args.overlapped_only:
        ev0.record(s0)
        L.issue(args.steps, 0)
        ev1.record(s0)
        torch.cuda.synchronize()
        err(f"[bench] overlapped-only: {ev0.elapsed_time(ev1) / args.steps:.4f} ms/step")
        return

    # ---- timed region: exactly --steps overlapped 1F1B steps -> value.  With
    # --graph on they are replays of one captured graph of Gk steps (plus one
    # eager step when --steps is odd); the library records only kernels and
    # events into the graph.
    K = args.steps
    Gk, rem = group_plan(K, args.group, unit) if args.graph == "on" else (None, K)
    replay_ms = []
    if Gk:
        g = L.capture(Gk, 0)
        for _ in range(max(1, args.warmup // Gk)):
            g.replay()
        torch.cuda.synchronize()
        reps = (K - rem) // Gk
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
        t0 = time.perf_counter()
        ev0.record(s0)
        for r in range(reps):
            g.replay()
            marks[r].record(s0)
        L.issue(rem, 0)
        ev1.record(s0)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        replay_ms = [ev0.elapsed_time(marks[0]) / Gk] + \
            [marks[r - 1].elapsed_time(marks[r]) / Gk for r in range(1, reps)]
        launch = f"hipGraph replay ({Gk} steps per graph)" + \
            (f" + {rem} eager step{'s' if rem > 1 else ''}" if rem else "")
    else:
        # one more group of warm-up steps, as the graph path replays its
        # captured group once before the timed region
        L.issue(args.group, 0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(s0)
        L.issue(K, 0)
        ev1.record(s0)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        launch = "eager launches"
    ms_step = ev0.elapsed_time(ev1) / K
    err(f"[bench] overlapped ({launch}): {ms_step:.4f} ms/step (wall {1e3 * wall / K:.4f})")

    # ---- overlapped against serialized, alternated (A/B) after the timed
    # region, as graph replays and as eager launches
    G = args.group
    if args.graph == "on":
        o_g, s_g = overlap_ab(L, G, args.ab_rounds, graph=True)
        err(f"[bench] A/B graph replays: overlapped {o_g:.4f} / serialized {s_g:.4f} ms/step "
            f"-> x{s_g / o_g:.3f}")
    o_e, s_e = overlap_ab(L, G, args.ab_rounds, graph=False)
    err(f"[bench] A/B eager: overlapped {o_e:.4f} / serialized {s_e:.4f} ms/step "
        f"-> x{s_e / o_e:.3f}")
    if args.graph != "on":  # no graphs: the eager comparison stands for both
        o_g, s_g = o_e, s_e

    # ---- per-kernel times: serialized steps with every kernel bracketed by
    # HIP events on its stream (no concurrency, so each kernel's interval is
    # its own execution); the events' own cost makes this step time no baseline
    L.issue(args.warmup, SER)
    M.moe_timing_reset()
    M.moe_timing_enable(64 * K)
    torch.cuda.synchronize()
    L.issue(K, SER)
    torch.cuda.synchronize()
    M.moe_timing_disable()
    kern = M.moe_timing_report()
    nonfinite = int(sum((~torch.isfinite(t.float())).sum().item()
                        for mb in L.mbs for t in (mb.out, mb.dx)))
    peak_mem = torch.cuda.max_memory_allocated()

    # ---- the two-micro-batch top-8 configuration's overlap figure
    c4 = None
    if args.overlap_workload != "none" and args.overlap_workload != w.name:
        w4 = WORKLOADS[args.overlap_workload]
        L4 = Layer(w4, args, s0, s1)
        L4.issue(args.warmup, 0)
        o4e, s4e = overlap_ab(L4, G, args.ab_rounds, graph=False)
        o4, s4 = (overlap_ab(L4, G, args.ab_rounds, graph=True) if args.graph == "on"
                  else (o4e, s4e))
        c4 = {"workload": w4.name, "T": w4.T, "E": w4.E, "K": w4.K, "routing": w4.route,
              "overlapped_ms_per_step": round(o4, 4), "serialized_ms_per_step": round(s4, 4),
              "overlap_speedup": round(s4 / o4, 4),
              "eager_overlapped_ms_per_step": round(o4e, 4),
              "eager_serialized_ms_per_step": round(s4e, 4),
              "eager_overlap_speedup": round(s4e / o4e, 4),
              "method": f"median of {args.ab_rounds} alternating {G}-step runs each"}
        err(f"[bench] {w4.name}: graph x{s4 / o4:.3f}, eager x{s4e / o4e:.3f}")
        del L4
        torch.cuda.synchronize()

    # ---- per-kernel achieved rates from the live kernel events
    work = algorithmic(w, N, T_loc, accumulate=True, fused=L.fused, fcb=L.fcb, group=L.group)
    traffic = stored_traffic(w.name) if args.tokens is None else {}
    kernels = {}
    for name, (tot_ms, n) in sorted(kern.items(), key=lambda kv: -kv[1][0]):
        avg_s = tot_ms / 1e3 / max(n, 1)
        ent = {"avg_us": round(avg_s * 1e6, 2), "launches_per_step": round(n / K, 3),
               "ms_per_step": round(tot_ms / K, 4)}
        step_s = tot_ms / 1e3 / K   # this kernel's time per step
        if name in work:
            t_s = avg_s if name in PER_LAUNCH else step_s
            bound, ach, peak, unit, frac = rate(work[name], t_s)
            ent.update(bound=bound, achieved=round(ach, 1), unit=unit, frac=round(frac, 4))
            if "flop" in work[name]:
                ent["mfma_frac"] = round(work[name]["flop"] / t_s / 1e12 / PEAK_BF16_TFLOPS, 4)
        if name in traffic:
            ent["traffic"] = traffic[name]
        kernels[name] = ent
        err(f"  {name:14s} {ent}")

    gemm = [k for k in GEMM_KERNELS if k in kern]
    dom = max(gemm, key=lambda k: kern[k][0])
    dom_avg_s = kern[dom][0] / 1e3 / kern[dom][1]
    dom_per_step = kern[dom][1] / K
    per_launch = (work[dom] if dom in PER_LAUNCH else
                  {u: v / dom_per_step for u, v in work[dom].items()})
    bound, ach, peak, unit, frac = rate(per_launch, dom_avg_s)
    roofline = {"kernel": dom, "bound": bound, "achieved": round(ach, 1), "peak": peak,
                "unit": unit, "frac": round(frac, 4), "traffic": traffic.get(dom),
                "algorithmic_per_launch": {"flop": f"{per_launch['flop']:.4g}",
                                           "byte": f"{per_launch['byte']:.4g}"},
                "mfma_frac": round(per_launch["flop"] / dom_avg_s / 1e12 / PEAK_BF16_TFLOPS, 4),
                "launches_per_step": round(dom_per_step, 3),
                "avg_launch_us": round(dom_avg_s * 1e6, 2)}
    gemm_flops = sum(work[k]["flop"] * (kern[k][1] if k in PER_LAUNCH else K) for k in gemm)
    gemm_s = sum(kern[k][0] / 1e3 for k in gemm)
    # the dispatch kernel; with the fused permute there is none (GEMM1 gathers x),
    # and the forward's remaining permute-class kernel, combine, is reported
    disp_kernel = "combine" if L.fused else "permute"
    disp = kernels.get(disp_kernel, {})

    tokens_per_s = w.T / (ms_step / 1e3)
    cpu = None
    if args.cpu_baseline == "on":
        cpu = cpu_oracle_baseline(w, L.inp)
        err(f"[bench] cpu oracle: {cpu}")

    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
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
                   "weight_grads": "float32, accumulated every step" + (
                       f"; the routed experts' of each group of {L.group} steps in one launch"
                       if L.pair else ""),
                   "launch": launch,
                   "pipeline": (f"moe_overlap_steps, {G} steps per call, stream roles "
                                "alternating" if L.pipelined else
                                "one moe_overlap_step per step, joined at each boundary"),
                   "permute": "fused into GEMM1 and wgrad" if L.fused else "separate kernel",
                   "y_layout": ("by (token, slot) pair, scattered by GEMM2's epilogue"
                                if L.scatter else "by dispatched row"),
                   "combine_backward": ("fused into dgrad and wgrad (no dy_p)" if L.fcb
                                        else "separate kernel writing dy_p"),
                   "shared_expert_F": w.F_s},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "grouped_gemm_mfma_util": round(gemm_flops / gemm_s / 1e12 / PEAK_BF16_TFLOPS, 4),
        "dispatch_hbm_gbs": disp.get("achieved"),
        "dispatch_hbm_kernel": disp_kernel,
        "median_replay_ms_per_step": (round(statistics.median(replay_ms), 4)
                                      if replay_ms else None),
        # overlapped vs serialized: medians of alternating runs of the same
        # steps (graph replays, then eager launches)
        "overlapped_ms_per_step_ab": round(o_g, 4),
        "serialized_ms_per_step": round(s_g, 4),
        "overlap_speedup": round(s_g / o_g, 4),
        "eager_overlapped_ms_per_step": round(o_e, 4),
        "eager_serialized_ms_per_step": round(s_e, 4),
        "eager_overlap_speedup": round(s_e / o_e, 4),
        "overlap_two_microbatch": c4,
        "peak_device_memory_gib": round(peak_mem / 2 ** 30, 2),
        "kernels": kernels,
        "nonfinite_outputs": nonfinite,
    }
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------------------
# rocprofv3 output -> profiles/ summaries (no GPU needed)
# ---------------------------------------------------------------------------
# kernel symbol -> the name the library times it under (MOE_LAUNCH); wgrad_kernel
# is split by its ROUTER template argument (the third: the router weight
# gradient reuses the kernel)
_CLASS = [("GateUpOp", "ffn_gate_up"), ("DownOp", "ffn_down"), ("DgradActOp", "dgrad_act"),
          ("DgradInOp", "dgrad_in"), ("combine_bwd_kernel", "combine_bwd"),
          ("dispatch_bwd_kernel", "dispatch_bwd"), ("combine_kernel", "combine"),
          ("permute_kernel", "permute"), ("transpose_batched_kernel", "transpose_w"),
          ("transpose_wr_kernel", "transpose_wr"), ("plan_hist_kernel", "plan_hist"),
          ("plan_scan_kernel", "plan_scan"), ("plan_rank_kernel", "plan_rank"),
          ("force_balance_kernel", "force_balance"), ("router_kernel", "router"),
          ("topk_kernel", "topk"), ("dlogits_kernel", "dlogits"),
          ("dwr_reduce", "dwr_reduce"), ("dwr_partial_kernel", "dwr_partial"),
          ("shared_plan_kernel", "shared_plan")]


def vendor_gemm(w, reps=10):
    """Dense bf16 torch.matmul (hipBLASLt / rocBLAS) on the expert GEMMs' shapes:
    the N dispatched rows (T*K, times E_l/E for a window, rounded to 256) as one
    matrix, so the same flops as the grouped kernels without their per-expert
    tiling; the weight gradients as [M, N] @ [N, K] products over the rows
    (bf16 output, where the library's kernels accumulate float32)."""
    import torch
    N = w.T * w.K * w.E_l // w.E // 256 * 256
    d, F = w.d, w.F
    g = torch.Generator(device="cuda").manual_seed(0)
    r = lambda *sh: torch.randn(*sh, generator=g, device="cuda", dtype=torch.bfloat16)
    shapes = {"ffn_gate_up": (N, d, 2 * F), "ffn_down": (N, F, d), "dgrad_act": (N, d, F),
              "dgrad_in": (N, 2 * F, d), "wgrad dW_gu": (2 * F, N, d),
              "wgrad dW_down": (d, N, F)}
    try:
        lib = str(torch.backends.cuda.preferred_blas_library())
    except Exception:  # noqa: BLE001 - older torch
        lib = "default"
    err(f"[vendor] torch {torch.__version__}, preferred BLAS library {lib}, N = {N} rows")
    for name, (m, k, n) in shapes.items():
        a, b = r(m, k), r(k, n)
        for _ in range(3):
            torch.matmul(a, b)
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            torch.matmul(a, b)
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        t = statistics.median(ts)
        fl = 2.0 * m * k * n
        print(f"[vendor] {name:14s} [{m} x {k}] @ [{k} x {n}]: {t * 1e6:8.1f} us, "
              f"{fl / t / 1e12:7.1f} TFLOP/s = {fl / t / 1e12 / PEAK_BF16_TFLOPS:.3f} of peak",
              flush=True)
        del a, b


def bench_name(sym):
    """The library's timing name of a kernel symbol, or None (not ours)."""
    if "moe::" not in sym:
        return None
    i = sym.find("wgrad_kernel<")
    if i >= 0 and "f32_wgrad" not in sym:
        depth, j, args, cur = 0, i + len("wgrad_kernel<"), [], ""
        while j < len(sym):
            ch = sym[j]
            if ch == "<":
                depth += 1
            elif ch == ">":
                if depth == 0:
                    break
                depth -= 1
            if ch == "," and depth == 0:
                args.append(cur.strip())
                cur = ""
            else:
                cur += ch
            j += 1
        args.append(cur.strip())
        # wgrad_kernel<GATHER, element type, ROUTER, ACC, GD, MULTI>
        if len(args) > 2 and args[2] == "true":
            return "dwr_mfma"
        return "wgrad_multi" if len(args) > 5 and args[5] == "true" else "wgrad"
    for k, v in _CLASS:
        if k in sym:
            return v
    return None


def read_trace(path):
    """[(symbol, start_ns, end_ns)] of a rocprofv3 kernel trace (csv or rocpd db)."""
    if path.endswith(".db"):
        import sqlite3
        c = sqlite3.connect(path)
        rows = c.execute("select name, start, end from kernels order by start")
        return [(r[0], int(r[1]), int(r[2])) for r in rows]
    out = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            out.append((r["Kernel_Name"], int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    out.sort(key=lambda r: r[1])
    return out


def read_counters(path):
    """{dispatch: (symbol, {counter: value summed over instances}, duration_ns)}."""
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    sym, dur = {}, {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            d = int(r["Dispatch_Id"])
            per[d][r["Counter_Name"]] += float(r["Counter_Value"])
            sym[d] = r["Kernel_Name"]
            dur[d] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    return {d: (sym[d], dict(per[d]), dur[d]) for d in per}


def _workload_for_summary(args):
    from combine_expert_ffn_amd.inputs import WORKLOADS
    w = WORKLOADS[args.workload]
    if args.tokens:
        w = w.with_tokens(args.tokens)
    # every expert local: N = T*K rows, all T tokens; a window: as given
    # (the bench line's config.N_rows and the tokens with a local expert)
    N, T_loc = (w.T * w.K, w.T) if w.E_l == w.E else (args.n_rows, args.t_loc)
    return w, N, T_loc


def _cmds(args):
    return "\n".join(args.profile_cmd) if args.profile_cmd else "(not given)"


def summarize(args):
    w, N, T_loc = _workload_for_summary(args)
    out = args.out or os.path.join(TRAFFIC_DIR, f"{args.summarize}_{w.name}.md")
    desc = (f"{w.name} (T={w.T}, d={w.d}, F={w.F}, {w.E_l} of {w.E} experts local, top-{w.K}, "
            f"{w.dtype}, {w.route})")
    txt = {"kernels": _sum_kernels, "traffic": _sum_traffic, "mfma": _sum_mfma,
           "overlap": _sum_overlap, "phases": _sum_phases}[args.summarize](args, w, N, T_loc,
                                                                         desc)
    with open(out, "w") as fh:
        fh.write(txt)
    err(f"[summarize] wrote {out}")


def _sum_kernels(args, w, N, T_loc, desc):
    rows = [(bench_name(s), s, a, b) for s, a, b in read_trace(args.inputs[0])]
    by = collections.OrderedDict()
    for name, sym, a, b in rows:
        if name:
            by.setdefault(name, []).append((b - a) / 1e3)
    total = sum(sum(v) for v in by.values())
    work = (algorithmic(w, N, T_loc, fused=args.fused_permute == "on",
                        fcb=args.fused_combine_bwd == "on", group=args.wgrad_group)
            if N is not None else {})
    lines = []
    for k, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        h = v[len(v) // 2:]
        rated = ""
        if k in work and k != "dwr_mfma":
            bound, ach, peak, unit, frac = rate(work[k], statistics.mean(h) / 1e6)
            rated = f"{bound} {ach:.1f} {unit} = {frac:.3f}"
        lines.append(f"| {k} | {len(v)} | {sum(v):.1f} | {sum(v) / len(v):.2f} | "
                     f"{statistics.median(h):.2f} | {statistics.mean(h):.2f} | "
                     f"{100 * sum(v) / total:.2f} | {rated} |")
    return f"""# Kernel trace: {desc}

Command (run from the repository root on one MI355X):

```
{_cmds(args)}
```

Kernel trace of the library's kernels (durations in microseconds), summarised
by `python bench.py --summarize kernels --workload {w.name} --inputs <trace>`.
`avg` is the mean over all calls; `steady median` / `steady mean` drop the
first half of each kernel's calls (the first calls of a fresh process run
slower while the clocks settle).  `rate` divides the kernel's algorithmic work
per launch (bench.py `algorithmic`: flops, and bytes with one pass over every
operand and result, float32 weight gradients read and written) by the steady
mean and rates it against whichever MI355X peak bounds it (2.5 PFLOP/s dense
bf16 or 8 TB/s HBM).

| kernel | calls | total us | avg us | steady median us | steady mean us | % | rate (bound, achieved = frac of peak) |
|---|---|---|---|---|---|---|---|
""" + "\n".join(lines) + "\n"


def _sum_traffic(args, w, N, T_loc, desc):
    F, W = read_counters(args.inputs[0]), read_counters(args.inputs[1])
    probe_kib = COPY_PROBE_BYTES / 1024

    def probe(rec, counter):
        v = [c.get(counter, 0.0) for s, c, _ in rec.values() if "neg_kernel" in s or
             ("neg" in s and "at::native" in s)]
        return statistics.median(v)

    pf, pw = probe(F, "FETCH_SIZE"), probe(W, "WRITE_SIZE")
    ff, fw = probe_kib / pf, probe_kib / pw

    def per_kernel(rec, counter):
        agg = collections.defaultdict(list)
        for s, c, _ in rec.values():
            b = bench_name(s)
            if b:
                agg[b].append(c.get(counter, 0.0))
        return agg

    aF, aW = per_kernel(F, "FETCH_SIZE"), per_kernel(W, "WRITE_SIZE")
    work = (algorithmic(w, N, T_loc, fused=args.fused_permute == "on",
                        fcb=args.fused_combine_bwd == "on", group=args.wgrad_group)
            if N is not None else {})
    rec = {"workload": w.name, "copy_probe_bytes": COPY_PROBE_BYTES,
           "fetch_factor": round(ff, 4), "write_factor": round(fw, 4), "kernels": {}}
    lines = []
    for k in sorted(aF, key=lambda k: -statistics.median(aF[k])):
        if k not in aW:
            continue
        f, wr = statistics.median(aF[k]), statistics.median(aW[k])
        rb, wb = f * ff * 1024, wr * fw * 1024
        alg = work.get(k, {}).get("byte")
        ent = {"fetch_kib_per_dispatch": round(f, 1), "write_kib_per_dispatch": round(wr, 1),
               "dispatches": len(aF[k]), "hbm_bytes_per_launch": int(round(rb + wb))}
        if k in KERNEL_SOURCE:
            ent["source_sha256"] = kernel_source_hash(k)
        rec["kernels"][k] = ent
        lines.append(f"| {k} | {len(aF[k])} | {f:.0f} | {wr:.0f} | {rb / 1e6:.1f} | "
                     f"{wb / 1e6:.1f} | " + (f"{alg / 1e6:.1f} | {(rb + wb) / alg:.2f} |"
                                             if alg else "- | - |"))
    return f"""# HBM traffic per kernel launch: {desc}

Counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch, as rocprofv3 reports
them), each from its own run of the same program, scaled by what the same
counter reads for a copy probe of known size (an elementwise negation reading
and writing {COPY_PROBE_BYTES} bytes, larger than the last-level cache); per
kernel the median over its dispatches.  Summarised by `python bench.py
--summarize traffic --workload {w.name} --inputs <fetch csv> <write csv>`.
Kernels are named by the library's launch names; the router weight gradient
(wgrad_kernel with its ROUTER template argument set) is `dwr_mfma`, not
`wgrad`.  `algorithmic` is one pass over every operand and result (bench.py
`algorithmic`, float32 weight gradients read and written).

Commands (run from the repository root on one MI355X):

```
{_cmds(args)}
```

Copy probe: FETCH_SIZE {pf:.0f} KiB (factor {ff:.4f}), WRITE_SIZE {pw:.0f} KiB (factor {fw:.4f}) for {probe_kib:.0f} KiB moved each way.

| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB (scaled) | written MB (scaled) | algorithmic MB | measured / algorithmic |
|---|---|---|---|---|---|---|---|
""" + "\n".join(lines) + """

Machine-readable record (bench.py reads `hbm_bytes_per_launch` while the kernel's source hash still matches):

```json
""" + json.dumps(rec, indent=1) + "\n```\n"


def _sum_mfma(args, w, N, T_loc, desc):
    rec = read_counters(args.inputs[0])
    work = (algorithmic(w, N, T_loc, fused=args.fused_permute == "on",
                        fcb=args.fused_combine_bwd == "on", group=args.wgrad_group)
            if N is not None else {})
    SIMDS, XCDS = 1024, 8
    peak_per_clk = PEAK_BF16_TFLOPS * 1e12 / 2.4e9
    agg = collections.defaultdict(list)
    for s, c, dur in rec.values():
        b = bench_name(s)
        if b in GEMM_KERNELS or b in ("router", "dwr_mfma"):
            agg[b].append((c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0),
                           c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0),
                           c.get("GRBM_GUI_ACTIVE", 0.0), dur))
    lines = []
    for k, v in sorted(agg.items(), key=lambda kv: -statistics.median(x[3] for x in kv[1])):
        busy = statistics.median(x[0] for x in v)
        mops = statistics.median(x[1] for x in v)
        gui = statistics.median(x[2] for x in v) / XCDS
        us = statistics.median(x[3] for x in v) / 1e3
        fl = mops * 512
        alg = work.get(k, {}).get("flop")
        lines.append(f"| {k} | {len(v)} | {us:.1f} | {gui / (us * 1e3):.2f} | "
                     f"{100 * busy / (gui * SIMDS):.1f} | {fl / 1e9:.1f} | "
                     + (f"{alg / 1e9:.1f} | " if alg else "- | ")
                     + f"{100 * fl / (gui * peak_per_clk):.1f} | {fl / (us * 1e-6) / 1e12:.0f} |")
    return f"""# Matrix-core counters per GEMM: {desc}

Counters SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16 and
GRBM_GUI_ACTIVE per dispatch (medians over each kernel's dispatches),
summarised by `python bench.py --summarize mfma --workload {w.name} --inputs
<counter csv>`.  `clock` = GPU-active cycles (per XCD) / duration; `MFMA busy`
= busy cycles / (active cycles x 1024 SIMDs); counted flops = MOPS x 512;
`of peak at clock` = counted flops / (active cycles x 2.5 PFLOP/s / 2.4 GHz),
i.e. the matrix cores' share at the clock the kernel actually ran at.

Command (run from the repository root on one MI355X):

```
{_cmds(args)}
```

| kernel | dispatches | us | clock GHz | MFMA busy % | counted GFLOP | algorithmic GFLOP | of peak at clock % | TFLOP/s |
|---|---|---|---|---|---|---|---|---|
""" + "\n".join(lines) + "\n"


def _union(iv):
    merged = []
    for s, e in sorted(iv):
        if merged and s <= merged[-1][1]:
            merged[-1][1] = max(merged[-1][1], e)
        else:
            merged.append([s, e])
    return merged


def _length(m):
    return sum(e - s for s, e in m)


def _intersect(a, b):
    i = j = 0
    out = []
    while i < len(a) and j < len(b):
        s, e = max(a[i][0], b[j][0]), min(a[i][1], b[j][1])
        if s < e:
            out.append((s, e))
        if a[i][1] < b[j][1]:
            i += 1
        else:
            j += 1
    return out


_GEMM_CLASS = GEMM_KERNELS + ("transpose_w", "router", "dwr_mfma")
_PERM_CLASS = ("permute", "combine", "combine_bwd", "dispatch_bwd", "plan_hist", "plan_scan",
               "plan_rank", "force_balance", "topk", "dlogits", "dwr_reduce", "transpose_wr")


def _sum_overlap(args, w, N, T_loc, desc):
    rows = [(bench_name(s), a, b) for s, a, b in read_trace(args.inputs[0])]
    rows = [r for r in rows if r[0]]
    t0, t1 = rows[0][1], max(r[2] for r in rows)
    cut = t0 + 0.4 * (t1 - t0)
    sel = [r for r in rows if r[1] >= cut]
    g = _union([(a, b) for n, a, b in sel if n in _GEMM_CLASS])
    p = _union([(a, b) for n, a, b in sel if n in _PERM_CLASS])
    busy = _union([(a, b) for n, a, b in sel])
    inter = _intersect(g, p)
    ng = sum(1 for r in sel if r[0] in _GEMM_CLASS)
    npm = sum(1 for r in sel if r[0] in _PERM_CLASS)
    # one routed wgrad per step, or one grouped wgrad per args.wgrad_group steps
    grouped = any(n == "wgrad_multi" for n, a, b in rows)
    per = args.wgrad_group if grouped else 1
    wend = [b for n, a, b in rows if n == ("wgrad_multi" if grouped else "wgrad")]
    half = wend[len(wend) // 2:]
    step_us = ((half[-1] - half[0]) / 1e3 / max(1, len(half) - 1) / per
               if len(half) > 1 else float("nan"))
    return f"""# Overlap of the two streams: pipelined 1F1B steps, {desc}

Command (run from the repository root on one MI355X):

```
{_cmds(args)}
```

The steps run through `moe_overlap_steps` (the streams' roles alternating each
step, routed wgrad between the two dgrad GEMMs), eager launches under the
profiler.  Interval analysis over the last 60 % of the trace, summarised by
`python bench.py --summarize overlap --workload {w.name} --inputs <trace>`.
GEMM class: expert GEMMs, router GEMMs and weight transposes; dispatch/combine
class: plan, top-k, permute, combine and their backwards.

| quantity | value |
|---|---|
| GEMM-class kernels / union (us) | {ng} / {_length(g) / 1e3:.1f} |
| dispatch/combine-class kernels / union (us) | {npm} / {_length(p) / 1e3:.1f} |
| intersection (us) | {_length(inter) / 1e3:.1f} |
| share of dispatch/combine time under a GEMM | {100 * _length(inter) / max(1, _length(p)):.2f} % |
| busy (any kernel) union (us) | {_length(busy) / 1e3:.1f} |
| steady step time under the profiler (us, wgrad to wgrad, second half{f", a grouped wgrad per {per} steps" if grouped else ""}) | {step_us:.1f} |
"""


def _rows(path):
    with open(path) as fh:
        return list(csv.DictReader(fh))


def _field(r, *names):
    for n in names:
        if n in r and r[n] != "":
            return r[n]
    raise KeyError(f"none of {names} in {sorted(r)}")


def _sum_phases(args, w, N, T_loc, desc):
    """Per-phase GPU time from a --roctx run: each kernel belongs to the roctx
    range (on the launching thread) that contains the host call launching it,
    matched through the launch's correlation id.  A phase's time per
    occurrence is the summed duration of the kernels of one of its ranges;
    the table gives the median over the second half of its occurrences (the
    first calls of a process run slower while the clocks settle)."""
    import bisect
    kern, api, mark = (_rows(p) for p in args.inputs[:3])
    launch = {}
    for r in api:
        launch[_field(r, "Correlation_Id")] = (_field(r, "Thread_Id"),
                                               int(_field(r, "Start_Timestamp")))
    ranges = collections.defaultdict(list)  # thread -> [(start, end, name)]
    for r in mark:
        name = _field(r, "Function", "Message", "Name")
        if not name.startswith("moe."):
            continue
        ranges[_field(r, "Thread_Id")].append((int(_field(r, "Start_Timestamp")),
                                               int(_field(r, "End_Timestamp")), name))
    for t in ranges:
        ranges[t].sort()
    starts = {t: [a for a, _, _ in v] for t, v in ranges.items()}
    inst = collections.defaultdict(lambda: collections.defaultdict(float))  # phase -> range -> us
    names = collections.defaultdict(set)
    count = collections.Counter()
    unmatched = 0
    for r in kern:
        n = bench_name(_field(r, "Kernel_Name"))
        if not n:
            continue
        a, b = int(_field(r, "Start_Timestamp")), int(_field(r, "End_Timestamp"))
        th, t = launch.get(_field(r, "Correlation_Id"), (None, None))
        key = None
        if th in ranges:
            i = bisect.bisect_right(starts[th], t) - 1
            if i >= 0 and ranges[th][i][1] >= t:
                key = (ranges[th][i][2], (th, i))
        if key is None:
            unmatched += 1
            key = ("(outside any range)", (None, 0))
        inst[key[0]][key[1]] += (b - a) / 1e3
        names[key[0]].add(n)
        count[key[0]] += 1
    rows = []
    for ph, d in inst.items():
        vals = [d[k] for k in sorted(d)]
        tail = vals[len(vals) // 2:]
        rows.append((statistics.median(tail), ph, len(vals), count[ph], sum(vals)))
    # per step: a phase's median times its occurrences per step (the phases
    # that run every step occur most often; the weight copies run once per
    # call, the grouped weight gradient once per group of steps)
    steps = max(r[2] for r in rows)
    per_step = lambda nr: 1.0 if nr > 0.75 * steps else nr / steps
    rows = [(med * per_step(nr), med, ph, nr, nk, tot) for med, ph, nr, nk, tot in rows]
    rows.sort(reverse=True)
    total = sum(r[0] for r in rows)
    lines = [f"| `{ph}` | {nr} | {nk} | {', '.join(sorted(names[ph]))} | {tot:.1f} | {med:.1f} | "
             f"{per:.1f} | {100 * per / max(total, 1e-9):.1f} |"
             for per, med, ph, nr, nk, tot in rows]
    table = "\n".join(lines)
    return f"""# Phases of the step (roctx ranges): {desc}

Command (run from the repository root on one MI355X):

```
{_cmds(args)}
```

`bench.py --roctx` sets MOE_ROCTX=1, so the library brackets each phase of the
step with a roctx range `moe.<phase>` (route, dispatch, expert FFN forward,
combine, and their backwards; the activation- and input-gradient halves of
the expert dgrad separately when the weight gradient runs between them; the
weight gradients; the dgrad weight copies made once per call).  The steps run
eagerly and serialized, so a phase's kernels run alone and their summed
durations are the phase's GPU time.  Each kernel is assigned to the range
that contains the host call that launched it (HIP API trace, matched by
correlation id), summarised by `python bench.py --summarize phases --workload
{w.name} --inputs <kernel trace> <HIP API trace> <marker trace>`.  `per
occurrence` is the median, over the second half of a phase's occurrences, of
the summed kernel time of one range (the first calls of a process run slower
while the clocks settle); `per step` scales it by the phase's occurrences
per step for the phases that run less than once a step (the weight copies
once per call, the grouped weight gradient once per group of steps; the phases
that run in most steps count once), and `share` is its part of the sum of
the per-step times.
Kernels outside every range: {unmatched}.

| phase | occurrences | kernels | kernel names | GPU time, all (us) | per occurrence (us) | per step (us) | share % |
|---|---|---|---|---|---|---|---|
{table}
"""


if __name__ == "__main__":
    main()
