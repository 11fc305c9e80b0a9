"""Full-size workloads on the GPU, in the launch configuration the benchmark times
(moe_overlap_step on two streams), checked against the oracle on sampled
outputs: the oracle recomputes sampled rows / tokens / weight-gradient entries
from the GPU's inputs to that stage.  Maps and indices are checked in full.
Also: overlapped == serialized == eager-wgrad, bit for bit (the pages' "loss
trajectory unchanged by overlap" criterion, skill card page 1, success criteria)."""

import numpy as np
import pytest
import torch

import combine_expert_ffn_amd as M
import oracle as O
from combine_expert_ffn_amd.inputs import WORKLOADS, Workload, make_inputs
from moe_harness import TAU, close, dev, exact, host, log, topk_gap

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()


class Net:
    """Device weights and gradient buffers of one workload."""

    def __init__(self, w, inp):
        D = lambda a: dev(a, w.dtype)
        self.w = w
        self.s = M.shape_of(w)
        self.topk = w.route == "topk"
        self.mode = M.MOE_ROUTE_TOPK if self.topk else M.MOE_ROUTE_FORCE_BALANCE
        self.W_gu, self.W_down = D(inp["W_gu"]), D(inp["W_down"])
        self.W_r = D(inp["W_r"]) if self.topk else None
        self.bias = dev(inp["bias"], "f32x") if inp["bias"] is not None else None
        self.dW_gu = torch.empty(w.E_l, 2 * w.F, w.d, dtype=torch.float32, device="cuda")
        self.dW_down = torch.empty(w.E_l, w.d, w.F, dtype=torch.float32, device="cuda")
        self.dW_r = torch.empty(w.d, w.E, dtype=torch.float32, device="cuda") if self.topk else None
        self.ws = torch.empty(M.moe_step_workspace_bytes(self.s), dtype=torch.uint8, device="cuda")

    def mb(self, x, dout, gates=None, fused=False):
        D = lambda a: dev(a, self.w.dtype)
        return M.MicroBatch(self.s, x=D(x), dout=D(dout),
                            gates=None if gates is None else dev(gates, "f32x"), fused=fused)

    def make(self, fwd, bwd, accumulate=0):
        return M.make_step(self.s, self.mode, self.W_gu, self.W_down, self.dW_gu, self.dW_down,
                           self.ws, fwd=fwd, bwd=bwd, W_r=self.W_r, bias=self.bias,
                           dW_r=self.dW_r, accumulate=accumulate)

    def step(self, fwd, bwd, s0, s1, flags, accumulate=0):
        M.moe_overlap_step(self.make(fwd, bwd, accumulate), s0, s1, flags)


def _rows(t, idx):
    return host(t[torch.from_numpy(np.asarray(idx, np.int64)).cuda()])


def sampled_check(w, inp, A, net, rng, nrows=192, ntok=96, wgrad_prev=None):
    """Check micro-batch A (forward and backward done) against the oracle on samples."""
    prec, tau = w.dtype, TAU[w.dtype]
    K = w.K
    x64 = np.asarray(inp["x"], np.float64)
    # ---- routing: in full
    if net.topk:
        ref_l = O.router_logits(x64, np.asarray(inp["W_r"], np.float64), inp["bias"], prec)
        gl = host(A.logits)
        close("logits", gl, ref_l, tau)
        i_o, g_o = O.topk_route(gl, K, prec)
        exact("idx vs oracle top-k of the GPU logits", host(A.idx), i_o)
        close("gates", host(A.gates), g_o, tau)
        i_ref, _ = O.topk_route(ref_l, K, prec)
        diff = np.any(i_o != i_ref, axis=1)
        assert np.all(topk_gap(ref_l, K)[diff] < 1e-4), "selection differs without a near tie"
        log(f"  routing: {diff.sum()} of {w.T} tokens differ from oracle-logit routing (near ties)")
    else:
        exact("idx", host(A.idx), O.force_balance_idx(w.T, K, w.E))
    idx = host(A.idx)
    gates = host(A.gates)
    # ---- plan: in full
    plan = O.dispatch_plan(idx, w.e_lo, w.E_l, M.moe_tile_m())
    for k in ("counts", "offsets", "tile_offsets", "row_of_pair", "pair_of_row"):
        exact(k, host(getattr(A, k)), plan[k])
    offsets = plan["offsets"]
    N = int(offsets[-1])
    log(f"  plan: N={N} rows, counts min {plan['counts'].min()} max {plan['counts'].max()}")
    # ---- sampled rows: permute, FFN forward, dgrad
    rows = np.sort(rng.choice(N, min(nrows, N), replace=False))
    exact("xp rows", _rows(A.xp, rows), x64[plan["pair_of_row"][rows] // K])
    xp_s, h_s, a_s, y_s = (_rows(getattr(A, k), rows) for k in ("xp", "h", "a", "yp"))
    dyp_s, dh_s, dxp_s = (_rows(getattr(A, k), rows) for k in ("dyp", "dh", "dxp"))
    e_of = np.searchsorted(offsets, rows, side="right") - 1
    for j in np.unique(e_of):
        sel = e_of == j
        o = np.array([0, sel.sum()])
        Wg = np.asarray(inp["W_gu"][j:j + 1], np.float64)
        Wd = np.asarray(inp["W_down"][j:j + 1], np.float64)
        hh, aa, yy = O.expert_ffn_fwd(xp_s[sel], o, Wg, Wd, prec)
        close(f"h (expert {j})", h_s[sel], hh, tau)
        close(f"a (expert {j})", a_s[sel], aa, tau)
        close(f"yp (expert {j})", y_s[sel], yy, tau)
        dh_r, dxp_r = O.ffn_dgrad(dyp_s[sel], h_s[sel], o, Wg, Wd, prec)
        close(f"dh (expert {j})", dh_s[sel], dh_r, tau)
        close(f"dxp (expert {j})", dxp_s[sel], dxp_r, tau)
    # ---- sampled tokens: combine, combine bwd, router bwd, dispatch bwd
    toks = np.sort(rng.choice(w.T, min(ntok, w.T), replace=False))
    rop = plan["row_of_pair"][toks]
    loc = np.unique(rop[rop >= 0])
    remap = {r: i for i, r in enumerate(loc)}
    rop_l = np.vectorize(lambda r: remap.get(r, -1))(rop) if rop.size else rop
    yp_l = _rows(A.yp, loc)
    dout = np.asarray(inp["dout"], np.float64)[toks]
    close("out", _rows(A.out, toks), O.combine(yp_l, gates[toks], rop_l, prec), tau)
    dyp_l, dg_l = O.combine_bwd(dout, yp_l, gates[toks], rop_l, len(loc), prec)
    close("dyp (token rows)", _rows(A.dyp, loc), dyp_l, tau)
    dgates = host(A.dgates)
    close("dgates", dgates[toks], dg_l, tau)
    dl_t = None
    if net.topk:
        dl_t, _ = O.route_bwd(dgates[toks], gates[toks], idx[toks], None, w.E, prec=prec)
        close("dlogits", _rows(A.dlogits, toks), dl_t, tau)
        if wgrad_prev is None:
            cols = np.sort(rng.choice(w.d, 16, replace=False))
            _, dwr = O.route_bwd(dgates, gates, idx, x64[:, cols], w.E, prec=prec)
            close("dW_r (columns)", host(net.dW_r)[cols], dwr, tau)
        dl_t = _rows(A.dlogits, toks)
    dxp_l = _rows(A.dxp, loc)
    W_r64 = np.asarray(inp["W_r"], np.float64) if net.topk else None
    close("dx", _rows(A.dx, toks), O.dispatch_bwd(dxp_l, rop_l, dl_t, W_r64, None, prec), tau)
    # ---- weight gradients: every entry of dW_gu[j] and dW_down[j] for eight
    # experts (the largest, the smallest and six drawn at random), from the
    # GPU's own stage inputs of those experts' rows
    if wgrad_prev is None:
        nz = np.nonzero(plan["counts"])[0]
        experts = np.unique(np.concatenate([
            nz[[np.argmax(plan["counts"][nz]), np.argmin(plan["counts"][nz])]],
            rng.choice(nz, min(6, nz.size), replace=False)]))
        for j in experts:
            r0, r1 = int(offsets[j]), int(offsets[j + 1])
            sl = lambda t: host(t[r0:r1])
            gu, dn = O.ffn_wgrad(sl(A.xp), sl(A.a), sl(A.dh), sl(A.dyp),
                                 np.array([0, r1 - r0]), prec=prec)
            close(f"dW_gu (expert {j}, all entries)", host(net.dW_gu[j]), gu[0], tau)
            close(f"dW_down (expert {j}, all entries)", host(net.dW_down[j]), dn[0], tau)
        log(f"  wgrad: all entries of {len(experts)} experts checked")


@pytest.mark.parametrize("name,T", [("ep16_rank_bf16", None), ("ep8_rank_zipf_bf16", None),
                                    ("ep1_128exp_bf16", 16384), ("ep16_rank_f16", None),
                                    # the size that matches the 524288 dispatched rows
                                    ("ep1_128exp_bf16", 65536)])
def test_fullsize_sampled(name, T):
    w = WORKLOADS[name] if T is None else WORKLOADS[name].with_tokens(T)
    log(f"[full size] {name}: T={w.T} d={w.d} F={w.F} E={w.E} E_l={w.E_l} K={w.K}")
    inp = make_inputs(w, seed=0)
    net = Net(w, inp)
    A = net.mb(inp["x"], inp["dout"], inp["gates"])
    s0 = torch.cuda.current_stream()
    s1 = torch.cuda.Stream()
    net.step(A, None, s0, s1, 0)
    net.step(None, A, s0, s1, 0)
    torch.cuda.synchronize()
    sampled_check(w, inp, A, net, np.random.default_rng(1))
    log(f"[full size] {name}: ok")


def test_overlap_equals_serialized_two_microbatch():
    w = WORKLOADS["two_microbatch_bf16"]
    log(f"[overlap] two micro-batches T={w.T} d={w.d} F={w.F} E={w.E} K={w.K}")
    inp = make_inputs(w, seed=0)
    net = Net(w, inp)
    s0 = torch.cuda.current_stream()
    s1 = torch.cuda.Stream()
    results = {}
    def late_wgrad(mb, acc):  # the wgrad a SKIP_WGRAD step leaves to the caller
        M.moe_ffn_wgrad(net.s, mb.xp, mb.a, mb.dh, mb.dyp, mb.offsets, net.dW_gu, net.dW_down,
                        acc, s0)

    fp = M.MOE_STEP_FUSED_PERMUTE
    mid = M.MOE_STEP_MID_WGRAD
    for tag, flags, copy in (("serial", M.MOE_STEP_SERIALIZE, s0), ("overlap", 0, s1),
                             ("eager", M.MOE_STEP_EAGER_WGRAD, s1),
                             ("skip", M.MOE_STEP_SKIP_WGRAD, s1),
                             ("fused", fp, s1), ("fused_serial", fp | M.MOE_STEP_SERIALIZE, s0),
                             ("mid", mid, s1), ("mid_serial", mid | M.MOE_STEP_SERIALIZE, s0),
                             ("mid_fused", mid | fp, s1), ("multi", -1, s1),
                             ("multi_mid", -1 ^ mid, s1)):
        multi = flags < 0       # the three steps in one pipelined moe_overlap_steps call
        flags = ~flags if multi else flags
        skip = flags == M.MOE_STEP_SKIP_WGRAD
        A = net.mb(inp["x"], inp["dout"], fused=bool(flags & fp))
        B = net.mb(inp["x_b"], inp["dout_b"], fused=bool(flags & fp))
        if multi:
            M.moe_overlap_steps([net.make(A, None), net.make(B, A),
                                 net.make(None, B, M.MOE_ACCUM_DW)], s0, copy, flags)
        else:
            net.step(A, None, s0, copy, flags)
            net.step(B, A, s0, copy, flags)                    # A's grads overwrite
            if skip:
                late_wgrad(A, 0)
            net.step(None, B, s0, copy, flags, M.MOE_ACCUM_DW)  # B's grads accumulate
            if skip:
                late_wgrad(B, M.MOE_ACCUM_DW)
        torch.cuda.synchronize()
        results[tag] = dict(A=A, B=B, dW_gu=net.dW_gu.clone(), dW_down=net.dW_down.clone(),
                            dW_r=net.dW_r.clone())
    ref = results["serial"]
    for tag in ("overlap", "eager", "skip", "fused", "fused_serial", "mid", "mid_serial",
                "mid_fused", "multi", "multi_mid"):
        r = results[tag]
        for mbn in ("A", "B"):
            for k in ("idx", "gates", "row_of_pair", "out", "dgates", "dlogits", "dx", "yp"):
                assert torch.equal(getattr(r[mbn], k), getattr(ref[mbn], k)), (tag, mbn, k)
        for k in ("dW_gu", "dW_down", "dW_r"):
            assert torch.equal(r[k], ref[k]), (tag, k)
    log("[overlap] overlapped, eager-wgrad, caller-deferred-wgrad, mid-wgrad, fused-permute "
        "and pipelined multi-step runs bit-identical to serialized")
    # oracle on samples of micro-batch A (weight grads hold A + B)
    r = results["overlap"]
    A, B = r["A"], r["B"]
    net.dW_gu.copy_(r["dW_gu"])
    net.dW_down.copy_(r["dW_down"])
    net.dW_r.copy_(r["dW_r"])
    rng = np.random.default_rng(2)
    sampled_check(w, inp, A, net, rng, wgrad_prev=True)
    # weight gradients: sum over both micro-batches, sampled entries
    prec, tau = w.dtype, TAU[w.dtype]
    cols = np.sort(rng.choice(w.d, 16, replace=False))
    prev = None
    for mb, xk in ((A, "x"), (B, "x_b")):
        _, prev = O.route_bwd(host(mb.dgates), host(mb.gates), host(mb.idx),
                              np.asarray(inp[xk], np.float64)[:, cols], w.E, dW_r_prev=prev,
                              prec=prec)
    close("dW_r A+B (columns)", host(net.dW_r)[cols], prev, tau)
    for j in (0, 5):
        I = np.sort(rng.choice(w.d, 8, replace=False))
        Fc = np.sort(rng.choice(w.F, 8, replace=False))
        Mc = np.sort(rng.choice(2 * w.F, 8, replace=False))
        Cc = np.sort(rng.choice(w.d, 8, replace=False))
        prev = None
        for mb in (A, B):
            off = host(mb.offsets)
            r0, r1 = int(off[j]), int(off[j + 1])
            sl = lambda t, c: host(t[r0:r1][:, torch.from_numpy(c).cuda()])
            gu, dn = O.ffn_wgrad(sl(mb.xp, Cc), sl(mb.a, Fc), sl(mb.dh, Mc), sl(mb.dyp, I),
                                 np.array([0, r1 - r0]),
                                 dW_gu_prev=None if prev is None else prev[0],
                                 dW_down_prev=None if prev is None else prev[1], prec=prec)
            prev = (gu, dn)
        close(f"dW_gu A+B (expert {j})", host(net.dW_gu[j])[np.ix_(Mc, Cc)], prev[0][0], tau)
        close(f"dW_down A+B (expert {j})", host(net.dW_down[j])[np.ix_(I, Fc)], prev[1][0], tau)


@pytest.mark.parametrize("pipelined", [False, True])
def test_step_graph_replay_matches_eager(pipelined):
    """G 1F1B steps captured into one HIP graph (stream 1 forked from and
    joined to the capture stream by the steps' own events) and replayed three
    times, with eager work and synchronisation between replays: after every
    replay the micro-batch outputs and the accumulated weight gradients equal
    those of the same steps launched eagerly one by one, bit for bit.  Captured
    either as G moe_overlap_step calls (G = 2) or as one pipelined
    moe_overlap_steps call with the wgrad between the dgrad GEMMs (G = 4), the
    form bench.py times."""
    w = Workload("graph_bf16", T=330, d=256, F=192, E=16, e_lo=4, E_l=8, K=4, dtype="bf16",
                 route="topk", zipf_s=1.1)
    inp = make_inputs(w, seed=3, microbatches=2)
    log(f"[graph] T={w.T} d={w.d} F={w.F} E={w.E} window [{w.e_lo},{w.e_lo + w.E_l}) K={w.K}")
    keys = ("out", "dx", "dgates", "dlogits", "idx", "row_of_pair")

    def state(net, mbs):
        snap = {f"{k}{j}": getattr(mbs[j], k).clone() for k in keys for j in (0, 1)}
        snap.update(dW_gu=net.dW_gu.clone(), dW_down=net.dW_down.clone(), dW_r=net.dW_r.clone())
        return snap

    def fresh():
        net = Net(w, inp)
        for t in (net.dW_gu, net.dW_down, net.dW_r):
            t.zero_()
        mbs = [net.mb(inp["x"], inp["dout"]), net.mb(inp["x_b"], inp["dout_b"])]
        return net, mbs

    G = 4 if pipelined else 2
    s1 = torch.cuda.Stream()
    # eager: prime, then 3 G steps, a snapshot after every G-th step
    net, mbs = fresh()
    s0 = torch.cuda.current_stream()
    net.step(mbs[0], None, s0, s1, 0)
    ref = []
    for j in range(3 * G):
        net.step(mbs[(j + 1) % 2], mbs[j % 2], s0, s1, 0, M.MOE_ACCUM_DW)
        if j % G == G - 1:
            torch.cuda.synchronize()
            ref.append(state(net, mbs))
    # graph: prime eagerly, capture G steps, replay three times
    net, mbs = fresh()
    net.step(mbs[0], None, s0, s1, 0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(s0)
    with torch.cuda.graph(g, stream=cap, capture_error_mode="thread_local"):
        c0 = torch.cuda.current_stream()
        if pipelined:
            M.moe_overlap_steps([net.make(mbs[(j + 1) % 2], mbs[j % 2], M.MOE_ACCUM_DW)
                                 for j in range(G)], c0, s1, M.MOE_STEP_MID_WGRAD)
        else:
            for j in range(G):
                net.step(mbs[(j + 1) % 2], mbs[j % 2], c0, s1, 0, M.MOE_ACCUM_DW)
    for r in range(3):
        g.replay()
        torch.cuda.synchronize()
        junk = torch.randn(4096, device="cuda").square().sum().item()  # eager work in between
        assert junk > 0
        got = state(net, mbs)
        for k, v in ref[r].items():
            assert torch.equal(got[k], v), (r, k)
        log(f"[graph] replay {r}: bit-identical to the eager steps")


@pytest.mark.parametrize("group", [2, 4])
def test_fullsize_grouped_steps(group):
    """The 128-expert layer in the schedule bench.py times: one pipelined
    moe_overlap_steps call with the wgrad between the dgrad GEMMs and grouped
    weight gradients (the first `group` back-propagated micro-batches' in one
    launch, the last one's alone), group + 1 micro-batch buffer sets.  Each
    micro-batch's forward and backward outputs on samples, and every entry of
    three experts' accumulated weight gradients (the sum over all the
    micro-batches, from the GPU's own stage inputs), against the oracle."""
    w = WORKLOADS["ep1_128exp_bf16"]
    nm = group + 1
    log(f"[full size grouped] {w.name}: T={w.T} E={w.E} K={w.K}, {nm} micro-batches, "
        f"groups of {group}")
    inp = make_inputs(w, seed=0, microbatches=2)
    net = Net(w, inp)
    for t in (net.dW_gu, net.dW_down, net.dW_r):
        t.zero_()
    srcs = [("", lambda a: a), ("_b", lambda a: a), ("", lambda a: a[::-1].copy()),
            ("_b", lambda a: a[::-1].copy()), ("", lambda a: np.roll(a, 28, axis=0))][:nm]
    xs = [f(inp["x" + k]) for k, f in srcs]
    ds = [f(inp["dout" + k]) for k, f in srcs]
    m = [net.mb(xs[i], ds[i]) for i in range(nm)]
    acc = M.MOE_ACCUM_DW
    steps = [net.make(m[0], None, acc)] + \
        [net.make(m[i + 1], m[i], acc) for i in range(nm - 1)] + [net.make(None, m[-1], acc)]
    flag = M.MOE_STEP_PAIR_WGRAD if group == 2 else M.MOE_STEP_GROUP4_WGRAD
    s0, s1 = torch.cuda.current_stream(), torch.cuda.Stream()
    M.moe_overlap_steps(steps, s0, s1, M.MOE_STEP_MID_WGRAD | flag)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for i in range(nm):
        log(f"  micro-batch {i}")
        sampled_check(w, dict(inp, x=xs[i], dout=ds[i]), m[i], net, rng, wgrad_prev=True)
    prec, tau = w.dtype, TAU[w.dtype]
    counts = host(m[0].counts)
    experts = [int(np.argmax(counts)), int(np.argmin(counts)), 77]
    for j in experts:
        prev = None
        for mb in m:
            off = host(mb.offsets)
            r0, r1 = int(off[j]), int(off[j + 1])
            sl = lambda t: host(t[r0:r1])
            prev = O.ffn_wgrad(sl(mb.xp), sl(mb.a), sl(mb.dh), sl(mb.dyp), np.array([0, r1 - r0]),
                               dW_gu_prev=None if prev is None else prev[0],
                               dW_down_prev=None if prev is None else prev[1], prec=prec)
        close(f"dW_gu of {nm} micro-batches (expert {j}, all entries)", host(net.dW_gu[j]),
              prev[0][0], tau)
        close(f"dW_down of {nm} micro-batches (expert {j}, all entries)",
              host(net.dW_down[j]), prev[1][0], tau)
    log(f"[full size grouped] ok: outputs of {nm} micro-batches, dW of experts {experts}")
