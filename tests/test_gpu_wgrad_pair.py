"""GPU tests of the paired weight gradient: moe_ffn_wgrad_pair (two micro-batches'
rows of each expert reduced in one launch) and MOE_STEP_PAIR_WGRAD in
moe_overlap_steps.

* the paired call against the oracle's weight gradients of both micro-batches
  (their sum, plus the prior values with accumulation), over ragged experts
  (empty, one-row, one past a 64-row stage) in bf16, fp16 and fp32;
* the paired steps, pipelined over two streams, bit-identical to the same
  paired steps serialized, and equal within float32 rounding to the unpaired
  steps;
* the checks: pairing needs the micro-batch back-propagated in step j intact
  in step j + 1, moe_overlap_step rejects the flag, the fused paths and
  stream capture are not supported with it.
"""

import numpy as np
import pytest
import torch

import combine_expert_ffn_amd as M
import oracle as O
from combine_expert_ffn_amd.inputs import Workload, make_inputs
from moe_harness import close_reduction, dev, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()


def _ops(rng, counts, d, F, prec, cap):
    """One micro-batch's wgrad operands (rows padded to the cap) and offsets."""
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    N = int(off[-1])

    def pad(a):
        return np.concatenate([a, np.zeros((cap - a.shape[0], a.shape[1]))])

    xp = pad(rng.standard_normal((N, d)))
    a = pad(0.3 * rng.standard_normal((N, F)))
    dh = pad(0.5 * rng.standard_normal((N, 2 * F)))
    dyp = pad(0.1 * rng.standard_normal((N, d)))
    return off, [dev(t, prec) for t in (xp, a, dh, dyp)]


@pytest.mark.parametrize("prec", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("countsA,countsB", [
    ((700, 0, 1313, 65), (64, 1, 0, 257)),      # empty and one-row experts, ragged stages
    ((1024,) * 4, (1000, 1100, 900, 1090)),     # full experts, second segment ragged
])
def test_wgrad_pair_against_oracle(prec, countsA, countsB):
    d, F = (256, 128) if prec != "f32" else (64, 64)
    E_l = len(countsA)
    cap = max(sum(countsA), sum(countsB))
    s = M.make_shape(cap, d, F, E_l, 0, E_l, 1, prec)
    rng = np.random.default_rng(23)
    offA, A = _ops(rng, countsA, d, F, prec, cap)
    offB, B = _ops(rng, countsB, d, F, prec, cap)
    oA, oB = dev(offA, "i32"), dev(offB, "i32")
    log(f"[wgrad pair] {prec} A={countsA} B={countsB}")
    prior = [torch.full((E_l, 2 * F, d), 0.75, device="cuda"),
             torch.full((E_l, d, F), -0.5, device="cuda")]
    XA = [host(t, int(offA[-1])) for t in A]
    XB = [host(t, int(offB[-1])) for t in B]
    ra = O.ffn_wgrad(*XA, offA, prec="f64")
    rb = O.ffn_wgrad(*XB, offB, prec="f64")
    ma = O.ffn_wgrad(*[np.abs(t) for t in XA], offA, prec="f64")
    mb = O.ffn_wgrad(*[np.abs(t) for t in XB], offB, prec="f64")
    tau = 1e-5
    for acc in (0, M.MOE_ACCUM_DW):
        dW = [t.clone() for t in prior]
        M.moe_ffn_wgrad_pair(s, *A, oA, *B, oB, dW[0], dW[1], acc)
        base = [host(t) if acc else 0.0 for t in prior]
        for k, name in ((0, "dW_gu"), (1, "dW_down")):
            close_reduction(f"{name} pair acc={acc}", host(dW[k]), base[k] + ra[k] + rb[k],
                            ma[k] + mb[k] + np.abs(base[k]), tau)
        # equal to two single calls within float32 rounding, and deterministic
        two = [t.clone() for t in prior]
        M.moe_ffn_wgrad(s, *A, oA, two[0], two[1], acc)
        M.moe_ffn_wgrad(s, *B, oB, two[0], two[1], M.MOE_ACCUM_DW)
        for k in range(2):
            close_reduction("pair vs two calls", host(dW[k]), host(two[k]),
                            ma[k] + mb[k] + np.abs(base[k] if acc else 0.0), tau)
        again = [t.clone() for t in prior]
        M.moe_ffn_wgrad_pair(s, *A, oA, *B, oB, again[0], again[1], acc)
        torch.cuda.synchronize()
        assert torch.equal(again[0], dW[0]) and torch.equal(again[1], dW[1])


@pytest.mark.parametrize("prec", ["bf16", "f32"])
@pytest.mark.parametrize("counts", [
    ((700, 0, 1313, 65), (64, 1, 0, 257), (0, 0, 129, 1000)),
    ((1024,) * 4, (1000, 1100, 900, 1090), (63, 65, 127, 1), (500, 0, 0, 2049)),
])
def test_wgrad_multi_against_oracle(prec, counts):
    """moe_ffn_wgrad_multi over three and four micro-batches against the oracle's
    sum of their weight gradients, and against single calls within float32
    rounding; deterministic."""
    d, F = (256, 128) if prec != "f32" else (64, 64)
    E_l = len(counts[0])
    cap = max(sum(c) for c in counts)
    s = M.make_shape(cap, d, F, E_l, 0, E_l, 1, prec)
    rng = np.random.default_rng(29)
    mbs = [_ops(rng, c, d, F, prec, cap) for c in counts]
    log(f"[wgrad multi] {prec} n={len(counts)} counts={counts}")
    prior = [torch.full((E_l, 2 * F, d), 0.75, device="cuda"),
             torch.full((E_l, d, F), -0.5, device="cuda")]
    ops = [tuple(t) + (dev(off, "i32"),) for off, t in mbs]
    X = [[host(t, int(off[-1])) for t in T_] for off, T_ in mbs]
    refs = [O.ffn_wgrad(*x, off, prec="f64") for x, (off, _) in zip(X, mbs)]
    mags = [O.ffn_wgrad(*[np.abs(t) for t in x], off, prec="f64") for x, (off, _) in zip(X, mbs)]
    tau = 1e-5
    for acc in (0, M.MOE_ACCUM_DW):
        dW = [t.clone() for t in prior]
        M.moe_ffn_wgrad_multi(s, ops, dW[0], dW[1], acc)
        base = [host(t) if acc else 0.0 for t in prior]
        for k, name in ((0, "dW_gu"), (1, "dW_down")):
            close_reduction(f"{name} multi acc={acc}", host(dW[k]),
                            base[k] + sum(r[k] for r in refs),
                            sum(m_[k] for m_ in mags) + np.abs(base[k]), tau)
        one = [t.clone() for t in prior]
        for i, o in enumerate(ops):
            M.moe_ffn_wgrad(s, *o, one[0], one[1], acc if i == 0 else M.MOE_ACCUM_DW)
        for k in range(2):
            close_reduction("multi vs single calls", host(dW[k]), host(one[k]),
                            sum(m_[k] for m_ in mags) + np.abs(base[k] if acc else 0.0), tau)
        again = [t.clone() for t in prior]
        M.moe_ffn_wgrad_multi(s, ops, again[0], again[1], acc)
        torch.cuda.synchronize()
        assert torch.equal(again[0], dW[0]) and torch.equal(again[1], dW[1])


def _steps(s, w, m, W, dW, ws, n, W_r, bias, rot, overwrite=(), shared=None):
    """n 1F1B steps over buffer sets m: step j forwards m[j % rot] (none in
    the last step) and back-propagates m[(j - 1) % rot] (none in the first);
    the steps in `overwrite` overwrite the weight gradients, the others add."""
    return [M.make_step(s, M.MOE_ROUTE_TOPK, W[0], W[1], dW[0], dW[1], ws,
                        fwd=m[j % rot] if j < n - 1 else None,
                        bwd=m[(j - 1) % rot] if j > 0 else None, W_r=W_r, bias=bias,
                        dW_r=dW[2], accumulate=0 if j in overwrite else M.MOE_ACCUM_DW,
                        shared=shared)
            for j in range(n)]


P2, G4 = M.MOE_STEP_PAIR_WGRAD, M.MOE_STEP_GROUP4_WGRAD


@pytest.mark.parametrize("name,n,flags,overwrite,group", [
    ("zipf_bf16", 8, M.MOE_STEP_MID_WGRAD, (), P2),
    ("zipf_bf16", 7, 0, (), P2),
    ("zipf_bf16", 9, M.MOE_STEP_SKIP_WGRAD, (), P2),
    ("mid_f32", 6, M.MOE_STEP_MID_WGRAD, (), P2),
    # the first backward overwrites: its pair starts from zero
    ("zipf_bf16", 7, M.MOE_STEP_MID_WGRAD, (1,), P2),
    # the second overwrites: steps 1 and 2 do not pair (2 discards 1's sums)
    ("zipf_bf16", 7, 0, (2,), P2),
    # an overwrite in the middle of the run
    ("mid_f32", 8, M.MOE_STEP_MID_WGRAD, (4,), P2),
    # groups of four: two whole groups and a remainder, with SKIP_WGRAD, with
    # an overwrite starting a group and one inside a would-be group
    ("zipf_bf16", 11, M.MOE_STEP_MID_WGRAD, (), G4),
    ("zipf_bf16", 10, M.MOE_STEP_SKIP_WGRAD, (), G4),
    ("mid_f32", 10, 0, (1,), G4),
    ("zipf_bf16", 10, M.MOE_STEP_MID_WGRAD, (3,), G4),
    # fp16 data through the same grouped launch
    ("zipf_f16", 10, M.MOE_STEP_MID_WGRAD, (), G4),
    # with a shared expert (its weight gradients stay per step)
    ("zipf_bf16_shared", 10, M.MOE_STEP_MID_WGRAD, (), G4),
    ("zipf_bf16_shared", 9, 0, (2,), P2),
])
def test_pair_steps_pipelined_equals_serialized(name, n, flags, overwrite, group):
    w = {
        "zipf_bf16": Workload("zipf_bf16", T=700, d=192, F=320, E=64, e_lo=0, E_l=8, K=6,
                              dtype="bf16", route="topk", zipf_s=1.1),
        "zipf_bf16_shared": Workload("zipf_bf16_shared", T=700, d=192, F=320, E=64, e_lo=0,
                                     E_l=8, K=6, dtype="bf16", route="topk", zipf_s=1.1),
        "zipf_f16": Workload("zipf_f16", T=700, d=192, F=320, E=64, e_lo=0, E_l=8, K=6,
                             dtype="f16", route="topk", zipf_s=1.1),
        "mid_f32": Workload("mid_f32", T=150, d=64, F=64, E=16, e_lo=5, E_l=3, K=4,
                            dtype="f32", route="topk"),
    }[name]
    prec = w.dtype
    log(f"[grouped steps] {name} n={n} flags={flags} overwrite={overwrite} group={group}")
    inp = make_inputs(w, seed=3, microbatches=2)
    s = M.shape_of(w)
    D = lambda a: dev(a, prec)
    W = (D(inp["W_gu"]), D(inp["W_down"]))
    W_r = D(inp["W_r"])
    bias = dev(inp["bias"], "f32x") if inp["bias"] is not None else None
    s0, s1 = torch.cuda.current_stream(), torch.cuda.Stream()
    Fs = 128 if name.endswith("_shared") else 0
    rng = np.random.default_rng(17)
    W_s = (D(O.store(0.05 * rng.standard_normal((2 * Fs, w.d)), prec)),
           D(O.store(0.05 * rng.standard_normal((w.d, Fs)), prec))) if Fs else None
    # a group of G steps keeps G micro-batches until its last step: G + 1
    # buffer sets rotate
    rot = 3 if group == P2 else 5
    xs = [inp["x"], inp["x_b"], inp["x"][::-1].copy(), inp["x_b"][::-1].copy(),
          np.roll(inp["x"], 7, axis=0)][:rot]
    ds = [inp["dout"], inp["dout_b"], inp["dout"][::-1].copy(), inp["dout_b"][::-1].copy(),
          np.roll(inp["dout"], 7, axis=0)][:rot]
    res = {}
    for tag, fl in (("serial", flags | group | M.MOE_STEP_SERIALIZE),
                    ("pipelined", flags | group),
                    ("unpaired", flags)):
        m = [M.MicroBatch(s, x=D(xs[i]), dout=D(ds[i]), F_s=Fs) for i in range(rot)]
        dW = (torch.full((w.E_l, 2 * w.F, w.d), 0.25, device="cuda"),
              torch.full((w.E_l, w.d, w.F), 0.25, device="cuda"),
              torch.full((w.d, w.E), 0.25, device="cuda"))
        sh = None
        if Fs:
            sh = (W_s[0], W_s[1], torch.full((2 * Fs, w.d), 0.25, device="cuda"),
                  torch.full((w.d, Fs), 0.25, device="cuda"))
        ws = torch.empty(M.moe_step_workspace_bytes_shared(s, Fs), dtype=torch.uint8,
                         device="cuda")
        M.moe_overlap_steps(_steps(s, w, m, W, dW, ws, n, W_r, bias, rot, overwrite, sh),
                            s0, s1, fl)
        if flags & M.MOE_STEP_SKIP_WGRAD:  # the caller's delayed wgrad of the last step
            b = m[(n - 2) % rot]
            M.moe_ffn_wgrad(s, b.xp, b.a, b.dh, b.dyp, b.offsets, dW[0], dW[1],
                            M.MOE_ACCUM_DW, stream=s0)
            assert not Fs, "the shared expert's delayed wgrad is not issued here"
        torch.cuda.synchronize()
        res[tag] = (m, dW, sh)
    (ma, ga, sa), (mb, gb, sb), (mu, gu, su) = res["serial"], res["pipelined"], res["unpaired"]
    if Fs:  # the shared expert's weight gradients are not grouped
        for k in (2, 3):
            assert torch.equal(sa[k], sb[k]) and torch.equal(sa[k], su[k]), ("shared dW", k)
    for i in range(rot):
        for k in ("out", "dx", "dgates", "dlogits", "idx") + (("y_s", "dx_s") if Fs else ()):
            assert torch.equal(getattr(mb[i], k), getattr(ma[i], k)), (i, k)
            assert torch.equal(getattr(mu[i], k), getattr(ma[i], k)), ("unpaired", i, k)
        # dh is sized to the cap; rows past N are never written
        N = int(ma[i].offsets[-1])
        assert torch.equal(mb[i].dh[:N], ma[i].dh[:N]) and torch.equal(mu[i].dh[:N], ma[i].dh[:N])
    for k in range(3):
        assert torch.equal(ga[k], gb[k]), ("dW", k)
    # the paired sums differ from the unpaired ones only in float32 rounding
    assert torch.equal(ga[2], gu[2])  # the router's dW_r is not paired
    for k in range(2):
        ref = gu[k].double()
        err = ((ga[k].double() - ref).abs() / ref.abs().clamp(min=1.0)).max().item()
        assert err <= 1e-5, (k, err)
    log("[grouped steps] pipelined == serialized; ungrouped within float32 rounding")


def test_pair_steps_checks():
    w = Workload("pc", T=64, d=64, F=64, E=4, e_lo=0, E_l=4, K=2, dtype="bf16", route="topk")
    inp = make_inputs(w, seed=4, microbatches=2)
    s = M.shape_of(w)
    D = lambda a: dev(a, "bf16")
    W = (D(inp["W_gu"]), D(inp["W_down"]))
    W_r = D(inp["W_r"])
    s0, s1 = torch.cuda.current_stream(), torch.cuda.Stream()
    dW = (torch.zeros((w.E_l, 2 * w.F, w.d), device="cuda"),
          torch.zeros((w.E_l, w.d, w.F), device="cuda"), torch.zeros((w.d, w.E), device="cuda"))
    ws = torch.empty(M.moe_step_workspace_bytes(s), dtype=torch.uint8, device="cuda")
    m2 = [M.MicroBatch(s, x=D(inp["x"]), dout=D(inp["dout"])),
          M.MicroBatch(s, x=D(inp["x_b"]), dout=D(inp["dout_b"]))]
    # two buffer sets: step 2 forwards into what step 1 back-propagated
    steps = _steps(s, w, m2, W, dW, ws, 4, W_r, None, 2)
    with pytest.raises(M.MoeError) as e:
        M.moe_overlap_steps(steps, s0, s1, M.MOE_STEP_PAIR_WGRAD)
    assert e.value.code == M.MOE_ERR_ARG
    with pytest.raises(M.MoeError) as e:
        M.moe_overlap_step(steps[1], s0, s1, M.MOE_STEP_PAIR_WGRAD)
    assert e.value.code == M.MOE_ERR_ARG
    with pytest.raises(M.MoeError) as e:
        M.moe_overlap_steps(steps, s0, s1, M.MOE_STEP_PAIR_WGRAD | M.MOE_STEP_FUSED_PERMUTE)
    assert e.value.code == M.MOE_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    # steps that accumulate into other weight-gradient buffers are not paired:
    # the same results, bit for bit, as the steps without the flag
    outs = []
    for fl in (M.MOE_STEP_PAIR_WGRAD, 0):
        m3x = [M.MicroBatch(s, x=D(inp["x"]), dout=D(inp["dout"])),
               M.MicroBatch(s, x=D(inp["x_b"]), dout=D(inp["dout_b"])),
               M.MicroBatch(s, x=D(inp["x"][::-1].copy()), dout=D(inp["dout"][::-1].copy()))]
        dWa = [torch.full_like(t, 0.5) for t in dW[:2]]
        dWb = [torch.full_like(t, -0.5) for t in dW[:2]]
        st4 = _steps(s, w, m3x, W, dW, ws, 5, W_r, None, 3)
        for j in range(5):  # odd steps into one pair of buffers, even into another
            g_ = dWa if j % 2 else dWb
            st4[j].dW_gu, st4[j].dW_down = g_[0].data_ptr(), g_[1].data_ptr()
        M.moe_overlap_steps(st4, s0, s1, fl)
        torch.cuda.synchronize()
        outs.append(dWa + dWb)
    for a_, b_ in zip(*outs):
        assert torch.equal(a_, b_)
    # groups of four need the deferred micro-batches intact for three steps:
    # three buffer sets are too few
    m3 = m2 + [M.MicroBatch(s, x=D(inp["x"][::-1].copy()), dout=D(inp["dout"][::-1].copy()))]
    steps6 = _steps(s, w, m3, W, dW, ws, 6, W_r, None, 3)
    with pytest.raises(M.MoeError) as e:
        M.moe_overlap_steps(steps6, s0, s1, M.MOE_STEP_GROUP4_WGRAD)
    assert e.value.code == M.MOE_ERR_ARG
    with pytest.raises(M.MoeError) as e:
        M.moe_overlap_step(steps6[1], s0, s1, M.MOE_STEP_GROUP4_WGRAD)
    assert e.value.code == M.MOE_ERR_ARG
    torch.cuda.synchronize()
    # paired steps are issued eagerly only: under stream capture the call
    # returns the error before it issues anything (the graph holds only the
    # fill around it)
    steps3 = _steps(s, w, m3, W, dW, ws, 4, W_r, None, 3)
    probe = torch.zeros(64, device="cuda")
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(s0)
    codes = []
    with torch.cuda.graph(g, stream=cap, capture_error_mode="thread_local"):
        probe.add_(1.0)
        try:
            M.moe_overlap_steps(steps3, torch.cuda.current_stream(), s1, M.MOE_STEP_PAIR_WGRAD)
        except M.MoeError as err:
            codes.append(err.code)
        probe.add_(1.0)
    torch.cuda.synchronize()
    assert codes == [M.MOE_ERR_UNSUPPORTED]
    g.replay()
    torch.cuda.synchronize()
    assert float(probe[0]) == 2.0
