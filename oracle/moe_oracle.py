"""Plain CPU definition of the MoE expert-parallel layer (test infrastructure only).

Each function computes one call of the layer in float64 with numpy, in the order
the pages give the phases (skill card page 1, "What it is"; 1F1B note page 2,
"how the 8 ops are split": forward dispatch -> expert MLP -> combine, backward
combine -> MLP (D before W, "MoE 1F1B overlap") -> dispatch).  There is no
blocking, fusion or reordering beyond the plain definition, so each line can be
checked against the formula it states.

Notation: T tokens, d hidden, F expert FFN width, E experts routed over, the
local expert window [e_lo, e_lo + E_l), K experts per token.  N = number of
(token, slot) pairs whose expert is local = rows of the permuted matrix.
"""

from __future__ import annotations

import numpy as np

PRECISIONS = ("f64", "f32", "bf16", "f16")


# ----------------------------------------------------------------------------
# rounding
# ----------------------------------------------------------------------------
def round_bf16(a) -> np.ndarray:
    """Round to bfloat16 with round-to-nearest-even, returned as float64 values.

    The value is first rounded to float32 (as a float32 accumulator holds it),
    then the low 16 bits of the float32 pattern are removed with RNE: add
    0x7FFF plus the lowest kept bit, then truncate.  Inputs are finite.
    """
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + keep_lsb) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def round_f16(a) -> np.ndarray:
    """Round to IEEE binary16 with round-to-nearest-even, returned as float64.

    As for bfloat16, the value is first rounded to float32 (the accumulator),
    then to the binary16 grid: with |v| = m * 2^e, 1 <= m < 2, the spacing of
    binary16 values is 2^(e - 10) for normal numbers (e >= -14) and the fixed
    2^-24 below, so v is divided by that spacing, rounded to the nearest
    integer with ties to even, and scaled back.  Magnitudes that round to
    2^16 or beyond overflow to infinity.
    """
    v = np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)
    _, ex = np.frexp(v)                      # v = f * 2^ex, 0.5 <= |f| < 1
    e = np.maximum(ex - 1, -14)
    q = np.ldexp(1.0, e - 10)
    r = np.rint(v / q) * q                   # rint: ties to even
    return np.where(np.abs(r) >= 65536.0, np.copysign(np.inf, v), r)


def round_f32(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def store(v, prec: str) -> np.ndarray:
    """Value of an activation-sized tensor as stored in precision ``prec``."""
    if prec == "f64":
        return np.asarray(v, dtype=np.float64)
    if prec == "f32":
        return round_f32(v)
    if prec == "bf16":
        return round_bf16(v)
    if prec == "f16":
        return round_f16(v)
    raise ValueError(prec)


def store_f32(v, prec: str) -> np.ndarray:
    """Value of a tensor that is float32 in every mode except ``f64``."""
    return np.asarray(v, dtype=np.float64) if prec == "f64" else round_f32(v)


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


# ----------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------
def router_logits(x, W_r, bias=None, prec="bf16") -> np.ndarray:
    """Router scores l = x . W_r (+ bias), float32 output.

    x [T, d], W_r [d, E], bias [E] or None.
    """
    l = np.asarray(x, np.float64) @ np.asarray(W_r, np.float64)
    if bias is not None:
        l = l + np.asarray(bias, np.float64)[None, :]
    return store_f32(l, prec)


def topk_route(logits, K: int, prec="bf16"):
    """Top-K selection and gates from router logits.

    idx[t, :] are the first K experts in descending-logit order, ties going to
    the lower expert index (a stable sort of -logits).  Gates: softmax over all
    E experts, the K selected probabilities, divided by their sum (equal to a
    softmax over the selected logits).  Returns (idx int32 [T,K], gates [T,K]).
    """
    l = np.asarray(logits, np.float64)
    T, E = l.shape
    if not (1 <= K <= E):
        raise ValueError("need 1 <= K <= E")
    idx = np.argsort(-l, axis=1, kind="stable")[:, :K].astype(np.int32)
    m = l.max(axis=1, keepdims=True)
    p = np.exp(l - m)
    p = p / p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    gates = sel / sel.sum(axis=1, keepdims=True)
    return idx, store_f32(gates, prec)


def force_balance_idx(T: int, K: int, E: int) -> np.ndarray:
    """Forced-balance routing: slot k of token t goes to expert (t*K + k) mod E."""
    t = np.arange(T, dtype=np.int64)[:, None]
    k = np.arange(K, dtype=np.int64)[None, :]
    return ((t * K + k) % E).astype(np.int32)


# ----------------------------------------------------------------------------
# dispatch (token -> expert-grouped rows)
# ----------------------------------------------------------------------------
def dispatch_plan(idx, e_lo: int, E_l: int, tile_m: int):
    """Stable counting sort of the local (token, slot) pairs by local expert.

    Pairs are ordered lexicographically by (t, k).  A pair is local when its
    expert e is in [e_lo, e_lo + E_l); its local id is j = e - e_lo.
    counts[j] = number of local pairs with id j; offsets = exclusive prefix sum
    (E_l + 1 entries, offsets[E_l] = N).  row_of_pair[t*K + k] = offsets[j] +
    number of earlier local pairs with the same id, or -1 for a non-local pair.
    pair_of_row is the inverse on rows [0, N) and -1 on rows [N, T*K).
    tile_offsets = exclusive prefix sum of ceil(counts / tile_m).
    """
    idx = np.asarray(idx)
    T, K = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    counts = np.zeros(E_l, np.int64)
    for e in flat:
        if e_lo <= e < e_lo + E_l:
            counts[e - e_lo] += 1
    offsets = np.zeros(E_l + 1, np.int64)
    for j in range(E_l):
        offsets[j + 1] = offsets[j] + counts[j]
    seen = np.zeros(E_l, np.int64)
    row_of_pair = np.full(T * K, -1, np.int64)
    for p, e in enumerate(flat):
        if e_lo <= e < e_lo + E_l:
            j = e - e_lo
            row_of_pair[p] = offsets[j] + seen[j]
            seen[j] += 1
    pair_of_row = np.full(T * K, -1, np.int64)
    for p in range(T * K):
        if row_of_pair[p] >= 0:
            pair_of_row[row_of_pair[p]] = p
    tiles = (counts + tile_m - 1) // tile_m
    tile_offsets = np.zeros(E_l + 1, np.int64)
    for j in range(E_l):
        tile_offsets[j + 1] = tile_offsets[j] + tiles[j]
    return dict(
        counts=counts.astype(np.int32),
        offsets=offsets.astype(np.int32),
        row_of_pair=row_of_pair.astype(np.int32).reshape(T, K),
        pair_of_row=pair_of_row.astype(np.int32),
        tile_offsets=tile_offsets.astype(np.int32),
    )


def permute(x, pair_of_row, K: int, N: int) -> np.ndarray:
    """xp[r] = x[token of pair pair_of_row[r]] for the N local rows (exact copy)."""
    x = np.asarray(x, np.float64)
    rows = np.asarray(pair_of_row[:N], np.int64)
    return x[rows // K].copy()


# ----------------------------------------------------------------------------
# expert FFN (SwiGLU) forward
# ----------------------------------------------------------------------------
def expert_ffn_fwd(xp, offsets, W_gu, W_down, prec="bf16"):
    """Per local expert j on its rows [offsets[j], offsets[j+1]):

    g = xp . W_gate[j]^T, u = xp . W_up[j]^T  (W_gu[j] rows [0,F) gate, [F,2F) up)
    h = [g, u] (stored), a = silu(g) * u from the unrounded g, u (stored),
    y_p = a_stored . W_down[j]^T (stored).   W_down[j] is [d, F].
    """
    xp = np.asarray(xp, np.float64)
    W_gu = np.asarray(W_gu, np.float64)
    W_down = np.asarray(W_down, np.float64)
    E_l, twoF, d = W_gu.shape
    F = twoF // 2
    N = int(offsets[E_l])
    h = np.zeros((N, 2 * F))
    a = np.zeros((N, F))
    yp = np.zeros((N, d))
    for j in range(E_l):
        r0, r1 = int(offsets[j]), int(offsets[j + 1])
        if r1 == r0:
            continue
        X = xp[r0:r1]
        g = X @ W_gu[j, :F].T
        u = X @ W_gu[j, F:].T
        h[r0:r1, :F] = store(g, prec)
        h[r0:r1, F:] = store(u, prec)
        a[r0:r1] = store(_silu(g) * u, prec)
        yp[r0:r1] = store(a[r0:r1] @ W_down[j].T, prec)
    return h, a, yp


# ----------------------------------------------------------------------------
# combine (expert-grouped rows -> tokens, gate-weighted)
# ----------------------------------------------------------------------------
def combine(yp, gates, row_of_pair, prec="bf16", add=None) -> np.ndarray:
    """out[t] = [add[t] +] sum over local slots k (ascending) of
    gates[t,k] * y_p[row(t,k)]; a token with no local slot gets add[t] (or 0).
    ``add`` is a token-aligned term, the shared expert's output."""
    yp = np.asarray(yp, np.float64)
    gates = np.asarray(gates, np.float64)
    T, K = row_of_pair.shape
    out = np.zeros((T, yp.shape[1])) if add is None else np.asarray(add, np.float64).copy()
    for k in range(K):
        r = row_of_pair[:, k]
        m = r >= 0
        out[m] += gates[m, k][:, None] * yp[r[m]]
    return store(out, prec)


def combine_bwd(dout, yp, gates, row_of_pair, N: int, prec="bf16"):
    """Backward of combine.  For a local pair (t,k) with row r:
    dy_p[r] = gates[t,k] * dout[t] (stored); dgates[t,k] = <dout[t], y_p[r]>.
    dgates is 0 for non-local pairs."""
    dout = np.asarray(dout, np.float64)
    yp = np.asarray(yp, np.float64)
    gates = np.asarray(gates, np.float64)
    T, K = row_of_pair.shape
    d = dout.shape[1]
    dyp = np.zeros((N, d))
    dgates = np.zeros((T, K))
    for k in range(K):
        r = row_of_pair[:, k]
        m = r >= 0
        dyp[r[m]] = gates[m, k][:, None] * dout[m]
        dgates[m, k] = np.sum(dout[m] * yp[r[m]], axis=1)
    return store(dyp, prec), store_f32(dgates, prec)


# ----------------------------------------------------------------------------
# expert FFN backward: activation gradient (D) and weight gradient (W)
# ----------------------------------------------------------------------------
def ffn_dgrad(dyp, h, offsets, W_gu, W_down, prec="bf16"):
    """Activation gradient of the SwiGLU expert FFN, per local expert j:

    da = dy_p . W_down[j] (kept unrounded); with g, u read from the stored h and
    s = sigmoid(g): dg = da * u * s * (1 + g (1 - s)), du = da * g * s;
    dh = [dg, du] (stored); dxp = dh_stored . W_gu[j] (stored).
    """
    dyp = np.asarray(dyp, np.float64)
    h = np.asarray(h, np.float64)
    W_gu = np.asarray(W_gu, np.float64)
    W_down = np.asarray(W_down, np.float64)
    E_l, twoF, d = W_gu.shape
    F = twoF // 2
    N = int(offsets[E_l])
    dh = np.zeros((N, 2 * F))
    dxp = np.zeros((N, d))
    for j in range(E_l):
        r0, r1 = int(offsets[j]), int(offsets[j + 1])
        if r1 == r0:
            continue
        da = dyp[r0:r1] @ W_down[j]
        g = h[r0:r1, :F]
        u = h[r0:r1, F:]
        s = _sigmoid(g)
        dh[r0:r1, :F] = store(da * u * s * (1.0 + g * (1.0 - s)), prec)
        dh[r0:r1, F:] = store(da * g * s, prec)
        dxp[r0:r1] = store(dh[r0:r1] @ W_gu[j], prec)
    return dh, dxp


def ffn_wgrad(xp, a, dh, dyp, offsets, dW_gu_prev=None, dW_down_prev=None, prec="bf16"):
    """Weight gradient of the expert FFN, reduced over each expert's rows:

    dW_down[j] = sum_r dy_p[r] (outer) a[r];   dW_gu[j] = sum_r dh[r] (outer) xp[r]
    (float32 output).  With the ``*_prev`` arguments the result is added to them
    (gradient accumulation); an expert with no rows gets 0 (or its prior value).
    """
    xp = np.asarray(xp, np.float64)
    a = np.asarray(a, np.float64)
    dh = np.asarray(dh, np.float64)
    dyp = np.asarray(dyp, np.float64)
    E_l = len(offsets) - 1
    twoF = dh.shape[1]
    F = a.shape[1]
    d = xp.shape[1]
    dW_gu = np.zeros((E_l, twoF, d))
    dW_down = np.zeros((E_l, d, F))
    for j in range(E_l):
        r0, r1 = int(offsets[j]), int(offsets[j + 1])
        dW_down[j] = dyp[r0:r1].T @ a[r0:r1]
        dW_gu[j] = dh[r0:r1].T @ xp[r0:r1]
    if dW_gu_prev is not None:
        dW_gu = np.asarray(dW_gu_prev, np.float64) + dW_gu
    if dW_down_prev is not None:
        dW_down = np.asarray(dW_down_prev, np.float64) + dW_down
    return store_f32(dW_gu, prec), store_f32(dW_down, prec)


# ----------------------------------------------------------------------------
# router backward and dispatch backward
# ----------------------------------------------------------------------------
def route_bwd(dgates, gates, idx, x, E: int, dW_r_prev=None, prec="bf16"):
    """Backward of the top-K softmax gates and of the router product.

    Gates are a softmax over the selected logits, so for a selected slot j
    dlogits[t, idx[t,j]] = g_j (dg_j - sum_k g_k dg_k); all other logits get 0.
    dW_r = x^T . dlogits (float32; added to ``dW_r_prev`` when given).
    Returns (dlogits [T,E], dW_r [d,E] or None when x is None).
    """
    dg = np.asarray(dgates, np.float64)
    g = np.asarray(gates, np.float64)
    T, K = g.shape
    inner = np.sum(g * dg, axis=1, keepdims=True)
    dsel = g * (dg - inner)
    dlogits = np.zeros((T, E))
    for k in range(K):
        dlogits[np.arange(T), idx[:, k]] += dsel[:, k]
    dlogits = store_f32(dlogits, prec)
    dW_r = None
    if x is not None:
        dW_r = np.asarray(x, np.float64).T @ dlogits
        if dW_r_prev is not None:
            dW_r = np.asarray(dW_r_prev, np.float64) + dW_r
        dW_r = store_f32(dW_r, prec)
    return dlogits, dW_r


def dispatch_bwd(dxp, row_of_pair, dlogits=None, W_r=None, dx_prev=None, prec="bf16",
                 add=None):
    """Gradient with respect to the layer input x:

    dx[t] = [dx_prev[t]] + [add[t]] + sum over local slots k of dxp[row(t,k)]
            [+ (dlogits . W_r^T)[t]   when the router is differentiated],
    stored once.  ``add`` is a token-aligned term, the shared expert's input
    gradient.
    """
    dxp = np.asarray(dxp, np.float64)
    T, K = row_of_pair.shape
    d = dxp.shape[1]
    dx = np.zeros((T, d)) if dx_prev is None else np.asarray(dx_prev, np.float64).copy()
    if add is not None:
        dx += np.asarray(add, np.float64)
    for k in range(K):
        r = row_of_pair[:, k]
        m = r >= 0
        dx[m] += dxp[r[m]]
    if dlogits is not None:
        dx += np.asarray(dlogits, np.float64) @ np.asarray(W_r, np.float64).T
    return store(dx, prec)


# ----------------------------------------------------------------------------
# shared expert: one SwiGLU FFN every token passes through, beside the routed
# experts (skill card page 1 names the shared-expert overlap), i.e. an expert
# over all T rows in token order with gate 1
# ----------------------------------------------------------------------------
def shared_expert_fwd(x, W_gu_s, W_down_s, prec="bf16"):
    """h_s = [g, u] = x . W_gu_s^T, a_s = silu(g) * u, y_s = a_s . W_down_s^T."""
    T = np.asarray(x).shape[0]
    return expert_ffn_fwd(x, np.array([0, T]), np.asarray(W_gu_s)[None],
                          np.asarray(W_down_s)[None], prec)


def shared_expert_dgrad(dout, h_s, W_gu_s, W_down_s, prec="bf16"):
    """dh_s and dx_s of the shared expert for output gradient dout."""
    T = np.asarray(dout).shape[0]
    return ffn_dgrad(dout, h_s, np.array([0, T]), np.asarray(W_gu_s)[None],
                     np.asarray(W_down_s)[None], prec)


def shared_expert_wgrad(x, a_s, dh_s, dout, dW_gu_prev=None, dW_down_prev=None, prec="bf16"):
    """dW_gu_s = dh_s^T . x, dW_down_s = dout^T . a_s (float32)."""
    T = np.asarray(x).shape[0]
    gu, dn = ffn_wgrad(x, a_s, dh_s, dout, np.array([0, T]),
                       None if dW_gu_prev is None else np.asarray(dW_gu_prev)[None],
                       None if dW_down_prev is None else np.asarray(dW_down_prev)[None], prec)
    return gu[0], dn[0]


# ----------------------------------------------------------------------------
# whole layer, in the pages' phase order
# ----------------------------------------------------------------------------
def layer_forward(x, K, e_lo, E_l, W_gu, W_down, *, W_r=None, bias=None, E=None,
                  logits=None, force_balance=False, gates=None, tile_m=256,
                  prec="bf16", shared=None):
    """route -> dispatch (plan + permute) -> expert FFN -> combine.

    Routing: ``force_balance`` (idx from the closed form, ``gates`` given), or
    top-K over ``logits`` when given, else over x . W_r + bias.  ``shared`` =
    (W_gu_s, W_down_s) adds the shared expert's output into the combine.
    """
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    if force_balance:
        if E is None:
            raise ValueError("E required")
        idx = force_balance_idx(T, K, E)
        g = np.asarray(gates, np.float64)
        lg = None
    else:
        lg = logits if logits is not None else router_logits(x, W_r, bias, prec)
        E = lg.shape[1]
        idx, g = topk_route(lg, K, prec)
    plan = dispatch_plan(idx, e_lo, E_l, tile_m)
    N = int(plan["offsets"][E_l])
    xp = permute(x, plan["pair_of_row"], K, N)
    h, a, yp = expert_ffn_fwd(xp, plan["offsets"], W_gu, W_down, prec)
    sh = {}
    if shared is not None:
        h_s, a_s, y_s = shared_expert_fwd(x, shared[0], shared[1], prec)
        sh = dict(h_s=h_s, a_s=a_s, y_s=y_s)
    out = combine(yp, g, plan["row_of_pair"], prec, add=sh.get("y_s"))
    return dict(logits=lg, idx=idx, gates=g, N=N, xp=xp, h=h, a=a, yp=yp, out=out,
                E=E, **plan, **sh)


def layer_backward(fwd, x, dout, W_gu, W_down, *, W_r=None, differentiate_router=True,
                   prec="bf16", shared=None):
    """combine bwd -> router bwd -> expert D (dgrad) -> dispatch bwd -> expert W (wgrad).
    With ``shared`` = (W_gu_s, W_down_s) the shared expert's D joins the
    dispatch backward and its W follows the routed W."""
    N = fwd["N"]
    dyp, dgates = combine_bwd(dout, fwd["yp"], fwd["gates"], fwd["row_of_pair"], N, prec)
    dlogits = dW_r = None
    if differentiate_router:
        dlogits, dW_r = route_bwd(dgates, fwd["gates"], fwd["idx"],
                                  x if W_r is not None else None, fwd["E"], prec=prec)
    dh, dxp = ffn_dgrad(dyp, fwd["h"], fwd["offsets"], W_gu, W_down, prec)
    sh = {}
    if shared is not None:
        dh_s, dx_s = shared_expert_dgrad(dout, fwd["h_s"], shared[0], shared[1], prec)
        sh = dict(dh_s=dh_s, dx_s=dx_s)
    dx = dispatch_bwd(dxp, fwd["row_of_pair"],
                      dlogits if (differentiate_router and W_r is not None) else None,
                      W_r, None, prec, add=sh.get("dx_s"))
    dW_gu, dW_down = ffn_wgrad(fwd["xp"], fwd["a"], dh, dyp, fwd["offsets"], prec=prec)
    if shared is not None:
        sh["dW_gu_s"], sh["dW_down_s"] = shared_expert_wgrad(
            np.asarray(x, np.float64), fwd["a_s"], sh["dh_s"], dout, prec=prec)
    return dict(dyp=dyp, dgates=dgates, dlogits=dlogits, dW_r=dW_r, dh=dh, dxp=dxp,
                dx=dx, dW_gu=dW_gu, dW_down=dW_down, **sh)
