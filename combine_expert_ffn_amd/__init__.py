"""combine_expert_ffn_amd - one GPU's share of a Mixture-of-Experts expert-parallel
layer on AMD Instinct MI355X (gfx950).

The compute lives in the HIP library ``libmoe.so`` (C ABI: ``include/moe.h``).
This module is a thin binding with the same entry-point names: it marshals
torch tensors (device memory) and streams into the C calls and raises
``MoeError`` on a non-zero status.  PyTorch supplies memory and streams only.
"""

from __future__ import annotations

import ctypes as C

from ._lib import (  # noqa: F401
    LIB_PATH, MB_FIELDS, MoeError, MoeMB, MoeShape, MoeStep, MoeWgradOps, check, lib,
    MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_WORKSPACE, MOE_ERR_HIP,
    MOE_ERR_UNSUPPORTED, MOE_ERR_ARG, MOE_F32, MOE_BF16, MOE_F16, MOE_ROUTE_TOPK,
    MOE_ROUTE_TOPK_FROM_LOGITS, MOE_ROUTE_FORCE_BALANCE, MOE_ACCUM_DX, MOE_ACCUM_DW,
    MOE_STEP_SERIALIZE, MOE_STEP_EAGER_WGRAD, MOE_STEP_SKIP_WGRAD, MOE_STEP_FUSED_PERMUTE,
    MOE_STEP_MID_WGRAD, MOE_STEP_FUSED_COMBINE_BWD, MOE_STEP_PAIR_WGRAD, MOE_STEP_FUSED_SCATTER,
    MOE_STEP_GROUP4_WGRAD,
)


_DATA, _F32, _I32 = "data", "f32", "i32"


def _torch_dtype(kind, s):
    import torch

    if kind == _F32:
        return torch.float32
    if kind == _I32:
        return torch.int32
    return {MOE_BF16: torch.bfloat16, MOE_F16: torch.float16}.get(s.dtype, torch.float32)


def _chk(s, fn, name, t, kind, numel, optional=False):
    """Host-side check of one tensor argument before it is passed as a raw
    pointer: on the GPU, contiguous, of the element type the shape implies,
    and holding at least ``numel`` elements (the size include/moe.h gives).
    Raises MoeError(MOE_ERR_ARG) instead of letting the library read or
    write past an allocation."""
    if t is None:
        if optional:
            return
        raise MoeError(MOE_ERR_NULL, f"{fn}: {name} is None")
    import torch

    if not isinstance(t, torch.Tensor):
        raise MoeError(MOE_ERR_ARG, f"{fn}: {name} is not a torch tensor")
    if not t.is_cuda:
        raise MoeError(MOE_ERR_ARG, f"{fn}: {name} is not on the GPU")
    if not t.is_contiguous():
        raise MoeError(MOE_ERR_ARG, f"{fn}: {name} is not contiguous")
    want = _torch_dtype(kind, s)
    if t.dtype != want:
        raise MoeError(MOE_ERR_ARG, f"{fn}: {name} is {t.dtype}, expected {want}")
    if t.numel() < int(numel):
        raise MoeError(MOE_ERR_ARG, f"{fn}: {name} has {t.numel()} elements, needs {int(numel)}")


def _chk_ws(fn, ws):
    if ws is None:
        return
    import torch

    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous():
        raise MoeError(MOE_ERR_ARG, f"{fn}: workspace must be a contiguous GPU tensor")


def _p(t):
    if t is None:
        return None
    ptr = t.data_ptr()
    if ptr == 0 and t.numel() == 0:  # empty view of a real allocation
        ptr = t.untyped_storage().data_ptr()
    return ptr


def _stream(stream):
    import torch

    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ws(ws):
    return (None, 0) if ws is None else (ws.data_ptr(), ws.numel() * ws.element_size())


def make_shape(T, d, F, E, e_lo, E_l, K, dtype) -> MoeShape:
    dt = {"bf16": MOE_BF16, "f16": MOE_F16, "f32": MOE_F32}.get(dtype, dtype)
    return MoeShape(int(T), int(d), int(F), int(E), int(e_lo), int(E_l), int(K), int(dt), 0)


def shape_of(w, T=None) -> MoeShape:
    """MoeShape of an ``inputs.Workload`` (optionally with another token count)."""
    return make_shape(w.T if T is None else T, w.d, w.F, w.E, w.e_lo, w.E_l, w.K, w.dtype)


def moe_workspace_bytes(s: MoeShape) -> int:
    return lib().moe_workspace_bytes(C.byref(s))


def moe_step_workspace_bytes_shared(s: MoeShape, F_s: int) -> int:
    return lib().moe_step_workspace_bytes_shared(C.byref(s), int(F_s))


def moe_shared_workspace_bytes(s: MoeShape, F_s: int) -> int:
    return lib().moe_shared_workspace_bytes(C.byref(s), int(F_s))


def moe_shared_expert_fwd(s, F_s, x, W_gu_s, W_down_s, h_s, a_s, y_s, ws, stream=None):
    fn, T, d, Fs = "moe_shared_expert_fwd", s.T, s.d, int(F_s)
    for n, t, k, c in (("x", x, _DATA, T * d), ("W_gu_s", W_gu_s, _DATA, 2 * Fs * d),
                       ("W_down_s", W_down_s, _DATA, d * Fs), ("h_s", h_s, _DATA, T * 2 * Fs),
                       ("a_s", a_s, _DATA, T * Fs), ("y_s", y_s, _DATA, T * d)):
        _chk(s, fn, n, t, k, c)
    _chk_ws(fn, ws)
    wp, wb = _ws(ws)
    check(lib().moe_shared_expert_fwd(C.byref(s), int(F_s), _p(x), _p(W_gu_s), _p(W_down_s),
                                      _p(h_s), _p(a_s), _p(y_s), wp, wb, _stream(stream)))


def moe_shared_expert_dgrad(s, F_s, dout, h_s, W_gu_s, W_down_s, dh_s, dx_s, ws, stream=None):
    fn, T, d, Fs = "moe_shared_expert_dgrad", s.T, s.d, int(F_s)
    for n, t, k, c in (("dout", dout, _DATA, T * d), ("h_s", h_s, _DATA, T * 2 * Fs),
                       ("W_gu_s", W_gu_s, _DATA, 2 * Fs * d), ("W_down_s", W_down_s, _DATA, d * Fs),
                       ("dh_s", dh_s, _DATA, T * 2 * Fs), ("dx_s", dx_s, _DATA, T * d)):
        _chk(s, fn, n, t, k, c)
    _chk_ws(fn, ws)
    wp, wb = _ws(ws)
    check(lib().moe_shared_expert_dgrad(C.byref(s), int(F_s), _p(dout), _p(h_s), _p(W_gu_s),
                                        _p(W_down_s), _p(dh_s), _p(dx_s), wp, wb,
                                        _stream(stream)))


def moe_shared_expert_wgrad(s, F_s, x, a_s, dh_s, dout, dW_gu_s, dW_down_s, accumulate, ws,
                            stream=None):
    fn, T, d, Fs = "moe_shared_expert_wgrad", s.T, s.d, int(F_s)
    for n, t, k, c in (("x", x, _DATA, T * d), ("a_s", a_s, _DATA, T * Fs),
                       ("dh_s", dh_s, _DATA, T * 2 * Fs), ("dout", dout, _DATA, T * d),
                       ("dW_gu_s", dW_gu_s, _F32, 2 * Fs * d), ("dW_down_s", dW_down_s, _F32, d * Fs)):
        _chk(s, fn, n, t, k, c)
    _chk_ws(fn, ws)
    wp, wb = _ws(ws)
    check(lib().moe_shared_expert_wgrad(C.byref(s), int(F_s), _p(x), _p(a_s), _p(dh_s),
                                        _p(dout), _p(dW_gu_s), _p(dW_down_s), int(accumulate),
                                        wp, wb, _stream(stream)))


def moe_step_workspace_bytes(s: MoeShape) -> int:
    return lib().moe_step_workspace_bytes(C.byref(s))


def moe_tile_m() -> int:
    return lib().moe_tile_m()


def moe_version() -> int:
    return lib().moe_version()


def moe_route(s, mode, x, W_r, bias, logits, idx, gates, ws, stream=None):
    fn, T, d, E, K = "moe_route", s.T, s.d, s.E, s.K
    topk = mode == MOE_ROUTE_TOPK
    fb = mode == MOE_ROUTE_FORCE_BALANCE
    _chk(s, fn, "x", x, _DATA, T * d, optional=not topk)
    _chk(s, fn, "W_r", W_r, _DATA, d * E, optional=not topk)
    _chk(s, fn, "bias", bias, _F32, E, optional=True)
    _chk(s, fn, "logits", logits, _F32, T * E, optional=fb)
    _chk(s, fn, "idx", idx, _I32, T * K)
    _chk(s, fn, "gates", gates, _F32, T * K, optional=fb)
    _chk_ws(fn, ws)
    wp, wb = _ws(ws)
    check(lib().moe_route(C.byref(s), mode, _p(x), _p(W_r), _p(bias), _p(logits), _p(idx),
                          _p(gates), wp, wb, _stream(stream)))


def moe_dispatch(s, x, idx, counts, offsets, row_of_pair, pair_of_row, tile_offsets, xp, ws,
                 stream=None):
    _chk_plan(s, "moe_dispatch", x, idx, counts, offsets, row_of_pair, pair_of_row, tile_offsets,
              xp)
    _chk_ws("moe_dispatch", ws)
    wp, wb = _ws(ws)
    check(lib().moe_dispatch(C.byref(s), _p(x), _p(idx), _p(counts), _p(offsets),
                             _p(row_of_pair), _p(pair_of_row), _p(tile_offsets), _p(xp), wp, wb,
                             _stream(stream)))


def _chk_plan(s, fn, x, idx, counts, offsets, row_of_pair, pair_of_row, tile_offsets, xp):
    T, d, E_l, K = s.T, s.d, s.E_l, s.K
    _chk(s, fn, "x", x, _DATA, T * d, optional=xp is None)
    _chk(s, fn, "xp", xp, _DATA, T * K * d, optional=True)
    for n, t, c in (("idx", idx, T * K), ("counts", counts, E_l), ("offsets", offsets, E_l + 1),
                    ("row_of_pair", row_of_pair, T * K), ("pair_of_row", pair_of_row, T * K),
                    ("tile_offsets", tile_offsets, E_l + 1)):
        _chk(s, fn, n, t, _I32, c)


def _chk_ffn(s, fn, offsets, tile_offsets, W_gu, W_down, **rows):
    """offsets/tile_offsets, the expert weights and row buffers of the given
    widths (name=(tensor, columns, kind))."""
    cap, d, F, E_l = s.T * s.K, s.d, s.F, s.E_l
    _chk(s, fn, "offsets", offsets, _I32, E_l + 1)
    if tile_offsets is not False:
        _chk(s, fn, "tile_offsets", tile_offsets, _I32, E_l + 1)
    if W_gu is not False:
        _chk(s, fn, "W_gu", W_gu, _DATA, E_l * 2 * F * d)
        _chk(s, fn, "W_down", W_down, _DATA, E_l * d * F)
    for n, (t, cols, kind) in rows.items():
        _chk(s, fn, n, t, kind, cols)


def moe_dispatch_noalloc(s, x, idx, counts, offsets, row_of_pair, pair_of_row, tile_offsets, xp,
                         stream=None):
    _chk_plan(s, "moe_dispatch_noalloc", x, idx, counts, offsets, row_of_pair, pair_of_row,
              tile_offsets, xp)
    check(lib().moe_dispatch_noalloc(C.byref(s), _p(x), _p(idx), _p(counts), _p(offsets),
                                     _p(row_of_pair), _p(pair_of_row), _p(tile_offsets), _p(xp),
                                     _stream(stream)))


def moe_dispatch_noalloc_max_scratch() -> int:
    return lib().moe_dispatch_noalloc_max_scratch()


def moe_expert_ffn_fwd(s, xp, offsets, tile_offsets, W_gu, W_down, h, a, yp, stream=None):
    cap, d, F = s.T * s.K, s.d, s.F
    _chk_ffn(s, "moe_expert_ffn_fwd", offsets, tile_offsets, W_gu, W_down,
             xp=(xp, cap * d, _DATA), h=(h, cap * 2 * F, _DATA), a=(a, cap * F, _DATA),
             yp=(yp, cap * d, _DATA))
    check(lib().moe_expert_ffn_fwd(C.byref(s), _p(xp), _p(offsets), _p(tile_offsets), _p(W_gu),
                                   _p(W_down), _p(h), _p(a), _p(yp), _stream(stream)))


def moe_expert_ffn_fwd_gather(s, x, pair_of_row, offsets, tile_offsets, W_gu, W_down, h, a, yp,
                              stream=None):
    cap, d, F = s.T * s.K, s.d, s.F
    _chk_ffn(s, "moe_expert_ffn_fwd_gather", offsets, tile_offsets, W_gu, W_down,
             x=(x, s.T * d, _DATA), pair_of_row=(pair_of_row, cap, _I32),
             h=(h, cap * 2 * F, _DATA), a=(a, cap * F, _DATA), yp=(yp, cap * d, _DATA))
    check(lib().moe_expert_ffn_fwd_gather(C.byref(s), _p(x), _p(pair_of_row), _p(offsets),
                                          _p(tile_offsets), _p(W_gu), _p(W_down), _p(h), _p(a),
                                          _p(yp), _stream(stream)))


def moe_expert_ffn_fwd_scatter(s, xp, x, pair_of_row, offsets, tile_offsets, W_gu, W_down, h,
                               a, yq, stream=None):
    """xp None: GEMM1 gathers x through pair_of_row (the fused permute)."""
    cap, d, F = s.T * s.K, s.d, s.F
    fn = "moe_expert_ffn_fwd_scatter"
    if xp is None and x is None:
        raise ValueError(f"{fn}: xp and x are both None")
    ops = dict(pair_of_row=(pair_of_row, cap, _I32), h=(h, cap * 2 * F, _DATA),
               a=(a, cap * F, _DATA), yq=(yq, cap * d, _DATA))
    if xp is not None:
        ops["xp"] = (xp, cap * d, _DATA)
    else:
        ops["x"] = (x, s.T * d, _DATA)
    _chk_ffn(s, fn, offsets, tile_offsets, W_gu, W_down, **ops)
    check(lib().moe_expert_ffn_fwd_scatter(C.byref(s), _p(xp), _p(x), _p(pair_of_row),
                                           _p(offsets), _p(tile_offsets), _p(W_gu), _p(W_down),
                                           _p(h), _p(a), _p(yq), _stream(stream)))


def moe_combine_pairs(s, yq, gates, row_of_pair, out, stream=None):
    fn, T, d, K = "moe_combine_pairs", s.T, s.d, s.K
    _chk(s, fn, "yq", yq, _DATA, T * K * d)
    _chk(s, fn, "gates", gates, _F32, T * K)
    _chk(s, fn, "row_of_pair", row_of_pair, _I32, T * K)
    _chk(s, fn, "out", out, _DATA, T * d)
    check(lib().moe_combine_pairs(C.byref(s), _p(yq), _p(gates), _p(row_of_pair), _p(out),
                                  _stream(stream)))


def moe_combine_bwd_pairs(s, dout, yq, gates, row_of_pair, dyp, dgates, stream=None):
    """dyp None: dgates only (the fused combine backward)."""
    fn, T, d, K = "moe_combine_bwd_pairs", s.T, s.d, s.K
    _chk(s, fn, "dout", dout, _DATA, T * d)
    _chk(s, fn, "yq", yq, _DATA, T * K * d)
    _chk(s, fn, "gates", gates, _F32, T * K)
    _chk(s, fn, "row_of_pair", row_of_pair, _I32, T * K)
    _chk(s, fn, "dyp", dyp, _DATA, T * K * d, optional=True)
    _chk(s, fn, "dgates", dgates, _F32, T * K)
    check(lib().moe_combine_bwd_pairs(C.byref(s), _p(dout), _p(yq), _p(gates), _p(row_of_pair),
                                      _p(dyp), _p(dgates), _stream(stream)))


def moe_combine(s, yp, gates, row_of_pair, out, stream=None):
    fn, T, d, K = "moe_combine", s.T, s.d, s.K
    _chk(s, fn, "yp", yp, _DATA, T * K * d)
    _chk(s, fn, "gates", gates, _F32, T * K)
    _chk(s, fn, "row_of_pair", row_of_pair, _I32, T * K)
    _chk(s, fn, "out", out, _DATA, T * d)
    check(lib().moe_combine(C.byref(s), _p(yp), _p(gates), _p(row_of_pair), _p(out),
                            _stream(stream)))


def moe_combine_bwd(s, dout, yp, gates, row_of_pair, dyp, dgates, stream=None):
    """dyp None: dgates only (the fused combine backward)."""
    fn, T, d, K = "moe_combine_bwd", s.T, s.d, s.K
    _chk(s, fn, "dout", dout, _DATA, T * d)
    _chk(s, fn, "yp", yp, _DATA, T * K * d)
    _chk(s, fn, "gates", gates, _F32, T * K)
    _chk(s, fn, "row_of_pair", row_of_pair, _I32, T * K)
    _chk(s, fn, "dyp", dyp, _DATA, T * K * d, optional=True)
    _chk(s, fn, "dgates", dgates, _F32, T * K)
    check(lib().moe_combine_bwd(C.byref(s), _p(dout), _p(yp), _p(gates), _p(row_of_pair),
                                _p(dyp), _p(dgates), _stream(stream)))


def moe_ffn_dgrad(s, dyp, h, offsets, tile_offsets, W_gu, W_down, dh, dxp, ws, stream=None):
    cap, d, F = s.T * s.K, s.d, s.F
    _chk_ffn(s, "moe_ffn_dgrad", offsets, tile_offsets, W_gu, W_down,
             dyp=(dyp, cap * d, _DATA), h=(h, cap * 2 * F, _DATA), dh=(dh, cap * 2 * F, _DATA),
             dxp=(dxp, cap * d, _DATA))
    _chk_ws("moe_ffn_dgrad", ws)
    wp, wb = _ws(ws)
    check(lib().moe_ffn_dgrad(C.byref(s), _p(dyp), _p(h), _p(offsets), _p(tile_offsets),
                              _p(W_gu), _p(W_down), _p(dh), _p(dxp), wp, wb, _stream(stream)))


def moe_ffn_wgrad(s, xp, a, dh, dyp, offsets, dW_gu, dW_down, accumulate=0, stream=None):
    cap, d, F, E_l = s.T * s.K, s.d, s.F, s.E_l
    _chk_ffn(s, "moe_ffn_wgrad", offsets, False, False, False,
             xp=(xp, cap * d, _DATA), a=(a, cap * F, _DATA), dh=(dh, cap * 2 * F, _DATA),
             dyp=(dyp, cap * d, _DATA), dW_gu=(dW_gu, E_l * 2 * F * d, _F32),
             dW_down=(dW_down, E_l * d * F, _F32))
    check(lib().moe_ffn_wgrad(C.byref(s), _p(xp), _p(a), _p(dh), _p(dyp), _p(offsets),
                              _p(dW_gu), _p(dW_down), int(accumulate), _stream(stream)))


def moe_ffn_wgrad_pair(s, xp, a, dh, dyp, offsets, xp2, a2, dh2, dyp2, offsets2, dW_gu, dW_down,
                       accumulate=0, stream=None):
    cap, d, F, E_l = s.T * s.K, s.d, s.F, s.E_l
    for sfx, (o, x_, a_, h_, y_) in (("", (offsets, xp, a, dh, dyp)),
                                     ("2", (offsets2, xp2, a2, dh2, dyp2))):
        _chk_ffn(s, "moe_ffn_wgrad_pair", o, False, False, False,
                 **{"xp" + sfx: (x_, cap * d, _DATA), "a" + sfx: (a_, cap * F, _DATA),
                    "dh" + sfx: (h_, cap * 2 * F, _DATA), "dyp" + sfx: (y_, cap * d, _DATA)})
    _chk(s, "moe_ffn_wgrad_pair", "dW_gu", dW_gu, _F32, E_l * 2 * F * d)
    _chk(s, "moe_ffn_wgrad_pair", "dW_down", dW_down, _F32, E_l * d * F)
    check(lib().moe_ffn_wgrad_pair(C.byref(s), _p(xp), _p(a), _p(dh), _p(dyp), _p(offsets),
                                   _p(xp2), _p(a2), _p(dh2), _p(dyp2), _p(offsets2), _p(dW_gu),
                                   _p(dW_down), int(accumulate), _stream(stream)))


def moe_ffn_wgrad_multi(s, ops, dW_gu, dW_down, accumulate=0, stream=None):
    """ops: a list of (xp, a, dh, dyp, offsets), one per micro-batch, 1 to 4."""
    cap, d, F, E_l = s.T * s.K, s.d, s.F, s.E_l
    fn = "moe_ffn_wgrad_multi"
    arr = (MoeWgradOps * max(1, len(ops)))()
    for i, (x_, a_, h_, y_, o) in enumerate(ops):
        _chk_ffn(s, fn, o, False, False, False,
                 **{f"xp{i}": (x_, cap * d, _DATA), f"a{i}": (a_, cap * F, _DATA),
                    f"dh{i}": (h_, cap * 2 * F, _DATA), f"dyp{i}": (y_, cap * d, _DATA)})
        arr[i] = MoeWgradOps(_p(x_), _p(a_), _p(h_), _p(y_), _p(o))
    _chk(s, fn, "dW_gu", dW_gu, _F32, E_l * 2 * F * d)
    _chk(s, fn, "dW_down", dW_down, _F32, E_l * d * F)
    check(lib().moe_ffn_wgrad_multi(C.byref(s), len(ops), arr, _p(dW_gu), _p(dW_down),
                                    int(accumulate), _stream(stream)))


def moe_ffn_wgrad_gather(s, x, pair_of_row, a, dh, dyp, offsets, dW_gu, dW_down, accumulate=0,
                         stream=None):
    cap, d, F, E_l = s.T * s.K, s.d, s.F, s.E_l
    _chk_ffn(s, "moe_ffn_wgrad_gather", offsets, False, False, False,
             x=(x, s.T * d, _DATA), pair_of_row=(pair_of_row, cap, _I32), a=(a, cap * F, _DATA),
             dh=(dh, cap * 2 * F, _DATA), dyp=(dyp, cap * d, _DATA),
             dW_gu=(dW_gu, E_l * 2 * F * d, _F32), dW_down=(dW_down, E_l * d * F, _F32))
    check(lib().moe_ffn_wgrad_gather(C.byref(s), _p(x), _p(pair_of_row), _p(a), _p(dh), _p(dyp),
                                     _p(offsets), _p(dW_gu), _p(dW_down), int(accumulate),
                                     _stream(stream)))


def moe_ffn_dgrad_gather(s, dout, pair_of_row, gates, h, offsets, tile_offsets, W_gu, W_down, dh,
                         dxp, ag, ws, stream=None):
    cap, d, F = s.T * s.K, s.d, s.F
    _chk_ffn(s, "moe_ffn_dgrad_gather", offsets, tile_offsets, W_gu, W_down,
             dout=(dout, s.T * d, _DATA), pair_of_row=(pair_of_row, cap, _I32),
             gates=(gates, cap, _F32), h=(h, cap * 2 * F, _DATA), dh=(dh, cap * 2 * F, _DATA),
             dxp=(dxp, cap * d, _DATA), ag=(ag, cap * F, _DATA))
    _chk_ws("moe_ffn_dgrad_gather", ws)
    wp, wb = _ws(ws)
    check(lib().moe_ffn_dgrad_gather(C.byref(s), _p(dout), _p(pair_of_row), _p(gates), _p(h),
                                     _p(offsets), _p(tile_offsets), _p(W_gu), _p(W_down), _p(dh),
                                     _p(dxp), _p(ag), wp, wb, _stream(stream)))


def moe_ffn_wgrad_fused(s, xp, x, pair_of_row, ag, dh, dout, offsets, dW_gu, dW_down,
                        accumulate=0, stream=None):
    """xp None: the dW_gu operand is gathered from x through pair_of_row too."""
    cap, d, F, E_l = s.T * s.K, s.d, s.F, s.E_l
    fn = "moe_ffn_wgrad_fused"
    _chk(s, fn, "xp", xp, _DATA, cap * d, optional=True)
    _chk(s, fn, "x", x, _DATA, s.T * d, optional=xp is not None)
    _chk_ffn(s, fn, offsets, False, False, False, pair_of_row=(pair_of_row, cap, _I32),
             ag=(ag, cap * F, _DATA), dh=(dh, cap * 2 * F, _DATA), dout=(dout, s.T * d, _DATA),
             dW_gu=(dW_gu, E_l * 2 * F * d, _F32), dW_down=(dW_down, E_l * d * F, _F32))
    check(lib().moe_ffn_wgrad_fused(C.byref(s), _p(xp), _p(x), _p(pair_of_row), _p(ag), _p(dh),
                                    _p(dout), _p(offsets), _p(dW_gu), _p(dW_down),
                                    int(accumulate), _stream(stream)))


def moe_route_bwd(s, mode, dgates, gates, idx, x, dlogits, dW_r, accumulate, ws, stream=None):
    fn, T, d, E, K = "moe_route_bwd", s.T, s.d, s.E, s.K
    _chk(s, fn, "dgates", dgates, _F32, T * K)
    _chk(s, fn, "gates", gates, _F32, T * K)
    _chk(s, fn, "idx", idx, _I32, T * K)
    _chk(s, fn, "x", x, _DATA, T * d, optional=True)
    _chk(s, fn, "dlogits", dlogits, _F32, T * E)
    _chk(s, fn, "dW_r", dW_r, _F32, d * E, optional=True)
    _chk_ws(fn, ws)
    wp, wb = _ws(ws)
    check(lib().moe_route_bwd(C.byref(s), mode, _p(dgates), _p(gates), _p(idx), _p(x),
                              _p(dlogits), _p(dW_r), int(accumulate), wp, wb, _stream(stream)))


def moe_dispatch_bwd(s, dxp, row_of_pair, idx, dlogits, W_r, dx, accumulate, ws, stream=None):
    fn, T, d, E, K = "moe_dispatch_bwd", s.T, s.d, s.E, s.K
    _chk(s, fn, "dxp", dxp, _DATA, T * K * d)
    _chk(s, fn, "row_of_pair", row_of_pair, _I32, T * K)
    router = dlogits is not None
    _chk(s, fn, "idx", idx, _I32, T * K, optional=not router)
    _chk(s, fn, "dlogits", dlogits, _F32, T * E, optional=True)
    _chk(s, fn, "W_r", W_r, _DATA, d * E, optional=not router)
    _chk(s, fn, "dx", dx, _DATA, T * d)
    _chk_ws(fn, ws)
    wp, wb = _ws(ws)
    check(lib().moe_dispatch_bwd(C.byref(s), _p(dxp), _p(row_of_pair), _p(idx), _p(dlogits),
                                 _p(W_r), _p(dx), int(accumulate), wp, wb, _stream(stream)))


def moe_overlap_step(step: MoeStep, s_compute=None, s_copy=None, flags=0):
    check(lib().moe_overlap_step(C.byref(step), _stream(s_compute), _stream(s_copy), int(flags)))


def moe_overlap_steps(steps, s_compute=None, s_copy=None, flags=0):
    """Run the MoeStep list `steps` as consecutive pipelined 1F1B steps."""
    arr = (MoeStep * len(steps))(*steps)
    check(lib().moe_overlap_steps(arr, len(steps), _stream(s_compute), _stream(s_copy),
                                  int(flags)))


def moe_timing_enable(max_records=4096):
    check(lib().moe_timing_enable(int(max_records)))


def moe_timing_disable():
    check(lib().moe_timing_disable())


def moe_timing_reset():
    check(lib().moe_timing_reset())


def moe_timing_report() -> dict:
    """{kernel name: (total ms, launches)} of the recorded launches (waits for them)."""
    L = lib()
    n = L.moe_timing_report(-1, None, 0, None, None)
    if n < 0:
        check(n)
    res = {}
    buf = C.create_string_buffer(64)
    for i in range(n):
        ms, cnt = C.c_double(), C.c_int()
        rc = L.moe_timing_report(i, buf, 64, C.byref(ms), C.byref(cnt))
        if rc < 0:
            check(rc)
        res[buf.value.decode()] = (ms.value, cnt.value)
    return res


# ---------------------------------------------------------------------------
# buffer plumbing (torch allocations only)
# ---------------------------------------------------------------------------
class MicroBatch:
    """Device buffers of one micro-batch for shape ``s`` (sizes per include/moe.h).
    With ``fused=True`` (steps run with MOE_STEP_FUSED_PERMUTE) no xp is allocated;
    with ``fused_bwd=True`` (MOE_STEP_FUSED_COMBINE_BWD) ag is allocated and dyp
    is not; with ``F_s > 0`` the shared expert's buffers are allocated too."""

    def __init__(self, s: MoeShape, device="cuda", x=None, dout=None, gates=None, logits=None,
                 fused=False, F_s=0, fused_bwd=False):
        import numpy as np
        import torch

        dt = {MOE_BF16: torch.bfloat16, MOE_F16: torch.float16}.get(s.dtype, torch.float32)
        T, d, F, E, E_l, K = s.T, s.d, s.F, s.E, s.E_l, s.K
        cap = T * K
        for n, t, kind, c in (("x", x, _DATA, T * d), ("dout", dout, _DATA, T * d),
                              ("gates", gates, _F32, T * K), ("logits", logits, _F32, T * E)):
            _chk(s, "MicroBatch", n, t, kind, c, optional=True)
        f32, i32 = torch.float32, torch.int32
        # at least one element per buffer, so that no pointer is NULL when T = 0
        e = lambda *sh, dtype=dt: torch.empty(max(1, int(np.prod(sh))), dtype=dtype,
                                              device=device)[: int(np.prod(sh))].view(*sh)
        self.x = x if x is not None else e(T, d)
        self.logits = logits if logits is not None else e(T, E, dtype=f32)
        self.idx = e(T, K, dtype=i32)
        self.gates = gates if gates is not None else e(T, K, dtype=f32)
        self.counts = e(E_l, dtype=i32)
        self.offsets = e(E_l + 1, dtype=i32)
        self.row_of_pair = e(T, K, dtype=i32)
        self.pair_of_row = e(cap, dtype=i32)
        self.tile_offsets = e(E_l + 1, dtype=i32)
        self.xp = None if fused else e(cap, d)
        self.h = e(cap, 2 * F)
        self.a = e(cap, F)
        self.yp = e(cap, d)
        self.out = e(T, d)
        self.dout = dout if dout is not None else e(T, d)
        self.dyp = None if fused_bwd else e(cap, d)
        self.dgates = e(T, K, dtype=f32)
        self.dlogits = e(T, E, dtype=f32)
        self.dh = e(cap, 2 * F)
        self.dxp = e(cap, d)
        self.dx = e(T, d)
        Fs = int(F_s)
        self.h_s = e(T, 2 * Fs) if Fs else None
        self.a_s = e(T, Fs) if Fs else None
        self.y_s = e(T, d) if Fs else None
        self.dh_s = e(T, 2 * Fs) if Fs else None
        self.dx_s = e(T, d) if Fs else None
        self.ag = e(cap, F) if fused_bwd else None

    def struct(self) -> MoeMB:
        return MoeMB(*[_p(getattr(self, n)) for n in MB_FIELDS])


def make_step(s: MoeShape, route_mode, W_gu, W_down, dW_gu, dW_down, ws, fwd=None, bwd=None,
              W_r=None, bias=None, dW_r=None, accumulate=0, shared=None):
    """Build a MoeStep; the returned object keeps the micro-batch structs alive.
    ``shared`` = (W_gu_s, W_down_s, dW_gu_s, dW_down_s) adds a shared expert."""
    fn, d, F, E, E_l = "make_step", s.d, s.F, s.E, s.E_l
    for n, t, kind, c, opt in (("W_gu", W_gu, _DATA, E_l * 2 * F * d, False),
                               ("W_down", W_down, _DATA, E_l * d * F, False),
                               ("dW_gu", dW_gu, _F32, E_l * 2 * F * d, True),
                               ("dW_down", dW_down, _F32, E_l * d * F, True),
                               ("W_r", W_r, _DATA, d * E, True), ("bias", bias, _F32, E, True),
                               ("dW_r", dW_r, _F32, d * E, True)):
        _chk(s, fn, n, t, kind, c, optional=opt)
    _chk_ws(fn, ws)
    if shared is not None:
        W_gu_s, W_down_s, dW_gu_s, dW_down_s = shared
        Fs = int(W_down_s.shape[1])
        for n, t, kind, c in (("W_gu_s", W_gu_s, _DATA, 2 * Fs * d),
                              ("W_down_s", W_down_s, _DATA, d * Fs),
                              ("dW_gu_s", dW_gu_s, _F32, 2 * Fs * d),
                              ("dW_down_s", dW_down_s, _F32, d * Fs)):
            _chk(s, fn, n, t, kind, c)
    fs = fwd.struct() if fwd is not None else None
    bs = bwd.struct() if bwd is not None else None
    st = MoeStep(s, int(route_mode), int(accumulate), _p(W_r), _p(bias), _p(W_gu), _p(W_down),
                 _p(dW_r), _p(dW_gu), _p(dW_down),
                 C.pointer(fs) if fs is not None else None,
                 C.pointer(bs) if bs is not None else None,
                 ws.data_ptr(), ws.numel() * ws.element_size())
    if shared is not None:
        W_gu_s, W_down_s, dW_gu_s, dW_down_s = shared
        st.F_s = int(W_down_s.shape[1])
        st.W_gu_s, st.W_down_s = _p(W_gu_s), _p(W_down_s)
        st.dW_gu_s, st.dW_down_s = _p(dW_gu_s), _p(dW_down_s)
    st._keep = (fs, bs)
    return st
