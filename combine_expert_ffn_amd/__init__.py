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
    LIB_PATH, MB_FIELDS, MoeError, MoeMB, MoeShape, MoeStep, check, lib,
    MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_WORKSPACE, MOE_ERR_HIP,
    MOE_ERR_UNSUPPORTED, MOE_ERR_ARG, MOE_F32, MOE_BF16, MOE_F16, MOE_ROUTE_TOPK,
    MOE_ROUTE_TOPK_FROM_LOGITS, MOE_ROUTE_FORCE_BALANCE, MOE_ACCUM_DX, MOE_ACCUM_DW,
    MOE_STEP_SERIALIZE, MOE_STEP_EAGER_WGRAD, MOE_STEP_SKIP_WGRAD, MOE_STEP_FUSED_PERMUTE,
    MOE_STEP_MID_WGRAD,
)


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
    wp, wb = _ws(ws)
    check(lib().moe_shared_expert_fwd(C.byref(s), int(F_s), _p(x), _p(W_gu_s), _p(W_down_s),
                                      _p(h_s), _p(a_s), _p(y_s), wp, wb, _stream(stream)))


def moe_shared_expert_dgrad(s, F_s, dout, h_s, W_gu_s, W_down_s, dh_s, dx_s, ws, stream=None):
    wp, wb = _ws(ws)
    check(lib().moe_shared_expert_dgrad(C.byref(s), int(F_s), _p(dout), _p(h_s), _p(W_gu_s),
                                        _p(W_down_s), _p(dh_s), _p(dx_s), wp, wb,
                                        _stream(stream)))


def moe_shared_expert_wgrad(s, F_s, x, a_s, dh_s, dout, dW_gu_s, dW_down_s, accumulate, ws,
                            stream=None):
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
    wp, wb = _ws(ws)
    check(lib().moe_route(C.byref(s), mode, _p(x), _p(W_r), _p(bias), _p(logits), _p(idx),
                          _p(gates), wp, wb, _stream(stream)))


def moe_dispatch(s, x, idx, counts, offsets, row_of_pair, pair_of_row, tile_offsets, xp, ws,
                 stream=None):
    wp, wb = _ws(ws)
    check(lib().moe_dispatch(C.byref(s), _p(x), _p(idx), _p(counts), _p(offsets),
                             _p(row_of_pair), _p(pair_of_row), _p(tile_offsets), _p(xp), wp, wb,
                             _stream(stream)))


def moe_expert_ffn_fwd(s, xp, offsets, tile_offsets, W_gu, W_down, h, a, yp, stream=None):
    check(lib().moe_expert_ffn_fwd(C.byref(s), _p(xp), _p(offsets), _p(tile_offsets), _p(W_gu),
                                   _p(W_down), _p(h), _p(a), _p(yp), _stream(stream)))


def moe_expert_ffn_fwd_gather(s, x, pair_of_row, offsets, tile_offsets, W_gu, W_down, h, a, yp,
                              stream=None):
    check(lib().moe_expert_ffn_fwd_gather(C.byref(s), _p(x), _p(pair_of_row), _p(offsets),
                                          _p(tile_offsets), _p(W_gu), _p(W_down), _p(h), _p(a),
                                          _p(yp), _stream(stream)))


def moe_combine(s, yp, gates, row_of_pair, out, stream=None):
    check(lib().moe_combine(C.byref(s), _p(yp), _p(gates), _p(row_of_pair), _p(out),
                            _stream(stream)))


def moe_combine_bwd(s, dout, yp, gates, row_of_pair, dyp, dgates, stream=None):
    check(lib().moe_combine_bwd(C.byref(s), _p(dout), _p(yp), _p(gates), _p(row_of_pair),
                                _p(dyp), _p(dgates), _stream(stream)))


def moe_ffn_dgrad(s, dyp, h, offsets, tile_offsets, W_gu, W_down, dh, dxp, ws, stream=None):
    wp, wb = _ws(ws)
    check(lib().moe_ffn_dgrad(C.byref(s), _p(dyp), _p(h), _p(offsets), _p(tile_offsets),
                              _p(W_gu), _p(W_down), _p(dh), _p(dxp), wp, wb, _stream(stream)))


def moe_ffn_wgrad(s, xp, a, dh, dyp, offsets, dW_gu, dW_down, accumulate=0, stream=None):
    check(lib().moe_ffn_wgrad(C.byref(s), _p(xp), _p(a), _p(dh), _p(dyp), _p(offsets),
                              _p(dW_gu), _p(dW_down), int(accumulate), _stream(stream)))


def moe_ffn_wgrad_gather(s, x, pair_of_row, a, dh, dyp, offsets, dW_gu, dW_down, accumulate=0,
                         stream=None):
    check(lib().moe_ffn_wgrad_gather(C.byref(s), _p(x), _p(pair_of_row), _p(a), _p(dh), _p(dyp),
                                     _p(offsets), _p(dW_gu), _p(dW_down), int(accumulate),
                                     _stream(stream)))


def moe_route_bwd(s, mode, dgates, gates, idx, x, dlogits, dW_r, accumulate, ws, stream=None):
    wp, wb = _ws(ws)
    check(lib().moe_route_bwd(C.byref(s), mode, _p(dgates), _p(gates), _p(idx), _p(x),
                              _p(dlogits), _p(dW_r), int(accumulate), wp, wb, _stream(stream)))


def moe_dispatch_bwd(s, dxp, row_of_pair, idx, dlogits, W_r, dx, accumulate, ws, stream=None):
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
    with ``F_s > 0`` the shared expert's buffers are allocated too."""

    def __init__(self, s: MoeShape, device="cuda", x=None, dout=None, gates=None, logits=None,
                 fused=False, F_s=0):
        import numpy as np
        import torch

        dt = {MOE_BF16: torch.bfloat16, MOE_F16: torch.float16}.get(s.dtype, torch.float32)
        T, d, F, E, E_l, K = s.T, s.d, s.F, s.E, s.E_l, s.K
        cap = T * K
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
        self.dyp = e(cap, d)
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

    def struct(self) -> MoeMB:
        return MoeMB(*[_p(getattr(self, n)) for n in MB_FIELDS])


def make_step(s: MoeShape, route_mode, W_gu, W_down, dW_gu, dW_down, ws, fwd=None, bwd=None,
              W_r=None, bias=None, dW_r=None, accumulate=0, shared=None):
    """Build a MoeStep; the returned object keeps the micro-batch structs alive.
    ``shared`` = (W_gu_s, W_down_s, dW_gu_s, dW_down_s) adds a shared expert."""
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
