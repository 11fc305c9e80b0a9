"""ctypes binding of libmoe (include/moe.h).  Argument marshalling only: every
step of the layer runs in the HIP library.  Loading fails loudly when the
library has not been built; there is no fallback."""

from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
MOE_ERR_NULL = -1
MOE_ERR_SHAPE = -2
MOE_ERR_DTYPE = -3
MOE_ERR_WORKSPACE = -4
MOE_ERR_HIP = -5
MOE_ERR_UNSUPPORTED = -6
MOE_ERR_ARG = -7

MOE_F32 = 0
MOE_BF16 = 1
MOE_F16 = 2

MOE_ROUTE_TOPK = 0
MOE_ROUTE_TOPK_FROM_LOGITS = 1
MOE_ROUTE_FORCE_BALANCE = 2

MOE_ACCUM_DX = 1
MOE_ACCUM_DW = 2

MOE_STEP_SERIALIZE = 1
MOE_STEP_EAGER_WGRAD = 2
MOE_STEP_SKIP_WGRAD = 4
MOE_STEP_FUSED_PERMUTE = 8
MOE_STEP_MID_WGRAD = 16
MOE_STEP_FUSED_COMBINE_BWD = 32
MOE_STEP_PAIR_WGRAD = 64
MOE_STEP_FUSED_SCATTER = 128
MOE_STEP_GROUP4_WGRAD = 256


class MoeShape(C.Structure):
    _fields_ = [("T", C.c_int64), ("d", C.c_int64), ("F", C.c_int64), ("E", C.c_int64),
                ("e_lo", C.c_int64), ("E_l", C.c_int64), ("K", C.c_int64),
                ("dtype", C.c_int32), ("reserved", C.c_int32)]


MB_FIELDS = ["x", "logits", "idx", "gates", "counts", "offsets", "row_of_pair",
             "pair_of_row", "tile_offsets", "xp", "h", "a", "yp", "out",
             "dout", "dyp", "dgates", "dlogits", "dh", "dxp", "dx",
             "h_s", "a_s", "y_s", "dh_s", "dx_s", "ag"]


class MoeMB(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in MB_FIELDS]


class MoeWgradOps(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("xp", "a", "dh", "dyp", "offsets")]


class MoeStep(C.Structure):
    _fields_ = [("shape", MoeShape), ("route_mode", C.c_int32), ("accumulate", C.c_int32),
                ("W_r", C.c_void_p), ("bias", C.c_void_p), ("W_gu", C.c_void_p),
                ("W_down", C.c_void_p), ("dW_r", C.c_void_p), ("dW_gu", C.c_void_p),
                ("dW_down", C.c_void_p), ("fwd", C.POINTER(MoeMB)), ("bwd", C.POINTER(MoeMB)),
                ("ws", C.c_void_p), ("ws_bytes", C.c_size_t),
                ("F_s", C.c_int64), ("W_gu_s", C.c_void_p), ("W_down_s", C.c_void_p),
                ("dW_gu_s", C.c_void_p), ("dW_down_s", C.c_void_p)]


_P = C.c_void_p
_SP = C.POINTER(MoeShape)
SIGNATURES = {
    "moe_workspace_bytes": (C.c_size_t, [_SP]),
    "moe_step_workspace_bytes": (C.c_size_t, [_SP]),
    "moe_step_workspace_bytes_shared": (C.c_size_t, [_SP, C.c_int64]),
    "moe_shared_workspace_bytes": (C.c_size_t, [_SP, C.c_int64]),
    "moe_shared_expert_fwd": (C.c_int, [_SP, C.c_int64, _P, _P, _P, _P, _P, _P, _P, C.c_size_t,
                                        _P]),
    "moe_shared_expert_dgrad": (C.c_int, [_SP, C.c_int64, _P, _P, _P, _P, _P, _P, _P,
                                          C.c_size_t, _P]),
    "moe_shared_expert_wgrad": (C.c_int, [_SP, C.c_int64, _P, _P, _P, _P, _P, _P, C.c_int, _P,
                                          C.c_size_t, _P]),
    "moe_tile_m": (C.c_int, []),
    "moe_last_error": (C.c_char_p, []),
    "moe_version": (C.c_int, []),
    "moe_route": (C.c_int, [_SP, C.c_int, _P, _P, _P, _P, _P, _P, _P, C.c_size_t, _P]),
    "moe_dispatch": (C.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, C.c_size_t, _P]),
    "moe_dispatch_noalloc": (C.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_dispatch_noalloc_max_scratch": (C.c_size_t, []),
    "moe_expert_ffn_fwd": (C.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_expert_ffn_fwd_gather": (C.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_combine": (C.c_int, [_SP, _P, _P, _P, _P, _P]),
    "moe_combine_bwd": (C.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P]),
    "moe_expert_ffn_fwd_scatter": (C.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_combine_pairs": (C.c_int, [_SP, _P, _P, _P, _P, _P]),
    "moe_combine_bwd_pairs": (C.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P]),
    "moe_ffn_dgrad": (C.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, C.c_size_t, _P]),
    "moe_ffn_wgrad": (C.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P, C.c_int, _P]),
    "moe_ffn_wgrad_pair": (C.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                     C.c_int, _P]),
    "moe_ffn_wgrad_gather": (C.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P, _P, C.c_int, _P]),
    "moe_ffn_wgrad_multi": (C.c_int, [_SP, C.c_int, C.POINTER(MoeWgradOps), _P, _P, C.c_int,
                                      _P]),
    "moe_ffn_dgrad_gather": (C.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                       C.c_size_t, _P]),
    "moe_ffn_wgrad_fused": (C.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, C.c_int, _P]),
    "moe_route_bwd": (C.c_int, [_SP, C.c_int, _P, _P, _P, _P, _P, _P, C.c_int, _P, C.c_size_t,
                                _P]),
    "moe_dispatch_bwd": (C.c_int, [_SP, _P, _P, _P, _P, _P, _P, C.c_int, _P, C.c_size_t, _P]),
    "moe_overlap_step": (C.c_int, [C.POINTER(MoeStep), _P, _P, C.c_int]),
    "moe_overlap_steps": (C.c_int, [C.POINTER(MoeStep), C.c_int, _P, _P, C.c_int]),
    "moe_timing_enable": (C.c_int, [C.c_int]),
    "moe_timing_disable": (C.c_int, []),
    "moe_timing_reset": (C.c_int, []),
    "moe_timing_report": (C.c_int, [C.c_int, C.c_char_p, C.c_size_t, C.POINTER(C.c_double),
                                    C.POINTER(C.c_int)]),
}

_lib = None


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libmoe error {code}: {msg}")
        self.code = code


def lib() -> C.CDLL:
    """The loaded libmoe.  Raises if the library is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built: run `python -c 'import __graft_entry__ as g; g.build()'` "
                "(hipcc, gfx950).  There is no CPU fallback.")
        l = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def check(rc: int) -> None:
    if rc != MOE_OK:
        raise MoeError(rc, lib().moe_last_error().decode())
