"""The C-ABI library loads, exports every symbol include/moe.h declares, and
rejects bad arguments on the host before any launch.  CPU only: no call here
reaches a kernel launch."""

import ctypes as C
import os
import re

import pytest

import combine_expert_ffn_amd as M
from combine_expert_ffn_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "moe.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("moe_route", "moe_dispatch", "moe_expert_ffn_fwd", "moe_combine", "moe_ffn_dgrad",
              "moe_ffn_wgrad", "moe_overlap_step", "moe_combine_bwd", "moe_dispatch_bwd",
              "moe_route_bwd", "moe_workspace_bytes", "moe_last_error", "moe_overlap_steps"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = C.CDLL(_lib.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), f"{n} declared in moe.h but not exported"
    assert set(_declared()) == set(_lib.SIGNATURES), "binding signatures out of sync with moe.h"


def test_struct_layouts_match_header():
    assert C.sizeof(_lib.MoeShape) == 7 * 8 + 2 * 4
    assert C.sizeof(_lib.MoeMB) == len(_lib.MB_FIELDS) * 8 == 27 * 8
    # shape + 2 ints + 7 pointers + 2 mb pointers + ws + ws_bytes + F_s + 4 shared pointers
    assert C.sizeof(_lib.MoeStep) == C.sizeof(_lib.MoeShape) + 8 + 7 * 8 + 2 * 8 + 8 + 8 + 8 + 4 * 8


def _shape(**kw):
    base = dict(T=64, d=128, F=128, E=8, e_lo=0, E_l=8, K=2, dtype="bf16")
    base.update(kw)
    return M.make_shape(**base)


FAKE = C.c_void_p(0x1000)  # never dereferenced: every call below fails validation


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), M.MOE_ERR_DTYPE),
    (dict(d=100), M.MOE_ERR_SHAPE),
    (dict(d=32), M.MOE_ERR_SHAPE),
    (dict(F=96), M.MOE_ERR_SHAPE),
    (dict(K=9), M.MOE_ERR_SHAPE),
    (dict(K=0), M.MOE_ERR_SHAPE),
    (dict(K=17, E=32, E_l=8), M.MOE_ERR_SHAPE),
    (dict(E=600, E_l=8), M.MOE_ERR_SHAPE),
    (dict(e_lo=4, E_l=8), M.MOE_ERR_SHAPE),
    (dict(E_l=0), M.MOE_ERR_SHAPE),
    (dict(T=-1), M.MOE_ERR_SHAPE),
    (dict(T=1 << 28, K=8), M.MOE_ERR_SHAPE),
])
def test_shape_validation(kw, code):
    s = _shape(**kw)
    rc = M.lib().moe_combine(C.byref(s), FAKE, FAKE, FAKE, FAKE, None)
    assert rc == code
    assert M.lib().moe_last_error()
    assert M.moe_workspace_bytes(s) == 0


def test_all_three_dtypes_accepted():
    for dt in ("f32", "bf16", "f16"):
        s = _shape(dtype=dt)
        assert M.moe_workspace_bytes(s) > 0, dt
        # validation passes the shape and stops at the first NULL pointer
        assert M.lib().moe_combine(C.byref(s), None, FAKE, FAKE, FAKE, None) == M.MOE_ERR_NULL
    # the 16-bit types both need the transposed-weight workspace of the dgrad
    # bf16's router weight gradient runs on the matrix cores and also holds the
    # split dlogits and per-chunk partials of [d, 2E]; fp16 needs no more than that
    assert M.moe_workspace_bytes(_shape(dtype="f16")) <= M.moe_workspace_bytes(_shape(dtype="bf16"))


def test_null_pointers_rejected():
    s = _shape()
    L = M.lib()
    assert L.moe_combine(C.byref(s), None, FAKE, FAKE, FAKE, None) == M.MOE_ERR_NULL
    assert b"yp" in L.moe_last_error()
    assert L.moe_combine(None, FAKE, FAKE, FAKE, FAKE, None) == M.MOE_ERR_NULL
    assert L.moe_expert_ffn_fwd(C.byref(s), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                None) == M.MOE_ERR_NULL
    assert L.moe_ffn_dgrad(C.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                           FAKE, 1 << 30, None) == M.MOE_ERR_NULL
    assert L.moe_ffn_dgrad(C.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                           FAKE, 16, None) == M.MOE_ERR_WORKSPACE
    assert L.moe_ffn_wgrad(C.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0,
                           None) == M.MOE_ERR_NULL
    # TOPK routing needs x, W_r, logits, gates
    assert L.moe_route(C.byref(s), M.MOE_ROUTE_TOPK, None, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                       1 << 20, None) == M.MOE_ERR_NULL
    # the router term of dispatch_bwd needs idx and W_r
    assert L.moe_dispatch_bwd(C.byref(s), FAKE, FAKE, None, FAKE, FAKE, FAKE, 0, FAKE, 1 << 20,
                              None) == M.MOE_ERR_NULL


def test_fused_permute_validation():
    L = M.lib()
    s = _shape()
    # NULL gather map / x
    assert L.moe_expert_ffn_fwd_gather(C.byref(s), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       FAKE, FAKE, None) == M.MOE_ERR_NULL
    assert L.moe_ffn_wgrad_gather(C.byref(s), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0,
                                  None) == M.MOE_ERR_NULL
    assert L.moe_ffn_wgrad_gather(C.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8,
                                  None) == M.MOE_ERR_ARG
    # x beyond the 32-bit offsets of the gathered loads
    big = _shape(T=1 << 17, d=16384, K=2)
    assert L.moe_expert_ffn_fwd_gather(C.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       FAKE, FAKE, None) == M.MOE_ERR_SHAPE
    assert b"2^31" in L.moe_last_error()
    # plan-only dispatch needs no x and no xp, but still its plan outputs
    assert L.moe_dispatch(C.byref(s), None, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE,
                          1 << 20, None) == M.MOE_ERR_NULL
    # a fused step needs x and pair_of_row in the backward micro-batch, not xp
    fields = {n: 0x1000 for n in _lib.MB_FIELDS}
    fields["xp"] = 0
    fields["pair_of_row"] = 0
    mb = _lib.MoeMB(*[fields[n] for n in _lib.MB_FIELDS])
    st = _lib.MoeStep(s, M.MOE_ROUTE_FORCE_BALANCE, 0, None, None, 0x1000, 0x1000, None, 0x1000,
                      0x1000, None, C.pointer(mb), 0x1000, 1 << 40)
    assert L.moe_overlap_step(C.byref(st), None, None, M.MOE_STEP_FUSED_PERMUTE) == M.MOE_ERR_NULL
    assert b"pair_of_row" in L.moe_last_error()
    assert L.moe_overlap_step(C.byref(st), None, None, 0) == M.MOE_ERR_NULL  # unfused needs xp
    assert b"xp" in L.moe_last_error()


def test_shared_expert_validation():
    L = M.lib()
    s = _shape()
    assert M.moe_shared_workspace_bytes(s, 96) == 0          # F_s not a multiple of 64
    assert M.moe_shared_workspace_bytes(s, 128) > 256
    assert M.moe_step_workspace_bytes_shared(s, 0) == M.moe_step_workspace_bytes(s)
    assert (M.moe_step_workspace_bytes_shared(s, 128)
            == M.moe_step_workspace_bytes(s) + 2 * M.moe_shared_workspace_bytes(s, 128))
    assert L.moe_shared_expert_fwd(C.byref(s), 100, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   1 << 30, None) == M.MOE_ERR_SHAPE
    assert L.moe_shared_expert_fwd(C.byref(s), 128, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   1 << 30, None) == M.MOE_ERR_NULL
    assert L.moe_shared_expert_dgrad(C.byref(s), 128, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     16, None) == M.MOE_ERR_WORKSPACE
    assert L.moe_shared_expert_wgrad(C.byref(s), 128, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8,
                                     FAKE, 1 << 30, None) == M.MOE_ERR_ARG
    # a step with a shared expert needs its weights, buffers and the larger workspace
    mb = _lib.MoeMB(*([0x1000] * len(_lib.MB_FIELDS)))
    st = _lib.MoeStep(s, M.MOE_ROUTE_FORCE_BALANCE, 0, None, None, 0x1000, 0x1000, None, 0x1000,
                      0x1000, C.pointer(mb), None, 0x1000, M.moe_step_workspace_bytes(s),
                      128, None, 0x1000, 0x1000, 0x1000)
    assert L.moe_overlap_step(C.byref(st), None, None, 0) == M.MOE_ERR_NULL
    assert b"W_gu_s" in L.moe_last_error()
    st.W_gu_s = 0x1000
    assert L.moe_overlap_step(C.byref(st), None, None, 0) == M.MOE_ERR_WORKSPACE
    st.F_s = 96
    assert L.moe_overlap_step(C.byref(st), None, None, 0) == M.MOE_ERR_SHAPE


def test_workspace_size_checked():
    s = _shape(T=4096, K=8)
    need = M.moe_workspace_bytes(s)
    assert need >= 256
    L = M.lib()
    rc = L.moe_dispatch(C.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None)
    assert rc == M.MOE_ERR_WORKSPACE
    rc = L.moe_route(C.byref(s), M.MOE_ROUTE_TOPK, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 16,
                     None)
    assert rc == M.MOE_ERR_WORKSPACE
    assert M.moe_step_workspace_bytes(s) == 2 * need


def test_modes_and_flags_rejected():
    s = _shape()
    L = M.lib()
    assert L.moe_route(C.byref(s), 9, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 20,
                       None) == M.MOE_ERR_ARG
    assert L.moe_route_bwd(C.byref(s), M.MOE_ROUTE_FORCE_BALANCE, FAKE, FAKE, FAKE, None, FAKE,
                           None, 0, None, 0, None) == M.MOE_ERR_UNSUPPORTED
    assert L.moe_ffn_wgrad(C.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8,
                           None) == M.MOE_ERR_ARG
    # the paired weight gradient: unknown accumulate bits, a missing operand
    assert L.moe_ffn_wgrad_pair(C.byref(s), *([FAKE] * 12), 8, None) == M.MOE_ERR_ARG
    assert L.moe_ffn_wgrad_pair(C.byref(s), *([FAKE] * 6), None, *([FAKE] * 5), 0,
                                None) == M.MOE_ERR_NULL
    st = _lib.MoeStep()
    st.shape = s
    st.route_mode = M.MOE_ROUTE_FORCE_BALANCE
    assert L.moe_overlap_step(C.byref(st), None, None, 512) == M.MOE_ERR_ARG
    assert L.moe_overlap_step(C.byref(st), None, None,
                              M.MOE_STEP_PAIR_WGRAD | M.MOE_STEP_GROUP4_WGRAD) == M.MOE_ERR_ARG
    # the grouped weight gradient: n out of [1, 4], a missing operand
    ops = (_lib.MoeWgradOps * 5)(*[_lib.MoeWgradOps(FAKE, FAKE, FAKE, FAKE, FAKE)] * 5)
    assert L.moe_ffn_wgrad_multi(C.byref(s), 0, ops, FAKE, FAKE, 0, None) == M.MOE_ERR_ARG
    assert L.moe_ffn_wgrad_multi(C.byref(s), 5, ops, FAKE, FAKE, 0, None) == M.MOE_ERR_ARG
    assert L.moe_ffn_wgrad_multi(C.byref(s), 3, ops, FAKE, FAKE, 8, None) == M.MOE_ERR_ARG
    ops[2].dh = None
    assert L.moe_ffn_wgrad_multi(C.byref(s), 3, ops, FAKE, FAKE, 0, None) == M.MOE_ERR_NULL
    assert L.moe_ffn_wgrad_multi(C.byref(s), 2, None, FAKE, FAKE, 0, None) == M.MOE_ERR_NULL
    # fused scatter: xp and x both missing, a missing map, missing y
    assert L.moe_expert_ffn_fwd_scatter(C.byref(s), None, None, *([FAKE] * 9),
                                        None) == M.MOE_ERR_NULL
    assert L.moe_expert_ffn_fwd_scatter(C.byref(s), FAKE, None, None, *([FAKE] * 8),
                                        None) == M.MOE_ERR_NULL
    assert L.moe_combine_pairs(C.byref(s), None, FAKE, FAKE, FAKE, None) == M.MOE_ERR_NULL
    assert L.moe_combine_bwd_pairs(C.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                   None) == M.MOE_ERR_NULL
    st.route_mode = 5
    assert L.moe_overlap_step(C.byref(st), None, None, 0) == M.MOE_ERR_ARG
    st.route_mode = M.MOE_ROUTE_FORCE_BALANCE
    assert L.moe_overlap_step(C.byref(st), None, None, 0) == M.MOE_ERR_NULL   # no weights
    assert L.moe_overlap_step(None, None, None, 0) == M.MOE_ERR_NULL


def test_step_rejects_small_workspace_and_same_microbatch():
    s = _shape()
    mb = _lib.MoeMB(*([0x1000] * len(_lib.MB_FIELDS)))
    st = _lib.MoeStep(s, M.MOE_ROUTE_FORCE_BALANCE, 0, None, None, 0x1000, 0x1000, None, 0x1000,
                      0x1000, C.pointer(mb), C.pointer(mb), 0x1000, 1 << 30)
    assert M.lib().moe_overlap_step(C.byref(st), None, None, 0) == M.MOE_ERR_ARG
    st.bwd = None
    st.ws_bytes = 8
    assert M.lib().moe_overlap_step(C.byref(st), None, None, 0) == M.MOE_ERR_WORKSPACE
    # eager and skipped wgrad exclude each other
    mb2 = _lib.MoeMB(*([0x2000] * len(_lib.MB_FIELDS)))
    st.bwd = C.pointer(mb2)
    st.ws_bytes = 1 << 40
    for flags in (M.MOE_STEP_EAGER_WGRAD | M.MOE_STEP_SKIP_WGRAD,
                  M.MOE_STEP_MID_WGRAD | M.MOE_STEP_SKIP_WGRAD,
                  M.MOE_STEP_MID_WGRAD | M.MOE_STEP_EAGER_WGRAD):
        assert M.lib().moe_overlap_step(C.byref(st), None, None, flags) == M.MOE_ERR_ARG
        assert b"exclude" in M.lib().moe_last_error()
    # an unknown flag bit is rejected
    assert M.lib().moe_overlap_step(C.byref(st), None, None, 64) == M.MOE_ERR_ARG


def test_multi_step_rejects_bad_chains():
    """moe_overlap_steps checks every step before it launches anything."""
    s = _shape()
    L = M.lib()
    m1 = _lib.MoeMB(*([0x1000] * len(_lib.MB_FIELDS)))
    m2 = _lib.MoeMB(*([0x2000] * len(_lib.MB_FIELDS)))
    m2_copy = _lib.MoeMB(*([0x2000] * len(_lib.MB_FIELDS)))   # same buffers, other struct
    m3 = _lib.MoeMB(*([0x3000] * len(_lib.MB_FIELDS)))

    def step(fwd, bwd, ws_bytes=1 << 40):
        return _lib.MoeStep(s, M.MOE_ROUTE_FORCE_BALANCE, 0, None, None, 0x1000, 0x1000, None,
                            0x1000, 0x1000, C.pointer(fwd) if fwd else None,
                            C.pointer(bwd) if bwd else None, 0x1000, ws_bytes)

    def run(steps, flags=0):
        arr = (_lib.MoeStep * len(steps))(*steps)
        return L.moe_overlap_steps(arr, len(steps), None, None, flags)

    assert L.moe_overlap_steps(None, 1, None, None, 0) == M.MOE_ERR_NULL
    arr = (_lib.MoeStep * 1)(step(m1, None))
    assert L.moe_overlap_steps(arr, 0, None, None, 0) == M.MOE_ERR_ARG
    # the backward of step 1 must be the micro-batch step 0 forwarded
    assert run([step(m1, None), step(m2, m3)]) == M.MOE_ERR_ARG
    assert b"must back-propagate" in L.moe_last_error()
    # forward and backward of one step on the same buffers (distinct structs)
    assert run([step(m2, None), step(m2_copy, m2)]) == M.MOE_ERR_ARG
    assert b"same" in L.moe_last_error()
    # the caller-deferred wgrad excludes the other wgrad placements
    assert run([step(m1, m2)], M.MOE_STEP_SKIP_WGRAD | M.MOE_STEP_MID_WGRAD) == M.MOE_ERR_ARG
    assert run([step(m1, m2)], M.MOE_STEP_MID_WGRAD | M.MOE_STEP_EAGER_WGRAD) == M.MOE_ERR_ARG
    # every step must use the same expert weights (their dgrad copies are made once)
    w2 = step(m2, m1)
    w2.W_gu = 0x5000
    assert run([step(m1, m2), w2]) == M.MOE_ERR_ARG
    assert b"expert weights" in L.moe_last_error()
    # a later step's small workspace is found before anything runs
    assert run([step(m1, m2), step(m2, m1, ws_bytes=8)]) == M.MOE_ERR_WORKSPACE
    # the streams' workspace halves are laid out once: every step shares the shape
    other = step(m2, m1)
    other.shape.T = s.T * 2
    assert run([step(m1, m2), other]) == M.MOE_ERR_ARG
    assert b"differs from step 0" in L.moe_last_error()
    other = step(m2, m1)
    other.ws = 0x2000
    assert run([step(m1, m2), other]) == M.MOE_ERR_ARG


def test_binding_rejects_bad_tensors_before_the_call():
    """The Python binding checks device, dtype, contiguity and size of every
    tensor against the shape before passing raw pointers (no GPU needed: a
    host tensor is rejected first)."""
    import torch

    s = _shape()
    t = torch.zeros(4)
    with pytest.raises(M.MoeError, match="not on the GPU"):
        M.moe_combine(s, t, t, t, t)
    with pytest.raises(M.MoeError, match="is None"):
        M.moe_combine(s, None, t, t, t)
    with pytest.raises(M.MoeError, match="not a torch tensor"):
        M.moe_combine(s, 123, t, t, t)


def test_noalloc_dispatch_rejects_shapes_beyond_its_scratch():
    """moe_dispatch_noalloc's plan scratch is a fixed 4 MiB array: a shape whose
    plan needs more is rejected on the host before anything runs (no GPU
    needed), with the limit in the message."""
    assert M.moe_dispatch_noalloc_max_scratch() == 4 << 20
    FAKE = C.c_void_p(0x1000)
    # 256 local experts x ceil(2^24 / 2048) plan blocks x 2 x 4 bytes = 16 MiB
    s = M.make_shape(1 << 21, 64, 64, 256, 0, 256, 8, "bf16")
    rc = M.lib().moe_dispatch_noalloc(C.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      None)
    assert rc == M.MOE_ERR_WORKSPACE
    assert b"4194304" in M.lib().moe_last_error()
    rc = M.lib().moe_dispatch_noalloc(C.byref(s), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      None)
    assert rc == M.MOE_ERR_NULL
