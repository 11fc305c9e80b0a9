"""moe_dispatch_noalloc (the dispatch that allocates nothing: its plan scratch
is a fixed device array of the library) against moe_dispatch with a caller
workspace, through the C ABI: the same counts, offsets, maps and permuted rows,
bit for bit, on two calls in a row, the second with a smaller input (the array
keeps the first call's contents)."""

import numpy as np
import pytest
import torch

import combine_expert_ffn_amd as M
from combine_expert_ffn_amd.inputs import Workload, make_inputs
from moe_harness import dev, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()


def _idx(T, K, E, seed):
    """K distinct experts per token, drawn at random (int32 [T, K])."""
    rng = np.random.default_rng(seed)
    return np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)


# the first call's plan scratch (E_l = 128, 64 plan blocks) is larger than
# the second's (8 experts, 1 block)
CASES = [Workload("noalloc_128exp", T=16384, d=256, F=64, E=128, e_lo=0, E_l=128, K=8,
                  dtype="bf16", route="topk"),
         Workload("noalloc_window", T=333, d=128, F=64, E=16, e_lo=4, E_l=8, K=4,
                  dtype="bf16", route="topk")]


def test_noalloc_dispatch_matches_workspace_dispatch():
    s0 = torch.cuda.current_stream()
    runs = []
    for n, w in enumerate(CASES):
        log(f"[no-alloc] call {n}: {w.name} T={w.T} d={w.d} E={w.E} window "
            f"[{w.e_lo},{w.e_lo + w.E_l}) K={w.K}")
        s = M.shape_of(w)
        x = dev(make_inputs(w, seed=n)["x"], "bf16")
        idx = dev(_idx(w.T, w.K, w.E, seed=10 + n), "i32")
        ref = M.MicroBatch(s)
        got = M.MicroBatch(s)
        for mb in (ref, got):  # rows a call must not touch keep this value
            mb.xp.fill_(5.0)
            for k in ("counts", "offsets", "row_of_pair", "pair_of_row", "tile_offsets"):
                getattr(mb, k).fill_(-7)
        ws = torch.empty(M.moe_workspace_bytes(s), dtype=torch.uint8, device="cuda")
        M.moe_dispatch(s, x, idx, ref.counts, ref.offsets, ref.row_of_pair, ref.pair_of_row,
                       ref.tile_offsets, ref.xp, ws, s0)
        M.moe_dispatch_noalloc(s, x, idx, got.counts, got.offsets, got.row_of_pair,
                               got.pair_of_row, got.tile_offsets, got.xp, s0)
        runs.append((w, ref, got, idx))
    torch.cuda.synchronize()
    for w, ref, got, idx in runs:
        for k in ("counts", "offsets", "row_of_pair", "pair_of_row", "tile_offsets", "xp"):
            assert torch.equal(getattr(got, k), getattr(ref, k)), (w.name, k)
        # and the plan is the stable counting sort: rows of an expert in (t, k) order
        N = int(ref.offsets[-1].item())
        assert N == int(((idx >= w.e_lo) & (idx < w.e_lo + w.E_l)).sum().item())
        log(f"[no-alloc] {w.name}: N={N}, identical to moe_dispatch")
