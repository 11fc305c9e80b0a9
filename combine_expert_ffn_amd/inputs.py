"""Seeded synthetic inputs for the MoE layer workloads.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic, so both the GPU path and the CPU oracle can be fed from it.
The workloads stand in for the pages' Qwen3-30B-A3B MoE training runs (skill
card page 1, "alltoall benchmark" and "HybridEP benchmark" sections), whose real
data is not used: shapes follow each workload's description, values are
synthetic.

Recipe: numpy PCG64 with the given seed; normals drawn in float64, cast to
float32, then (for bf16 / f16 workloads) rounded to bfloat16 by torch's RNE cast
or to IEEE binary16 by numpy's RNE cast.
Draw order: x, W_r, W_gu, W_down, dout, then gates (forced-balance workloads).
A second micro-batch draws its x and dout after all of the above.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    F: int
    E: int
    e_lo: int
    E_l: int
    K: int
    dtype: str                 # "f32", "bf16" or "f16"
    route: str                 # "topk" or "force_balance"
    weight_std: float = 0.02
    zipf_s: float = 0.0        # >0: per-expert router bias -s*ln(e+1)
    microbatches: int = 1
    note: str = ""
    F_s: int = 0               # >0: a shared expert of this FFN width

    def with_tokens(self, T: int) -> "Workload":
        return replace(self, T=T)


WORKLOADS = {
    # Tiny layer for the oracle: fp32, top-2 softmax-renormalised gates.
    "tiny_f32": Workload("tiny_f32", T=256, d=128, F=256, E=8, e_lo=0, E_l=8, K=2,
                         dtype="f32", route="topk"),
    # One EP16 rank's share: 4096 tokens x top-8, forced balance over the 8 local
    # experts (4096 rows each), gates Dirichlet(1).
    "ep16_rank_bf16": Workload("ep16_rank_bf16", T=4096, d=2048, F=768, E=8, e_lo=0,
                               E_l=8, K=8, dtype="bf16", route="force_balance"),
    # One EP8 rank's share of a 64-expert layer: local window [0, 8), top-6,
    # Zipf(1.1) per-expert router bias for skewed load.
    "ep8_rank_zipf_bf16": Workload("ep8_rank_zipf_bf16", T=8192, d=2048, F=1408, E=64,
                                   e_lo=0, E_l=8, K=6, dtype="bf16", route="topk",
                                   zipf_s=1.1),
    # Two micro-batches of the 8-expert top-8 layer for the two-stream step.
    "two_microbatch_bf16": Workload("two_microbatch_bf16", T=4096, d=2048, F=768, E=8,
                                    e_lo=0, E_l=8, K=8, dtype="bf16", route="topk",
                                    microbatches=2),
    # Whole 128-expert layer on one GPU (EP=1), top-8.
    "ep1_128exp_bf16": Workload("ep1_128exp_bf16", T=16384, d=2048, F=768, E=128, e_lo=0,
                                E_l=128, K=8, dtype="bf16", route="topk"),
    # the forced-balance EP16 rank shapes in IEEE fp16 (the pages' other
    # mixed-precision setting)
    "ep16_rank_f16": Workload("ep16_rank_f16", T=4096, d=2048, F=768, E=8, e_lo=0,
                              E_l=8, K=8, dtype="f16", route="force_balance"),
    # the ep16 step with a shared expert of width 2F beside the routed experts
    "ep16_rank_shared_bf16": Workload("ep16_rank_shared_bf16", T=4096, d=2048, F=768, E=8,
                                      e_lo=0, E_l=8, K=8, dtype="bf16",
                                      route="force_balance", F_s=1536),
}


def _normal(rng, shape, scale, chunk_rows=None):
    """float64 normals (scaled), cast to float32; drawn slab by slab along axis 0
    so that large weight tensors do not need a full float64 copy."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, np.float32)
    if len(shape) == 0 or shape[0] == 0:
        return out
    per = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    step = chunk_rows or max(1, (1 << 24) // max(per, 1))
    for i in range(0, shape[0], step):
        j = min(shape[0], i + step)
        out[i:j] = (rng.standard_normal((j - i,) + shape[1:]) * scale).astype(np.float32)
    return out


def _to_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage type (RNE for bf16 and f16) and return
    them as float32 arrays holding exactly representable values."""
    if dtype == "f32":
        return a
    if dtype == "f16":
        return a.astype(np.float16).astype(np.float32)
    import torch

    return torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()


def make_inputs(w: Workload, seed: int = 0, microbatches: int | None = None) -> dict:
    """All inputs of one workload as float32 numpy arrays (values representable
    in ``w.dtype``).  Keys: x, W_r (None for forced balance), bias (or None),
    W_gu [E_l,2F,d], W_down [E_l,d,F], dout, gates (forced balance only), and
    x_b, dout_b (, gates_b) for a second micro-batch, and W_gu_s [2F_s,d],
    W_down_s [d,F_s] for a shared expert (drawn last, so the other draws do not
    depend on it)."""
    microbatches = w.microbatches if microbatches is None else microbatches
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    out["x"] = _to_dtype(_normal(rng, (w.T, w.d), 1.0), w.dtype)
    if w.route == "topk":
        out["W_r"] = _to_dtype(_normal(rng, (w.d, w.E), w.weight_std), w.dtype)
    else:
        out["W_r"] = None
    if w.zipf_s > 0:
        out["bias"] = np.array([-w.zipf_s * math.log(e + 1.0) for e in range(w.E)],
                               dtype=np.float32)
    else:
        out["bias"] = None
    out["W_gu"] = _to_dtype(_normal(rng, (w.E_l, 2 * w.F, w.d), w.weight_std, 1), w.dtype)
    out["W_down"] = _to_dtype(_normal(rng, (w.E_l, w.d, w.F), w.weight_std, 1), w.dtype)
    out["dout"] = _to_dtype(_normal(rng, (w.T, w.d), 1.0), w.dtype)
    if w.route == "force_balance":
        # Dirichlet(1) over the K slots: K Exp(1) draws per token, normalised.
        e = rng.standard_exponential((w.T, w.K))
        out["gates"] = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    else:
        out["gates"] = None
    if microbatches > 1:
        out["x_b"] = _to_dtype(_normal(rng, (w.T, w.d), 1.0), w.dtype)
        out["dout_b"] = _to_dtype(_normal(rng, (w.T, w.d), 1.0), w.dtype)
        if w.route == "force_balance":
            e = rng.standard_exponential((w.T, w.K))
            out["gates_b"] = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    if w.F_s > 0:
        out["W_gu_s"] = _to_dtype(_normal(rng, (2 * w.F_s, w.d), w.weight_std, 1), w.dtype)
        out["W_down_s"] = _to_dtype(_normal(rng, (w.d, w.F_s), w.weight_std, 1), w.dtype)
    return out


def to_device(arrays: dict, dtype: str, device="cuda"):
    """torch tensors on ``device``: data tensors in the workload dtype, gates and
    bias in float32."""
    import torch

    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}.get(dtype, torch.float32)
    res = {}
    for k, v in arrays.items():
        if v is None:
            res[k] = None
        elif k in ("gates", "gates_b", "bias"):
            res[k] = torch.from_numpy(np.ascontiguousarray(v)).to(device)
        else:
            res[k] = torch.from_numpy(np.ascontiguousarray(v)).to(device=device, dtype=tdt)
    return res
