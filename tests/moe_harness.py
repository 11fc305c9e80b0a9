"""Shared helpers for the GPU parity tests: device transfer, the oracle reference
for a workload, tolerance checks.  Parity bar: bit-exact for indices, counts,
maps and the permuted copy; |gpu - ref| <= tau * max(1, |ref|) elementwise for
floating point, tau = 2e-2 (bf16 data, float32 accumulation), 4e-3 (fp16 data,
float32 accumulation) or 1e-5 (float32)."""

from __future__ import annotations

import sys

import numpy as np
import torch

import combine_expert_ffn_amd as M
import oracle as O

TAU = {"bf16": 2e-2, "f16": 4e-3, "f32": 1e-5}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a, dtype, device="cuda"):
    """numpy -> device tensor; dtype 'bf16' | 'f16' | 'f32' | 'i32' | 'f32x' (float32 always)."""
    a = np.ascontiguousarray(a)
    if dtype == "i32":
        return torch.from_numpy(a.astype(np.int32)).to(device)
    if dtype in ("f32", "f32x"):
        return torch.from_numpy(a.astype(np.float32)).to(device)
    if dtype == "f16":
        return torch.from_numpy(a.astype(np.float32)).to(device=device, dtype=torch.float16)
    return torch.from_numpy(a.astype(np.float32)).to(device=device, dtype=torch.bfloat16)


def host(t, rows=None):
    """device tensor -> numpy (float64 for floating point, as-is for integers).
    With ``rows`` only the first ``rows`` rows are copied: row buffers are sized
    to the cap T*K and rows [N, cap) hold whatever the allocation held."""
    if rows is not None:
        t = t[: int(rows)]
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    a = t.detach().cpu().numpy()
    return a.astype(np.float64) if a.dtype.kind == "f" else a


def close(name, gpu, ref, tau):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    if gpu.size == 0:
        return 0.0
    assert np.all(np.isfinite(gpu)), f"{name}: non-finite values"
    err = np.abs(gpu - ref) / np.maximum(1.0, np.abs(ref))
    worst = float(err.max())
    i = np.unravel_index(int(err.argmax()), err.shape)
    nbad = int((err > tau).sum())
    assert worst <= tau, (f"{name}: max scaled error {worst:.3e} > {tau} at {i}: gpu {gpu[i]} "
                          f"ref {ref[i]}; {nbad} of {err.size} elements over tolerance")
    return worst


def exact(name, gpu, ref):
    gpu = np.asarray(gpu)
    ref = np.asarray(ref)
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    bad = np.nonzero(gpu.reshape(-1) != ref.reshape(-1))[0]
    assert bad.size == 0, f"{name}: {bad.size} mismatches, first at {bad[:5]}: " \
                          f"gpu {gpu.reshape(-1)[bad[:5]]} ref {ref.reshape(-1)[bad[:5]]}"


def topk_gap(logits, K):
    """Per-token gap between the K-th and (K+1)-th largest logit, relative to
    max(1, |logit|).  Tokens with a tiny gap may legitimately select differently
    when logits are computed in another precision/order."""
    l = np.sort(np.asarray(logits, np.float64), axis=1)[:, ::-1]
    if K >= l.shape[1]:
        return np.full(l.shape[0], np.inf)
    return (l[:, K - 1] - l[:, K]) / np.maximum(1.0, np.abs(l[:, K - 1]))


def oracle_inputs(w, inp):
    """Inputs as float64 arrays holding exactly the values the GPU sees."""
    return {k: (None if v is None else np.asarray(v, np.float64)) for k, v in inp.items()}


def close_reduction(name, gpu, ref, mag, tau):
    """Bound for a reduction whose terms are themselves rounded results that the
    GPU and the oracle may round to neighbouring values: |gpu - ref| <=
    tau * max(1, sum of |terms|) (mag = that sum, computed by the oracle on the
    absolute values of the terms)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(gpu - ref) / np.maximum(1.0, np.asarray(mag, np.float64))
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tau, f"{name}: max error / max(1, sum|terms|) = {worst:.3e} > {tau}"
    return worst
