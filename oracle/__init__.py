"""CPU oracle for one GPU's share of a Mixture-of-Experts expert-parallel layer.

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
(``combine_expert_ffn_amd``) never imports, calls or links anything here, and
nothing here imports the product: the two share no code.

The oracle is written from the pages' statement of the layer: the expert-parallel
overlap skill card (page 1, "What it is": token dispatch and combine around the
expert FFN, optionally with the expert weight gradient computed later) and the
1F1B EP-overlap note (page 2, "MoE 1F1B overlap": the MLP backward split into
activation gradient D before weight gradient W; "how the 8 ops are split": the
backward chain combine -> mlp -> dispatch).  The pages do not spell out the
routing function, the FFN type or the permutation order; this oracle takes
top-k softmax routing (gates renormalised over the chosen experts), SwiGLU
experts and a stable counting-sort permutation (pairs in token-major order
within each expert) as the plainest readings.

Every function is numpy in float64.  Precision modes:

* ``"f64"``  – no rounding anywhere (used for finite-difference pins);
* ``"f32"``  – outputs rounded to float32 (the fp32 configuration);
* ``"bf16"`` – activation-sized outputs rounded to bfloat16 (round to nearest
  even) at the contract points; router logits, gates, gate gradients, logit
  gradients and weight gradients are float32;
* ``"f16"``  – the same with IEEE binary16 in place of bfloat16.

Pinned by ``tests/test_oracle_pins.py`` (brute force, closed forms, invariants,
finite differences, library routines) and the hand-worked fixture in
``tests/golden/``.  Parity unpinned: absolute values against the pages, which
print no worked example for this layer.
"""

from .moe_oracle import (  # noqa: F401
    round_bf16,
    round_f16,
    store,
    router_logits,
    topk_route,
    force_balance_idx,
    dispatch_plan,
    permute,
    expert_ffn_fwd,
    combine,
    combine_bwd,
    ffn_dgrad,
    route_bwd,
    dispatch_bwd,
    ffn_wgrad,
    layer_forward,
    layer_backward,
    shared_expert_fwd,
    shared_expert_dgrad,
    shared_expert_wgrad,
)
