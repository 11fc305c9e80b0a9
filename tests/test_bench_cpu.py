"""bench.py's timing plan (host logic, no GPU): any --steps K is timed exactly,
as replays of a graph whose length is a multiple of the unit (2 steps; 6 with
the paired weight gradient over three buffer sets) plus fewer than a unit of
eager steps; the grouped weight gradient's algorithmic work per launch."""

import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402


def test_group_plan_covers_every_step_count():
    for G0 in (2, 10, 16):
        for K in range(1, 201):
            g, rem = bench.group_plan(K, G0)
            if g is None:
                assert rem == K and K < 3, (G0, K)
                continue
            assert g % 2 == 0 and 2 <= g <= 2 * G0, (G0, K, g)
            assert rem in (0, 1) and (K - rem) % g == 0 and K - rem >= g, (G0, K, g, rem)
            if K % G0 == 0:
                assert (g, rem) == (G0, 0), (G0, K, g, rem)


def test_group_plan_paired_unit():
    for G0 in (6, 12, 24):
        for K in range(1, 201):
            g, rem = bench.group_plan(K, G0, 6)
            if g is None:
                assert rem == K and K < 6, (G0, K)
                continue
            assert g % 6 == 0 and 6 <= g <= 2 * G0, (G0, K, g)
            assert 0 <= rem < 6 and (K - rem) % g == 0 and K - rem >= g, (G0, K, g, rem)
            if K % G0 == 0:
                assert (g, rem) == (G0, 0), (G0, K, g, rem)


def test_grouped_wgrad_work_per_launch():
    """The grouped launch reduces the rows of `group` micro-batches (that many
    times the flops and operand bytes of one wgrad) and reads and writes the
    float32 dW once."""
    from combine_expert_ffn_amd.inputs import WORKLOADS
    w = WORKLOADS["ep1_128exp_bf16"]
    N, T_loc = w.T * w.K, w.T
    for group in (2, 3, 4):
        for acc in (True, False):
            a = bench.algorithmic(w, N, T_loc, accumulate=acc, group=group)
            dW = 4.0 * w.E_l * 3 * w.F * w.d * (2 if acc else 1)
            one, many = a["wgrad"], a["wgrad_multi"]
            assert many["flop"] == group * one["flop"]
            assert abs(many["byte"] - (group * (one["byte"] - dW) + dW)) < 1.0
    assert "wgrad_multi" in bench.PER_LAUNCH and "wgrad_multi" in bench.GEMM_KERNELS
