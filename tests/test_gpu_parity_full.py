"""GPU parity at the full workload shapes, in the launch configuration the bench times.

The oracle computes every logit of a full decode step (OpenMP over rows), so each case compares
whole steps element by element: logits within 1e-2 max relative error, identical greedy ids where
the oracle's top-2 gap exceeds 1e-2, per-layer mid-states within 2e-3 normwise, and for the hybrid
the recurrent and conv states of every delta-rule layer (gpu_harness).  0.6B and the hybrid run
their whole 64 steps; 8B eight and 13B four, the oracle's share there being several seconds a step.
"""
import pytest

import synth
from gpu_harness import run_parity, say

pytestmark = pytest.mark.gpu

CASES = {
    # the whole 64-step runs of the two smaller workloads (every logit, mid-state and state each step)
    "0.6b": (synth.CONFIGS["0.6b"], 64),
    "hybrid": (synth.CONFIGS["hybrid"], 64),
    "8b": (synth.CONFIGS["8b"], 8),
    # batch 8, ragged contexts 512-4096, shuffled pages, matrix-core projections
    "13b": (synth.CONFIGS["13b"], 4),
}


@pytest.mark.parametrize("case", list(CASES))
def test_parity_full_size(case):
    cfg, steps = CASES[case]
    rep = run_parity(cfg, steps)
    say(f"[{case}] {rep.steps} steps, worst logits rel {rep.worst_rel:.2e}, worst mid {rep.worst_mid:.2e}, "
        f"greedy {rep.greedy_agree}/{rep.greedy_checked}")
    assert not rep.failures, rep.failures
    assert rep.steps == steps
