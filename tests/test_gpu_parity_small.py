"""GPU parity at oracle-friendly sizes: every tile kind, ragged batches, paging, single-key attention.

Each case runs the megakernel through the C ABI and compares, element by element, with the oracle
on the same seeded inputs: logits within 1e-2 max relative error, identical greedy ids wherever the
oracle's top-2 gap exceeds 1e-2, and per-layer mid-states (residual after each sub-layer, attention /
delta output, SwiGLU product) within 2e-3 normwise.
"""
import pytest

import synth
from gpu_harness import Step, run_parity, say

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": (synth.CONFIGS["tiny"], 8),
    "tiny-gain": (synth.SMALL["tiny-gain"], 4),
    "tiny-qknorm-tied": (synth.SMALL["tiny-qknorm"], 4),
    # ragged batch of 3 with a shuffled page table; one sequence starts from an empty cache
    "tiny-ragged": (synth.SMALL["tiny-gain"].replace(name="tiny-ragged", batch=3, ctx=[0, 77, 19], shuffle_pages=True), 5),
    # delta-rule hybrid at toy size (dk = dv = 64), batch 2
    "tiny-hybrid": (synth.SMALL["tiny-hybrid"].replace(delta_dk=64, delta_dv=64), 8),
    # head_dim 128, MHA, batch 4 with contexts that straddle chunk and page boundaries
    "small-mha-b4": (synth.Config("small-mha-b4", n_layers=2, hidden=512, n_q_heads=4, n_kv_heads=4, head_dim=128,
                                  ffn=1024, vocab=2048, batch=4, ctx=[1, 16, 33, 300], steps=3, seed=11,
                                  gain_range=(0.5, 1.5)), 3),
    # head_dim 128, GQA group 4 (the 8B grouping), batch 2, contexts across several chunks
    "small-gqa4-d128": (synth.Config("small-gqa4-d128", n_layers=2, hidden=512, n_q_heads=8, n_kv_heads=2,
                                     head_dim=128, ffn=1024, vocab=2048, batch=2, ctx=[200, 61], steps=3, seed=12), 3),
    # batch 8 (matrix-core projections), MHA, ragged contexts incl. an empty cache, shuffled pages
    "small-b8": (synth.Config("small-b8", n_layers=2, hidden=512, n_q_heads=4, n_kv_heads=4, head_dim=128,
                              ffn=1024, vocab=2048, batch=8, ctx=[5, 40, 0, 17, 100, 3, 64, 31], steps=3, seed=14,
                              shuffle_pages=True, gain_range=(0.5, 1.5)), 3),
    # chunks of nine ring slots (one past a full round of the eight waves), the new token in a
    # partly filled last slot
    "small-split9": (synth.Config("small-split9", n_layers=2, hidden=512, n_q_heads=8, n_kv_heads=8, head_dim=128,
                                  ffn=1024, vocab=2048, batch=1, ctx=[4390], steps=3, seed=15), 3),
    # head_dim 64 with the largest group the kernel takes (8 query heads per KV head)
    "small-gqa8-d64": (synth.Config("small-gqa8-d64", n_layers=2, hidden=512, n_q_heads=16, n_kv_heads=2,
                                    head_dim=64, ffn=1024, vocab=2048, batch=1, ctx=[150], steps=3, seed=13), 3),
}


@pytest.mark.parametrize("case", list(CASES))
def test_parity_small(case):
    cfg, steps = CASES[case]
    rep = run_parity(cfg, steps)
    say(f"[{case}] {rep.steps} steps, worst logits rel {rep.worst_rel:.2e}, worst mid {rep.worst_mid:.2e}, "
        f"greedy {rep.greedy_agree}/{rep.greedy_checked}")
    assert not rep.failures, "\n".join(rep.failures[:20])
    assert rep.steps == steps


@pytest.mark.parametrize("case", ["tiny-ragged", "tiny-hybrid", "small-b8"])
def test_parity_small_counters(case, monkeypatch):
    """The same checks with every dependency taken through the stage counters (the diagnostic
    plan): the counter path stays correct while the tagged one is the default."""
    monkeypatch.setenv("MK_STAGE_COUNTERS", "1")
    cfg, steps = CASES[case]
    rep = run_parity(cfg, steps)
    say(f"[{case}, counters] {rep.steps} steps, worst logits rel {rep.worst_rel:.2e}, worst mid {rep.worst_mid:.2e}")
    assert not rep.failures, "\n".join(rep.failures[:20])
    assert rep.steps == steps


# Launch sequences whose attention plan changes from step to step (the cases the tag protocol must
# survive): contexts that cross chunk boundaries as they grow, a slot refilled with a shorter
# context (its chunk count drops, then recovers), and batches that shrink and grow back.
RAGGED = synth.Config("ragged-gqa4", n_layers=2, hidden=512, n_q_heads=16, n_kv_heads=4, head_dim=128, ffn=1024,
                      vocab=2048, batch=4, ctx=[250, 120, 1020, 17], steps=36, seed=16, shuffle_pages=True,
                      gain_range=(0.5, 1.5))
SCHEDULES = {
    # 36 steps of batch 4 (hybrid attention shape: 4 KV heads); sequence 1 restarts at context 20 at
    # step 12 and sequence 3 at context 5 at step 20
    "ragged-plan-changes": (RAGGED, [Step(4, {1: 20} if i == 12 else ({3: 5} if i == 20 else {})) for i in range(36)]),
    # batch 3 -> 2 -> 3: the third sequence sits out and comes back at the position it left
    "batch-3-2-3": (synth.SMALL["tiny-gain"].replace(name="batch-3-2-3", batch=3, ctx=[40, 9, 130]),
                    [Step(b) for b in (3, 3, 2, 2, 3, 3, 2, 3, 1, 3)]),
    # the same with batch 8 (matrix-core projections)
    "batch-8-5-8": (synth.Config("batch-8-5-8", n_layers=2, hidden=512, n_q_heads=4, n_kv_heads=4, head_dim=128,
                                 ffn=1024, vocab=2048, batch=8, ctx=[5, 40, 1, 17, 100, 3, 64, 31], steps=6, seed=17,
                                 shuffle_pages=True), [Step(b) for b in (8, 5, 8, 3, 8, 8)]),
    # delta-rule hybrid: a sequence outside the step keeps its recurrent and conv states untouched
    "hybrid-2-1-2": (synth.SMALL["tiny-hybrid"].replace(name="hybrid-2-1-2", delta_dk=64, delta_dv=64),
                     [Step(b) for b in (2, 1, 1, 2, 2, 1, 2, 2)]),
}


@pytest.mark.parametrize("case", list(SCHEDULES))
def test_parity_changing_batch_and_plan(case):
    cfg, sched = SCHEDULES[case]
    rep = run_parity(cfg, len(sched), schedule=sched)
    say(f"[{case}] {rep.steps} steps, worst logits rel {rep.worst_rel:.2e}, worst mid {rep.worst_mid:.2e}, "
        f"greedy {rep.greedy_agree}/{rep.greedy_checked}")
    assert not rep.failures, "\n".join(rep.failures[:20])
    assert rep.steps == len(sched)
