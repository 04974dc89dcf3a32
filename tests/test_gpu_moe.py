"""Mixture-of-experts MLPs against the oracle, through the C ABI.

Every step the oracle runs the experts the GPU's router chose (read back from the workspace), as
both sides consume the GPU's greedy token; wherever the oracle's own k-th router margin exceeds
1e-2 its choice must be the GPU's.  Gates as for the dense models: logits within 1e-2 relative, the
greedy id where the top-2 gap exceeds 1e-2, per-layer residuals, attention outputs and router
logits within 2e-3 normwise.  Cases: one sequence (the vector path), batches of 2 and 4 (the
matrix-core row-group path) with ragged contexts, sequences leaving and re-entering the batch (every
expert's SwiGLU rows are rewritten each step), multi-step launches, and the workload's full shape.
"""
import numpy as np
import pytest

import synth
from gpu_harness import Step, run_parity, say

pytestmark = pytest.mark.gpu

CASES = {
    "tiny-moe": (synth.SMALL["tiny-moe"], 8, None),
    # batch 2: 16 experts of width 512, top 4, GQA, gains
    "small-moe-b2": (synth.Config("small-moe-b2", n_layers=2, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=64,
                                  ffn=512, vocab=2048, batch=2, ctx=[40, 7], steps=4, seed=51, n_experts=16, top_k=4,
                                  gain_range=(0.5, 1.5)), 4, None),
    # batch 4, ragged contexts, shuffled pages; batch 4 -> 2 -> 4 (two sequences skip two steps)
    "tiny-moe-b4": (synth.SMALL["tiny-moe"].replace(name="tiny-moe-b4", batch=4, ctx=[128, 3, 60, 17],
                                                     shuffle_pages=True), 6,
                    [Step(4), Step(2), Step(2), Step(4), Step(3), Step(4)]),
    # the mixture-of-experts workload: 16 layers, hidden 2048, 8 of 64 experts of width 1024
    "moe": (synth.CONFIGS["moe"], 3, None),
}


@pytest.mark.parametrize("case", list(CASES))
def test_moe_parity(case):
    cfg, steps, schedule = CASES[case]
    rep = run_parity(cfg, steps, schedule=schedule)
    say(f"[{case}] {rep.steps} steps, worst logits rel {rep.worst_rel:.2e}, worst mid {rep.worst_mid:.2e}, "
        f"greedy {rep.greedy_agree}/{rep.greedy_checked}, routing {rep.route_agree}/{rep.route_checked}")
    assert not rep.failures, "\n".join(rep.failures[:20])
    assert rep.steps == steps and rep.route_checked > 0


def test_moe_multistep_matches_single_steps():
    """Eight greedy steps in one launch on the mixture-of-experts kernels: the same tokens and, bit for
    bit, the same logits as eight single-step launches."""
    import torch

    import persistent_megakernel_decode_amd as mkd
    cfg = synth.SMALL["tiny-moe"].replace(name="tiny-moe-ms")
    w = synth.make_weights(cfg)
    ctx0 = synth.context_lengths(cfg)
    cache = synth.make_cache(cfg, ctx0, 8)
    max_ctx = int(cache["max_pages_per_seq"]) * cfg.page_size
    a = mkd.DecodeContext(synth.shape_of(cfg, max_ctx), w, cache, "cuda:0")
    b = mkd.DecodeContext(synth.shape_of(cfg, max_ctx), w, cache, "cuda:0")
    try:
        toks = [int(t) for t in synth.first_tokens(cfg)]
        rc, logits, tout = a.steps(toks, ctx0, [c + 1 for c in ctx0], 8)
        assert rc == 0, mkd.mk_last_error()
        torch.cuda.synchronize()
        assert a.sync() == 0, mkd.mk_last_error()
        L, T = logits.cpu().numpy(), tout.cpu().numpy()
        for s in range(8):
            st = toks if s == 0 else [int(T[s - 1, 0])]
            pos = [c + s for c in ctx0]
            assert b.step(st, pos, [p + 1 for p in pos]) == 0, mkd.mk_last_error()
            torch.cuda.synchronize()
            assert b.sync() == 0
            R = b.logits[0].cpu().numpy()
            assert int(T[s, 0]) == int(np.argmax(L[s, 0]))
            assert np.array_equal(L[s, 0].view(np.uint32), R.view(np.uint32)), f"step {s}"
        say("[moe multi-step] 8 steps in one launch equal 8 single-step launches")
    finally:
        a.close()
        b.close()


def test_moe_refuses_verify_windows():
    import persistent_megakernel_decode_amd as mkd
    cfg = synth.SMALL["tiny-moe"].replace(name="tiny-moe-win", batch=4, ctx=[20, 20, 20, 20])
    w = synth.make_weights(cfg)
    ctx0 = synth.context_lengths(cfg)
    cache = synth.make_cache(cfg, ctx0, 4)
    max_ctx = int(cache["max_pages_per_seq"]) * cfg.page_size
    g = mkd.DecodeContext(synth.shape_of(cfg, max_ctx), w, cache, "cuda:0")
    try:
        rc, _ = g.window([[1, 2], [3, 4]], [20, 20], [21, 21])
        assert rc == mkd.MK_ERR_UNSUPPORTED, rc
    finally:
        g.close()


@pytest.mark.parametrize("case", ["small-moe-b2", "tiny-moe-b4"])
def test_moe_parity_counters(case, monkeypatch):
    """The same checks with every dependency taken through the stage counters (the diagnostic plan):
    the router, gate / up and down stages of the mixture-of-experts layers signal and wait by counter."""
    monkeypatch.setenv("MK_STAGE_COUNTERS", "1")
    cfg, steps, schedule = CASES[case]
    rep = run_parity(cfg, steps, schedule=schedule)
    say(f"[{case}, counters] {rep.steps} steps, worst logits rel {rep.worst_rel:.2e}, worst mid {rep.worst_mid:.2e}, "
        f"routing {rep.route_agree}/{rep.route_checked}")
    assert not rep.failures, "\n".join(rep.failures[:20])
    assert rep.steps == steps
