"""MX fp4 weight streaming (E2M1 codes, one E8M0 scale per 32 weights) against the oracle, through the
C ABI.

Same gates as the bf16 parity tests (gpu_harness): logits within 1e-2 max relative error, the
oracle's greedy id wherever its top-2 gap exceeds 1e-2, per-layer mid-states within 2e-3 normwise,
and for the delta-rule layers the recurrent and conv states.  fp4 runs one sequence per step; the
cases cover every shape of that projection path: pieces per row group 1, 2 and 4 (slots holding
several row groups), 8 with and without padding pieces, 16 (two input fragments of 32 per wave,
with padding), the RMSNorm gains, q/k norm with a tied bf16 LM head, the delta-rule projections,
multi-step launches, and the 0.6B and 8B shapes at full size.
"""
import numpy as np
import pytest

import synth
from gpu_harness import run_parity, say

pytestmark = pytest.mark.gpu

CASES = {
    # hidden 256 / ffn 768: one piece per row group (slots of eight groups)
    "tiny-fp4": (synth.CONFIGS["tiny"].replace(name="tiny-fp4", weights="fp4"), 8),
    "tiny-gain-fp4": (synth.SMALL["tiny-gain"].replace(name="tiny-gain-fp4", weights="fp4"), 4),
    "tiny-qknorm-fp4": (synth.SMALL["tiny-qknorm"].replace(name="tiny-qknorm-fp4", weights="fp4"), 4),
    # delta-rule layers (in_proj, gates and readout projections in fp4), one sequence
    "hybrid-fp4": (synth.SMALL["tiny-hybrid"].replace(name="hybrid-fp4", weights="fp4", delta_dk=64, delta_dv=64,
                                                      batch=1, ctx=[16]), 6),
    # QKV / gate-up over 2048 inputs (2 pieces), o_proj over 6144 (8 pieces, 2 of them padding),
    # down over 10240 (16 pieces, 6 of them padding: two fragments of 32 inputs per wave)
    "mid-fp4": (synth.Config("mid-fp4", n_layers=2, hidden=2048, n_q_heads=48, n_kv_heads=12, head_dim=128,
                             ffn=10240, vocab=4096, batch=1, ctx=[300], steps=3, seed=41, gain_range=(0.5, 1.5),
                             weights="fp4"), 3),
    # gate-up over 1024 inputs (1 piece), down over 8192 (8 pieces, no padding)
    "wide-fp4": (synth.Config("wide-fp4", n_layers=2, hidden=1024, n_q_heads=8, n_kv_heads=4, head_dim=128,
                              ffn=8192, vocab=2048, batch=1, ctx=[77], steps=3, seed=42, weights="fp4"), 3),
    # the 0.6B shape (q/k norm, tied bf16 LM head over 151936 rows; QKV / gate-up over 1024 inputs:
    # 1 piece, o_proj over 2048: 2, down over 3072: 3 padded to 4)
    "0.6b-fp4": (synth.CONFIGS["0.6b"].replace(name="0.6b-fp4", weights="fp4"), 3),
    # the 8B shape (QKV / o_proj / gate-up over 4096 inputs: 4 pieces; down over 14336: 16 pieces,
    # 2 of them padding), bf16 LM head over 128256 rows
    "8b-fp4": (synth.CONFIGS["8b"].replace(name="8b-fp4", weights="fp4"), 3),
}


@pytest.mark.parametrize("case", list(CASES))
def test_fp4_parity(case):
    cfg, steps = CASES[case]
    rep = run_parity(cfg, steps)
    say(f"[{case}] {rep.steps} steps, worst logits rel {rep.worst_rel:.2e}, worst mid {rep.worst_mid:.2e}, "
        f"greedy {rep.greedy_agree}/{rep.greedy_checked}")
    assert not rep.failures, "\n".join(rep.failures[:20])
    assert rep.steps == steps


def test_fp4_multistep_matches_single_steps():
    """Eight greedy steps in one launch on the fp4 kernels: the same tokens and, bit for bit, the same
    logits as eight single-step launches."""
    import torch

    import persistent_megakernel_decode_amd as mkd
    cfg = synth.SMALL["tiny-gain"].replace(name="tiny-gain-fp4-ms", weights="fp4")
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
        say("[fp4 multi-step] 8 steps in one launch equal 8 single-step launches")
    finally:
        a.close()
        b.close()


def test_fp4_create_rejects_a_missing_block_scale():
    import persistent_megakernel_decode_amd as mkd
    cfg = synth.CONFIGS["tiny"].replace(name="tiny-fp4-bad", weights="fp4")
    w = synth.make_weights(cfg)
    ctx0 = synth.context_lengths(cfg)
    cache = synth.make_cache(cfg, ctx0, 2)
    max_ctx = int(cache["max_pages_per_seq"]) * cfg.page_size
    g = mkd.DecodeContext(synth.shape_of(cfg, max_ctx), w, cache, "cuda:0")
    try:
        keep = g.layers[1].w_up_scale
        g.layers[1].w_up_scale = None
        with pytest.raises(mkd.MKError) as e:
            mkd.mk_create(g.desc, g.w, g.c, g.ws_ptr, g.ws_bytes)
        assert e.value.status == mkd.MK_ERR_INVALID_ARG and "w_up_scale" in str(e.value)
        g.layers[1].w_up_scale = keep
    finally:
        g.close()
