"""fp8 weight streaming (E4M3 codes with fp32 row scales) against the oracle, through the C ABI.

Same gates as the bf16 parity tests (gpu_harness): logits within 1e-2 max relative error, the
oracle's greedy id wherever its top-2 gap exceeds 1e-2, per-layer mid-states within 2e-3 normwise,
and for the delta-rule layers the recurrent and conv states.  The cases cover every shape of the
batch-1 fp8 projection: pieces per row group 1, 2 and 4 (slots holding several row groups), 8 with
and without row groups staged in registers, 16 (two input fragments per wave, padded pieces) and
24 / 32 (four fragments), the RMSNorm gains, q/k norm with a tied bf16 LM head, the delta-rule
projections, and the 8B shape at full size; the row-group matrix-core path at batches 2 to 4
(dense and delta-rule, up to the hybrid workload's shape); and the batch-8 matrix-core path
(batches 6 and 8, ragged contexts, shuffled pages) up to the 13B shape.
"""
import numpy as np
import pytest

import synth
from gpu_harness import run_parity, say

pytestmark = pytest.mark.gpu

CASES = {
    # hidden 256 / ffn 768: 1 and 2 pieces per row group
    "tiny-fp8": (synth.CONFIGS["tiny"].replace(name="tiny-fp8", weights="fp8"), 8),
    "tiny-gain-fp8": (synth.SMALL["tiny-gain"].replace(name="tiny-gain-fp8", weights="fp8"), 4),
    "tiny-qknorm-fp8": (synth.SMALL["tiny-qknorm"].replace(name="tiny-qknorm-fp8", weights="fp8"), 4),
    # delta-rule layers (in_proj, gates and readout projections in fp8), one sequence
    "hybrid-fp8": (synth.SMALL["tiny-hybrid"].replace(name="hybrid-fp8", weights="fp8", delta_dk=64, delta_dv=64,
                                                      batch=1, ctx=[16]), 6),
    # QKV over 2048 inputs (4 pieces), o_proj over 6144 (16 pieces, 4 of them padding), down over
    # 10240 (24 pieces: three fragments of 16 inputs per wave)
    "mid-fp8": (synth.Config("mid-fp8", n_layers=2, hidden=2048, n_q_heads=48, n_kv_heads=12, head_dim=128,
                             ffn=10240, vocab=4096, batch=1, ctx=[300], steps=3, seed=31, gain_range=(0.5, 1.5),
                             weights="fp8"), 3),
    # the 8B shape (QKV / o_proj / gate-up over 4096 inputs: 8 pieces, gate-up staged; down over
    # 14336: 32 pieces), bf16 LM head over 128256 rows
    "8b-fp8": (synth.CONFIGS["8b"].replace(name="8b-fp8", weights="fp8"), 4),
    # batch 8 (the matrix-core k-outer path, 512 codes per segment), ragged contexts incl. an empty
    # cache, shuffled pages, gains
    "small-b8-fp8": (synth.Config("small-b8-fp8", n_layers=2, hidden=512, n_q_heads=4, n_kv_heads=4, head_dim=128,
                                  ffn=1536, vocab=2048, batch=8, ctx=[5, 40, 0, 17, 100, 3, 64, 31], steps=3, seed=32,
                                  shuffle_pages=True, gain_range=(0.5, 1.5), weights="fp8"), 3),
    # batch 6 on the batch-8 kernel, GQA
    "small-b6-fp8": (synth.Config("small-b6-fp8", n_layers=2, hidden=1024, n_q_heads=8, n_kv_heads=2, head_dim=128,
                                  ffn=2048, vocab=4096, batch=6, ctx=[7, 300, 33, 1, 90, 129], steps=3, seed=33,
                                  weights="fp8"), 3),
    # the 13B shape at batch 8 (ragged contexts 512-4096, shuffled pages)
    "13b-fp8": (synth.CONFIGS["13b"].replace(name="13b-fp8", weights="fp8"), 2),
    # batch 2 and 3 (the row-group matrix-core path: 8 and 4 input parts per tile)
    "tiny-b2-fp8": (synth.SMALL["tiny-gain"].replace(name="tiny-b2-fp8", batch=2, ctx=[128, 33], weights="fp8"), 4),
    "tiny-ragged-fp8": (synth.SMALL["tiny-gain"].replace(name="tiny-ragged-fp8", batch=3, ctx=[0, 77, 19],
                                                         shuffle_pages=True, weights="fp8"), 4),
    # delta-rule hybrid at batch 4, and the hybrid workload's shape at full size
    "hybrid-b4-fp8": (synth.SMALL["tiny-hybrid"].replace(name="hybrid-b4-fp8", weights="fp8", delta_dk=64, delta_dv=64,
                                                         batch=4, ctx=[16, 40, 9, 9]), 4),
    "hybrid-full-fp8": (synth.CONFIGS["hybrid"].replace(name="hybrid-full-fp8", weights="fp8"), 4),
}


@pytest.mark.parametrize("case", list(CASES))
def test_fp8_parity(case):
    cfg, steps = CASES[case]
    rep = run_parity(cfg, steps)
    say(f"[{case}] {rep.steps} steps, worst logits rel {rep.worst_rel:.2e}, worst mid {rep.worst_mid:.2e}, "
        f"greedy {rep.greedy_agree}/{rep.greedy_checked}")
    assert not rep.failures, "\n".join(rep.failures[:20])
    assert rep.steps == steps


def test_fp8_multistep_matches_single_steps():
    """Eight greedy steps in one launch on the fp8 kernels: the same tokens and, bit for bit, the same
    logits as eight single-step launches."""
    import torch

    import persistent_megakernel_decode_amd as mkd
    cfg = synth.SMALL["tiny-gain"].replace(name="tiny-gain-fp8-ms", weights="fp8")
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
        say("[fp8 multi-step] 8 steps in one launch equal 8 single-step launches")
    finally:
        a.close()
        b.close()


def test_fp8_create_rejects_a_missing_row_scale():
    import persistent_megakernel_decode_amd as mkd
    cfg = synth.CONFIGS["tiny"].replace(name="tiny-fp8-bad", weights="fp8")
    w = synth.make_weights(cfg)
    ctx0 = synth.context_lengths(cfg)
    cache = synth.make_cache(cfg, ctx0, 2)
    max_ctx = int(cache["max_pages_per_seq"]) * cfg.page_size
    g = mkd.DecodeContext(synth.shape_of(cfg, max_ctx), w, cache, "cuda:0")
    try:
        keep = g.layers[1].w_down_scale
        g.layers[1].w_down_scale = None
        with pytest.raises(mkd.MKError) as e:
            mkd.mk_create(g.desc, g.w, g.c, g.ws_ptr, g.ws_bytes)
        assert e.value.status == mkd.MK_ERR_INVALID_ARG and "w_down_scale" in str(e.value)
        g.layers[1].w_down_scale = keep + 4  # misaligned
        with pytest.raises(mkd.MKError) as e:
            mkd.mk_create(g.desc, g.w, g.c, g.ws_ptr, g.ws_bytes)
        assert e.value.status == mkd.MK_ERR_INVALID_ARG
    finally:
        g.close()
