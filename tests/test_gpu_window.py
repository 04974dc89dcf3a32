"""Verify windows (mk_decode_window): several tokens of each sequence in one step, against the oracle.

Token t of sequence b's window is checked against the oracle's step t, the oracle fed the same
window tokens one step at a time (the window's semantics: a speculative draft verified in one
pass): logits within 1e-2 max relative error, the oracle's greedy id wherever its top-2 gap exceeds
1e-2.  A decode step after the window then checks the K/V rows the window appended.  Cases: batch
1 and 2, windows of 2 to 8 tokens (the rows run on the batch-2, batch-4 and batch-8 kernels),
head_dim 64 and 128, windows that cross a page and a chunk boundary, the delta-rule hybrid with
windows shorter and longer than its conv history (its recurrent and conv states checked against the
oracle's after the window), and a one-token window equal bit for bit to mk_decode_step.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_harness import GREEDY_GAP, LOGIT_REL_TOL, STATE_RUN_TOL, make_pair, say, top2_gap

pytestmark = pytest.mark.gpu

# (config with batch = the rows the context must hold, sequences, window)
CASES = {
    "tiny-b1-w4": (synth.CONFIGS["tiny"].replace(name="tiny-w", batch=4, ctx=[128] * 4), 1, 4),
    "tiny-gain-b2-w3": (synth.SMALL["tiny-gain"].replace(name="tiny-gain-w", batch=6, ctx=[14, 77, 30, 5, 9, 40]), 2, 3),
    "d128-b1-w8-page": (synth.Config("d128-w8", n_layers=2, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
                                     ffn=1024, vocab=2048, batch=8, ctx=[60] * 8, steps=3, seed=21,
                                     gain_range=(0.5, 1.5)), 1, 8),
    "d64-b2-w2": (synth.Config("d64-w2", n_layers=2, hidden=512, n_q_heads=16, n_kv_heads=2, head_dim=64,
                               ffn=1024, vocab=2048, batch=4, ctx=[150, 31, 7, 7], steps=3, seed=22), 2, 2),
    "d128-b1-w5-chunks": (synth.Config("d128-w5", n_layers=2, hidden=512, n_q_heads=4, n_kv_heads=4, head_dim=128,
                                       ffn=1024, vocab=2048, batch=8, ctx=[1700] * 8, steps=3, seed=23), 1, 5),
    # delta-rule hybrid (dk = dv = 64): windows shorter and longer than the conv history of 3
    "hybrid-b1-w2": (synth.SMALL["tiny-hybrid"].replace(name="hyb-w2", delta_dk=64, delta_dv=64, batch=2, ctx=[16, 16]), 1, 2),
    "hybrid-b2-w2": (synth.SMALL["tiny-hybrid"].replace(name="hyb-b2-w2", delta_dk=64, delta_dv=64, batch=4, ctx=[16, 40, 9, 9]), 2, 2),
    "hybrid-d128-b2-w4": (synth.SMALL["tiny-hybrid"].replace(name="hyb-d128-w4", delta_dk=128, delta_dv=128, batch=8,
                                                             ctx=[16, 40] + [9] * 6), 2, 4),
    "hybrid-d128-b1-w8": (synth.SMALL["tiny-hybrid"].replace(name="hyb-d128-w8", delta_dk=128, delta_dv=128, batch=8,
                                                             ctx=[33] * 8), 1, 8),
    # the 0.6B-shape workload at full size, a window of 8 drafted tokens
    "0.6b-w8": (synth.CONFIGS["0.6b"].replace(name="0.6b-w8", batch=8, ctx=[1024] * 8), 1, 8),
    # fp8 projections: the window's 8 rows on the batch-8 fp8 kernel
    "d128-fp8-b1-w8": (synth.Config("d128-fp8-w8", n_layers=2, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
                                    ffn=1024, vocab=2048, batch=8, ctx=[60] * 8, steps=3, seed=34,
                                    gain_range=(0.5, 1.5), weights="fp8"), 1, 8),
}


def draft_tokens(cfg, B, W):
    """The window's tokens: the first tokens of the workload, then seeded draft tokens."""
    first = [int(t) for t in synth.first_tokens(cfg)][:B]
    draws = synth.u32(B * W, cfg.seed, "window_drafts").reshape(B, W) % cfg.vocab
    toks = np.array(draws, dtype=np.int64)
    toks[:, 0] = first
    return toks


@pytest.mark.parametrize("case", list(CASES))
def test_window_parity(case):
    import torch

    import persistent_megakernel_decode_amd as mkd
    cfg, B, W = CASES[case]
    w, cache, orc, gpu, ctx0 = make_pair(cfg, W + 2)
    try:
        ctx = list(ctx0[:B])
        toks = draft_tokens(cfg, B, W)
        say(f"[{case}] window of {W} for {B} sequence(s) at positions {ctx}")
        rc, logits = gpu.window(toks.tolist(), ctx, [c + 1 for c in ctx])
        assert rc == 0, mkd.mk_last_error()
        torch.cuda.synchronize()
        assert gpu.sync() == 0, mkd.mk_last_error()
        L = logits.cpu().numpy()
        errs, worst, checked = [], 0.0, 0
        for t in range(W):
            o = orc.step([int(x) for x in toks[:, t]], [c + t for c in ctx], [c + 1 + t for c in ctx])
            for b in range(B):
                g = L[b, t]
                if not np.isfinite(g).all():
                    errs.append(f"token {t} seq {b}: non-finite logits")
                    continue
                rel = float(np.max(np.abs(g.astype(np.float64) - o[b])) / np.max(np.abs(o[b])))
                worst = max(worst, rel)
                if rel > LOGIT_REL_TOL:
                    errs.append(f"token {t} seq {b}: logits rel err {rel:.3e}")
                if top2_gap(o[b]) > GREEDY_GAP:
                    checked += 1
                    if int(np.argmax(g)) != oracle.argmax(o[b]):
                        errs.append(f"token {t} seq {b}: greedy id {int(np.argmax(g))} != {oracle.argmax(o[b])}")
        # one ordinary step after the window reads every K/V row the window appended
        nxt = [int(np.argmax(L[b, W - 1])) for b in range(B)]
        pos = [c + W for c in ctx]
        assert gpu.step(nxt, pos, [p + 1 for p in pos]) == 0, mkd.mk_last_error()
        torch.cuda.synchronize()
        assert gpu.sync() == 0, mkd.mk_last_error()
        g2 = gpu.logits[:B].cpu().numpy()
        o2 = orc.step(nxt, pos, [p + 1 for p in pos])
        for b in range(B):
            rel = float(np.max(np.abs(g2[b].astype(np.float64) - o2[b])) / np.max(np.abs(o2[b])))
            worst = max(worst, rel)
            if rel > LOGIT_REL_TOL:
                errs.append(f"step after the window, seq {b}: logits rel err {rel:.3e}")
        if gpu.delta_state is not None:  # the states after the window and the step after it
            for name, gv, ov in (("S", gpu.delta_state, orc.delta_state), ("conv state", gpu.conv_state, orc.conv_state)):
                g, o = gv.cpu().numpy()[:, :B], np.asarray(ov)[:, :B]
                e = float(np.linalg.norm(g.astype(np.float64) - o) / np.linalg.norm(o))
                if e > STATE_RUN_TOL:
                    errs.append(f"{name} normwise err {e:.3e} against the oracle run")
        say(f"[{case}] worst logits rel {worst:.2e}, greedy checked {checked}")
        assert not errs, "\n".join(errs[:20])
    finally:
        gpu.close()


def test_one_token_window_equals_a_decode_step():
    import torch

    import persistent_megakernel_decode_amd as mkd
    cfg = synth.CONFIGS["tiny"]
    w, cache, orc, gpu, ctx0 = make_pair(cfg, 2)
    max_ctx = int(cache["max_pages_per_seq"]) * cfg.page_size
    ref = mkd.DecodeContext(synth.shape_of(cfg, max_ctx), w, cache, "cuda:0")
    try:
        toks = [int(t) for t in synth.first_tokens(cfg)]
        rc, logits = gpu.window([toks], ctx0, [c + 1 for c in ctx0])
        assert rc == 0, mkd.mk_last_error()
        assert ref.step(toks, ctx0, [c + 1 for c in ctx0]) == 0
        torch.cuda.synchronize()
        assert gpu.sync() == 0 and ref.sync() == 0
        a = logits[0, 0].cpu().numpy()
        b = ref.logits[0].cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    finally:
        gpu.close()
        ref.close()


def test_window_rejects_bad_arguments():
    import persistent_megakernel_decode_amd as mkd
    cfg = synth.CONFIGS["tiny"].replace(name="tiny-w", batch=4, ctx=[128] * 4)
    w, cache, orc, gpu, ctx0 = make_pair(cfg, 2)
    try:
        a = (gpu.tokens.data_ptr(), gpu.positions.data_ptr(), gpu.ctx_lens.data_ptr())
        lg = gpu.logits.data_ptr()
        assert mkd.mk_decode_window(gpu.ctx, *a, 1, mkd.MK_MAX_WINDOW + 1, lg) == mkd.MK_ERR_INVALID_ARG
        assert mkd.mk_decode_window(gpu.ctx, *a, 1, 0, lg) == mkd.MK_ERR_INVALID_ARG
        assert mkd.mk_decode_window(gpu.ctx, *a, 2, 3, lg) == mkd.MK_ERR_INVALID_ARG  # 6 rows > max_batch 4
    finally:
        gpu.close()
