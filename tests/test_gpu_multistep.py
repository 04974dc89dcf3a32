"""Several greedy decode steps in one launch (mk_decode_steps), against the oracle.

The launch feeds each step's argmax back on the device.  Per step and sequence:
  * the token the device chose is the first index of the largest logit it wrote (bit-exact);
  * logits against the oracle stepped on the device's tokens: max relative error <= 1e-2, and the
    oracle's greedy id wherever its top-2 gap exceeds 1e-2;
  * logits equal, bit for bit, those of a second context stepped one launch per step on the same
    tokens (the step-by-step path is the one the single-step parity tests gate);
and at the end of the run the delta-rule states against the oracle's trajectory (normwise <= 1e-4)
and, bit for bit, against the step-by-step context.  Cases cover batch widths 1 / 2 / 4 / 8, GQA and
MHA, head_dim 64 and 128, contexts that cross page and chunk boundaries within a launch (rows appended
by earlier steps of the launch on other compute units), several launches in a row, and the
0.6B-shape workload at full size.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_harness import GREEDY_GAP, LOGIT_REL_TOL, STATE_RUN_TOL, make_pair, normwise, say, top2_gap

pytestmark = pytest.mark.gpu

CASES = {
    # the tiny decoder: 8 greedy steps per launch, two launches
    "tiny": (synth.CONFIGS["tiny"], 8, 2),
    # delta-rule hybrid at toy size (dk = dv = 64), batch 2 (kernel width 2)
    "tiny-hybrid": (synth.SMALL["tiny-hybrid"].replace(delta_dk=64, delta_dv=64), 6, 2),
    # batch 3 on the width-4 kernel, ragged contexts that cross page boundaries inside the launch
    "tiny-ragged": (synth.SMALL["tiny-gain"].replace(name="tiny-ragged", batch=3, ctx=[14, 77, 30],
                                                     shuffle_pages=True), 5, 1),
    # head_dim 128 MHA, batch 4, contexts across chunk boundaries
    "small-mha-b4": (synth.Config("small-mha-b4", n_layers=2, hidden=512, n_q_heads=4, n_kv_heads=4, head_dim=128,
                                  ffn=1024, vocab=2048, batch=4, ctx=[1, 16, 33, 300], steps=3, seed=11,
                                  gain_range=(0.5, 1.5)), 6, 1),
    # batch 8 (matrix-core projections), shuffled pages
    "small-b8": (synth.Config("small-b8", n_layers=2, hidden=512, n_q_heads=4, n_kv_heads=4, head_dim=128,
                              ffn=1024, vocab=2048, batch=8, ctx=[5, 40, 1, 17, 100, 3, 64, 31], steps=3, seed=14,
                              shuffle_pages=True, gain_range=(0.5, 1.5)), 4, 1),
    # one long context split over many chunks: the rows the launch appends land in its last chunk
    "small-split9": (synth.Config("small-split9", n_layers=2, hidden=512, n_q_heads=8, n_kv_heads=8, head_dim=128,
                                  ffn=1024, vocab=2048, batch=1, ctx=[4390], steps=3, seed=15), 5, 1),
    # the 0.6B-shape workload at full size (28 layers, tied LM head over 151936 rows): 8 steps per launch
    "0.6b": (synth.CONFIGS["0.6b"], 8, 1),
    # fp8 projections at batch 3 on the width-4 kernel, ragged contexts across page boundaries
    "tiny-ragged-fp8": (synth.SMALL["tiny-gain"].replace(name="tiny-ragged-fp8", batch=3, ctx=[14, 77, 30],
                                                         shuffle_pages=True, weights="fp8"), 5, 1),
    # fp8 projections at batch 8 (the batch-8 fp8 multi-step kernel)
    "small-b8-fp8": (synth.Config("small-b8-fp8", n_layers=2, hidden=512, n_q_heads=4, n_kv_heads=4, head_dim=128,
                                  ffn=1024, vocab=2048, batch=8, ctx=[5, 40, 1, 17, 100, 3, 64, 31], steps=3, seed=35,
                                  shuffle_pages=True, gain_range=(0.5, 1.5), weights="fp8"), 4, 1),
}


def first_argmax(v: np.ndarray) -> int:
    return int(np.argmax(v))  # numpy returns the first index of the maximum


@pytest.mark.parametrize("case", list(CASES))
def test_multistep_parity(case):
    import torch

    import persistent_megakernel_decode_amd as mkd
    cfg, K, launches = CASES[case]
    total = K * launches
    w, cache, orc, gpu, ctx0 = make_pair(cfg, total)
    max_ctx = int(cache["max_pages_per_seq"]) * cfg.page_size
    ref = mkd.DecodeContext(synth.shape_of(cfg, max_ctx), w, cache, "cuda:0")  # stepped one launch per step
    B = cfg.batch
    toks = [int(t) for t in synth.first_tokens(cfg)]
    ctx = list(ctx0)
    worst = 0.0
    checked = agree = 0
    errs = []
    try:
        for li in range(launches):
            pos = list(ctx)
            lens = [c + 1 for c in ctx]
            say(f"[{case}] launch {li}: {K} steps, tokens {toks} positions {pos}")
            rc, logits, tout = gpu.steps(toks, pos, lens, K)
            assert rc == 0, mkd.mk_last_error()
            torch.cuda.synchronize()
            assert gpu.sync() == 0, mkd.mk_last_error()
            L = logits.cpu().numpy()
            T = tout.cpu().numpy()
            for s in range(K):
                st_toks = toks if s == 0 else [int(t) for t in T[s - 1]]
                st_pos = [p + s for p in pos]
                st_lens = [c + s for c in lens]
                assert ref.step(st_toks, st_pos, st_lens) == 0, mkd.mk_last_error()
                torch.cuda.synchronize()
                assert ref.sync() == 0, mkd.mk_last_error()
                R = ref.logits[:B].cpu().numpy()
                o = orc.step(st_toks, st_pos, st_lens)
                for b in range(B):
                    g = L[s, b]
                    where = f"launch {li} step {s} row {b}"
                    if not np.isfinite(g).all():
                        errs.append(f"{where}: non-finite logits")
                        continue
                    if T[s, b] != first_argmax(g):
                        t = int(T[s, b])
                        errs.append(f"{where}: device token {t} (logit {g[t] if 0 <= t < g.size else 'n/a'}) != argmax "
                                    f"{first_argmax(g)} (logit {g.max()}); step-by-step argmax {first_argmax(R[b])}")
                    if not np.array_equal(g.view(np.uint32), R[b].view(np.uint32)):
                        errs.append(f"{where}: logits differ from the step-by-step launch in {int(np.sum(g != R[b]))} "
                                    f"values (max abs diff {float(np.max(np.abs(g - R[b]))):.3e})")
                    rel = float(np.max(np.abs(g.astype(np.float64) - o[b])) / np.max(np.abs(o[b])))
                    worst = max(worst, rel)
                    if rel > LOGIT_REL_TOL:
                        errs.append(f"{where}: logits rel err {rel:.3e}")
                    if top2_gap(o[b]) > GREEDY_GAP:
                        checked += 1
                        if int(T[s, b]) == oracle.argmax(o[b]):
                            agree += 1
                        else:
                            errs.append(f"{where}: greedy id {int(T[s, b])} differs from the oracle's {oracle.argmax(o[b])}")
            if errs:
                break
            toks = [int(t) for t in T[K - 1]]
            ctx = [c + K for c in ctx]
        assert not errs, "\n".join(errs[:20])
        if gpu.delta_state is not None:
            for name, gv, rv, ov in (("S", gpu.delta_state, ref.delta_state, orc.delta_state),
                                     ("conv state", gpu.conv_state, ref.conv_state, orc.conv_state)):
                g = gv.cpu().numpy()
                assert np.array_equal(g.view(np.uint32), rv.cpu().numpy().view(np.uint32)), \
                    f"{name} differs from the step-by-step launch"
                e = normwise(g, ov)
                assert e <= STATE_RUN_TOL, f"{name} normwise err {e:.3e} against the oracle run"
        say(f"[{case}] {launches} x {K} steps: worst logits rel {worst:.2e}, greedy {agree}/{checked}")
    finally:
        gpu.close()
        ref.close()


def test_multistep_row_leaving_the_contract():
    """A row whose position runs past its mapped pages during the launch: its logits are finite
    until then and NaN from that step on (token -1), the other row is unaffected, and the launch
    reports the sticky device-input error."""
    import torch

    import persistent_megakernel_decode_amd as mkd
    cfg = synth.SMALL["tiny-gain"].replace(name="leaves-contract", batch=2, ctx=[30, 10])
    w = synth.make_weights(cfg)
    cache = synth.make_cache(cfg, [30, 10], 2)  # row 0: pages for positions < 32
    max_ctx = int(cache["max_pages_per_seq"]) * cfg.page_size
    gpu = mkd.DecodeContext(synth.shape_of(cfg, max_ctx), w, cache, "cuda:0")
    try:
        toks = [int(t) for t in synth.first_tokens(cfg)]
        say("[leaves-contract] 4 steps, row 0 from position 30 (pages end at 32)")
        rc, logits, tout = gpu.steps(toks, [30, 10], [31, 11], 4)
        assert rc == 0, mkd.mk_last_error()
        torch.cuda.synchronize()
        assert gpu.sync() == mkd.MK_ERR_DEVICE_INPUT
        L = logits.cpu().numpy()
        T = tout.cpu().numpy()
        for s in range(4):
            assert np.isfinite(L[s, 1]).all() and T[s, 1] == first_argmax(L[s, 1])
            if s < 2:
                assert np.isfinite(L[s, 0]).all() and T[s, 0] == first_argmax(L[s, 0])
            else:
                assert np.isnan(L[s, 0]).all() and T[s, 0] == -1
        assert gpu.reset() == 0
    finally:
        gpu.close()


def test_multistep_rejects_bad_arguments():
    import torch

    import persistent_megakernel_decode_amd as mkd
    cfg = synth.CONFIGS["tiny"]
    w = synth.make_weights(cfg)
    cache = synth.make_cache(cfg, synth.context_lengths(cfg), 4)
    max_ctx = int(cache["max_pages_per_seq"]) * cfg.page_size
    gpu = mkd.DecodeContext(synth.shape_of(cfg, max_ctx), w, cache, "cuda:0")
    try:
        lg = torch.empty((2, 1, cfg.vocab), dtype=torch.float32, device="cuda:0")
        tk = torch.empty((4, 4), dtype=torch.int32, device="cuda:0")
        args = (gpu.tokens.data_ptr(), gpu.positions.data_ptr(), gpu.ctx_lens.data_ptr(), 1)
        assert mkd.mk_decode_steps(gpu.ctx, *args, 0, lg.data_ptr(), tk.data_ptr()) == mkd.MK_ERR_INVALID_ARG
        assert mkd.mk_decode_steps(gpu.ctx, *args, mkd.MK_MAX_STEPS + 1, lg.data_ptr(), tk.data_ptr()) == mkd.MK_ERR_INVALID_ARG
        assert mkd.mk_decode_steps(gpu.ctx, *args, 2, lg.data_ptr(), 0) == mkd.MK_ERR_INVALID_ARG
        assert mkd.mk_decode_steps(gpu.ctx, *args, 2, lg.data_ptr(), tk.data_ptr() + 4) == mkd.MK_ERR_INVALID_ARG
        assert mkd.mk_decode_steps(gpu.ctx, *args, 2, 0, tk.data_ptr()) == mkd.MK_ERR_INVALID_ARG
    finally:
        gpu.close()
