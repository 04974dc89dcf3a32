"""mk_create_static, the entry point for callers that cannot allocate device memory: the same decode
through the library's static device scratch instead of a caller-provided workspace.

Two calls in a row, the second with a smaller model: each static context's logits must equal, bit
for bit, those of the ordinary mk_create path on the same inputs (same kernels, same plan), and the
second call must not see anything the first left in the shared scratch.  The first static context
is refused once the second has taken the scratch over; a model whose workspace exceeds the scratch
is rejected before anything is touched.
"""
import ctypes

import numpy as np
import pytest

import persistent_megakernel_decode_amd as mkd
import synth
from gpu_harness import say

pytestmark = pytest.mark.gpu

BIG = synth.Config("static-mha-b4", n_layers=4, hidden=512, n_q_heads=4, n_kv_heads=4, head_dim=128, ffn=1024,
                   vocab=2048, batch=4, ctx=[1, 16, 33, 300], seed=21, gain_range=(0.5, 1.5))
SMALL = synth.CONFIGS["tiny"]


def _run(cfg, static, steps=3):
    import torch
    ctx0 = synth.context_lengths(cfg)
    w = synth.make_weights(cfg)
    cache = synth.make_cache(cfg, ctx0, steps)
    max_ctx = int(cache["max_pages_per_seq"]) * cfg.page_size
    g = mkd.DecodeContext(synth.shape_of(cfg, max_ctx), w, cache, static_workspace=static)
    toks = [int(t) for t in synth.first_tokens(cfg)]
    ctx = list(ctx0)
    out = []
    for _ in range(steps):
        assert g.step(toks, ctx, [c + 1 for c in ctx]) == 0
        torch.cuda.synchronize()
        assert g.sync() == 0
        lg = g.logits[:cfg.batch].cpu().numpy().copy()
        out.append(lg)
        toks = [int(np.argmax(r)) for r in lg]
        ctx = [c + 1 for c in ctx]
    return g, np.stack(out)


def test_static_scratch_matches_the_workspace_path():
    contexts = []
    sizes = []
    for cfg in (BIG, SMALL):  # the second call with a smaller input
        say(f"static scratch: {cfg.name}")
        ref_ctx, ref = _run(cfg, static=False)
        sizes.append(ref_ctx.ws_bytes)
        ref_ctx.close()
        g, got = _run(cfg, static=True)
        assert np.isfinite(got).all()
        assert np.array_equal(ref, got), f"{cfg.name}: static-scratch logits differ from the workspace path"
        contexts.append(g)
    assert sizes[1] < sizes[0] <= mkd.MK_STATIC_SCRATCH_BYTES
    # the second mk_create_static took the scratch over: the first context is refused
    first, second = contexts
    assert mkd.mk_decode_step(first.ctx, first.tokens.data_ptr(), first.positions.data_ptr(),
                              first.ctx_lens.data_ptr(), 1, first.logits.data_ptr(), first.stream_ptr()) == mkd.MK_ERR_STATE
    assert first.sync() == mkd.MK_ERR_STATE
    assert second.sync() == 0
    for g in contexts:
        g.close()


def test_static_scratch_rejects_a_model_that_does_not_fit():
    """13B shape, batch 8: its workspace (attention partials of 40 layers) exceeds the scratch.
    Rejected from the description alone, before any weight or cache pointer is looked at."""
    cfg = synth.CONFIGS["13b"]
    s = synth.shape_of(cfg, 4096 + 80)
    d = mkd.make_desc(s["n_layers"], s["hidden"], s["vocab"], s["ffn"], s["n_q_heads"], s["n_kv_heads"],
                      s["head_dim"], s["qk_norm"], s["tied"], s["rms_eps"], s["rope_base"], s["layer_kinds"],
                      s["max_batch"], s["max_ctx"])
    assert mkd.mk_workspace_size(d) > mkd.MK_STATIC_SCRATCH_BYTES
    out = ctypes.c_void_p()
    rc = mkd.lib().mk_create_static(ctypes.byref(d), ctypes.byref(mkd.mk_weights()), ctypes.byref(mkd.mk_kv_cache()),
                                    ctypes.byref(out))
    assert rc == mkd.MK_ERR_INVALID_ARG and not out.value
    assert "static scratch" in mkd.mk_last_error()
