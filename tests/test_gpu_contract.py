"""Behaviour at the C-ABI boundary on the GPU: host-side rejections, device-side input errors
(sticky, NaN row, no cache write), reset, determinism, and paging invariance."""
import numpy as np
import pytest

import persistent_megakernel_decode_amd as mkd
import synth
from gpu_harness import say

pytestmark = pytest.mark.gpu


def _ctx(cfg, steps=4):
    ctx0 = synth.context_lengths(cfg)
    w = synth.make_weights(cfg)
    cache = synth.make_cache(cfg, ctx0, steps)
    max_ctx = int(cache["max_pages_per_seq"]) * cfg.page_size
    return mkd.DecodeContext(synth.shape_of(cfg, max_ctx), w, cache), ctx0, cache


def test_host_rejects_bad_calls():
    import torch
    g, ctx0, _ = _ctx(synth.CONFIGS["tiny"])
    say("host rejections")
    assert g.step([1], [ctx0[0]], [ctx0[0] + 1]) == 0
    assert g.sync() == 0
    bad_batch = mkd.mk_decode_step(g.ctx, g.tokens.data_ptr(), g.positions.data_ptr(), g.ctx_lens.data_ptr(), 0,
                                   g.logits.data_ptr(), g.stream_ptr())
    assert bad_batch == mkd.MK_ERR_INVALID_ARG
    too_big = mkd.mk_decode_step(g.ctx, g.tokens.data_ptr(), g.positions.data_ptr(), g.ctx_lens.data_ptr(), 2,
                                 g.logits.data_ptr(), g.stream_ptr())
    assert too_big == mkd.MK_ERR_INVALID_ARG
    misaligned = mkd.mk_decode_step(g.ctx, g.tokens.data_ptr() + 4, g.positions.data_ptr(), g.ctx_lens.data_ptr(), 1,
                                    g.logits.data_ptr(), g.stream_ptr())
    assert misaligned == mkd.MK_ERR_INVALID_ARG
    null = mkd.mk_decode_step(g.ctx, 0, g.positions.data_ptr(), g.ctx_lens.data_ptr(), 1, g.logits.data_ptr(),
                              g.stream_ptr())
    assert null == mkd.MK_ERR_INVALID_ARG
    torch.cuda.synchronize()
    g.close()


@pytest.mark.parametrize("bad", ["token", "position", "ctx"])
def test_device_input_errors_are_sticky_and_contained(bad):
    import torch
    cfg = synth.SMALL["tiny-gain"].replace(batch=2, ctx=[10, 20])
    g, ctx0, cache = _ctx(cfg)
    toks, pos, lens = [3, 4], [10, 20], [11, 21]
    if bad == "token":
        toks[1] = cfg.vocab + 5
    elif bad == "position":
        pos[1] = 7
    else:
        lens[1] = 10 ** 6
        pos[1] = lens[1] - 1
    say(f"device input error: {bad}")
    k_before = g.k_pages.cpu().numpy().copy()
    assert g.step(toks, pos, lens) == 0
    torch.cuda.synchronize()
    assert g.sync() == mkd.MK_ERR_DEVICE_INPUT
    lg = g.logits[:2].cpu().numpy()
    assert np.isfinite(lg[0]).all() and np.isnan(lg[1]).all()
    k_after = g.k_pages.cpu().numpy()
    # row 0 appended its K at position 10 of its own pages; row 1 wrote nothing
    t = cache["page_table"]
    changed = np.argwhere((k_before != k_after).any(axis=-1))
    rows1 = set(int(p) for p in t[1][t[1] >= 0])
    assert not any(int(c[1]) in rows1 for c in changed)
    assert g.step(toks, pos, lens) == mkd.MK_ERR_STATE
    assert g.reset() == 0
    assert g.step([3, 4], [11, 21], [12, 22]) == 0
    torch.cuda.synchronize()
    assert g.sync() == 0
    g.close()


def test_same_inputs_give_bitwise_identical_logits():
    import torch
    cfg = synth.SMALL["tiny-gain"].replace(batch=3, ctx=[5, 50, 120])
    say("determinism")
    out = []
    for _ in range(2):
        g, ctx0, _ = _ctx(cfg)
        assert g.step([7, 7, 9], ctx0, [c + 1 for c in ctx0]) == 0
        torch.cuda.synchronize()
        assert g.sync() == 0
        out.append(g.logits[:3].cpu().numpy().copy())
        g.close()
    assert np.array_equal(out[0], out[1])
    # identical inputs in different batch rows give identical outputs
    cfg2 = cfg.replace(ctx=[40, 40, 40])
    g, ctx0, cache = _ctx(cfg2)
    # make rows 0 and 2 hold the same cache contents
    kp, vp, t = g.k_pages, g.v_pages, cache["page_table"]
    for p in range(-(-41 // 16)):
        kp[:, int(t[2][p])] = kp[:, int(t[0][p])]
        vp[:, int(t[2][p])] = vp[:, int(t[0][p])]
    assert g.step([5, 6, 5], [40, 40, 40], [41, 41, 41]) == 0
    torch.cuda.synchronize()
    assert g.sync() == 0
    lg = g.logits[:3].cpu().numpy()
    assert np.array_equal(lg[0], lg[2])
    g.close()


def test_shuffled_pages_match_identity_pages_bitwise():
    import torch
    base = synth.SMALL["tiny-gain"].replace(batch=3, ctx=[33, 70, 5])
    say("paging invariance")
    res = []
    for shuffle in (False, True):
        cfg = base.replace(shuffle_pages=shuffle)
        g, ctx0, _ = _ctx(cfg)
        lg = []
        toks = [1, 2, 3]
        for s in range(3):
            assert g.step(toks, [c + s for c in ctx0], [c + s + 1 for c in ctx0]) == 0
            torch.cuda.synchronize()
            assert g.sync() == 0
            lg.append(g.logits[:3].cpu().numpy().copy())
        res.append(np.stack(lg))
        g.close()
    assert np.array_equal(res[0], res[1])


def test_step_queued_behind_a_failed_step_does_nothing():
    """A step enqueued before the host has seen a device error (no sync in between) leaves at
    entry: it writes no logits, and the error is reported once the host syncs."""
    import torch
    cfg = synth.SMALL["tiny-gain"].replace(batch=2, ctx=[10, 20])
    g, ctx0, _ = _ctx(cfg)
    say("queued behind a failed step")
    assert g.step([3, cfg.vocab + 1], [10, 20], [11, 21]) == 0   # row 1: token out of range
    g.logits.fill_(123.0)                                        # stream-ordered between the launches
    assert g.step([3, 4], [11, 21], [12, 22]) == 0               # accepted: the host does not know yet
    torch.cuda.synchronize()
    assert g.sync() == mkd.MK_ERR_DEVICE_INPUT
    assert (g.logits[:2].cpu().numpy() == 123.0).all()
    assert g.reset() == 0
    assert g.step([3, 4], [11, 21], [12, 22]) == 0
    torch.cuda.synchronize()
    assert g.sync() == 0 and np.isfinite(g.logits[:2].cpu().numpy()).all()
    g.close()


def test_watchdog_timeout_is_reported_and_reset(monkeypatch):
    """The timeout path forced from the host: a watchdog limit of 1 us ends the step's waits
    (every wait in the kernel is bounded), the step reports MK_ERR_TIMEOUT, later steps are refused
    until mk_reset, and a context with the normal limit works afterwards in the same process."""
    import torch
    cfg = synth.CONFIGS["tiny"]
    monkeypatch.setenv("MK_WATCHDOG_MS", "0.001")
    g, ctx0, _ = _ctx(cfg)
    say("forced watchdog timeout")
    assert g.step([1], [ctx0[0]], [ctx0[0] + 1]) == 0
    torch.cuda.synchronize()
    assert g.sync() == mkd.MK_ERR_TIMEOUT
    assert g.step([1], [ctx0[0]], [ctx0[0] + 1]) == mkd.MK_ERR_STATE
    assert g.reset() == 0
    assert g.sync() == 0
    g.close()
    monkeypatch.delenv("MK_WATCHDOG_MS")
    g, ctx0, _ = _ctx(cfg)
    assert g.step([1], [ctx0[0]], [ctx0[0] + 1]) == 0
    torch.cuda.synchronize()
    assert g.sync() == 0 and np.isfinite(g.logits[:1].cpu().numpy()).all()
    g.close()
