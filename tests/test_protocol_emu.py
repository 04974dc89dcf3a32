"""The dependency protocol on the CPU: the compiled queues replayed by the library's emulator
(mk_emulate) over launch sequences with changing batches and contexts, in random interleavings.

The megakernel's consumers poll their inputs for the launch's parity, which is sound only if every
value they may poll is written exactly once per launch.  These tests check, with no GPU, that the
plan the GPU path uploads keeps that invariant -- no poll accepts an earlier launch's value, no
value is written twice or left unwritten, no launch deadlocks -- across attention plans whose chunk
counts drop and recover and batches that shrink and grow back.  Two further cases model the
earlier kernel that broke it (attention items without a chunk writing nothing; mixer rows of
sequences outside the step left unwritten) and check that the emulator reports the hazard.
"""
import numpy as np
import pytest

import persistent_megakernel_decode_amd as mkd
import synth

MAX_CTX = 8192


def _desc(cfg, max_ctx=MAX_CTX):
    s = synth.shape_of(cfg, max_ctx)
    return mkd.make_desc(s["n_layers"], s["hidden"], s["vocab"], s["ffn"], s["n_q_heads"], s["n_kv_heads"],
                         s["head_dim"], s["qk_norm"], s["tied"], s["rms_eps"], s["rope_base"], s["layer_kinds"],
                         s["max_batch"], s["max_ctx"], s["n_delta_heads"], s["delta_dk"], s["delta_dv"],
                         s["conv_width"], n_experts=s["n_experts"], top_k=s["top_k"])


def _clean(rep):
    return (rep.stale_accepts, rep.unsynced_reads, rep.double_writes, rep.unwritten_cells, rep.deadlocks) == (0,) * 5


def random_sequence(rng, max_batch, n, lo=1, hi=600, p_refill=0.1, p_dead=0.05):
    """Launch batches and contexts: sequences grow by one per launch while in the batch, the batch
    shrinks and grows back, a slot is sometimes refilled with a new context, and a context is
    sometimes out of range (the row is then outside the step's attention)."""
    ctx = list(rng.integers(lo, hi, size=max_batch))
    batches, ctxs = [], []
    for _ in range(n):
        b = int(rng.integers(1, max_batch + 1))
        row = []
        for j in range(max_batch):
            if j < b:
                if rng.random() < p_refill:
                    ctx[j] = int(rng.integers(lo, hi))
                ctx[j] += 1
            row.append(0 if rng.random() < p_dead else ctx[j])
        batches.append(b)
        ctxs.append(row)
    return batches, ctxs


SHAPES = {
    "tiny-gqa-d64": synth.CONFIGS["tiny"].replace(batch=3),
    "mha-d128-b4": synth.Config("mha-d128-b4", n_layers=2, hidden=512, n_q_heads=4, n_kv_heads=4, head_dim=128,
                                ffn=1024, vocab=2048, batch=4),
    "mha-b8": synth.Config("mha-b8", n_layers=2, hidden=512, n_q_heads=4, n_kv_heads=4, head_dim=128, ffn=1024,
                           vocab=2048, batch=8),
    "gqa8-d64": synth.Config("gqa8-d64", n_layers=2, hidden=512, n_q_heads=16, n_kv_heads=2, head_dim=64,
                             ffn=1024, vocab=2048, batch=2),
    "tiny-hybrid": synth.SMALL["tiny-hybrid"].replace(batch=3, delta_dk=64, delta_dv=64),
    # mixture of experts: every expert's SwiGLU rows written each launch (zeros when not chosen)
    "tiny-moe-b4": synth.SMALL["tiny-moe"].replace(batch=4),
}


@pytest.mark.parametrize("shape", list(SHAPES))
@pytest.mark.parametrize("n_cus", [3, 8, 13])
def test_protocol_holds_over_changing_batches_and_contexts(shape, n_cus):
    cfg = SHAPES[shape]
    rng = np.random.default_rng(hash((shape, n_cus)) % 2**32)
    batches, ctxs = random_sequence(rng, cfg.batch, 40)
    for seed in (1, 2):
        rep, msg = mkd.mk_emulate(_desc(cfg), n_cus, batches, ctxs, seed=seed)
        assert _clean(rep), msg
        assert rep.ops_run > 0 and rep.polls > 0


def test_protocol_holds_for_the_hybrid_attention_shape_on_256_units():
    """Batch 4 with 4 KV heads (the hybrid model's attention layers) on all 256 compute units:
    ragged contexts that change the chunk plan as they grow, one slot refilled partway."""
    cfg = synth.CONFIGS["hybrid"].replace(n_layers=4, layer_kinds=synth.hybrid_kinds(4))
    ctx0 = [2541, 810, 5979, 605]
    ctxs = [[c + i for c in ctx0] for i in range(24)]
    for i in range(12, 24):
        ctxs[i][1] = 40 + i  # sequence 1 restarts with a short context: fewer chunks, then more
    rep, msg = mkd.mk_emulate(_desc(cfg), 256, [4] * 24, ctxs, seed=3)
    assert _clean(rep), msg


def test_counter_plan_holds():
    cfg = SHAPES["tiny-hybrid"]
    rng = np.random.default_rng(7)
    batches, ctxs = random_sequence(rng, cfg.batch, 30)
    rep, msg = mkd.mk_emulate(_desc(cfg), 8, batches, ctxs, seed=5, flags=mkd.MK_EMU_COUNTERS)
    assert _clean(rep), msg


def _drop_and_recover():
    # a second sequence leaves for one launch, then returns: its chunk slots go unwritten for a launch
    return [2, 1, 2, 2], [[200, 200], [201, 0], [202, 201], [203, 202]]


def test_emulator_catches_idle_items_that_write_nothing():
    cfg = SHAPES["mha-d128-b4"].replace(batch=2)
    batches, ctxs = _drop_and_recover()
    rep, msg = mkd.mk_emulate(_desc(cfg), 8, batches, ctxs, seed=1, flags=mkd.MK_EMU_IDLE_ITEMS_SILENT)
    assert rep.unwritten_cells > 0
    assert rep.stale_accepts > 0, msg
    rep, msg = mkd.mk_emulate(_desc(cfg), 8, batches, ctxs, seed=1)
    assert _clean(rep), msg


def test_emulator_catches_unwritten_rows_of_sequences_outside_the_step():
    cfg = synth.SMALL["tiny-gain"].replace(batch=3)
    batches = [3, 2, 3, 3]
    ctxs = [[10, 20, 30], [11, 21, 0], [12, 22, 31], [13, 23, 32]]
    rep, msg = mkd.mk_emulate(_desc(cfg), 8, batches, ctxs, seed=1, flags=mkd.MK_EMU_DEAD_ROWS_SILENT)
    assert rep.stale_accepts > 0 and rep.first_bad_launch >= 0
    rep, msg = mkd.mk_emulate(_desc(cfg), 8, batches, ctxs, seed=1)
    assert _clean(rep), msg


def test_a_stuck_producer_is_reported_not_hung():
    cfg = SHAPES["tiny-hybrid"]
    rep, msg = mkd.mk_emulate(_desc(cfg), 8, [3, 3], [[5, 6, 7], [6, 7, 8]], seed=1, flags=mkd.MK_EMU_STALL_ONE_OP)
    assert rep.deadlocks == 1 and rep.first_bad_launch == 0
    assert "watchdog" in msg


def test_emulator_rejects_bad_arguments():
    cfg = SHAPES["tiny-gqa-d64"]
    with pytest.raises(mkd.MKError):
        mkd.mk_emulate(_desc(cfg), 0, [1], [[5]])
    with pytest.raises(mkd.MKError):
        mkd.mk_emulate(_desc(cfg), 4, [9], [[5]])
