"""The per-op timing trace (MK_TRACE=1): every queue entry is stamped in order on its CU, every
stage of the plan shows up, and tracing leaves the results unchanged."""
import numpy as np
import pytest

import persistent_megakernel_decode_amd as mkd
from persistent_megakernel_decode_amd import trace
import synth
from gpu_harness import run_parity, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny-hybrid", "small-b8"])
def test_trace_records_every_op(name, monkeypatch):
    monkeypatch.setenv("MK_TRACE", "1")
    cfg = synth.SMALL["tiny-hybrid"].replace(delta_dk=64, delta_dv=64) if name == "tiny-hybrid" else synth.Config(
        "small-b8", n_layers=2, hidden=512, n_q_heads=4, n_kv_heads=4, head_dim=128, ffn=1024, vocab=2048,
        batch=8, ctx=[5, 40, 0, 17, 100, 3, 64, 31], steps=3, seed=14)
    ctx0 = synth.context_lengths(cfg)
    cache = synth.make_cache(cfg, ctx0, 2)
    max_ctx = int(cache["max_pages_per_seq"]) * cfg.page_size
    g = mkd.DecodeContext(synth.shape_of(cfg, max_ctx), synth.make_weights(cfg), cache)
    say(f"[{name}] trace: two steps")
    tokens = list(range(1, len(ctx0) + 1))
    for s in range(2):
        pos = [c + s for c in ctx0]
        assert g.step(tokens, pos, [p + 1 for p in pos]) == 0
    assert g.sync() == 0
    tr = g.trace()
    g.close()
    n_ops = len(tr["opcode"])
    assert n_ops == int(tr["queue_off"][-1]) and len(tr["cu"]) == n_ops
    assert set(np.unique(tr["opcode"]).tolist()) <= set(trace.OPCODES)
    assert np.all(tr["t"] != 0), "an op was never stamped"
    assert trace.check(tr) == []
    rows = trace.stage_table(tr)
    stages = sorted({int(s) for s in tr["stage"]})
    assert [r["stage"] for r in rows] == stages
    assert all(r["us"] >= 0 and r["waiting_us"] >= 0 and r["tail_us"] >= 0 for r in rows)
    total = trace.unwrap(tr)[:, 2].max()
    say(f"[{name}] {n_ops} ops in {len(rows)} stages, {total:.1f} us from first start to last end")


def test_trace_leaves_results_unchanged(monkeypatch):
    monkeypatch.setenv("MK_TRACE", "1")
    cfg = synth.SMALL["tiny-gain"].replace(name="tiny-ragged", batch=3, ctx=[0, 77, 19], shuffle_pages=True)
    rep = run_parity(cfg, 3)
    say(f"[tiny-ragged, traced] worst logits rel {rep.worst_rel:.2e}, worst mid {rep.worst_mid:.2e}")
    assert not rep.failures, "\n".join(rep.failures[:20])
