"""The decode oracle against brute-force full-sequence recomputation (oracle/brute.py).

brute.py shares no code with oracle.c: it recomputes the whole sequence with a
causal mask in float64, and the delta rule through its closed product form.
The oracle decodes the same prompt one token at a time from an empty cache;
the last position must agree to 1e-5 relative.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import brute


def _run_prompt(cfg, tokens, states=None, dump=False):
    T = len(tokens)
    cache = synth.make_cache(cfg, [0] * cfg.batch, T, prompt_mode=True)
    if states is not None:
        cache["delta_state"], cache["conv_state"] = states
    w = synth.make_weights(cfg)
    orc = oracle.DecodeOracle(cfg, w, cache)
    out = None
    for t in range(T):
        out = orc.step([tokens[t]] * cfg.batch, [t] * cfg.batch, [t + 1] * cfg.batch, dump=dump)
    return w, orc, out


def _rel(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - b)) / np.max(np.abs(b)))


@pytest.mark.parametrize("name,T", [("tiny-gain", 40), ("tiny-qknorm", 33), ("tiny", 136)])
def test_dense_decode_matches_full_sequence(name, T):
    cfg = synth.SMALL.get(name, synth.CONFIGS.get(name))
    tokens = (synth.u32(T, cfg.seed, "prompt") % cfg.vocab).astype(int).tolist()
    w, orc, (logits, mid) = _run_prompt(cfg, tokens, dump=True)
    want, xs, _ = brute.forward(cfg, w, tokens)
    assert _rel(logits[0], want) < 1e-5
    for l in range(cfg.n_layers):
        assert _rel(mid["x_mlp"][l, 0], xs[l]) < 1e-5


@pytest.mark.parametrize("random_states", [False, True])
def test_hybrid_decode_matches_product_form(random_states):
    cfg = synth.SMALL["tiny-hybrid"].replace(batch=1, ctx=[0])
    T = 12
    tokens = (synth.u32(T, cfg.seed, "prompt") % cfg.vocab).astype(int).tolist()
    nD = cfg.n_delta_layers
    C = cfg.n_delta_heads * (2 * cfg.delta_dk + cfg.delta_dv)
    states = None
    if random_states:
        states = (synth.normal_f32((nD, 1, cfg.n_delta_heads, cfg.delta_dv, cfg.delta_dk), 9, "S0"),
                  synth.normal_f32((nD, 1, C, cfg.conv_width - 1), 9, "conv0"))
    w, orc, (logits, mid) = _run_prompt(cfg, tokens, states=states, dump=True)
    S0 = None if states is None else [states[0][i, 0] for i in range(nD)]
    c0 = None if states is None else [states[1][i, 0] for i in range(nD)]
    want, xs, fin = brute.forward(cfg, w, tokens, S0=S0, conv0=c0)
    # Cached K/V are rounded to bf16 (both sides).  The oracle rounds from fp32-stored values and
    # brute.py from float64, so an element within ~1e-7 of a bf16 midpoint can round one ulp apart
    # (2^-8 relative on one element of one key).  Layers up to the first attention layer have no
    # such decision and must agree to 1e-5; after it a single flip moves the residual by ~3e-5.
    first_attn = cfg.kinds().index(0)
    for l in range(cfg.n_layers):
        assert _rel(mid["x_mlp"][l, 0], xs[l]) < (1e-5 if l < first_attn else 1e-4)
    assert _rel(logits[0], want) < 1e-4
    for i in range(nD):
        Sf, cf = fin[i]
        assert _rel(orc.delta_state[i, 0], Sf) < 1e-5
        # the rolling conv window holds the last W-1 pre-conv inputs
        assert _rel(orc.conv_state[i, 0], cf) < 1e-6


def test_decay_first_reading_matches_its_product_form():
    cfg = synth.SMALL["tiny-hybrid"].replace(batch=1, ctx=[0])
    T = 6
    tokens = (synth.u32(T, cfg.seed, "prompt") % cfg.vocab).astype(int).tolist()
    cache = synth.make_cache(cfg, [0], T, prompt_mode=True)
    w = synth.make_weights(cfg)
    orc = oracle.DecodeOracle(cfg, w, cache, decay_first=1)
    for t in range(T):
        logits = orc.step([tokens[t]], [t], [t + 1])
    want, _, _ = brute.forward(cfg, w, tokens, decay_first=True)
    lit, _, _ = brute.forward(cfg, w, tokens, decay_first=False)
    assert _rel(logits[0], want) < 1e-5
    assert _rel(logits[0], lit) > 1e-5  # the two readings are distinguishable at this size


def test_batch_rows_are_independent():
    cfg = synth.SMALL["tiny-gain"].replace(batch=3, ctx=[7, 30, 19])
    w = synth.make_weights(cfg)
    cache = synth.make_cache(cfg, cfg.ctx, 4)
    toks = [3, 500, 77]
    joint = oracle.DecodeOracle(cfg, w, cache).step(toks, [c for c in cfg.ctx], [c + 1 for c in cfg.ctx])
    for b in range(3):
        solo_cache = dict(cache)
        solo_cache["page_table"] = cache["page_table"][b:b + 1]
        solo = oracle.DecodeOracle(cfg.replace(batch=1, ctx=[cfg.ctx[b]]), w, solo_cache)
        one = solo.step([toks[b]], [cfg.ctx[b]], [cfg.ctx[b] + 1])
        assert np.array_equal(one[0], joint[b])


def test_mha_equals_gqa_with_replicated_kv_heads():
    gqa = synth.SMALL["tiny-gain"].replace(batch=1, ctx=[20])
    mha = gqa.replace(n_kv_heads=gqa.n_q_heads)
    w = synth.make_weights(gqa)
    rep = gqa.n_q_heads // gqa.n_kv_heads
    d = gqa.head_dim
    w2 = dict(w)
    w2["layers"] = []
    for L in w["layers"]:
        L2 = dict(L)
        for nm in ("wk", "wv"):
            L2[nm] = np.repeat(L[nm].reshape(gqa.n_kv_heads, d, -1), rep, axis=0).reshape(-1, gqa.hidden)
        w2["layers"].append(L2)
    c1 = synth.make_cache(gqa, gqa.ctx, 2)
    c2 = dict(c1)
    c2["k_pages"] = np.repeat(c1["k_pages"], rep, axis=2)
    c2["v_pages"] = np.repeat(c1["v_pages"], rep, axis=2)
    a = oracle.DecodeOracle(gqa, w, c1).step([5], [20], [21])
    b = oracle.DecodeOracle(mha, w2, c2).step([5], [20], [21])
    assert np.array_equal(a, b)


def test_tied_lm_head_is_the_embedding():
    cfg = synth.SMALL["tiny-qknorm"].replace(batch=1, ctx=[9])
    w = synth.make_weights(cfg)
    logits, mid = oracle.DecodeOracle(cfg, w, synth.make_cache(cfg, cfg.ctx, 2)).step([11], [9], [10], dump=True)
    E = synth.bf16_to_f32(w["embed"]).astype(np.float64)
    np.testing.assert_allclose(logits[0], E @ mid["final_r"][0], rtol=1e-5, atol=1e-6)


def test_out_of_contract_inputs_are_rejected():
    cfg = synth.CONFIGS["tiny"]
    w = synth.make_weights(cfg)
    orc = oracle.DecodeOracle(cfg, w, synth.make_cache(cfg, [128], 8))
    for toks, pos, ctx in (([cfg.vocab], [128], [129]), ([1], [127], [129]), ([1], [500], [501]), ([-1], [128], [129])):
        with pytest.raises(ValueError):
            orc.step(toks, pos, ctx)


def test_moe_decode_matches_full_sequence():
    """Mixture-of-experts MLPs: the incremental oracle against the full-sequence recomputation.  The
    router's choice is discrete, so the prompt is also checked to keep every top-k margin well above
    the two sides' rounding (no near-tie decides between them)."""
    cfg = synth.SMALL["tiny-moe"]
    T = 24
    tokens = (synth.u32(T, cfg.seed, "prompt") % cfg.vocab).astype(int).tolist()
    w, orc, (logits, mid) = _run_prompt(cfg, tokens, dump=True)
    want, xs, _ = brute.forward(cfg, w, tokens)
    srt = np.sort(mid["router"][:, 0], axis=-1)[:, ::-1]
    assert float(np.min(srt[:, cfg.top_k - 1] - srt[:, cfg.top_k])) > 1e-4
    assert _rel(logits[0], want) < 1e-5
    for l in range(cfg.n_layers):
        assert _rel(mid["x_mlp"][l, 0], xs[l]) < 1e-5
