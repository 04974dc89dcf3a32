"""Pins of the oracle's mixture-of-experts MLP (no GPU): the router's top-k choice and weights, the
one-expert and identical-experts special cases that reduce it to the dense SwiGLU MLP, and forced
expert choices (how the GPU parity tests feed the GPU's routing back)."""
import numpy as np
import pytest

import oracle
import synth


def test_select_takes_the_k_largest_in_descending_order_ties_to_the_lower_index():
    z = np.array([0.5, 2.0, -1.0, 2.0, 0.5, 3.0, 0.5], np.float32)
    assert oracle.moe_select(z, 1).tolist() == [5]
    assert oracle.moe_select(z, 3).tolist() == [5, 1, 3]
    assert oracle.moe_select(z, 5).tolist() == [5, 1, 3, 0, 4]
    assert oracle.moe_select(z, 7).tolist() == [5, 1, 3, 0, 4, 6, 2]


def test_weights_are_the_softmax_renormalised_over_the_chosen():
    rng = np.random.default_rng(3)
    z = rng.standard_normal(16).astype(np.float32)
    sel = oracle.moe_select(z, 4)
    w = oracle.moe_weights(z, sel)
    p = np.exp(z.astype(np.float64) - z.max())
    p /= p.sum()
    assert np.allclose(w, p[sel] / p[sel].sum(), rtol=1e-14, atol=0)
    assert abs(w.sum() - 1.0) < 1e-15 and np.all(np.diff(w) <= 0)
    # softmax of the chosen logits alone: the renormalisation cancels the unchosen experts
    q = np.exp(z[sel].astype(np.float64) - z[sel].max())
    assert np.allclose(w, q / q.sum(), rtol=1e-14, atol=0)


def _step(cfg, w, steps=2, force=None):
    ctx = synth.context_lengths(cfg)
    cache = synth.make_cache(cfg, ctx, steps)
    orc = oracle.DecodeOracle(cfg, w, cache)
    toks = [int(t) for t in synth.first_tokens(cfg)]
    outs = []
    for s in range(steps):
        pos = [c + s for c in ctx]
        lg, mid = orc.step(toks, pos, [p + 1 for p in pos], dump=True,
                           force_experts=None if force is None else force[s])
        outs.append((lg, mid))
        toks = [oracle.argmax(r) for r in lg]
    return outs


def _dense_from_expert(w, e):
    d = dict(w)
    d["layers"] = []
    for L in w["layers"]:
        L = {k: v for k, v in L.items() if k != "w_router"}
        L["w_gate"], L["w_up"], L["w_down"] = (np.ascontiguousarray(L[f][e]) for f in ("w_gate", "w_up", "w_down"))
        d["layers"].append(L)
    return d


def test_one_expert_is_the_dense_mlp_bit_for_bit():
    cfg = synth.SMALL["tiny-moe"].replace(n_experts=1, top_k=1)
    w = synth.make_weights(cfg)
    dense = cfg.replace(n_experts=0, top_k=0)
    a = _step(cfg, w)
    b = _step(dense, _dense_from_expert(w, 0))
    for (la, _), (lb, _) in zip(a, b):
        assert np.array_equal(la.view(np.uint32), lb.view(np.uint32))


def test_identical_experts_are_the_dense_mlp():
    """Every expert the same: whichever k are chosen, their weights sum to one."""
    cfg = synth.SMALL["tiny-moe"]
    w = synth.make_weights(cfg)
    for L in w["layers"]:
        for f in ("w_gate", "w_up", "w_down"):
            L[f] = np.ascontiguousarray(np.broadcast_to(L[f][3], L[f].shape))
    a = _step(cfg, w)
    b = _step(cfg.replace(n_experts=0, top_k=0), _dense_from_expert(w, 3))
    for (la, _), (lb, _) in zip(a, b):
        assert float(np.max(np.abs(la - lb)) / np.max(np.abs(lb))) < 1e-6


def test_routing_uses_every_chosen_expert_and_only_those():
    """Changing the weights of an expert no sequence chose leaves the step unchanged; changing a chosen
    one moves it."""
    cfg = synth.SMALL["tiny-moe"]
    w = synth.make_weights(cfg)
    (lg, mid), = _step(cfg, w, steps=1)
    chosen = set(mid["sel"][1, 0].tolist())
    unchosen = next(e for e in range(cfg.n_experts) if e not in chosen)
    for e, moves in ((unchosen, False), (min(chosen), True)):
        w2 = dict(w)
        w2["layers"] = [dict(L) for L in w["layers"]]
        w2["layers"][1]["w_down"] = w["layers"][1]["w_down"].copy()
        w2["layers"][1]["w_down"][e] ^= np.uint16(0x0100)
        (lg2, _), = _step(cfg, w2, steps=1)
        assert np.array_equal(lg, lg2) != moves, e


def test_forcing_the_own_choice_changes_nothing_and_another_choice_does():
    cfg = synth.SMALL["tiny-moe"]
    w = synth.make_weights(cfg)
    base = _step(cfg, w)
    own = [m["sel"] for _, m in base]
    same = _step(cfg, w, force=own)
    for (la, _), (lb, _) in zip(base, same):
        assert np.array_equal(la.view(np.uint32), lb.view(np.uint32))
    other = [s.copy() for s in own]
    other[0][0, 0, -1] = next(e for e in range(cfg.n_experts) if e not in other[0][0, 0])
    moved = _step(cfg, w, force=other)
    assert not np.array_equal(base[0][0], moved[0][0])
    # the forced step reports the oracle's own choice, not the forced one
    assert np.array_equal(moved[0][1]["sel"], own[0])
