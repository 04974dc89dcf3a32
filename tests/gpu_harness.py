"""Shared GPU-vs-oracle harness for the parity tests and the smoke check (test infrastructure).

Both sides consume the same seeded inputs from synth; the oracle keeps its own KV / state history,
and both are fed the GPU's greedy token every step so the histories never fork.

Gates, per step (the mid-state oracle of the ForgeMegakernel abstract; the separate output /
conv-state / recurrent-state gates of the MK-KDA pull request's summary):
  * logits: max_v |g - o| / max_v |o| <= 1e-2 per sequence, greedy ids equal where the oracle's top-2
    gap exceeds 1e-2;
  * per-layer mid-states (residual after each sub-layer, attention / delta output, SwiGLU product):
    normwise <= 2e-3;
  * delta-rule layers, every step and every sequence in the step:
      - the recurrent state S the GPU wrote against the oracle's delta mixer applied to the GPU's own
        projections, conv state and S from before the step: normwise <= 1e-5 per head;
      - the conv state the GPU wrote equals, bit for bit, its previous state shifted by one with the
        GPU's own new projection appended (the rolling-window regression of the MK-KDA review);
      - GPU S and conv state against the oracle's own trajectory: normwise <= 1e-4;
    and the states of sequences outside the step are unchanged, bit for bit.
A step schedule can shrink and regrow the batch and move a sequence to a shorter context (a slot
refilled with a new request), which changes the attention plan from launch to launch.
"""
from __future__ import annotations

import sys
import time
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

import oracle
import synth

LOGIT_REL_TOL = 1e-2   # max_v |g - o| / max_v |o| per (sequence, step): bf16 weights, fp32 accumulation
GREEDY_GAP = 1e-2      # greedy ids must agree wherever the oracle's top-2 logit gap exceeds this
MID_TOL = 2e-3         # normwise relative error of per-layer mid-states (fp32 activations)
STATE_OP_TOL = 1e-5    # delta-rule S from the GPU's own inputs (fp32 update of fp32 state)
STATE_RUN_TOL = 1e-4   # GPU S / conv state against the oracle's own trajectory
ROUTE_GAP = 1e-2       # mixture of experts: the oracle's own top-k choice must be the GPU's wherever its
                       # k-th and (k+1)-th router logits differ by more than this (the oracle then runs
                       # the GPU's choice, as both sides consume the GPU's greedy token)


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def normwise(g, o) -> float:
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    return float(np.linalg.norm(g - o) / max(np.linalg.norm(o), 1e-30))


def top2_gap(v) -> float:
    s = np.sort(np.asarray(v, np.float64))
    return float(s[-1] - s[-2])


@dataclass
class ParityReport:
    name: str
    steps: int = 0
    worst_rel: float = 0.0
    worst_mid: float = 0.0
    worst_state_op: float = 0.0
    worst_state_run: float = 0.0
    conv_checked: int = 0
    greedy_checked: int = 0
    greedy_agree: int = 0
    route_checked: int = 0   # (layer, sequence) routing choices compared (oracle's k-th margin > ROUTE_GAP)
    route_agree: int = 0
    failures: List[str] = field(default_factory=list)


@dataclass
class Step:
    """One launch: the sequences 0..batch-1 take part; `jump` moves sequence b to context jump[b]
    (its cache positions below that are kept) before the step."""
    batch: int
    jump: Dict[int, int] = field(default_factory=dict)


def make_pair(cfg: synth.Config, steps: int, device: str = "cuda:0"):
    import persistent_megakernel_decode_amd as mkd
    ctx0 = synth.context_lengths(cfg)
    t0 = time.time()
    w = synth.make_weights(cfg)
    cache = synth.make_cache(cfg, ctx0, steps)
    say(f"[{cfg.name}] inputs generated in {time.time() - t0:.1f}s (batch {cfg.batch}, ctx {ctx0})")
    orc = oracle.DecodeOracle(cfg, w, cache)
    max_ctx = int(cache["max_pages_per_seq"]) * cfg.page_size  # what the mapped pages can hold
    gpu = mkd.DecodeContext(synth.shape_of(cfg, max_ctx), w, cache, device)
    say(f"[{cfg.name}] device model ready ({gpu.ws_bytes / 2**20:.1f} MiB workspace)")
    return w, cache, orc, gpu, ctx0


def _delta_layers(cfg) -> List[int]:
    return [l for l, k in enumerate(cfg.kinds()) if k == synth.DELTA]


def run_parity(cfg: synth.Config, steps: int, mid: bool = True, device: str = "cuda:0", mid_every: int = 1,
               schedule: Optional[Sequence[Step]] = None, states: bool = True) -> ParityReport:
    import torch
    w, cache, orc, gpu, ctx0 = make_pair(cfg, steps, device)
    B = cfg.batch
    rep = ParityReport(cfg.name)
    toks = [int(t) for t in synth.first_tokens(cfg)]
    ctx = list(ctx0)
    dls = _delta_layers(cfg) if states else []
    C = cfg.n_delta_heads * (2 * cfg.delta_dk + cfg.delta_dv) if dls else 0
    for step in range(steps):
        st = schedule[step] if schedule is not None else Step(B)
        nb = st.batch
        for b, c in st.jump.items():
            ctx[b] = c
        pos = ctx[:nb]
        lens = [c + 1 for c in pos]
        say(f"[{cfg.name}] step {step}: batch {nb} tokens {toks[:nb]} positions {pos}")
        if dls:
            s_old = gpu.delta_state.cpu().numpy().copy()
            c_old = gpu.conv_state.cpu().numpy().copy()
        rc = gpu.step(toks[:nb], pos, lens)
        if rc != 0:
            rep.failures.append(f"step {step}: mk_decode_step returned {rc}")
            return rep
        torch.cuda.synchronize()
        rc = gpu.sync()
        if rc != 0:
            rep.failures.append(f"step {step}: mk_sync_status returned {rc}")
            return rep
        g = gpu.logits[:nb].cpu().numpy()
        gmid = {}
        do_mid = mid and step % mid_every == 0
        moe = cfg.n_experts > 0
        if moe:  # the GPU's router logits and the experts it chose from them, fed to the oracle
            E, k = cfg.n_experts, cfg.top_k
            glog = np.stack([gpu.midstate(6, l, E, nb).cpu().numpy() for l in range(cfg.n_layers)])
            gsel = np.array([[oracle.moe_select(glog[l, b], k) for b in range(nb)] for l in range(cfg.n_layers)],
                            dtype=np.int32)
        if do_mid:
            H, F, X = cfg.hidden, cfg.ffn, orc.mix_dim
            for l in range(cfg.n_layers):
                gmid[("x_mixer", l)] = gpu.midstate(0, l, H, nb).cpu().numpy()
                gmid[("x_mlp", l)] = gpu.midstate(1, l, H, nb).cpu().numpy()
                gmid[("mixer_o", l)] = gpu.midstate(2, l, X, nb).cpu().numpy()
                if moe:
                    gmid[("router", l)] = glog[l]
                else:
                    gmid[("mlp_m", l)] = gpu.midstate(3, l, F, nb).cpu().numpy()
        if dls:
            s_new = gpu.delta_state.cpu().numpy()
            c_new = gpu.conv_state.cpu().numpy()
            proj = {l: gpu.midstate(4, l, C + 2 * cfg.n_delta_heads, nb).cpu().numpy() for l in dls}
            mixo = {l: gpu.midstate(2, l, orc.mix_dim, nb).cpu().numpy() for l in dls}
        t0 = time.time()
        o, omid = orc.step(toks[:nb], pos, lens, dump=True, force_experts=gsel if moe else None)
        if moe:  # where the oracle's own choice is clear, it must be the GPU's
            for l in range(cfg.n_layers):
                for b in range(nb):
                    srt = np.sort(omid["router"][l, b])[::-1]
                    if k < E and float(srt[k - 1] - srt[k]) <= ROUTE_GAP:
                        continue
                    rep.route_checked += 1
                    if sorted(omid["sel"][l, b].tolist()) == sorted(gsel[l, b].tolist()):
                        rep.route_agree += 1
                    else:
                        rep.failures.append(f"step {step} layer {l} row {b}: experts {sorted(gsel[l, b].tolist())} "
                                            f"!= the oracle's {sorted(omid['sel'][l, b].tolist())}")
        say(f"[{cfg.name}] step {step}: oracle {time.time() - t0:.2f}s")
        for b in range(nb):
            rel = float(np.max(np.abs(g[b].astype(np.float64) - o[b])) / np.max(np.abs(o[b])))
            rep.worst_rel = max(rep.worst_rel, rel)
            if not np.isfinite(g[b]).all():
                rep.failures.append(f"step {step} row {b}: non-finite logits")
            if rel > LOGIT_REL_TOL:
                rep.failures.append(f"step {step} row {b}: logits rel err {rel:.3e}")
            if top2_gap(o[b]) > GREEDY_GAP:
                rep.greedy_checked += 1
                if int(np.argmax(g[b])) == oracle.argmax(o[b]):
                    rep.greedy_agree += 1
                else:
                    rep.failures.append(f"step {step} row {b}: greedy id {int(np.argmax(g[b]))} != {oracle.argmax(o[b])}")
        for (kind, l), gv in gmid.items():
            for b in range(nb):
                e = normwise(gv[b], omid[kind][l, b])
                rep.worst_mid = max(rep.worst_mid, e)
                if e > MID_TOL:
                    rep.failures.append(f"step {step} layer {l} row {b}: {kind} normwise err {e:.3e}")
        if dls:
            _check_delta_states(cfg, orc, dls, nb, C, s_old, c_old, s_new, c_new, proj, mixo, step, rep)
        say(f"[{cfg.name}] step {step}: worst logits rel {rep.worst_rel:.2e}, worst mid-state {rep.worst_mid:.2e}"
            + (f", S vs oracle on GPU inputs {rep.worst_state_op:.2e}, states vs oracle run {rep.worst_state_run:.2e}"
               if dls else ""))
        for b in range(nb):
            toks[b] = int(np.argmax(g[b]))  # both sides consume the GPU's token
            ctx[b] += 1
        rep.steps += 1
        if rep.failures:
            break
    gpu.close()
    return rep


def _check_delta_states(cfg, orc, dls, nb, C, s_old, c_old, s_new, c_new, proj, mixo, step, rep) -> None:
    nh, dv = cfg.n_delta_heads, cfg.delta_dv
    for i, l in enumerate(dls):
        for b in range(cfg.batch):
            if b >= nb:  # outside the step: untouched
                if not (np.array_equal(s_new[i, b], s_old[i, b]) and np.array_equal(c_new[i, b], c_old[i, b])):
                    rep.failures.append(f"step {step} layer {l} row {b}: state of a sequence outside the step changed")
                continue
            u, a = proj[l][b, :C], proj[l][b, C:C + 2 * nh]
            o_ref, cs_ref, st_ref = orc.delta_mixer(l, u, a, c_old[i, b], s_old[i, b])
            # conv state: the previous window shifted by one with the GPU's own projection appended
            if not np.array_equal(c_new[i, b].view(np.uint32), cs_ref.view(np.uint32)):
                bad = int(np.sum(c_new[i, b].view(np.uint32) != cs_ref.view(np.uint32)))
                rep.failures.append(f"step {step} layer {l} row {b}: conv state differs in {bad} values")
            rep.conv_checked += 1
            for h in range(nh):
                e = normwise(s_new[i, b, h], st_ref[h])
                rep.worst_state_op = max(rep.worst_state_op, e)
                if e > STATE_OP_TOL:
                    rep.failures.append(f"step {step} layer {l} row {b} head {h}: S normwise err {e:.3e} "
                                        f"against the oracle on the GPU's inputs")
            e = normwise(mixo[l][b, :nh * dv], o_ref)
            rep.worst_state_op = max(rep.worst_state_op, e)
            if e > STATE_OP_TOL:
                rep.failures.append(f"step {step} layer {l} row {b}: delta readout normwise err {e:.3e}")
            for what, gv, ov in (("S", s_new[i, b], orc.delta_state[i, b]), ("conv state", c_new[i, b], orc.conv_state[i, b])):
                e = normwise(gv, ov)
                rep.worst_state_run = max(rep.worst_state_run, e)
                if e > STATE_RUN_TOL:
                    rep.failures.append(f"step {step} layer {l} row {b}: {what} normwise err {e:.3e} against the oracle run")
