"""Shared GPU-vs-oracle harness for the parity tests and the smoke check (test infrastructure).

Both sides consume the same seeded inputs from synth; the oracle keeps its own KV / state history,
and both are fed the GPU's greedy token every step so the histories never fork.
"""
from __future__ import annotations

import sys
import time
from dataclasses import dataclass, field
from typing import List

import numpy as np

import oracle
import synth

LOGIT_REL_TOL = 1e-2   # max_v |g - o| / max_v |o| per (sequence, step): bf16 weights, fp32 accumulation
GREEDY_GAP = 1e-2      # greedy ids must agree wherever the oracle's top-2 logit gap exceeds this
MID_TOL = 2e-3         # normwise relative error of per-layer mid-states (fp32 activations)


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
    greedy_checked: int = 0
    greedy_agree: int = 0
    failures: List[str] = field(default_factory=list)


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


def run_parity(cfg: synth.Config, steps: int, mid: bool = True, device: str = "cuda:0") -> ParityReport:
    import torch
    w, cache, orc, gpu, ctx0 = make_pair(cfg, steps, device)
    B = cfg.batch
    rep = ParityReport(cfg.name)
    toks = [int(t) for t in synth.first_tokens(cfg)]
    ctx = list(ctx0)
    for step in range(steps):
        pos = list(ctx)
        lens = [c + 1 for c in ctx]
        say(f"[{cfg.name}] step {step}: tokens {toks} positions {pos}")
        rc = gpu.step(toks, pos, lens)
        if rc != 0:
            rep.failures.append(f"step {step}: mk_decode_step returned {rc}")
            return rep
        torch.cuda.synchronize()
        st = gpu.sync()
        if st != 0:
            rep.failures.append(f"step {step}: mk_sync_status returned {st}")
            return rep
        g = gpu.logits[:B].cpu().numpy()
        gmid = {}
        if mid:
            H, F, X = cfg.hidden, cfg.ffn, orc.mix_dim
            for l in range(cfg.n_layers):
                gmid[("x_mixer", l)] = gpu.midstate(0, l, H, B).cpu().numpy()
                gmid[("x_mlp", l)] = gpu.midstate(1, l, H, B).cpu().numpy()
                gmid[("mixer_o", l)] = gpu.midstate(2, l, X, B).cpu().numpy()
                gmid[("mlp_m", l)] = gpu.midstate(3, l, F, B).cpu().numpy()
        t0 = time.time()
        o, omid = orc.step(toks, pos, lens, dump=True)
        say(f"[{cfg.name}] step {step}: oracle {time.time() - t0:.2f}s")
        for b in range(B):
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
            for b in range(B):
                e = normwise(gv[b], omid[kind][l, b])
                rep.worst_mid = max(rep.worst_mid, e)
                if e > MID_TOL:
                    rep.failures.append(f"step {step} layer {l} row {b}: {kind} normwise err {e:.3e}")
        say(f"[{cfg.name}] step {step}: worst logits rel {rep.worst_rel:.2e}, worst mid-state {rep.worst_mid:.2e}")
        toks = [int(np.argmax(g[b])) for b in range(B)]  # both sides consume the GPU's token
        ctx = lens
        rep.steps += 1
        if rep.failures:
            break
    gpu.close()
    return rep
