#!/usr/bin/env python3
"""Decode throughput of the persistent megakernel on one MI355X.

One step = one mk_decode_step: the whole decode of one token per sequence
(embedding, every layer's RMSNorm / QKV / RoPE / paged attention / o_proj /
SwiGLU MLP, final norm, LM head) in one kernel launch.  Inputs are seeded
synthetic weights and caches of the named shape, resident in HBM before the
timed region; tokens and positions for every timed step are staged on the
device beforehand, so nothing but launches happens between steps.

Prints ONE JSON line: decode tokens/s (value), MBU, the roofline of the
megakernel (algorithmic bytes per launch / measured launch time vs 8 TB/s)
and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth

WORKLOADS = {
    "8b": "8B-shape decoder (32 layers, hidden 4096, GQA 32/8, head_dim 128, FFN 14336, vocab 128256), batch 1, ctx 4096",
    "0.6b": "0.6B-shape decoder (28 layers, hidden 1024, GQA 16/8, q/k norm, FFN 3072, vocab 151936, tied), batch 1, ctx 1024",
    "hybrid": "hybrid decoder (24 layers, hidden 2048, 6 GQA + 18 gated delta-rule layers, FFN 6144, vocab 65536), batch 4, ctx 2048",
    "13b": "13B-shape MHA decoder (40 layers, hidden 5120, 40 heads, FFN 13824, vocab 32000), batch 8, ctx U[512,4096], paged",
    "tiny": "tiny decoder (2 layers, hidden 256, GQA 4/2, head_dim 64, FFN 768, vocab 1024), batch 1, ctx 128",
}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def bytes_per_step(cfg, ctx_lens) -> float:
    """Algorithmic HBM bytes of one decode step: every projection weight once, one embedding row per
    sequence, the LM head once, K/V of every cached position per attention layer (plus the append),
    the delta-rule and conv states read and written, and the logits written."""
    H, F, V, B = cfg.hidden, cfg.ffn, cfg.vocab, cfg.batch
    w = 0.0
    attn_kv = 0.0
    for kind in cfg.kinds():
        w += 3.0 * F * H * 2
        if kind == 0:
            w += 2.0 * H * cfg.head_dim * (cfg.n_q_heads + cfg.n_kv_heads) * 2
            attn_kv += sum(2.0 * c * cfg.n_kv_heads * cfg.head_dim * 2 for c in ctx_lens)  # read K and V
        else:
            C = cfg.n_delta_heads * (2 * cfg.delta_dk + cfg.delta_dv)
            w += (C + 2.0 * cfg.n_delta_heads + cfg.n_delta_heads * cfg.delta_dv) * H * 2
            w += C * cfg.conv_width * 2
            attn_kv += B * cfg.n_delta_heads * cfg.delta_dk * cfg.delta_dv * 4 * 2     # S read + write
            attn_kv += B * C * (cfg.conv_width - 1) * 4 * 2                             # conv state
    w += V * H * 2                      # LM head (the embedding when tied, counted once)
    w += B * H * 2                      # embedding rows
    norms = (2 * cfg.n_layers + 1) * H * 2
    return w + attn_kv + norms + B * V * 4


PMC_FILE = os.path.join(ROOT, "profiles", "megakernel_8b_b1_ctx4096_pmc.txt")


def kernel_source_hash() -> str:
    """Hash of the device sources the counters were taken with (kernel + shared header)."""
    import hashlib
    h = hashlib.sha256()
    for f in ("mk_kernel.hip", "mk_internal.h"):
        with open(os.path.join(ROOT, "persistent_megakernel_decode_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(config: str):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE summary, calibrated against a
    plain copy kernel; None when the summary is missing, for another workload, or for other sources."""
    if config != "8b" or not os.path.exists(PMC_FILE):
        return None
    vals = {}
    with open(PMC_FILE) as fh:
        for line in fh:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def calibrate_copy(nbytes: int) -> int:
    """A plain device-to-device copy of known size, for scaling the HBM byte counters."""
    import torch
    n = nbytes // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda:0").uniform_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 3}), flush=True)
    return 0


def cpu_baseline(cfg, w, cache, ctx0, budget_s: float, max_steps: int) -> dict:
    """The oracle as it stands, on the host cores, over the same workload's first steps (at most
    `max_steps`: the cache it is given has room for that many new positions)."""
    import oracle
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    orc = oracle.DecodeOracle(cfg, w, cache)
    toks = [int(t) for t in __import__("synth").first_tokens(cfg)]
    ctx = list(ctx0)
    times = []
    t_start = time.time()
    while True:
        t0 = time.perf_counter()
        logits = orc.step(toks, ctx, [c + 1 for c in ctx])
        times.append(time.perf_counter() - t0)
        toks = [oracle.argmax(l) for l in logits]
        ctx = [c + 1 for c in ctx]
        if time.time() - t_start > budget_s or len(times) >= max_steps:
            break
    step = float(np.mean(times))
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    import resource
    rss_gb = resource.getrusage(resource.RUSAGE_SELF).ru_maxrss / 2**20  # KiB -> GiB
    return {"value": cfg.batch / step, "unit": "tokens/s", "cores": min(threads, cores), "kind": "oracle",
            "cpu_model": model, "host_peak_rss_gib": round(rss_gb, 1), "step_s_median": round(float(np.median(times)), 3),
            "sample": f"{len(times)} full decode steps of the same workload from its first position "
                      f"(mean {step:.3f} s/step, fp64-accumulating C oracle, OpenMP over output rows)"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="8b", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--trace", metavar="PATH", default="",
                    help="run the traced kernels (per-op stamps) and write the last step as a Perfetto JSON")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration) and exit")
    args = ap.parse_args()
    if args.calibrate_copy:
        return calibrate_copy(args.calibrate_copy)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the megakernel is a single-GPU decode step (asked for {args.gpus})",
              file=sys.stderr)
        return 2

    if args.trace:
        os.environ["MK_TRACE"] = "1"  # read at context creation: selects the traced kernels
    import torch
    import synth
    import persistent_megakernel_decode_amd as mkd

    cfg = synth.CONFIGS[args.config]
    B = cfg.batch
    total = args.warmup + args.steps
    ctx0 = synth.context_lengths(cfg)
    t0 = time.time()
    w = synth.make_weights(cfg)
    cache = synth.make_cache(cfg, ctx0, total)
    log(f"{args.config}: inputs generated in {time.time() - t0:.1f}s")
    t0 = time.time()
    max_ctx = int(cache["max_pages_per_seq"]) * cfg.page_size
    g = mkd.DecodeContext(synth.shape_of(cfg, max_ctx), w, cache, "cuda:0")
    torch.cuda.synchronize()
    log(f"device model ready in {time.time() - t0:.1f}s, workspace {g.ws_bytes / 2**20:.1f} MiB")

    # per-step device inputs, each row padded to 16 bytes
    stride = max(4, (B + 3) // 4 * 4)
    toks_h = np.zeros((total, stride), np.int32)
    pos_h = np.zeros((total, stride), np.int32)
    len_h = np.zeros((total, stride), np.int32)
    draws = synth.u32(total * B, cfg.seed, "bench_tokens").reshape(total, B) % cfg.vocab
    for s in range(total):
        toks_h[s, :B] = draws[s]
        pos_h[s, :B] = [c + s for c in ctx0]
        len_h[s, :B] = [c + s + 1 for c in ctx0]
    toks_d = torch.from_numpy(toks_h).cuda()
    pos_d = torch.from_numpy(pos_h).cuda()
    len_d = torch.from_numpy(len_h).cuda()
    stream = torch.cuda.current_stream()
    sp = int(stream.cuda_stream)
    row = stride * 4

    def launch(s: int) -> None:
        rc = mkd.mk_decode_step(g.ctx, toks_d.data_ptr() + s * row, pos_d.data_ptr() + s * row,
                                len_d.data_ptr() + s * row, B, g.logits.data_ptr(), sp)
        if rc != 0:
            raise mkd.MKError(rc, f"mk_decode_step (step {s})")

    for s in range(args.warmup):
        launch(s)
    torch.cuda.synchronize()
    mkd.check(g.sync(), "warm-up")
    log(f"warm-up done ({args.warmup} steps)")

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        launch(args.warmup + i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    mkd.check(g.sync(), "timed steps")
    kms = np.array([a.elapsed_time(b) for a, b in ev])  # per-launch kernel time on its stream
    log(f"timed {args.steps} steps: {elapsed * 1e3:.1f} ms wall, kernel median {np.median(kms) * 1e3:.1f} us")

    step_bytes = [bytes_per_step(cfg, [c + args.warmup + i for c in ctx0]) for i in range(args.steps)]
    mean_bytes = float(np.mean(step_bytes))
    ms_per_step = elapsed * 1e3 / args.steps
    tok_s = B * args.steps / elapsed
    kernel_s = float(np.mean(kms)) * 1e-3
    achieved = mean_bytes / kernel_s / 1e9
    out = {
        "metric": "decode tokens/s and MBU (% of HBM peak) per step, 8B-shape batch 1 ctx 4096"
        if args.config == "8b" else f"decode tokens/s and MBU (% of HBM peak) per step, {args.config}",
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random-init weights and KV cache of the named shape)",
        "config": {"workload": WORKLOADS[args.config], "batch": B, "ctx": ctx0 if B > 1 else ctx0[0],
                   "layers": cfg.n_layers, "hidden": cfg.hidden},
        "mbu": round(mean_bytes / (ms_per_step * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
        "bytes_per_step": mean_bytes,
        "kernel_us_median": round(float(np.median(kms)) * 1e3, 2),
        "kernel_us_p90": round(float(np.percentile(kms, 90)) * 1e3, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.config)},
    }
    # context: what a plain streaming read reaches on this GPU in the same run (torch's sum over a
    # 2 GiB buffer, i.e. one read of every byte)
    buf = torch.empty(1 << 29, dtype=torch.float32, device="cuda")
    buf.fill_(1.0)
    rd = []
    for _ in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        buf.sum()
        e1.record(stream)
        torch.cuda.synchronize()
        rd.append(e0.elapsed_time(e1))
    stream_gbs = buf.numel() * 4 / (float(np.median(rd[1:])) * 1e-3) / 1e9
    dst = torch.empty_like(buf)
    cp = []
    for _ in range(6):  # device-to-device copy (the runtime's blit kernel): read + write bytes
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dst.copy_(buf)
        e1.record(stream)
        torch.cuda.synchronize()
        cp.append(e0.elapsed_time(e1))
    copy_gbs = 2 * buf.numel() * 4 / (float(np.median(cp[1:])) * 1e-3) / 1e9
    del buf, dst
    out["stream_read"] = {"gbs": round(stream_gbs, 1), "kernel": "torch.sum over 2 GiB fp32",
                          "achieved_frac": round(achieved / stream_gbs, 4),
                          "copy_gbs": round(copy_gbs, 1), "copy": "2 GiB device-to-device copy, read + write bytes"}
    if args.trace:  # the last timed step, per op (the traced kernels were timed above)
        from persistent_megakernel_decode_amd import trace as mktrace
        tr = g.trace()
        with open(args.trace, "w") as f:
            json.dump(mktrace.chrome_trace(tr), f)
        out["traced"] = {"path": args.trace, "per_op_kind_us": {
            k: {kk: round(vv, 1) if isinstance(vv, float) else vv for kk, vv in v.items()}
            for k, v in mktrace.op_summary(tr).items()}}
        log(f"trace of the last step written to {args.trace}")
    if not args.no_cpu:
        log("timing the CPU oracle on a bounded sample")
        g.close()
        del g
        torch.cuda.empty_cache()
        room = 64  # new positions the oracle's cache can take
        out["cpu_baseline"] = cpu_baseline(cfg, w, synth.make_cache(cfg, ctx0, room), ctx0, args.cpu_budget, room)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
