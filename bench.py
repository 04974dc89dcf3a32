#!/usr/bin/env python3
"""Decode throughput of the persistent megakernel on one MI355X.

One step = one mk_decode_step: the whole decode of one token per sequence
(embedding, every layer's RMSNorm / QKV / RoPE / paged attention / o_proj /
SwiGLU MLP, final norm, LM head) in one kernel launch.  Inputs are seeded
synthetic weights and caches of the named shape, resident in HBM before the
timed region; tokens and positions for every timed step are staged on the
device beforehand, so nothing but launches happens between steps.

Prints ONE JSON line: decode tokens/s of the headline workload (value), MBU,
the roofline of the megakernel (algorithmic bytes per launch / measured launch
time vs 8 TB/s), the same decode continued as launches of several steps with
the greedy token chosen on the device (multistep), the CPU oracle timed on a
bounded sample of the same workload, the read ceiling of this GPU measured in
the same run (stream_read), the same figures for the other workloads
(per_config), and verify windows of 8 tokens (verify_window).
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
    "8b-fp8": "8B-shape decoder with fp8 E4M3 projections (fp32 row scales; bf16 embedding, LM head and KV "
              "cache), batch 1, ctx 4096",
    "8b-fp4": "8B-shape decoder with MX fp4 projections (E2M1 codes, E8M0 scales per 32 weights; bf16 "
              "embedding, LM head and KV cache), batch 1, ctx 4096",
    "moe": "mixture-of-experts decoder (16 layers, hidden 2048, GQA 16/4, every MLP top-8 of 64 SwiGLU experts "
           "of width 1024, vocab 50304), batch 1, ctx 4096",
}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def bytes_per_step(cfg, ctx_lens) -> float:
    """Algorithmic HBM bytes of one decode step: every projection weight once (2 bytes a bf16 weight,
    or 1 an fp8 code plus 4 a row scale, or half a byte an fp4 code plus 1 a block scale of 32),
    one embedding row per sequence, the LM head once, K/V of
    every cached position per attention layer (plus the append), the delta-rule and conv states read
    and written, and the logits written."""
    H, F, V, B = cfg.hidden, cfg.ffn, cfg.vocab, cfg.batch
    fp8, fp4 = cfg.weights == "fp8", cfg.weights == "fp4"

    def proj(rows, cols):
        if fp4:
            return rows * (cols / 2.0 + cols / 32.0)
        return rows * (cols + 4.0) if fp8 else rows * cols * 2.0

    w = 0.0
    attn_kv = 0.0
    for kind in cfg.kinds():
        if cfg.n_experts:  # the router, and the chosen experts' rows (exactly top_k of them at batch 1;
            # at larger batches the union of the sequences' choices, bounded here by top_k * batch)
            w += cfg.n_experts * H * 2 + min(cfg.n_experts, cfg.top_k * B) * (2 * proj(F, H) + proj(H, F))
        else:
            w += 2 * proj(F, H) + proj(H, F)
        if kind == 0:
            w += proj((cfg.n_q_heads + 2 * cfg.n_kv_heads) * cfg.head_dim, H) + proj(H, cfg.n_q_heads * cfg.head_dim)
            attn_kv += sum(2.0 * c * cfg.n_kv_heads * cfg.head_dim * 2 for c in ctx_lens)  # read K and V
        else:
            C = cfg.n_delta_heads * (2 * cfg.delta_dk + cfg.delta_dv)
            w += proj(C + 2.0 * cfg.n_delta_heads, H) + proj(H, cfg.n_delta_heads * cfg.delta_dv)
            w += C * cfg.conv_width * 2
            attn_kv += B * cfg.n_delta_heads * cfg.delta_dk * cfg.delta_dv * 4 * 2     # S read + write
            attn_kv += B * C * (cfg.conv_width - 1) * 4 * 2                             # conv state
    w += V * H * 2                      # LM head (the embedding when tied, counted once)
    w += B * H * 2                      # embedding rows
    norms = (2 * cfg.n_layers + 1) * H * 2
    return w + attn_kv + norms + B * V * 4


PMC_FILES = {"8b": os.path.join(ROOT, "profiles", "megakernel_8b_b1_ctx4096_pmc.txt"),
             "8b-fp8": os.path.join(ROOT, "profiles", "megakernel_8b_fp8_b1_ctx4096_pmc.txt"),
             "8b-fp4": os.path.join(ROOT, "profiles", "megakernel_8b_fp4_b1_ctx4096_pmc.txt"),
             "moe": os.path.join(ROOT, "profiles", "megakernel_moe_b1_ctx4096_pmc.txt")}


def kernel_source_hash(texts=None) -> str:
    """Hash of the device code the counters were taken with (kernel and the headers it includes),
    comments and blank lines left out, so that a change to comments alone keeps the figure."""
    import hashlib
    import re
    h = hashlib.sha256()
    if texts is None:
        texts = []
        for f in ("mk_kernel.hip", "mk_internal.h", "mk_attn_plan.h"):
            with open(os.path.join(ROOT, "persistent_megakernel_decode_amd", "csrc", f)) as fh:
                texts.append(fh.read())
    for t in texts:
        t = re.sub(r"/\*.*?\*/", "", t, flags=re.S)
        for line in t.splitlines():
            line = re.sub(r"//.*", "", line).rstrip()
            if line:
                h.update(line.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(config: str):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE summary, calibrated against a
    plain copy kernel; None when the summary is missing, for another workload, or for other sources."""
    path = PMC_FILES.get(config)
    if path is None or not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if (vals.get("kernel_source_sha256_16", "").split() or [""])[0] != kernel_source_hash():
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


def stream_read_ceiling(mkd, torch, stream) -> dict:
    """What a plain streaming read reaches on this GPU in the same run: the library's own read kernel
    over a 2 GiB buffer (every byte once), best over a few grid sizes; and the runtime's
    device-to-device copy for context."""
    nbytes = 1 << 31
    buf = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    buf.fill_(1.0)
    out = torch.empty(65536, dtype=torch.int32, device="cuda")
    sp = int(stream.cuda_stream)
    best = (0.0, 0)
    for blocks in (2048, 4096, 8192, 16384):
        ts = []
        for _ in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            mkd.check(mkd.mk_stream_read(buf.data_ptr(), nbytes, out.data_ptr(), blocks, sp), "mk_stream_read")
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        gbs = nbytes / (float(np.median(ts[1:])) * 1e-3) / 1e9
        if gbs > best[0]:
            best = (gbs, blocks)
    dst = torch.empty_like(buf)
    cp = []
    for _ in range(6):  # read + write bytes
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dst.copy_(buf)
        e1.record(stream)
        torch.cuda.synchronize()
        cp.append(e0.elapsed_time(e1))
    copy_gbs = 2 * nbytes / (float(np.median(cp[1:])) * 1e-3) / 1e9
    del buf, dst, out
    torch.cuda.empty_cache()
    return {"gbs": round(best[0], 1), "kernel": f"mk_stream_read over 2 GiB, {best[1]} workgroups x 256 threads, "
            "non-temporal 16-byte loads, 8 in flight per thread, best of 2048/4096/8192/16384 workgroups",
            "copy_gbs": round(copy_gbs, 1), "copy": "2 GiB device-to-device copy (runtime blit), read + write bytes"}


def staged_inputs(torch, B, rows):
    """Device int32 arrays [len(rows)][stride] (each row padded to 16 bytes) from host rows."""
    stride = max(4, (B + 3) // 4 * 4)
    a = np.zeros((len(rows), stride), np.int32)
    for i, r in enumerate(rows):
        a[i, :B] = r
    return torch.from_numpy(a).cuda(), stride * 4


def run_config(name: str, steps: int, warmup: int, multi_k: int, cpu_budget: float, trace_path: str = "") -> dict:
    """Times `steps` single-step launches (after `warmup`), then `steps` decode steps as launches of
    `multi_k` steps each (mk_decode_steps, tokens chosen on the device), on one seeded workload;
    then the CPU oracle on a bounded sample (cpu_budget > 0)."""
    import torch
    import synth
    import persistent_megakernel_decode_amd as mkd

    cfg = synth.CONFIGS[name]
    B = cfg.batch
    n_launch = max(1, steps // multi_k) if multi_k else 0
    room = warmup + steps + (multi_k * (1 + n_launch) if multi_k else 0)
    ctx0 = synth.context_lengths(cfg)
    t0 = time.time()
    w = synth.make_weights(cfg)
    cache = synth.make_cache(cfg, ctx0, room)
    log(f"{name}: inputs generated in {time.time() - t0:.1f}s")
    t0 = time.time()
    max_ctx = int(cache["max_pages_per_seq"]) * cfg.page_size
    g = mkd.DecodeContext(synth.shape_of(cfg, max_ctx), w, cache, "cuda:0")
    del cache
    entry = {}
    try:
        torch.cuda.synchronize()
        log(f"{name}: device model ready in {time.time() - t0:.1f}s, workspace {g.ws_bytes / 2**20:.1f} MiB")
        total = warmup + steps
        draws = synth.u32(total * B, cfg.seed, "bench_tokens").reshape(total, B) % cfg.vocab
        toks_d, row = staged_inputs(torch, B, [draws[s] for s in range(total)])
        pos_d, _ = staged_inputs(torch, B, [[c + s for c in ctx0] for s in range(total)])
        len_d, _ = staged_inputs(torch, B, [[c + s + 1 for c in ctx0] for s in range(total)])
        stream = torch.cuda.current_stream()
        sp = int(stream.cuda_stream)

        def launch(s: int) -> None:
            rc = mkd.mk_decode_step(g.ctx, toks_d.data_ptr() + s * row, pos_d.data_ptr() + s * row,
                                    len_d.data_ptr() + s * row, B, g.logits.data_ptr(), sp)
            if rc != 0:
                raise mkd.MKError(rc, f"mk_decode_step (step {s})")

        for s in range(warmup):
            launch(s)
        torch.cuda.synchronize()
        mkd.check(g.sync(), "warm-up")
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for i in range(steps):
            ev[i][0].record(stream)
            launch(warmup + i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t_start
        mkd.check(g.sync(), "timed steps")
        kms = np.array([a.elapsed_time(b) for a, b in ev])  # per-launch kernel time on its stream
        log(f"{name}: timed {steps} steps: {elapsed * 1e3:.1f} ms wall, kernel median {np.median(kms) * 1e3:.1f} us")
        step_bytes = [bytes_per_step(cfg, [c + warmup + i for c in ctx0]) for i in range(steps)]
        mean_bytes = float(np.mean(step_bytes))
        ms_per_step = elapsed * 1e3 / steps
        kernel_s = float(np.mean(kms)) * 1e-3
        achieved = mean_bytes / kernel_s / 1e9
        entry = {
            "workload": WORKLOADS[name], "weights": cfg.weights, "batch": B, "ctx": ctx0 if B > 1 else ctx0[0],
            "steps": steps,
            "warmup": warmup, "ms_per_step": round(ms_per_step, 4), "tokens_per_s": round(B * steps / elapsed, 2),
            "mbu": round(mean_bytes / (ms_per_step * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
            "bytes_per_step": mean_bytes,
            "kernel_us_mean": round(kernel_s * 1e6, 2),
            "kernel_us_median": round(float(np.median(kms)) * 1e3, 2),
            "kernel_us_p90": round(float(np.percentile(kms, 90)) * 1e3, 2),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(name)},
        }
        if trace_path:  # the last timed step, per op (the traced kernels were timed above)
            from persistent_megakernel_decode_amd import trace as mktrace
            tr = g.trace()
            with open(trace_path, "w") as f:
                json.dump(mktrace.chrome_trace(tr), f)
            entry["traced"] = {"path": trace_path, "per_op_kind_us": {
                k: {kk: round(vv, 1) if isinstance(vv, float) else vv for kk, vv in v.items()}
                for k, v in mktrace.op_summary(tr).items()}}
            log(f"trace of the last step written to {trace_path}")
        elif multi_k:
            # the same decode continued as launches of multi_k steps (greedy tokens chosen on the device)
            base = [c + total for c in ctx0]
            first = [int(t) for t in draws[-1]]
            starts = [[c + multi_k * j for c in base] for j in range(1 + n_launch)]
            mtok_d, mrow = staged_inputs(torch, B, [first] * (1 + n_launch))
            mpos_d, _ = staged_inputs(torch, B, starts)
            mlen_d, _ = staged_inputs(torch, B, [[c + 1 for c in st] for st in starts])
            mlogits = torch.empty((multi_k, B, cfg.vocab), dtype=torch.float32, device="cuda")
            mtoks = torch.empty((multi_k, max(4, B)), dtype=torch.int32, device="cuda")

            def mlaunch(j: int) -> None:
                rc = mkd.mk_decode_steps(g.ctx, mtok_d.data_ptr() + j * mrow, mpos_d.data_ptr() + j * mrow,
                                         mlen_d.data_ptr() + j * mrow, B, multi_k, mlogits.data_ptr(),
                                         mtoks.data_ptr(), sp)
                if rc != 0:
                    raise mkd.MKError(rc, f"mk_decode_steps (launch {j})")

            mlaunch(0)
            torch.cuda.synchronize()
            mkd.check(g.sync(), "multi-step warm-up")
            mev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_launch)]
            t_start = time.perf_counter()
            for j in range(n_launch):
                mev[j][0].record(stream)
                mlaunch(1 + j)
                mev[j][1].record(stream)
            torch.cuda.synchronize()
            m_elapsed = time.perf_counter() - t_start
            mkd.check(g.sync(), "multi-step launches")
            mk_ms = np.array([a.elapsed_time(b) for a, b in mev])
            m_steps = n_launch * multi_k
            m_bytes = float(np.mean([bytes_per_step(cfg, [c + k for c in starts[1 + j]])
                                     for j in range(n_launch) for k in range(multi_k)]))
            m_ms = m_elapsed * 1e3 / m_steps
            m_kernel_s = float(np.mean(mk_ms)) * 1e-3 / multi_k
            entry["multistep"] = {
                "steps_per_launch": multi_k, "launches": n_launch, "ms_per_step": round(m_ms, 4),
                "tokens_per_s": round(B * m_steps / m_elapsed, 2),
                "mbu": round(m_bytes / (m_ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
                "kernel_us_per_step": round(m_kernel_s * 1e6, 2),
                "roofline_frac": round(m_bytes / m_kernel_s / 1e9 / HBM_PEAK_GBS, 4)}
            log(f"{name}: {n_launch} launches of {multi_k} steps: {m_ms * 1e3:.1f} us per step")
    finally:
        g.close()
        del g
        torch.cuda.empty_cache()
    if cpu_budget > 0:
        log(f"{name}: timing the CPU oracle on a bounded sample")
        room = 64  # new positions the oracle's cache can take
        entry["cpu_baseline"] = cpu_baseline(cfg, w, synth.make_cache(cfg, ctx0, room), ctx0, cpu_budget, room)
    return entry


def run_window(name: str, window: int, launches: int, warmup: int) -> dict:
    """Verify windows (mk_decode_window): `window` tokens of each sequence per step, the same
    workload's weights and cache, a context compiled for batch x window rows."""
    import torch
    import synth
    import persistent_megakernel_decode_amd as mkd

    cfg = synth.CONFIGS[name]
    B = cfg.batch
    total = warmup + launches
    ctx0 = synth.context_lengths(cfg)
    w = synth.make_weights(cfg)
    cache = synth.make_cache(cfg, ctx0, total * window)
    max_ctx = int(cache["max_pages_per_seq"]) * cfg.page_size
    shape = synth.shape_of(cfg, max_ctx)
    shape["max_batch"] = B * window
    g = mkd.DecodeContext(shape, w, cache, "cuda:0")
    del cache
    try:
        draws = synth.u32(total * B * window, cfg.seed, "bench_window_tokens").reshape(total, B * window) % cfg.vocab
        toks_d, trow = staged_inputs(torch, B * window, [draws[i] for i in range(total)])
        pos_d, row = staged_inputs(torch, B, [[c + i * window for c in ctx0] for i in range(total)])
        len_d, _ = staged_inputs(torch, B, [[c + i * window + 1 for c in ctx0] for i in range(total)])
        logits = torch.empty((B, window, cfg.vocab), dtype=torch.float32, device="cuda")
        stream = torch.cuda.current_stream()
        sp = int(stream.cuda_stream)

        def launch(i: int) -> None:
            rc = mkd.mk_decode_window(g.ctx, toks_d.data_ptr() + i * trow, pos_d.data_ptr() + i * row,
                                      len_d.data_ptr() + i * row, B, window, logits.data_ptr(), sp)
            if rc != 0:
                raise mkd.MKError(rc, f"mk_decode_window (launch {i})")

        for i in range(warmup):
            launch(i)
        torch.cuda.synchronize()
        mkd.check(g.sync(), "window warm-up")
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
        t_start = time.perf_counter()
        for i in range(launches):
            ev[i][0].record(stream)
            launch(warmup + i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t_start
        mkd.check(g.sync(), "window launches")
        kms = np.array([a.elapsed_time(b) for a, b in ev])
    finally:
        g.close()
        del g
        torch.cuda.empty_cache()
    ms = elapsed * 1e3 / launches
    log(f"{name}: {launches} windows of {window}: {ms * 1e3:.1f} us per window")
    return {"window": window, "sequences": B, "launches": launches, "ms_per_window": round(ms, 4),
            "tokens_per_s": round(B * window * launches / elapsed, 2),
            "kernel_us_median": round(float(np.median(kms)) * 1e3, 2),
            "note": "tokens verified per second: every window token's logits per launch"}


PER_CONFIG = ("0.6b", "hybrid", "13b", "8b-fp8", "8b-fp4", "moe")  # measured beside the headline 8B workload
WINDOWS = {"8b": 8, "0.6b": 8}            # verify windows timed beside them
RUN_STEPS = {"8b": 128, "0.6b": 64, "hybrid": 64, "13b": 64, "tiny": 8, "8b-fp8": 128, "8b-fp4": 128, "moe": 64}  # decode steps per run


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="8b", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--per-config-cpu-budget", type=float, default=6.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-per-config", action="store_true", help="time the headline workload only")
    ap.add_argument("--multi-k", type=int, default=8, help="steps per launch of the multi-step timing (0 = skip)")
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
    import persistent_megakernel_decode_amd as mkd

    head = run_config(args.config, args.steps, args.warmup, args.multi_k,
                      0.0 if args.no_cpu else args.cpu_budget, args.trace)
    B = head["batch"]
    out = {
        "metric": "decode tokens/s and MBU (% of HBM peak) per step, 8B-shape batch 1 ctx 4096"
        if args.config == "8b" else f"decode tokens/s and MBU (% of HBM peak) per step, {args.config}",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["weights"] if head["weights"] in ("fp8", "fp4") else "bf16",
        "data": "synthetic (seeded random-init weights and KV cache of the named shape)",
        "config": {"workload": head["workload"], "batch": B, "ctx": head["ctx"]},
    }
    for k in ("mbu", "bytes_per_step", "kernel_us_mean", "kernel_us_median", "kernel_us_p90", "roofline",
              "multistep", "traced", "cpu_baseline"):
        if k in head:
            out[k] = head[k]
    out["stream_read"] = stream_read_ceiling(mkd, torch, torch.cuda.current_stream())
    out["stream_read"]["achieved_frac"] = round(head["roofline"]["achieved"] / out["stream_read"]["gbs"], 4)
    if not args.no_per_config and not args.trace and args.config == "8b":
        out["verify_window"] = {name: run_window(name, win, 16, 2) for name, win in WINDOWS.items()}
        out["per_config"] = {}
        for name in PER_CONFIG:
            n = min(args.steps, RUN_STEPS[name])
            out["per_config"][name] = run_config(name, n, args.warmup, args.multi_k,
                                                 0.0 if args.no_cpu else args.per_config_cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
