"""Summaries of the per-op timing trace (contexts created with MK_TRACE=1).

Times are the GPU's 100 MHz real-time clock (low 32 bits), so every figure is in microseconds
after unwrapping against the first op.  A stage's time is measured from the previous stage's last
op end to its own last op end; "waiting" is the median time its ops spend before their inputs are
in hand, "tail" how long its last op ends after its median op.
"""
import numpy as np

OPCODES = {1: "embed", 2: "gemv", 3: "attention", 4: "delta", 5: "mmv", 6: "moe_gate_up", 7: "moe_down"}


def unwrap(tr: dict) -> np.ndarray:
    """Stamps [n_ops, 3] (start, ready, end) in us relative to the earliest start."""
    t = tr["t"].astype(np.int64)
    # differences to one stamp, taken modulo 2^32 (every stamp of a step lies within 21 s of it)
    d = (t - int(t[0, 0]) + (1 << 31)) % (1 << 32) - (1 << 31)
    return (d - d[:, 0].min()) / 100.0


def stage_table(tr: dict) -> list:
    """One row per stage: opcode, ops, time from the previous stage's end, waiting, tail."""
    us = unwrap(tr)
    rows, prev_end = [], 0.0
    for s in range(int(tr["stage"].max()) + 1):
        m = tr["stage"] == s
        if not m.any():
            continue
        end = us[m, 2]
        rows.append({"stage": s, "op": OPCODES.get(int(tr["opcode"][m][0]), "?"), "ops": int(m.sum()),
                     "us": float(end.max() - prev_end), "waiting_us": float(np.median(us[m, 1] - us[m, 0])),
                     "tail_us": float(end.max() - np.median(end))})
        prev_end = float(end.max())
    return rows


def check(tr: dict) -> list:
    """Consistency problems: stamps out of order within an op or across a CU's queue."""
    us = unwrap(tr)
    bad = []
    if np.any(us[:, 1] < us[:, 0]) or np.any(us[:, 2] < us[:, 1]):
        bad.append("an op's stamps are out of order")
    off = tr["queue_off"]
    for c in range(tr["n_cus"]):
        a, b = int(off[c]), int(off[c + 1])
        if b - a > 1 and np.any(us[a + 1:b, 0] < us[a:b - 1, 2]):
            bad.append(f"cu {c}: an op starts before the previous one ends")
            break
    return bad


def op_summary(tr: dict) -> dict:
    """Stage time summed per op kind (embed / gemv / attention / delta / mmv / moe_gate_up / moe_down) over the step, in us,
    with the part of it the median op spent waiting for its inputs."""
    out = {}
    for r in stage_table(tr):
        s = out.setdefault(r["op"], {"stages": 0, "us": 0.0, "waiting_us": 0.0, "tail_us": 0.0})
        s["stages"] += 1
        for k in ("us", "waiting_us", "tail_us"):
            s[k] += r[k]
    return out


def chrome_trace(tr: dict) -> dict:
    """The step as a Chrome / Perfetto trace (load the JSON in ui.perfetto.dev): one track per CU,
    each op split into its input wait and its work."""
    us = unwrap(tr)
    ev = []
    for i in range(len(us)):
        name = f"{OPCODES.get(int(tr['opcode'][i]), '?')} s{int(tr['stage'][i])}"
        cu = int(tr["cu"][i])
        t0, t1, t2 = (float(x) for x in us[i])
        if t1 > t0:
            ev.append({"name": name + " wait", "ph": "X", "pid": 0, "tid": cu, "ts": t0, "dur": t1 - t0,
                       "cat": "wait"})
        ev.append({"name": name, "ph": "X", "pid": 0, "tid": cu, "ts": t1, "dur": max(t2 - t1, 0.0),
                   "cat": "op", "args": {"queue_index": i}})
    return {"traceEvents": ev, "displayTimeUnit": "ns"}
