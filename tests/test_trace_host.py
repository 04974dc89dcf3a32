"""Host logic of the per-op trace summaries on a hand-built trace (no GPU)."""
import json

import numpy as np

from persistent_megakernel_decode_amd import trace


def _trace():
    # two CUs; stages 0 (gemv, 2 ops) and 1 (attention, 2 ops); clock ticks are 10 ns
    t = np.array([[100, 150, 400], [110, 110, 380],   # cu 0: gemv s0, attention s1
                  [105, 300, 420], [420, 500, 900]], np.int64)
    return {"n_cus": 2, "queue_off": np.array([0, 2, 4]), "cu": np.array([0, 0, 1, 1]),
            "opcode": np.array([2, 3, 2, 3]), "stage": np.array([0, 1, 0, 1], np.int16), "t": t}


def test_unwrap_handles_clock_wrap():
    tr = _trace()
    tr["t"] = (tr["t"] + (1 << 32) - 200) % (1 << 32)  # the low 32 bits wrap inside the step
    us = trace.unwrap(tr)
    assert us.min() == 0.0
    assert np.allclose(us, (_trace()["t"] - 100) / 100.0)


def test_stage_table_and_summary():
    tr = _trace()
    tr["t"][1] = [410, 410, 700]  # cu 0's second op starts after its first ends
    assert trace.check(tr) == []
    rows = trace.stage_table(tr)
    assert [r["stage"] for r in rows] == [0, 1]
    assert rows[0]["op"] == "gemv" and rows[1]["op"] == "attention"
    assert rows[0]["us"] == (420 - 100) / 100.0          # stage 0 ends at its last op end
    assert rows[1]["us"] == (900 - 420) / 100.0          # measured from stage 0's end
    assert rows[0]["waiting_us"] == np.median([0.5, 1.95])
    s = trace.op_summary(tr)
    assert s["gemv"]["stages"] == 1 and s["attention"]["us"] == rows[1]["us"]


def test_check_flags_disorder():
    tr = _trace()  # cu 0's second op starts (110) before its first ends (400)
    assert any("cu 0" in b for b in trace.check(tr))
    tr["t"][3] = [420, 410, 900]
    assert any("out of order" in b for b in trace.check(tr))


def test_chrome_trace_is_json():
    tr = _trace()
    ev = json.loads(json.dumps(trace.chrome_trace(tr)))["traceEvents"]
    ops = [e for e in ev if e["cat"] == "op"]
    assert len(ops) == 4 and {e["tid"] for e in ops} == {0, 1}
    waits = [e for e in ev if e["cat"] == "wait"]
    assert len(waits) == 3  # the op with ready == start has no wait slice
