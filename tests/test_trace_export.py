"""The Perfetto (Chrome trace-event) export of unit traces, on a synthetic
trace: one process per XCD, non-overlapping slices per track, three slices
per unit with the right times."""
import json

import numpy as np

from persistent_micro_dispatch_amd import gpuos as G
from persistent_micro_dispatch_amd.trace_export import to_chrome_trace, write_perfetto


def _trace():
    t = np.zeros(5, G.TRACE_DTYPE)
    # (seq, tile, xcc, wg, claim, ready, body, done) in 100 MHz ticks
    rows = [(10, 0, 0, 3, 100, 150, 250, 300), (11, 0, 0, 3, 120, 160, 200, 260),  # overlap in WG 3
            (11, 1, 0, 3, 310, 310, 400, 420), (12, 0, 5, 7, 90, 95, 130, 140), (12, 1, 5, 8, 90, 95, 131, 141)]
    for i, (s, u, x, w, a, b, c, d) in enumerate(rows):
        t[i]["seq"], t[i]["tile"], t[i]["hw"] = s, u, (x << 16) | w
        t[i]["t_claim"], t[i]["t_ready"], t[i]["t_body"], t[i]["t_done"] = a, b, c, d
    return t


def test_chrome_trace_layout(tmp_path):
    tr = _trace()
    out = to_chrome_trace(tr, clock_khz=100_000, names=lambda s: f"op{s}")
    ev = [e for e in out["traceEvents"] if e["ph"] == "X"]
    assert len(ev) == 3 * len(tr)
    procs = {e["args"]["name"] for e in out["traceEvents"] if e["name"] == "process_name"}
    assert procs == {"XCD 0", "XCD 5"}
    # t0 = 90 ticks; 10 ns per tick
    first = next(e for e in ev if e["args"]["seq"] == 10 and e["name"] == "op10")
    assert abs(first["ts"] - 0.6) < 1e-9 and abs(first["dur"] - 1.0) < 1e-9
    # the two overlapping units of WG 3 sit on different tracks; the third reuses the first
    tids = {(e["args"]["seq"], e["args"]["unit"]): e["tid"] for e in ev}
    assert tids[(10, 0)] != tids[(11, 0)] and tids[(11, 1)] == tids[(10, 0)]
    for tid in set(tids.values()):
        sl = sorted((e["ts"], e["ts"] + e["dur"]) for e in ev if e["tid"] == tid)
        assert all(a[1] <= b[0] + 1e-9 for a, b in zip(sl, sl[1:]))
    p = tmp_path / "t.json"
    write_perfetto(tr, str(p))
    assert len(json.load(open(p))["traceEvents"]) == len(out["traceEvents"])


def test_empty_trace():
    assert to_chrome_trace(np.zeros(0, G.TRACE_DTYPE))["traceEvents"] == []
