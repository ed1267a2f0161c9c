"""Unit traces (gpuos_trace_read) as Chrome trace-event JSON, which the
Perfetto UI and chrome://tracing open.

One process per XCD, one track per workgroup (split into as many sub-tracks
as the workgroup had units in flight at once, so events on a track never
overlap); each unit becomes three slices: "wait" (claimed and published ->
dependencies satisfied), its body ("run", or the name `names` gives its
descriptor) and "publish" (body done -> completion written).  Times are the
device's constant-rate wall clock, converted with `clock_khz`
(hipDeviceAttributeWallClockRate; 100 MHz on MI355X).
"""
from __future__ import annotations

import json
from typing import Callable, Dict, Optional

import numpy as np


def to_chrome_trace(trace: np.ndarray, clock_khz: float = 100_000.0,
                    names: Optional[Callable[[int], str]] = None) -> Dict:
    """trace: records as returned by gpuos.gpuos_trace_read.  names(seq) -> a
    label for the descriptor's body slices (default "run")."""
    if len(trace) == 0:
        return {"traceEvents": [], "displayTimeUnit": "ns"}
    us = 1000.0 / float(clock_khz)  # microseconds per tick
    t0 = int(min(int(trace["t_claim"].min()), int(trace["t_ready"].min())))
    xcc = (trace["hw"].astype(np.int64) >> 16)
    wg = (trace["hw"].astype(np.int64) & 0xFFFF)
    events = []
    seen_pid = set()
    # greedy interval partitioning per workgroup: a unit goes to the first
    # sub-track whose last unit has ended
    order = np.lexsort((trace["t_claim"], wg, xcc))
    lanes: Dict[tuple, list] = {}
    for i in order:
        r = trace[i]
        key = (int(xcc[i]), int(wg[i]))
        start, end = int(r["t_claim"]), int(r["t_done"])
        ends = lanes.setdefault(key, [])
        lane = next((k for k, e in enumerate(ends) if e <= start), len(ends))
        if lane == len(ends):
            ends.append(end)
        else:
            ends[lane] = end
        pid, tid = key[0], key[1] * 64 + lane
        if pid not in seen_pid:
            seen_pid.add(pid)
            events.append({"name": "process_name", "ph": "M", "pid": pid, "args": {"name": f"XCD {pid}"}})
        seq, tile = int(r["seq"]), int(r["tile"])
        args = {"seq": seq, "unit": tile, "workgroup": key[1]}
        label = names(seq) if names else "run"
        for nm, a, b in (("wait", r["t_claim"], r["t_ready"]), (label, r["t_ready"], r["t_body"]),
                         ("publish", r["t_body"], r["t_done"])):
            a, b = int(a), int(b)
            if b < a:
                continue
            events.append({"name": nm, "ph": "X", "pid": pid, "tid": tid, "ts": (a - t0) * us,
                           "dur": (b - a) * us, "args": args})
    for (p, w), ends in lanes.items():
        for lane in range(len(ends)):
            events.append({"name": "thread_name", "ph": "M", "pid": p, "tid": w * 64 + lane,
                           "args": {"name": f"WG {w}" + (f" / {lane}" if lane else "")}})
    return {"traceEvents": events, "displayTimeUnit": "ns"}


def write_perfetto(trace: np.ndarray, path: str, clock_khz: float = 100_000.0,
                   names: Optional[Callable[[int], str]] = None) -> None:
    with open(path, "w") as f:
        json.dump(to_chrome_trace(trace, clock_khz, names), f)
