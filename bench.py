"""Benchmark of the persistent micro-op dispatcher on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the whole hot path (fetch, claim, dependency wait,
op body, completion) over one seeded synthetic descriptor stream:
  elementwise (default)  100,000 descriptors over 32 fp32 + 32 bf16 tensors
                         of 65536 values; n log-uniform in [256, 65536];
                         {add, mul, relu, gelu}; 10% in place; bursts 1-64
  pr1                    1,000 fp32 add/mul/relu descriptors over 16 x 4096
  rows                   50,000 row ops (sum/max/min/softmax/LayerNorm) on
                         [r in 1..64, h in {768,1024,2048,4096}] fp32 slices
                         of a 2 GiB pool
  decode                 2,000 decode steps x 32 layers x {RoPE, KV append,
                         SDPA}: B in {1,2,4,8}, 32 heads x 128, bf16 KV cache
                         of 4096 per sequence (16 GiB), L in [128, 4096]
  decode_gqa             the same with 32 query heads sharing 8 key/value
                         heads (grouped-query attention, 4 GiB of cache)
  copy                   one 1 GiB COPY descriptor (calibrates HBM counters)
  copy64                 the same 1 GiB copied by 64 independent 16 MiB descriptors
  mixed                  500 tokens x 32 layers x 11 ops at hidden 1024 (LN,
                         GEMV 1024x3072, RoPE, KV append, SDPA, add, LN, GEMV
                         1024x3072, GELU, GEMV 3072x1024, add); with --gemm a
                         bf16 8192^3 GEMM loop co-runs on a second stream
Pools larger than the host generator fills quickly (rows, decode, mixed) are
drawn on the GPU with torch's seeded generator.

The executor is launched at the start of each step and paused (it drains and
exits) at its end, so one launch covers exactly one step; its duration comes
from HIP events recorded on the executor's own stream.

Printed: one JSON line with micro-ops/s (the headline value), p50/p99
closed-loop per-op latency, the eager hipLaunchKernel-per-op and hipGraph
baselines, null-launch cost, host submission cost, element-wise ops/s and
GB/s per log2-size bucket (in stream order with hazard ordering, and as
independent ops), the latency of binding an injected element-wise program
and its throughput beside the built-in op, the achievable HBM read and copy
bandwidth with the op
bodies' memory instructions (a plain streaming kernel), the roofline of
the executor kernel and the CPU oracle timed on a bounded sample of the
stream.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
# sources of the executor kernel: recorded counter values hold only for these
KERNEL_SOURCES = ["persistent_micro_dispatch_amd/csrc/gpuos_device.hip",
                  "persistent_micro_dispatch_amd/csrc/gpuos_ops.h",
                  "persistent_micro_dispatch_amd/csrc/gpuos_internal.h",
                  "persistent_micro_dispatch_amd/csrc/rope_math.h",
                  "include/gpuos.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gpuos_executor_hbm_traffic.md")


CORUN_CAP_S = 120.0  # longest the co-run steps go on while GEMMs are queued


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload):
    """HBM bytes per executor launch for `workload`, from the rocprofv3
    FETCH_SIZE/WRITE_SIZE runs summarised under profiles/ (scaled by a copy
    of known size), or None when none was taken or the kernel changed since."""
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    cur = kernel_source_hash()
    for line in lines:
        f = line.split()
        if len(f) == 4 and f[0] == "traffic" and f[1] == workload and f[2] == cur:
            return float(f[3])
    return None


def jit_injection(sub, nbk, by, waves, ring, num_wgs):
    """Compiled injection, in a context whose executor build calls injected
    code: the latency of binding a new program (hipRTC compile, code-object
    load, table flip; five programs that differ in a constant, so each is
    compiled anew), and the stream's independent add/mul descriptors run as
    the built-in bodies, as compiled a+b / a*b and as interpreted a+b / a*b
    in that same executor."""
    import workloads as W
    from persistent_micro_dispatch_amd import gpuos as G
    ctx = G.gpuos_init(ring_entries=ring, waves_per_wg=waves, num_wgs=num_wgs, flags=G.GPUOS_INIT_JIT)
    try:
        X, P = W.xins, W.program
        # bound while the executor is paused, as for the interpreted programs
        assert G.gpuos_pause(ctx, 30_000_000_000) == 0
        reg, comp, load, flip = [], [], [], []
        vgprs = 0
        for i in range(5):
            prog = P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_ADD, 0, 1, 2), X(W.X_CONST, 3, 0, 0, 0),
                      X(W.X_ADD, 0, 0, 3)], [0.5 * (i + 1)])
            ta = time.perf_counter()
            rc, info = G.gpuos_register_jit(ctx, 210 + i, prog)
            assert rc == 0, (rc, info)
            reg.append((time.perf_counter() - ta) * 1e3)
            comp.append(info["compile_ms"]); load.append(info["load_ms"]); flip.append(info["flip_ms"])
            vgprs = max(vgprs, info["vgprs"])
        p_add = P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_ADD, 0, 1, 2)])
        p_mul = P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_MUL, 0, 1, 2)])
        assert G.gpuos_register_jit(ctx, 200, p_add)[0] == 0 and G.gpuos_register_jit(ctx, 201, p_mul)[0] == 0
        assert G.gpuos_register_expr(ctx, 202, p_add) == 0 and G.gpuos_register_expr(ctx, 203, p_mul) == 0
        assert G.gpuos_resume(ctx) == 0
        row = {"register_ms_p50": float(np.median(reg)), "compile_ms_p50": float(np.median(comp)),
               "load_ms_p50": float(np.median(load)), "flip_ms_p50": float(np.median(flip)),
               "max_vgprs": int(vgprs), "descriptors": int(len(sub))}
        fl = G.GPUOS_SUBMIT_BLOCK | G.GPUOS_SUBMIT_NOHAZARD
        for key, ids in (("builtin", None), ("compiled", (200, 201)), ("interpreted", (202, 203))):
            dd = sub.copy()
            if ids:
                dd["op_id"] = np.where(dd["op_id"] == W.OP_ADD, ids[0], ids[1]).astype(np.uint32)
            best = 0.0
            for _ in range(2):
                ta = time.perf_counter()
                rc, _, _ = G.gpuos_submit_bursts(ctx, dd, nbk, fl)
                assert rc == 0 and G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 60_000_000_000)[0] == 0
                best = max(best, len(sub) / (time.perf_counter() - ta))
            row[key + "_ops_per_s"] = best
            row[key + "_gbs"] = best * by / len(sub) / 1e9
        return row
    finally:
        assert G.gpuos_shutdown(ctx) == 0


def chain_hops_by_xcd(num_wgs=512, n=4000, n_elem=256):
    """A dependent chain of `n` single-unit adds on one buffer, traced: the
    median time from one descriptor's completion to the next one's (a hop),
    and from a completion to the consumer finding it, split by whether the
    producer's last unit and the consumer's unit ran on the same XCD.  With
    more workgroups than CUs the executor uses one claim shard, so
    consecutive units land on any XCD."""
    import torch
    from persistent_micro_dispatch_amd import gpuos as G
    buf = torch.zeros(n_elem, dtype=torch.float32, device="cuda")
    one = torch.ones(n_elem, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    ctx = G.gpuos_init(num_wgs=num_wgs, waves_per_wg=1, ring_entries=512, flags=G.GPUOS_INIT_TRACE)
    try:
        d = G.new_descs(n)
        d["op_id"] = G.GPUOS_OP_ADD
        d["flags"] = G.flags(G.GPUOS_F32)
        d["size"] = n_elem
        d["input_a"] = d["output"] = buf.data_ptr()
        d["input_b"] = one.data_ptr()
        for i in range(0, n, 512):
            assert G.gpuos_submit(ctx, d[i:i + 512], G.GPUOS_SUBMIT_BLOCK)[0] == 0
        assert G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 60_000_000_000)[0] == 0
        assert G.gpuos_pause(ctx, 30_000_000_000) == 0
        tr = G.gpuos_trace_read(ctx)
    finally:
        assert G.gpuos_shutdown(ctx) == 0
    assert float(buf[0].item()) == float(n)
    done, xcc_done, ready, xcc_ready, claim, body = {}, {}, {}, {}, {}, {}
    for r in tr:
        q = int(r["seq"])
        if q not in done or r["t_done"] > done[q]:
            done[q], xcc_done[q] = int(r["t_done"]), int(r["hw"]) >> 16
            body[q] = int(r["t_body"])
        if q not in ready or r["t_ready"] < ready[q]:
            ready[q], xcc_ready[q], claim[q] = int(r["t_ready"]), int(r["hw"]) >> 16, int(r["t_claim"])
    hop, seen = {"same": [], "other": []}, {"same": [], "other": []}
    # where a hop's time goes (all hops): the consumer's unit claimed (and
    # its descriptor read) before or after the producer completed; from the
    # producer's completion to the consumer's dependencies found satisfied
    # (detect); the consumer's body; its completion written (publish)
    waiting, detect, bodies, publish = [], [], [], []
    us = 1e-2  # 100 MHz wall clock -> us
    qs = sorted(done)
    for a, b in zip(qs[:-1], qs[1:]):
        if b == a + 1:
            k = "same" if xcc_done[a] == xcc_ready[b] else "other"
            hop[k].append((done[b] - done[a]) * us)
            seen[k].append((ready[b] - done[a]) * us)
            waiting.append(claim[b] <= done[a])
            detect.append((ready[b] - done[a]) * us)
            bodies.append((body[b] - ready[b]) * us)
            publish.append((done[b] - body[b]) * us)
    out = {k: {"hops": len(hop[k]), "hop_us_p50": float(np.median(hop[k])) if hop[k] else None,
               "seen_after_done_us_p50": float(np.median(seen[k])) if seen[k] else None} for k in hop}
    if waiting:
        w = np.asarray(waiting)
        pct = lambda x, p: float(np.percentile(np.asarray(x), p))  # noqa: E731
        out["phases"] = {
            "consumer_claimed_before_producer_done": float(w.mean()),
            "detect_us_p50": pct(detect, 50), "detect_us_p90": pct(detect, 90),
            "detect_us_p50_when_claimed_before": pct(np.asarray(detect)[w], 50) if w.any() else None,
            "detect_us_p50_when_claimed_after": pct(np.asarray(detect)[~w], 50) if (~w).any() else None,
            "body_us_p50": pct(bodies, 50), "publish_us_p50": pct(publish, 50),
            "hop_us_p50": pct(np.asarray(detect) + np.asarray(bodies) + np.asarray(publish), 50),
        }
    return out



def critical_path(recs, descs, bursts, waves, ring, num_wgs, units_per_wave):
    """The element-wise stream once more, in the timed configuration but
    with the unit trace on, and its critical path: from the descriptor that
    completed last, each step goes to its dependency (read-after-write,
    write-after-read, write-after-write on whole prefixes of pool tensors,
    which is exact for this stream) that completed last.  Each hop of the
    path (from that dependency's completion to the consumer's) splits into
    claim-late (the consumer's first unit claimed only after the dependency
    completed), detect (until the first unit found its dependencies
    satisfied), spread (until the last unit did) and tail (the last unit's
    body and the descriptor's completion).  Times are device wall-clock
    stamps (100 MHz)."""
    import workloads as W
    from persistent_micro_dispatch_amd import gpuos as G
    ctx = G.gpuos_init(waves_per_wg=waves, ring_entries=ring, num_wgs=num_wgs,
                       units_per_wave=units_per_wave, flags=G.GPUOS_INIT_TRACE)
    try:
        assert G.gpuos_pause(ctx, 30_000_000_000) == 0
        for _ in range(2):  # the trace keeps the last launch
            assert G.gpuos_resume(ctx) == 0
            rc, first, n = G.gpuos_submit_bursts(ctx, descs, bursts, G.GPUOS_SUBMIT_BLOCK)
            assert rc == 0 and n == len(descs), (rc, n)
            assert G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 300_000_000_000)[0] == 0
            assert G.gpuos_pause(ctx, 30_000_000_000) == 0
        tr = G.gpuos_trace_read(ctx, 1 << 21)
    finally:
        assert G.gpuos_shutdown(ctx) == 0
    tr = tr[tr["seq"] >= first]
    order = np.argsort(tr["seq"], kind="stable")
    tr = tr[order]
    u, idx = np.unique(tr["seq"].astype(np.int64), return_index=True)
    if len(u) != len(recs):
        return {"error": f"trace holds {len(u)} of {len(recs)} descriptors"}
    t = {f: tr[f].astype(np.int64) for f in ("t_claim", "t_ready", "t_body", "t_done")}
    claim0 = np.minimum.reduceat(t["t_claim"], idx)
    ready0 = np.minimum.reduceat(t["t_ready"], idx)
    ready1 = np.maximum.reduceat(t["t_ready"], idx)
    done1 = np.maximum.reduceat(t["t_done"], idx)
    nunits = np.diff(np.append(idx, len(tr)))
    assert (recs["off"][:, [W.A, W.B, W.OUT]] == 0).all()
    crit = np.full(len(recs), -1, np.int64)
    last_w, readers = {}, {}
    ops, bufs = recs["op"], recs["buf"]
    for i in range(len(recs)):
        ins = [int(bufs[i, W.A])] + ([int(bufs[i, W.B])] if ops[i] in (W.OP_ADD, W.OP_MUL) else [])
        o = int(bufs[i, W.OUT])
        deps = {last_w[x] for x in ins + [o] if x in last_w}
        deps.update(readers.get(o, ()))
        if deps:
            dl = np.fromiter(deps, np.int64, len(deps))
            crit[i] = dl[np.argmax(done1[dl])]
        for x in ins:
            readers.setdefault(x, []).append(i)
        last_w[o] = i
        readers[o] = []
    k, path = int(np.argmax(done1)), []
    while k >= 0:
        path.append(k)
        k = int(crit[k])
    q = np.asarray(path[::-1][1:], np.int64)
    c = crit[q]
    us = 1e-2
    hop = (done1[q] - done1[c]) * us
    ph = {"claim_late": np.maximum(0, claim0[q] - done1[c]) * us,
          "detect": (ready0[q] - np.maximum(done1[c], claim0[q])) * us,
          "spread": (ready1[q] - ready0[q]) * us,
          "tail": (done1[q] - ready1[q]) * us}
    span = (done1.max() - claim0.min()) * us
    out = {"span_us": float(span), "hops": int(len(q)), "hop_us_mean": float(hop.mean()),
           "hop_us_p50": float(np.median(hop)), "path_share_of_span": float(hop.sum() / span),
           "claimed_after_dependency_done": float((claim0[q] > done1[c]).mean()),
           "phases_us_mean": {k2: float(v.mean()) for k2, v in ph.items()},
           "units_mean_on_path": float(nunits[q].mean()), "units_mean_all": float(nunits.mean())}
    by_units = {}
    for lo, hi in ((1, 1), (2, 4), (5, 16), (17, 1 << 30)):
        m = (nunits[q] >= lo) & (nunits[q] <= hi)
        if m.any():
            key = str(lo) if lo == hi else (f"{lo}-{hi}" if hi < (1 << 30) else f"{lo}+")
            by_units[key] = {"hops": int(m.sum()), "hop_us_mean": float(hop[m].mean()),
                             **{k2 + "_us_mean": float(v[m].mean()) for k2, v in ph.items()}}
    out["by_units"] = by_units
    names = {W.OP_ADD: "add", W.OP_MUL: "mul", W.OP_RELU: "relu", W.OP_GELU: "gelu"}
    dts = {W.F32: "f32", W.BF16: "bf16"}
    by_op = {}
    for o, on in names.items():
        for dt, dn in dts.items():
            m = (ops[q] == o) & (recs["dtype"][q] == dt)
            if m.any():
                by_op[f"{on}/{dn}"] = {"hops": int(m.sum()), "hop_us_mean": float(hop[m].mean()),
                                       "tail_us_mean": float(ph["tail"][m].mean()),
                                       "share_of_path": float(hop[m].sum() / hop.sum())}
    out["by_op"] = by_op
    return out

def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dag_levels(recs):
    """Depth of the dependency DAG of an element-wise stream under sequential
    semantics (read-after-write, write-after-read, write-after-write).  Every
    access of these streams covers a prefix of one pool tensor, so any two
    accesses to the same tensor overlap and tensor granularity is exact."""
    import workloads as W
    assert (recs["off"][:, [W.A, W.B, W.OUT]] == 0).all()
    last_w, readers = {}, {}
    depth = np.zeros(len(recs), np.int64)
    ops, bufs = recs["op"], recs["buf"]
    for i in range(len(recs)):
        ins = [int(bufs[i, W.A])] + ([int(bufs[i, W.B])] if ops[i] in (W.OP_ADD, W.OP_MUL) else [])
        o = int(bufs[i, W.OUT])
        d = 0
        for t in ins:
            if t in last_w:
                d = max(d, depth[last_w[t]])
        if o in last_w:
            d = max(d, depth[last_w[o]])
        for r in readers.get(o, ()):
            d = max(d, depth[r])
        depth[i] = d + 1
        for t in ins:
            readers.setdefault(t, []).append(i)
        last_w[o] = i
        readers[o] = []
    return int(depth.max())


def torch_eager_calls(recs, pool, nmax):
    """The pages' eager baseline: each descriptor as the PyTorch op a framework
    would call, on views of the same device pool (one op call per descriptor;
    out= variants where torch has them).  Only for streams whose ops all map
    onto single torch ops (element-wise and row ops); None otherwise."""
    import functools
    import torch
    import torch.nn.functional as F
    import workloads as W
    TD = {W.F32: torch.float32, W.BF16: torch.bfloat16}

    def view(r, role, count):
        b, off = int(r["buf"][role]), int(r["off"][role])
        es = W.DTYPE_BYTES[int(r["dtype"])]
        return pool.tensors[b][off: off + count * es].view(TD[int(r["dtype"])])

    calls = []
    for r in recs[:nmax]:
        op, n, h = int(r["op"]), int(r["size"]), int(r["dim"][0])
        P = functools.partial
        if op in (W.OP_ADD, W.OP_MUL):
            fn = torch.add if op == W.OP_ADD else torch.mul
            calls.append(P(fn, view(r, W.A, n), view(r, W.B, n), out=view(r, W.OUT, n)))
        elif op == W.OP_RELU:
            calls.append(P(torch.clamp, view(r, W.A, n), min=0, out=view(r, W.OUT, n)))
        elif op == W.OP_GELU:
            calls.append(P(torch.ops.aten.gelu.out, view(r, W.A, n), approximate="tanh", out=view(r, W.OUT, n)))
        elif op in (W.OP_SUM, W.OP_MAX, W.OP_MIN):
            fn = {W.OP_SUM: torch.sum, W.OP_MAX: torch.amax, W.OP_MIN: torch.amin}[op]
            calls.append(P(fn, view(r, W.A, n * h).view(n, h), 1, out=view(r, W.OUT, n)))
        elif op == W.OP_SOFTMAX:
            calls.append(P(torch.ops.aten._softmax.out, view(r, W.A, n * h).view(n, h), 1, False,
                           out=view(r, W.OUT, n * h).view(n, h)))
        elif op == W.OP_LAYERNORM:
            x, o = view(r, W.A, n * h).view(n, h), view(r, W.OUT, n * h).view(n, h)
            g, b, eps = view(r, W.AUX0, h), view(r, W.AUX1, h), float(r["fparam"][0])
            calls.append(lambda x=x, o=o, g=g, b=b, eps=eps, h=h: o.copy_(F.layer_norm(x, (h,), g, b, eps)))
        else:
            return None
    return calls


def make_stream(name):
    import workloads as W
    fill = "host"
    if name == "elementwise":
        s = W.make_elementwise()
        desc = ("element-wise micro-op stream: 100,000 descriptors over 32 fp32 + 32 bf16 tensors of 65536 "
                "values N(0,1); n log-uniform in [256, 65536]; op uniform over {add, mul, relu, gelu(tanh)}; "
                "10% in place; bursts of 1-64")
    elif name == "pr1":
        s = W.make_pr1()
        s.bursts = np.full(len(s) // 8, 8)
        desc = ("PR1: 1,000 fp32 descriptors over 16 vectors of 4096 values U[-1,1]; op uniform over "
                "{add, mul, relu}; operands and outputs uniform over the pool")
    elif name in ("copy", "copy64"):
        parts = 1 if name == "copy" else 64
        s = W.Stream(name, [W.Buffer("src", W.F32, 1 << 28, ("uniform", -1.0, 1.0), 77), W.Buffer("dst", W.F32, 1 << 28, ("zeros",))],
                     np.zeros(parts, W.REC_DTYPE), np.array([parts]))
        s.recs["buf"] = -1
        s.recs["op"] = W.OP_COPY
        s.recs["size"] = (1 << 30) // parts
        s.recs["buf"][:, W.A], s.recs["buf"][:, W.OUT] = 0, 1
        s.recs["off"][:, W.A] = np.arange(parts) * ((1 << 30) // parts)
        s.recs["off"][:, W.OUT] = s.recs["off"][:, W.A]
        fill = "device"
        desc = ("one 1 GiB copy descriptor (counter calibration: 1 GiB read + 1 GiB written)" if parts == 1 else
                "1 GiB copied by 64 independent descriptors of 16 MiB")
    elif name == "rows":
        s, fill = W.make_rows(), "device"
        desc = ("row ops: 50,000 descriptors of [r, h] fp32, r in {1,2,...,64}, h in {768,1024,2048,4096}, "
                "x ~ N(0,2) from a 2 GiB pool; op uniform over {sum, max, min, softmax, LayerNorm}")
    elif name == "decode":
        s, fill = W.make_decode(steps=2000), "device"
        desc = ("attention decoding: 2,000 decode steps x 32 layers x {RoPE(theta 1e4), KV append, SDPA}; "
                "B in {1,2,4,8}, 32 heads x 128, bf16 KV cache 4096/sequence, L in [128, 4096] +1 per step")
    elif name == "decode_gqa":
        s, fill = W.make_decode(steps=2000, kv_heads=8), "device"
        desc = ("attention decoding with grouped-query attention: 2,000 decode steps x 32 layers x {RoPE(theta 1e4), "
                "KV append, SDPA}; B in {1,2,4,8}, 32 query heads sharing 8 key/value heads x 128, bf16 KV cache "
                "4096/sequence, L in [128, 4096] +1 per step")
    elif name == "decode_paged":
        s, fill = W.make_decode(steps=2000, page_size=64), "device"
        desc = ("attention decoding on paged KV caches: the decode stream (2,000 steps x 32 layers x {RoPE, KV "
                "append, SDPA}, B in {1,2,4,8}, 32 heads x 128, L in [128, 4096]) with each layer's caches in pages "
                "of 64 positions placed at random through a block table per layer")
    elif name == "matmul":
        s, fill = W.make_matmul(), "device"
        desc = ("small matmuls of batched decoding on the matrix cores: 32 tokens through the QKV (1024->3072), "
                "up (1024->3072) and down (3072->1024) projections of 32 layers, bf16, weights [out, in] N(0,0.02) "
                "(604 MB), 20 passes (1,920 independent descriptors)")
    elif name == "mixed":
        s, fill = W.make_mixed(tokens=500), "device"
        desc = ("mixed decode pipeline: 500 tokens x 32 layers x 11 ops at hidden 1024, 8 heads x 128, bf16: "
                "LN, GEMV 1x1024.1024x3072, RoPE, KV append, SDPA (L in [64, 2048]), add, LN, GEMV 1024x3072, "
                "GELU, GEMV 3072x1024, add")
    else:
        raise SystemExit(f"unknown workload {name}")
    return s, desc, fill


WAVES_DEFAULT = {"elementwise": 2, "rows": 4, "decode": 4, "decode_gqa": 4, "decode_paged": 4, "copy": 4, "copy64": 4, "matmul": 4}
UPW_DEFAULT = {"decode": 2, "decode_gqa": 2, "decode_paged": 2, "rows": 2}
# the workloads reported beside the headline in a default run, with the
# steps each times (the decode and mixed streams run about 1-2 s per step)
SUB_WORKLOADS = ("pr1", "rows", "decode", "decode_gqa", "decode_paged", "mixed", "matmul")
SUB_STEPS = {"pr1": 20, "rows": 10, "decode": 2, "decode_gqa": 3, "decode_paged": 2, "mixed": 3, "matmul": 10}


def host_cpu():
    """Core count and CPU model of this host (the oracle leg's machine)."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "usable_cpus": len(os.sched_getaffinity(0)), "model": model}


def cpu_oracle(stream, recs, arrays, fill, budget_s):
    """The oracle on a bounded prefix of the same stream, grown until it
    takes about budget_s, on one host core (the process is pinned to one
    CPU for the duration).  Host-filled streams use the same inputs as the
    GPU; device-filled ones (pools of GiBs) use zero-filled host buffers of
    the same shapes, which leaves the oracle's work (every op runs the same
    loops whatever the values) unchanged."""
    import oracle
    nd = len(recs)
    if fill == "host":
        def make_pool():
            return oracle.Pool([a.copy() for a in arrays])
        n_cpu, what = min(nd, 1000), "the same inputs"
    else:
        def make_pool():
            return oracle.Pool([np.zeros(b.nbytes, np.uint8) for b in stream.buffers])
        n_cpu, what = min(nd, 8), "zero-filled host buffers of the stream's shapes"
    before = os.sched_getaffinity(0)
    core = min(before)
    os.sched_setaffinity(0, {core})
    try:
        while True:
            p = make_pool()
            ta = time.perf_counter()
            p.run(recs[:n_cpu])
            el = time.perf_counter() - ta
            del p
            if el > budget_s or n_cpu >= nd:
                break
            n_cpu = min(nd, n_cpu * (4 if el < budget_s / 5 else 2))
    finally:
        os.sched_setaffinity(0, before)
    hc = host_cpu()
    return {"value": n_cpu / el, "unit": "micro-ops/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n_cpu} of {nd} descriptors of the same stream on {what}, sequential C "
                      f"oracle (fp64), one thread pinned to CPU {core}, {el:.1f} s",
            "host_nproc": hc["nproc"], "host_cpu_model": hc["model"]}


def run_workload(name, steps, warmup, waves=0, units_per_wave=0, ring=512, num_wgs=0, backoff=0,
                 headline=False, baselines=True, cpu_budget_s=10.0, gemm=False, probe=None):
    """Time `steps` executor launches over one workload's stream (after
    `warmup` untimed ones) and measure its closed-loop latency, roofline,
    baselines and CPU oracle.  Returns the record (the headline adds the
    dispatch micro-benchmarks, size buckets and injection figures)."""
    import torch

    import workloads as W
    from persistent_micro_dispatch_amd import gpuos as G
    from workloads.gpu import DevicePool, to_descs

    waves = waves or WAVES_DEFAULT.get(name, 1)
    units_per_wave = units_per_wave or UPW_DEFAULT.get(name, 1)
    stream, wdesc, fill = make_stream(name)
    recs = stream.recs
    nd = len(recs)
    log(f"workload {name}: {nd} descriptors, {len(stream.bursts)} bursts, fill={fill}")
    arrays = [b.host_bytes() for b in stream.buffers] if fill == "host" else None
    pool = DevicePool(arrays) if fill == "host" else DevicePool.from_stream(stream, fill="device")
    descs = to_descs(recs, pool.ptrs)
    bursts = np.asarray(stream.bursts, np.uint32)
    step_bytes = int(W.algorithmic_bytes(recs).sum())

    # buffers of the dependent-chain test are made now: while the executor is
    # resident no other kernel is launched (a profiler that serialises
    # dispatches would otherwise queue it behind the executor)
    chain_buf = torch.zeros(256, dtype=torch.float32, device="cuda")
    one_buf = torch.ones(256, dtype=torch.float32, device="cuda")
    torch.cuda.current_stream().synchronize()
    ctx = G.gpuos_init(waves_per_wg=waves, ring_entries=ring, num_wgs=num_wgs,
                       units_per_wave=units_per_wave, backoff_max=backoff)
    assert G.gpuos_pause(ctx, 30_000_000_000) == 0
    st0 = G.gpuos_stats_get(ctx)

    def one_step():
        assert G.gpuos_resume(ctx) == 0
        rc, first, n = G.gpuos_submit_bursts(ctx, descs, bursts, G.GPUOS_SUBMIT_BLOCK)
        assert rc == 0 and n == nd, (rc, n)
        rc, es, stc = G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 300_000_000_000)
        assert rc == 0, (rc, es, stc)
        assert G.gpuos_pause(ctx, 30_000_000_000) == 0
        return G.gpuos_stats_get(ctx)["last_launch_ms"]

    for i in range(warmup):
        one_step()
        log(f"{name}: warmup step {i} done")
    st_w = G.gpuos_stats_get(ctx)
    launch_ms = []
    t0 = time.perf_counter()
    for i in range(steps):
        launch_ms.append(one_step())
        log(f"{name}: step {i}: executor launch {launch_ms[-1]:.2f} ms")
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps
    ops_per_s = nd * steps / (t1 - t0)
    st = G.gpuos_stats_get(ctx)
    extra = {}

    # ---- co-running GEMM: a bf16 8192^3 loop on its own stream, alone and
    # while the micro-op stream runs
    if gemm:
        gs = torch.cuda.Stream()
        with torch.cuda.stream(gs):
            a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
            b = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
            c = torch.empty(8192, 8192, device="cuda", dtype=torch.bfloat16)
            torch.matmul(a, b, out=c)
        gs.synchronize()
        n_gemm = 40
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(gs):
            e0.record(gs)
            for _ in range(n_gemm):
                torch.matmul(a, b, out=c)
            e1.record(gs)
        gs.synchronize()
        gemm_alone_ms = e0.elapsed_time(e1) / n_gemm
        # enough GEMMs to cover about two seconds, so that the steps timed
        # beside them run while they do
        n_gemm = max(n_gemm, int(2000.0 / gemm_alone_ms))
        with torch.cuda.stream(gs):
            e0.record(gs)
            for _ in range(n_gemm):
                torch.matmul(a, b, out=c)
            e1.record(gs)
        tc0 = time.perf_counter()
        k_co = 0
        capped = False
        while not e1.query():
            one_step()
            k_co += 1
            log(f"{name}: step {k_co} beside the GEMMs")
            # with an executor wave on every CU no GEMM workgroup fits, and
            # the GEMMs only advance between launches: stop after CORUN_CAP_S
            if time.perf_counter() - tc0 > CORUN_CAP_S:
                capped = True
                log(f"{name}: GEMMs still queued after {CORUN_CAP_S:.0f} s of steps; stopping the steps")
                break
        tc1 = time.perf_counter()
        gs.synchronize()
        gemm_co_ms = e0.elapsed_time(e1) / n_gemm
        flop = 2.0 * 8192 ** 3
        extra.update({
            "gemm_tflops_alone": flop / (gemm_alone_ms * 1e-3) / 1e12,
            "gemm_tflops_corun": flop / (gemm_co_ms * 1e-3) / 1e12,
            "gemm_retained": gemm_alone_ms / gemm_co_ms,
            "corun_steps": k_co,
            "corun_capped": capped,  # the GEMMs outlasted the steps: their time includes a tail run alone
            "ops_per_s_with_gemm": nd * k_co / (tc1 - tc0) if k_co else None,
        })
        del a, b, c
        log(f"gemm alone {gemm_alone_ms:.3f} ms, co-run {gemm_co_ms:.3f} ms; {k_co} steps during the GEMMs")

    # ---- closed-loop latency: one descriptor at a time, waited for
    # (measured inside the library, as a C caller sees it; the same loop
    # through the Python binding adds its call overhead, reported beside)
    assert G.gpuos_resume(ctx) == 0
    nlat = min(nd, 2000 if headline else 500)
    lat = G.gpuos_latency_bench(ctx, descs[:nlat])
    lat_py = None
    nop_s = chain_s = None
    buckets = injection = jit_in = None
    chain = nop = None
    if headline:
        lat_py = np.zeros(min(nlat, 500))
        for i in range(len(lat_py)):
            ta = time.perf_counter_ns()
            rc, f = G.gpuos_submit(ctx, descs[i:i + 1], G.GPUOS_SUBMIT_BLOCK)
            rc2 = G.gpuos_sync(ctx, f, 10_000_000_000)[0]
            lat_py[i] = (time.perf_counter_ns() - ta) / 1e3
            assert rc == 0 and rc2 == 0
        # ---- dispatch micro-benchmarks: NOP stream (bursts of 64) and a chain
        nop = G.new_descs(100_000)
        nb = np.full(len(nop) // 64, 64, np.uint32)
        ta = time.perf_counter()
        rc, _, _ = G.gpuos_submit_bursts(ctx, nop, nb, G.GPUOS_SUBMIT_BLOCK)
        assert rc == 0 and G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 60_000_000_000)[0] == 0
        nop_s = time.perf_counter() - ta
        chain = G.new_descs(5000)
        chain["op_id"] = G.GPUOS_OP_ADD
        chain["flags"] = G.flags(G.GPUOS_F32)
        chain["size"] = 256
        chain["input_a"] = chain["output"] = chain_buf.data_ptr()
        chain["input_b"] = one_buf.data_ptr()
        ta = time.perf_counter()
        rc, _, _ = G.gpuos_submit_bursts(ctx, chain, np.full(len(chain) // 50, 50, np.uint32), G.GPUOS_SUBMIT_BLOCK)
        assert rc == 0 and G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 60_000_000_000)[0] == 0
        chain_s = time.perf_counter() - ta
    # ---- element-wise throughput per log2-size bucket: the bucket's
    # descriptors in stream order, once with hazard ordering and once as
    # independent ops (NOHAZARD; outputs race, nothing reads them after)
    if headline and name in ("elementwise", "pr1"):
        buckets = {}
        lg = np.minimum(np.floor(np.log2(recs["size"])).astype(np.int64), 15)
        per_op = W.algorithmic_bytes(recs)
        for b in range(int(lg.min()), int(lg.max()) + 1):
            idx = np.nonzero(lg == b)[0]
            if len(idx) < 64:
                continue
            sub = descs[idx].copy()
            nbk = np.full(len(sub) // 64, 64, np.uint32)
            rem = len(sub) - int(nbk.sum())
            if rem:
                nbk = np.append(nbk, np.uint32(rem))
            row = {"descriptors": int(len(idx)), "bytes_per_op": float(per_op[idx].mean())}
            for key, fl in (("ordered", G.GPUOS_SUBMIT_BLOCK),
                            ("independent", G.GPUOS_SUBMIT_BLOCK | G.GPUOS_SUBMIT_NOHAZARD)):
                ta = time.perf_counter()
                rc, _, _ = G.gpuos_submit_bursts(ctx, sub, nbk, fl)
                assert rc == 0 and G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 60_000_000_000)[0] == 0
                el = time.perf_counter() - ta
                row[key + "_ops_per_s"] = len(idx) / el
                row[key + "_gbs"] = float(per_op[idx].sum()) / el / 1e9
            buckets[f"2^{b}"] = row
    # ---- injected operator (an element-wise program bound by a table flip):
    # registration latency, and add/mul descriptors of the stream run as
    # built-in ops and as the program a+b / a*b (independent ops)
    if headline and name == "elementwise":
        sel = np.nonzero((recs["op"] == W.OP_ADD) | (recs["op"] == W.OP_MUL))[0][:20000]
        sub = descs[sel].copy()
        nbk = np.full(len(sub) // 64, 64, np.uint32)
        sub = sub[:int(nbk.sum())]
        fl = G.GPUOS_SUBMIT_BLOCK | G.GPUOS_SUBMIT_NOHAZARD
        X, P = W.xins, W.program
        progs = {W.OP_ADD: P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_ADD, 0, 1, 2)]),
                 W.OP_MUL: P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_MUL, 0, 1, 2)])}
        # bound while the executor is paused: the table copy is a separate
        # dispatch, which a profiler that serialises dispatches would queue
        # behind a resident executor (binding during execution is tested)
        assert G.gpuos_pause(ctx, 30_000_000_000) == 0
        t_reg = []
        for i in range(20):
            ta = time.perf_counter_ns()
            assert G.gpuos_register_expr(ctx, 200 + (i & 1), progs[W.OP_ADD if i & 1 else W.OP_MUL]) == 0
            t_reg.append((time.perf_counter_ns() - ta) / 1e3)
        assert G.gpuos_register_expr(ctx, 200, progs[W.OP_ADD]) == 0
        assert G.gpuos_register_expr(ctx, 201, progs[W.OP_MUL]) == 0
        assert G.gpuos_resume(ctx) == 0
        by = float(W.algorithmic_bytes(recs[sel[:len(sub)]]).sum())
        row = {"register_us_p50": float(np.median(t_reg)), "descriptors": int(len(sub)),
               "bytes_per_op": by / max(1, len(sub))}
        for key, ids in (("builtin", None), ("program", (200, 201))):
            dd = sub.copy()
            if ids:
                dd["op_id"] = np.where(dd["op_id"] == W.OP_ADD, ids[0], ids[1]).astype(np.uint32)
            ta = time.perf_counter()
            rc, _, _ = G.gpuos_submit_bursts(ctx, dd, nbk, fl)
            assert rc == 0 and G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 60_000_000_000)[0] == 0
            el = time.perf_counter() - ta
            row[key + "_ops_per_s"] = len(sub) / el
            row[key + "_gbs"] = by / el / 1e9
        injection = row
        jit_in = (sub, nbk, by)
    assert G.gpuos_pause(ctx, 30_000_000_000) == 0
    chain_ok = float(chain_buf.cpu()[0]) == 5000.0 if headline else None

    if baselines:
        # ---- eager: one hipLaunchKernel per descriptor (same op bodies) on
        # a torch stream
        s_eager = torch.cuda.Stream()
        nb_e = min(nd, 20_000 if headline else 5_000)
        scratch_b = G.gpuos_eager_scratch_bytes(descs[:nb_e])
        scratch = torch.zeros(scratch_b, dtype=torch.uint8, device="cuda")
        torch.cuda.current_stream().synchronize()
        sp = s_eager.cuda_stream
        assert G.gpuos_eager_submit(descs[:min(nd, 200)], sp, scratch.data_ptr(), scratch_b) == 0
        s_eager.synchronize()
        ta = time.perf_counter()
        assert G.gpuos_eager_submit(descs[:nb_e], sp, scratch.data_ptr(), scratch_b) == 0
        s_eager.synchronize()
        eager_s = time.perf_counter() - ta
        eager_lat = np.zeros(min(nd, 500))
        for i in range(len(eager_lat)):
            ta = time.perf_counter_ns()
            assert G.gpuos_eager_submit(descs[i:i + 1], sp, scratch.data_ptr(), scratch_b) == 0
            s_eager.synchronize()
            eager_lat[i] = (time.perf_counter_ns() - ta) / 1e3
        # ---- hipGraph: captured per burst; stable = replay prebuilt graphs,
        #      variable = capture + instantiate + launch for every burst
        ng = min(len(bursts), 300 if headline else 100)
        offs = np.r_[0, np.cumsum(bursts[:ng])].astype(np.int64)
        ta = time.perf_counter()
        graphs = []
        for i in range(ng):
            ge = G.gpuos_graph_build(descs[offs[i]:offs[i + 1]], sp, scratch.data_ptr(), scratch_b)
            G.gpuos_graph_launch(ge, sp)
            graphs.append(ge)
        s_eager.synchronize()
        var_s = time.perf_counter() - ta
        ta = time.perf_counter()
        for ge in graphs:
            G.gpuos_graph_launch(ge, sp)
        s_eager.synchronize()
        stable_s = time.perf_counter() - ta
        for ge in graphs:
            G.gpuos_graph_destroy(ge)
        gdesc = int(offs[ng])
        # ---- PyTorch eager, the pages' baseline: one torch op per descriptor
        calls = torch_eager_calls(recs, pool, 20_000 if headline else 5_000)
        if calls:
            for c in calls[:200]:
                c()
            torch.cuda.current_stream().synchronize()
            ta = time.perf_counter()
            for c in calls:
                c()
            torch.cuda.current_stream().synchronize()
            torch_rate = len(calls) / (time.perf_counter() - ta)
            extra.update({"torch_eager_ops_per_s": torch_rate, "speedup_vs_torch_eager": ops_per_s / torch_rate})
        extra.update({
            "eager_ops_per_s": nb_e / eager_s,
            "eager_p50_us": float(np.percentile(eager_lat, 50)),
            "speedup_vs_eager": ops_per_s / (nb_e / eager_s),
            "graph_stable_ops_per_s": gdesc / stable_s,
            "graph_variable_ops_per_s": gdesc / var_s,
            "speedup_vs_graph_stable": ops_per_s / (gdesc / stable_s),
        })
        if headline:
            null_async, null_sync = G.gpuos_null_launch_bench(sp, 20000)
            extra.update({"null_launch_us": null_async / 1e3, "null_launch_sync_us": null_sync / 1e3})
        del scratch
    assert G.gpuos_shutdown(ctx) == 0
    if jit_in is not None:
        injection["compiled"] = jit_injection(*jit_in, waves=waves, ring=ring, num_wgs=num_wgs)
    xcd_hops = chain_hops_by_xcd() if headline else None
    cpath = critical_path(recs, descs, bursts, waves, ring, num_wgs, units_per_wave) \
        if headline and name == "elementwise" else None

    # ---- roofline of the executor kernel (one launch = one step)
    mean_launch_ms = float(np.mean(launch_ms))
    achieved = step_bytes / (mean_launch_ms * 1e-3) / 1e9
    tb = recorded_traffic(name if units_per_wave == 1 else f"{name}/upw2")
    roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": tb / (mean_launch_ms * 1e-3) / 1e9 if tb else None,
            "traffic_bytes_per_launch": tb,
            "kernel": "gpuos_executor_s2" if units_per_wave == 2 else "gpuos_executor",
            "launch_ms": mean_launch_ms, "bytes_per_launch": step_bytes}
    if name == "matmul":
        # the matrix cores' own roofline beside the HBM one: the products are
        # bf16 at M = 32 rows per weight element (32 flop per byte of weights)
        tflops = stream.meta["flops"] / (mean_launch_ms * 1e-3) / 1e12
        extra["roofline_mfma"] = {"bound": "mfma", "achieved": tflops, "peak": 2500.0, "unit": "TFLOP/s",
                                  "frac": tflops / 2500.0, "flops_per_launch": stream.meta["flops"]}
    levels = dag_levels(recs) if name in ("elementwise", "pr1") else None
    cpu = cpu_oracle(stream, recs, arrays, fill, cpu_budget_s) if cpu_budget_s > 0 else None

    # host cost over the warmup and timed steps only
    dsub = max(1, st["submitted"] - st0["submitted"])
    steps_total = max(1, steps + warmup)
    rec = {
        "value": ops_per_s,
        "unit": "micro-ops/s",
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "config": {"workload": wdesc, "descriptors_per_step": nd, "waves_per_wg": waves,
                   "num_wgs": st["num_wgs"], "ring_entries": st["ring_entries"],
                   "units_per_wave": units_per_wave, "fill": fill},
        "p50_us": float(np.percentile(lat, 50)),
        "p99_us": float(np.percentile(lat, 99)),
        "stream_gbs": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "dag_levels": levels,
        "us_per_dag_level": ms_per_step * 1e3 / levels if levels else None,
        "units_per_step": (st["units"] - st0["units"]) / steps_total,
        "dep_waits_per_step": (st["dep_waits"] - st0["dep_waits"]) / steps_total,
        "fetch_batches_per_step": (st["fetch_batches"] - st0["fetch_batches"]) / steps_total,
        "host_submit_ns_per_desc": (st["ns_submit"] - st0["ns_submit"]) / dsub,
        "host_blocked_ns_per_desc": (st["ns_blocked"] - st0["ns_blocked"]) / dsub,
        "host_annotate_ns_per_desc": (st["ns_annotate"] - st0["ns_annotate"]) / dsub,
        "timed_steps_host_submit_ns_per_desc": (st["ns_submit"] - st_w["ns_submit"]) / max(1, st["submitted"] - st_w["submitted"]),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if headline:
        rec.update({
            "p50_us_python": float(np.percentile(lat_py, 50)),
            "dispatch_interval_us_nop": nop_s / len(nop) * 1e6,
            "dependent_chain_us_per_op": chain_s / len(chain) * 1e6,
            "dependent_chain_ok": chain_ok,
            "size_buckets": buckets,
            "injection": injection,
            "chain_hops_by_xcd": xcd_hops,
            "critical_path": cpath,
        })
    rec.update(extra)
    del pool, descs, chain_buf, one_buf
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="elementwise")
    ap.add_argument("--waves", type=int, default=0,
                    help="wave64s per workgroup (one workgroup per CU); 0: 4 for rows, decode, decode_gqa "
                         "and copy, else 1")
    ap.add_argument("--ring", type=int, default=512,
                    help="ring entries: descriptors in flight, which is also the window of hazard tracking")
    ap.add_argument("--units-per-wave", type=int, default=0, choices=(0, 1, 2),
                    help="units a worker wave holds at once (2 lets a ready unit overtake a waiting one); "
                         "0: 2 for decode, decode_gqa and rows, else 1")
    ap.add_argument("--num-wgs", type=int, default=0,
                    help="executor workgroups (0: one per CU); fewer leave whole CUs to other kernels")
    ap.add_argument("--backoff", type=int, default=0,
                    help="s_sleep cap of idle waits, 1..127 (0: the library's default)")
    ap.add_argument("--gemm", action="store_true", help="co-run a bf16 8192^3 GEMM loop")
    ap.add_argument("--no-baselines", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-sub", action="store_true",
                    help="skip the other workloads' records (pr1, rows, decode, decode_gqa, mixed)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the dispatcher is a "
              "single-device path; the design notes describe how it would shard.", file=sys.stderr)
        sys.exit(2)

    import torch

    from persistent_micro_dispatch_amd import gpuos as G

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    # achievable HBM bandwidth with the op bodies' memory instructions (1 GiB
    # read and copy), measured before the executor is resident
    pb = 1 << 30
    p_src = torch.empty(pb, dtype=torch.uint8, device="cuda").fill_(7)
    p_dst = torch.empty(pb, dtype=torch.uint8, device="cuda")
    torch.cuda.current_stream().synchronize()
    sp0 = torch.cuda.current_stream().cuda_stream
    hbm_probe = {"bytes": pb,
                 "read_gbs": G.gpuos_hbm_probe(p_src.data_ptr(), p_dst.data_ptr(), pb, 0, 5, sp0),
                 "copy_gbs": G.gpuos_hbm_probe(p_src.data_ptr(), p_dst.data_ptr(), pb, 1, 5, sp0)}
    # bandwidth against the number of active CUs: one workgroup (four waves,
    # 64 KiB of loads in flight) per CU; by Little's law the latency is
    # in-flight bytes / bandwidth while few CUs are active, and the bytes in
    # flight per CU that half of the peak needs follow from it
    sweep = []
    sb = 256 << 20
    for wg in (8, 16, 32, 64, 128, 256):
        sweep.append({"workgroups": wg,
                      "read_gbs": G.gpuos_hbm_probe_grid(p_src.data_ptr(), p_dst.data_ptr(), sb, 0, 3, wg, sp0),
                      "copy_gbs": G.gpuos_hbm_probe_grid(p_src.data_ptr(), p_dst.data_ptr(), sb, 1, 3, wg, sp0)})
    inflight_wg = 256 * 16 * 16
    lat_s = sweep[0]["workgroups"] * inflight_wg / (sweep[0]["read_gbs"] * 1e9)
    half = next((p["workgroups"] for p in sweep if p["read_gbs"] >= HBM_PEAK_GBS / 2), None)
    hbm_probe.update({"sweep_bytes": sb, "sweep": sweep, "inflight_bytes_per_workgroup": inflight_wg,
                      "latency_us_little": lat_s * 1e6,
                      "inflight_bytes_per_cu_for_half_peak": HBM_PEAK_GBS / 2 * 1e9 * lat_s / 256,
                      "cus_reaching_half_peak": half})
    del p_src, p_dst
    torch.cuda.current_stream().synchronize()
    torch.cuda.empty_cache()
    log(f"hbm probe: read {hbm_probe['read_gbs']:.0f} GB/s, copy {hbm_probe['copy_gbs']:.0f} GB/s")

    head = run_workload(args.workload, args.steps, args.warmup, waves=args.waves,
                        units_per_wave=args.units_per_wave, ring=args.ring, num_wgs=args.num_wgs,
                        backoff=args.backoff, headline=True, baselines=not args.no_baselines,
                        cpu_budget_s=0.0 if args.no_cpu else 10.0, gemm=args.gemm)
    subs = {}
    if not args.no_sub and args.workload == "elementwise":
        for name in SUB_WORKLOADS:
            k = min(args.steps, SUB_STEPS[name])
            subs[name] = run_workload(name, k, 1, baselines=not args.no_baselines,
                                      cpu_budget_s=0.0 if args.no_cpu else 4.0)
            log(f"{name}: {subs[name]['value']:.0f} micro-ops/s, {subs[name]['ms_per_step']:.2f} ms per step")
        # the mixed pipeline beside a bf16 8192^3 GEMM loop, with the executor
        # on 64 workgroups of two waves (the rest of the chip left to the GEMM)
        subs["mixed_with_gemm"] = run_workload("mixed", 1, 1, waves=2, num_wgs=64, baselines=False,
                                               cpu_budget_s=0.0, gemm=True)
    out = {
        "metric": "micro-ops/sec (+ p50 per-op latency us, vs per-op hipLaunch; HBM GB/s frac)",
        "value": head.pop("value"),
        "unit": head.pop("unit"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 (bf16 operands computed in f32)",
        "data": "synthetic",
        "config": head.pop("config"),
    }
    head.pop("steps")
    head.pop("warmup")
    out.update(head)
    out["hbm_probe"] = hbm_probe
    out["host_cpu"] = host_cpu()
    if subs:
        out["workloads"] = subs
    print(json.dumps(out))


if __name__ == "__main__":
    main()
