"""Run symbolic records on the GPU through the C ABI and on the oracle, and
compare outputs with the per-op metrics of parity.py."""
from __future__ import annotations

import sys
from typing import List, Sequence

import numpy as np

import oracle
import workloads as W
from parity import TOL, as_float, bits_equal, rel_check, ulp_bf16
from persistent_micro_dispatch_amd import gpuos as G
from workloads.gpu import DevicePool, split_bursts, to_descs

SYNC_NS = 120_000_000_000


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_gpu(arrays: Sequence[np.ndarray], recs: np.ndarray, bursts=None, flags=G.GPUOS_SUBMIT_BLOCK,
            ctx=None, **init) -> List[np.ndarray]:
    """Upload arrays, submit recs, sync, download every buffer (uint8)."""
    pool = DevicePool(arrays)
    descs = to_descs(recs, pool.ptrs)
    own = ctx is None
    if own:
        ctx = G.gpuos_init(**init)
    try:
        if bursts is None:
            bursts = np.full((len(descs) + 63) // 64, 64)
        for sl in split_bursts(len(descs), np.asarray(bursts)):
            if sl.stop <= sl.start:
                continue
            rc, _ = G.gpuos_submit(ctx, descs[sl], flags)
            assert rc == 0, f"submit: {G.ERR_NAMES.get(rc)}"
        rc, es, st = G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, SYNC_NS)
        assert rc == 0, f"sync: {G.ERR_NAMES.get(rc)} seq={es} status={st}"
        out = [pool.download(i) for i in range(len(arrays))]
    finally:
        if own:
            assert G.gpuos_shutdown(ctx) == 0
    return out


def run_oracle(arrays: Sequence[np.ndarray], recs: np.ndarray) -> List[np.ndarray]:
    p = oracle.Pool([np.array(a, copy=True) for a in arrays])
    p.run(recs)
    return p.arrays


def _f(buf: np.ndarray, off: int, n: int, dt: int) -> np.ndarray:
    es = W.DTYPE_BYTES[dt]
    return as_float(buf[off: off + n * es].copy(), dt)


def check_record(r, inputs: List[np.ndarray], gpu: List[np.ndarray], orc: List[np.ndarray]) -> dict:
    """Compare the outputs of one record (its inputs are `inputs`, the pool
    before it ran).  Returns a dict with 'ok' and details."""
    op = int(r["op"])
    dt, do = int(r["dtype"]), int(r["out_dtype"])
    size = int(r["size"])
    d = [int(v) for v in r["dim"]]
    buf, off = r["buf"], r["off"]
    res = {"op": W.OP_NAMES[op], "ok": True, "worst": 0.0}
    exact = op in (W.OP_NOP, W.OP_ADD, W.OP_MUL, W.OP_RELU, W.OP_MAX, W.OP_MIN, W.OP_KV_APPEND, W.OP_COPY)
    if op == W.OP_EXPR:
        pw = inputs[int(buf[W.AUX2])][int(off[W.AUX2]): int(off[W.AUX2]) + 4 * d[2]].copy().view(np.uint32)
        exact = W.program_is_exact(pw)
    tol = TOL["f32"] if do == W.F32 else TOL["bf16"]
    for (b, o, nbytes) in W.output_ranges(r):
        g = gpu[b][o: o + nbytes]
        rr = orc[b][o: o + nbytes]
        if exact or op == W.OP_COPY:
            if op in (W.OP_KV_APPEND, W.OP_COPY):
                eq = g == rr
            else:
                eq = bits_equal(g.copy(), rr.copy(), do)
            if not eq.all():
                res.update(ok=False, mismatches=int((~eq).sum()))
            continue
        gf, rf = as_float(g.copy(), do if op != W.OP_ROPE else dt), as_float(rr.copy(), do if op != W.OP_ROPE else dt)
        extra = ulp_bf16(rf) if (do == W.BF16 and op != W.OP_ROPE) else 0.0
        if op == W.OP_GELU:
            denom = np.maximum(np.abs(rf), 2.0 ** -126)
            ok, worst = rel_check(gf, rf, denom + extra / tol, tol)
        elif op == W.OP_SOFTMAX:
            ok, worst = rel_check(gf, rf, np.abs(rf) + extra / tol, tol)
        elif op in (W.OP_LAYERNORM, W.OP_EXPR):
            # EXPR with exp/log/tanh/sigmoid steps: library functions within a
            # few ulps, compared on the unit scale like LayerNorm
            ok, worst = rel_check(gf, rf, np.maximum(np.abs(rf), 1.0) + extra / tol, tol)
        elif op == W.OP_SUM:
            h = d[0]
            x = _f(inputs[int(buf[W.A])], int(off[W.A]), size * h, dt).reshape(size, h)
            ok, worst = rel_check(gf, rf, np.abs(x).sum(axis=1) + extra / tol, tol)
        elif op == W.OP_ROPE:
            # within one bf16 ulp (or 2^-23 relative for fp32) of the oracle
            if dt == W.BF16:
                ok = np.abs(gf - rf) <= ulp_bf16(rf) * 1.0001
                ok |= np.isnan(gf) & np.isnan(rf)
                worst = float(np.max(np.abs(gf - rf) / ulp_bf16(rf))) if gf.size else 0.0
            else:
                ok, worst = rel_check(gf, rf, np.maximum(np.abs(rf), 1e-30), 2.0 ** -22)
        elif op == W.OP_SDPA:
            H, D, C = d[0], d[1], d[2]
            Hkv = d[3] or H  # grouped-query attention: kv head h // (H // Hkv)
            q = _f(inputs[int(buf[W.A])], int(off[W.A]), size * H * D, dt).reshape(size, H, D)
            K = _f(inputs[int(buf[W.AUX0])], int(off[W.AUX0]), size * Hkv * C * D, dt).reshape(size, Hkv, C, D)
            V = _f(inputs[int(buf[W.AUX1])], int(off[W.AUX1]), size * Hkv * C * D, dt).reshape(size, Hkv, C, D)
            K, V = np.repeat(K, H // Hkv, axis=1), np.repeat(V, H // Hkv, axis=1)
            denom = np.zeros((size, H, D))
            scale = float(r["fparam"][1]) or 1.0 / np.sqrt(D)
            for bb in range(size):
                L = int(r["lens"][bb])
                s = np.einsum("hd,hjd->hj", q[bb], K[bb, :, :L]) * scale
                p = np.exp(s - s.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                denom[bb] = np.einsum("hj,hjd->hd", p, np.abs(V[bb, :, :L]))
            t = TOL["sdpa"] if do == W.F32 else TOL["bf16"]
            ok, worst = rel_check(gf, rf, denom.reshape(-1) + extra / t, t)
        elif op == W.OP_GEMV:
            K_, N_ = d[0], d[1]
            x = _f(inputs[int(buf[W.A])], int(off[W.A]), K_, dt)
            Wm = _f(inputs[int(buf[W.B])], int(off[W.B]), K_ * N_, dt).reshape(K_, N_)
            denom = np.abs(x) @ np.abs(Wm)
            t = TOL["f32"] if do == W.F32 else TOL["bf16"]
            ok, worst = rel_check(gf, rf, denom + extra / t, t)
        else:
            raise AssertionError(op)
        res["worst"] = max(res["worst"], worst)
        if not np.all(ok):
            res.update(ok=False, mismatches=int((~ok).sum()))
    return res


def untouched_equal(recs, gpu, orc) -> bool:
    """Bytes that no record writes must be bit-identical (no stray writes)."""
    masks = [np.ones(len(a), bool) for a in gpu]
    for r in recs:
        for (b, o, n) in W.output_ranges(r):
            masks[b][o: o + n] = False
    return all(np.array_equal(g[m], o[m]) for g, o, m in zip(gpu, orc, masks))


# --------------------------------------------------------------------------
# Verify mode: record every output on the GPU, replay on the oracle with
# teacher forcing (compare each op's output with the oracle's result from the
# same inputs, then adopt the GPU's bytes so differences never cascade).
# --------------------------------------------------------------------------
def with_log(recs: np.ndarray, n_arrays: int):
    """Insert after each logged record a COPY of each output range into a log
    buffer (index n_arrays).  KV appends are not logged (bit copies, checked
    on the final pool).  Returns (augmented records, log layout, log bytes)."""
    from oracle_util import rec as mkrec
    out, layout, pos = [], [], 0
    for k, r in enumerate(recs):
        out.append(r.reshape(1))
        if int(r["op"]) in (W.OP_NOP, W.OP_COPY, W.OP_KV_APPEND):
            continue
        for (b, o, n) in W.output_ranges(r):
            out.append(mkrec(W.OP_COPY, size=n, a=(b, o), out=(n_arrays, pos)))
            layout.append((k, b, o, n, pos))
            pos += (n + 255) // 256 * 256
    return np.concatenate(out), layout, max(pos, 256)


def verify_stream(arrays: Sequence[np.ndarray], recs: np.ndarray, bursts=None, ctx=None, **init) -> dict:
    arrays = [np.ascontiguousarray(a).view(np.uint8).reshape(-1) for a in arrays]
    aug, layout, log_bytes = with_log(recs, len(arrays))
    gpu = run_gpu(list(arrays) + [np.zeros(log_bytes, np.uint8)], aug, bursts=bursts, ctx=ctx, **init)
    log = gpu[-1]
    by_rec = {}
    for (k, b, o, n, p) in layout:
        by_rec.setdefault(k, []).append((b, o, n, p))
    pool = oracle.Pool([a.copy() for a in arrays])
    worst = {}
    fails = []
    for k, r in enumerate(recs):
        # ops that read their inputs in the check (sum, sdpa, gemv) never write them
        before = list(pool.arrays)
        pool.run(r.reshape(1))
        if k not in by_rec:
            continue
        gview = [a for a in pool.arrays]  # oracle state after the op
        # build a "gpu" view: oracle state with the logged ranges substituted
        gsub = [a.copy() for a in gview]
        for (b, o, n, p) in by_rec[k]:
            gsub[b][o: o + n] = log[p: p + n]
        res = check_record(r, before, gsub, gview)
        nm = res["op"]
        worst[nm] = max(worst.get(nm, 0.0), res["worst"])
        if not res["ok"]:
            fails.append((k, res))
        # teacher forcing: adopt the GPU's bytes
        for (b, o, n, p) in by_rec[k]:
            pool.arrays[b][o: o + n] = log[p: p + n]
    # buffers written only by unlogged ops (KV caches) must match bit for bit
    logged_bufs = {b for (_, b, _, _, _) in layout}
    kv_bufs = set()
    for r in recs:
        if int(r["op"]) == W.OP_KV_APPEND:
            kv_bufs |= {int(r["buf"][W.AUX0]), int(r["buf"][W.AUX1])}
    kv_ok = all(np.array_equal(gpu[b], pool.arrays[b]) for b in kv_bufs - logged_bufs)
    return {"fails": fails, "worst": worst, "kv_ok": kv_ok, "n_logged": len(layout)}
