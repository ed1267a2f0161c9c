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


def run_gpu(arrays, recs: np.ndarray, bursts=None, flags=G.GPUOS_SUBMIT_BLOCK,
            ctx=None, download=None, **init) -> List[np.ndarray]:
    """Upload arrays (or take an already filled DevicePool), submit recs,
    sync, download the buffers listed in `download` (default: every buffer;
    uint8 arrays, None for those not downloaded)."""
    pool = arrays if isinstance(arrays, DevicePool) else DevicePool(arrays)
    descs = to_descs(recs, pool.ptrs)
    own = ctx is None
    if own:
        ctx = G.gpuos_init(**init)
    try:
        if bursts is None:
            bursts = np.full((len(descs) + 63) // 64, 64)
        ring = G.gpuos_stats_get(ctx)["ring_entries"]
        for sl in split_bursts(len(descs), np.asarray(bursts)):
            for lo in range(sl.start, sl.stop, ring):  # a burst longer than the ring goes in parts
                rc, _ = G.gpuos_submit(ctx, descs[lo:min(sl.stop, lo + ring)], flags)
                assert rc == 0, f"submit: {G.ERR_NAMES.get(rc)}"
        rc, es, st = G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, SYNC_NS)
        assert rc == 0, f"sync: {G.ERR_NAMES.get(rc)} seq={es} status={st}"
        want = range(len(pool.tensors)) if download is None else set(download)
        out = [pool.download(i) if i in want else None for i in range(len(pool.tensors))]
    finally:
        if own:
            assert G.gpuos_shutdown(ctx) == 0
    return out


EXACT_OPS = (W.OP_NOP, W.OP_ADD, W.OP_MUL, W.OP_RELU, W.OP_MAX, W.OP_MIN, W.OP_KV_APPEND, W.OP_COPY)


def _is_exact(r, inputs) -> bool:
    op = int(r["op"])
    if op == W.OP_EXPR:
        d2 = int(r["dim"][2])
        pb, po = int(r["buf"][W.AUX2]), int(r["off"][W.AUX2])
        return W.program_is_exact(inputs[pb][po: po + 4 * d2].copy().view(np.uint32))
    return op in EXACT_OPS


def capture_windows(r):
    """Output windows whose unrounded oracle values a toleranced record is
    compared against: (buffer, byte offset, bytes, element bytes)."""
    es = W.DTYPE_BYTES[int(r["dtype"]) if int(r["op"]) == W.OP_ROPE else int(r["out_dtype"])]
    return [(b, o, n, es) for (b, o, n) in W.output_ranges(r)]


def run_record_oracle(pool: "oracle.Pool", r, exact: bool):
    """Run one record on the oracle pool in place; for a toleranced record
    also return the unrounded double of each output element (one array per
    output range), else None."""
    if exact or int(r["op"]) in EXACT_OPS:
        pool.run(r.reshape(1))
        return None
    return pool.run_capture(r, capture_windows(r))


def run_oracle(arrays: Sequence[np.ndarray], recs: np.ndarray, capture: bool = False):
    """Run recs on host copies of arrays.  With capture, records run one at a
    time and the unrounded outputs of each toleranced record are returned
    too: (final arrays, [per-record list of arrays or None])."""
    p = oracle.Pool([np.array(a, copy=True) for a in arrays])
    if not capture:
        p.run(recs)
        return p.arrays
    hps = []
    for r in recs:
        hps.append(run_record_oracle(p, r, _is_exact(r, p.arrays)))
    return p.arrays, hps


def _f(buf: np.ndarray, off: int, n: int, dt: int) -> np.ndarray:
    es = W.DTYPE_BYTES[dt]
    return as_float(buf[off: off + n * es].copy(), dt)


def plain_rel(g: np.ndarray, r: np.ndarray) -> float:
    """Plain max |g - r| / |r| over the elements with |r| at least 1e-3 of the
    range's largest finite |r| and at least 2^-126 (subnormal results carry
    an absolute rounding error, not a relative one); reported beside the
    conditioned metrics."""
    a = np.abs(r)
    fin = np.isfinite(a) & np.isfinite(g)
    if not fin.any():
        return 0.0
    m = fin & (a >= max(1e-3 * a[fin].max(), 2.0 ** -126))
    if not m.any():
        return 0.0
    return float(np.max(np.abs(g[m] - r[m]) / a[m]))


def kv_rows(inputs: List[np.ndarray], r, bb: int, hk: int, L: int):
    """Key and value rows 0..L-1 of batch row bb and key/value head hk of an
    SDPA record, as float arrays [L, D], from contiguous caches or through the
    block table of paged ones; `kept` is False for keys whose page lies
    outside the pool (they take no part)."""
    d = [int(v) for v in r["dim"]]
    buf, off = r["buf"], r["off"]
    dt = int(r["dtype"])
    H, D = d[0], d[1]
    Hkv = d[3] or H
    es = W.DTYPE_BYTES[dt]
    kb, ko = inputs[int(buf[W.AUX0])], int(off[W.AUX0])
    vb, vo = inputs[int(buf[W.AUX1])], int(off[W.AUX1])
    if not int(r["flags"]) & W.FLAG_KV_PAGED:
        row = (bb * Hkv + hk) * d[2] * D * es
        return (_f(kb, ko + row, L * D, dt).reshape(L, D), _f(vb, vo + row, L * D, dt).reshape(L, D),
                np.ones(L, bool))
    PS, MP, NP = d[2], (int(r["size"]) >> 16) & 0xFFFF, int(r["size"]) >> 32
    tb, to = inputs[int(buf[W.B])], int(off[W.B])
    table = tb[to + bb * MP * 4: to + (bb + 1) * MP * 4].copy().view(np.int32).astype(np.int64)
    j = np.arange(L)
    page = table[j // PS]
    kept = (page >= 0) & (page < NP)
    start = (((np.where(kept, page, 0) * Hkv + hk) * PS + j % PS) * D * es)[:, None] + np.arange(D * es)[None, :]
    K = as_float(kb[ko + start].reshape(-1).copy(), dt).reshape(L, D)
    V = as_float(vb[vo + start].reshape(-1).copy(), dt).reshape(L, D)
    return np.where(kept[:, None], K, 0.0), np.where(kept[:, None], V, 0.0), kept


def check_outputs(r, inputs: List[np.ndarray], pairs, hp=None) -> dict:
    """Compare the outputs of one record.  inputs: the pool before it ran;
    pairs: (gpu bytes, oracle bytes) per output range in W.output_ranges
    order; hp: the oracle's unrounded values per range (toleranced records;
    run_record_oracle).  Returns a dict with 'ok', the worst ratio to the
    allowance ('worst', <= 1 passes) and the plain relative error ('plain')."""
    op = int(r["op"])
    dt, do = int(r["dtype"]), int(r["out_dtype"])
    size = int(r["size"])
    d = [int(v) for v in r["dim"]]
    buf, off = r["buf"], r["off"]
    res = {"op": W.OP_NAMES[op], "ok": True, "worst": 0.0, "plain": 0.0}
    exact = _is_exact(r, inputs)
    tol = TOL["f32"] if do == W.F32 else TOL["bf16"]
    for k, (g, rr) in enumerate(pairs):
        if exact:
            if op in (W.OP_KV_APPEND, W.OP_COPY):
                eq = g == rr
            else:
                eq = bits_equal(g.copy(), rr.copy(), do)
            if not eq.all():
                res.update(ok=False, mismatches=int((~eq).sum()))
            continue
        if op == W.OP_ROPE:
            # within one bf16 ulp (or 2^-22 relative for fp32) of the rounded
            # oracle value; the distance to the exact value is reported
            gf, rf = as_float(g.copy(), dt), as_float(rr.copy(), dt)
            if dt == W.BF16:
                ok = np.abs(gf - rf) <= ulp_bf16(rf) * 1.0001
                ok |= np.isnan(gf) & np.isnan(rf)
                worst = float(np.max(np.abs(gf - rf) / ulp_bf16(rf))) if gf.size else 0.0
                if hp is not None and gf.size:
                    res["ulps_vs_exact"] = max(res.get("ulps_vs_exact", 0.0),
                                               float(np.max(np.abs(gf - hp[k]) / ulp_bf16(hp[k]))))
            else:
                ok, worst = rel_check(gf, rf, np.maximum(np.abs(rf), 1e-30), 2.0 ** -22)
            res["worst"] = max(res["worst"], worst)
            if not np.all(ok):
                res.update(ok=False, mismatches=int((~ok).sum()))
            continue
        # toleranced ops: against the oracle's unrounded double
        assert hp is not None, "toleranced records need the oracle's unrounded outputs"
        gf, rf = as_float(g.copy(), do), hp[k]
        if op == W.OP_GELU:
            ok, worst = rel_check(gf, rf, np.maximum(np.abs(rf), 2.0 ** -126), tol)
        elif op == W.OP_SOFTMAX:
            ok, worst = rel_check(gf, rf, np.abs(rf), tol)
        elif op in (W.OP_LAYERNORM, W.OP_EXPR):
            # EXPR with exp/log/tanh/sigmoid steps: library functions within a
            # few ulps, compared on the unit scale like LayerNorm
            ok, worst = rel_check(gf, rf, np.maximum(np.abs(rf), 1.0), tol)
        elif op == W.OP_SUM:
            h = d[0]
            x = _f(inputs[int(buf[W.A])], int(off[W.A]), size * h, dt).reshape(size, h)
            ok, worst = rel_check(gf, rf, np.abs(x).sum(axis=1), tol)
        elif op == W.OP_SDPA:
            H, D = d[0], d[1]
            size = W.rec_rows(r)
            paged = bool(int(r["flags"]) & W.FLAG_KV_PAGED)
            C = ((int(r["size"]) >> 16) & 0xFFFF) * d[2] if paged else d[2]
            Hkv = d[3] or H  # grouped-query attention: kv head h // (H // Hkv)
            q = _f(inputs[int(buf[W.A])], int(off[W.A]), size * H * D, dt).reshape(size, H, D)
            denom = np.zeros((size, H, D))
            scale = float(r["fparam"][1]) or 1.0 / np.sqrt(D)
            mask = None
            if int(r["flags"]) & W.FLAG_SDPA_MASK:
                mask = _f(inputs[int(buf[W.AUX2])], int(off[W.AUX2]), size * C, W.F32).reshape(size, C)
            for bb in range(size):
                L = int(r["lens"][bb])
                for hk in range(Hkv):
                    K, V, kept = kv_rows(inputs, r, bb, hk, L)
                    hs = slice(hk * (H // Hkv), (hk + 1) * (H // Hkv))
                    s = (q[bb, hs] @ K.T) * scale
                    s[:, ~kept] = -np.inf
                    if mask is not None:
                        s = s + mask[bb, :L]
                    with np.errstate(invalid="ignore"):
                        p = np.exp(s - s.max(axis=1, keepdims=True))
                    p /= p.sum(axis=1, keepdims=True)
                    denom[bb, hs] = p @ np.abs(V)
            t = TOL["sdpa"] if do == W.F32 else TOL["bf16"]
            ok, worst = rel_check(gf, rf, denom.reshape(-1), t)
        elif op == W.OP_MATMUL:
            M_, K_, N_ = size, d[0], d[1]
            x = _f(inputs[int(buf[W.A])], int(off[W.A]), M_ * K_, dt).reshape(M_, K_)
            Wt = _f(inputs[int(buf[W.B])], int(off[W.B]), N_ * K_, dt).reshape(N_, K_)
            denom = (np.abs(x) @ np.abs(Wt).T).reshape(-1)
            t = TOL["f32"] if do == W.F32 else TOL["bf16"]
            ok, worst = rel_check(gf, rf, denom, t)
        elif op == W.OP_GEMV:
            K_, N_ = d[0], d[1]
            x = _f(inputs[int(buf[W.A])], int(off[W.A]), K_, dt)
            Wm = _f(inputs[int(buf[W.B])], int(off[W.B]), K_ * N_, dt).reshape(K_, N_)
            denom = np.abs(x) @ np.abs(Wm)
            t = TOL["f32"] if do == W.F32 else TOL["bf16"]
            ok, worst = rel_check(gf, rf, denom, t)
        else:
            raise AssertionError(op)
        res["worst"] = max(res["worst"], worst)
        res["plain"] = max(res["plain"], plain_rel(gf, rf))
        if not np.all(ok):
            res.update(ok=False, mismatches=int((~ok).sum()))
    return res


def check_record(r, inputs: List[np.ndarray], gpu: List[np.ndarray], orc: List[np.ndarray], hp=None) -> dict:
    """check_outputs with the outputs taken from whole-pool lists."""
    pairs = [(gpu[b][o: o + n], orc[b][o: o + n]) for (b, o, n) in W.output_ranges(r)]
    return check_outputs(r, inputs, pairs, hp)


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


def verify_stream(arrays, recs: np.ndarray, bursts=None, ctx=None, pool: DevicePool = None, **init) -> dict:
    """Verify mode: log every output on the GPU, replay on the oracle with
    teacher forcing.  The pool is either host arrays (uploaded) or a filled
    DevicePool (its initial contents are downloaded for the oracle first)."""
    if pool is not None:
        arrays = [pool.download(i) for i in range(len(pool.tensors))]
    arrays = [np.ascontiguousarray(a).view(np.uint8).reshape(-1) for a in arrays]
    aug, layout, log_bytes = with_log(recs, len(arrays))
    kv_bufs = set()
    for r in recs:
        if int(r["op"]) == W.OP_KV_APPEND:
            kv_bufs |= {int(r["buf"][W.AUX0]), int(r["buf"][W.AUX1])}
    if pool is None:
        pool = DevicePool(arrays)
    pool.append_zeros(log_bytes)
    gpu = run_gpu(pool, aug, bursts=bursts, ctx=ctx, download=kv_bufs | {len(arrays)}, **init)
    log = gpu[-1]
    by_rec = {}
    for (k, b, o, n, p) in layout:
        by_rec.setdefault(k, []).append((b, o, n, p))
    pool = oracle.Pool([a.copy() for a in arrays])
    worst, plain = {}, {}
    fails = []
    for k, r in enumerate(recs):
        # ops that read their inputs in the check (sum, sdpa, gemv) never
        # write them, so the pool after the op still holds those inputs
        exact = _is_exact(r, pool.arrays)
        hp = run_record_oracle(pool, r, exact)
        if k not in by_rec:
            continue
        pairs = [(log[p: p + n], pool.arrays[b][o: o + n]) for (b, o, n, p) in by_rec[k]]
        res = check_outputs(r, pool.arrays, pairs, hp)
        nm = res["op"]
        worst[nm] = max(worst.get(nm, 0.0), res["worst"])
        plain[nm] = max(plain.get(nm, 0.0), res["plain"])
        if not res["ok"]:
            fails.append((k, res))
        # teacher forcing: adopt the GPU's bytes
        for (b, o, n, p) in by_rec[k]:
            pool.arrays[b][o: o + n] = log[p: p + n]
    # buffers written only by unlogged ops (KV caches) must match bit for bit
    logged_bufs = {b for (_, b, _, _, _) in layout}
    kv_ok = all(np.array_equal(gpu[b], pool.arrays[b]) for b in kv_bufs - logged_bufs)
    return {"fails": fails, "worst": worst, "plain": plain, "kv_ok": kv_ok, "n_logged": len(layout)}
